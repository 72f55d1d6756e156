/*
 * rar.h -- C ABI of the MI355X ring AllReduce library (librar.so).
 *
 * One GPU hosts N virtual ranks.  Every rank owns a send and a receive buffer
 * in device memory; neighbouring ranks on the ring exchange data through FIFOs
 * of NCCL_STEPS (8) slots that the library owns.  One call launches one HIP
 * kernel that runs every (rank, channel) of the collective.
 *
 * Sources for the semantics (two public course pages on NCCL, and notes):
 *   [C12] "NCCL 专家课程 12：Ring AllReduce 逐步推导、真实 Ring 与 Channel 并行"
 *         (ring AllReduce step by step, real rings and channel parallelism)
 *   [C23] "NCCL 专家课程 23：Device Kernel、Primitives、Step/Credit 与 LL Flag"
 *         (device kernel, primitives, step/credit and the LL flag)
 *   [C2]  NCCL notes at cishoon.github.io/posts/ai-infra/nccl (symmetric
 *         memory, the LSA device API, the one-shot AllReduce)
 *
 * General rules
 *   - All entry points are plain C; nothing throws across the boundary.
 *   - Device pointers are HIP device addresses (hipMalloc or a framework
 *     allocator on the same device).  Host arrays of pointers are read during
 *     the call and not kept.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Calls are stream ordered and asynchronous: the caller must keep every
 *     buffer alive and unmodified until the stream has passed the call
 *     [C23 "排障树": reusing a buffer before the stream completes corrupts it].
 *   - Calls on one communicator must be issued in order on one stream.
 *   - On any error nothing is launched; rar_get_last_error() gives detail.
 *   - HIP graphs: rar_allreduce, rar_allreduce_premul and rar_group_end may
 *     be called while their stream is being captured, on a communicator made
 *     with launch_mode 1, when the launch plan fits in the 3,584 bytes that
 *     travel inside the kernel arguments (every single AllReduce up to 16
 *     channels and 8 ranks; small groups).  The captured kernel node reads
 *     the buffers named at capture time; each replay is one more launch on
 *     the communicator, stream-ordered with its other launches like an eager
 *     call.  Otherwise the capturing call fails with RAR_UNSUPPORTED before
 *     anything is enqueued.  The one-shot entry points capture as they are.
 */
#ifndef RAR_H
#define RAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Result codes.  As the pages' library reports every failure as a result
 * code (the ring builder returns an internal error with the message "ring
 * does not loop back") [C12 "Graph 如何变成完整 ring"], each entry point
 * returns one of these and never throws; the message of the last failure on
 * the calling thread is kept for rar_get_last_error(). */
typedef enum {
  RAR_SUCCESS = 0,
  RAR_INVALID_ARGUMENT = 1, /* a precondition below is violated            */
  RAR_UNSUPPORTED = 2,      /* valid request this build or device cannot run */
  RAR_HIP_ERROR = 3,        /* the HIP runtime reported an error            */
  RAR_INTERNAL_ERROR = 4,   /* a library invariant failed                   */
  RAR_ABORTED = 5           /* a previous launch hit the wait watchdog; the
                               communicator is poisoned and must be destroyed */
} rar_result_t;

/* Protocols [C23 "Simple 的 Credit 与 Step", "LL：Data 与 Flag 同 Line",
 * "LL128：15/16 Payload"]. */
typedef enum { RAR_PROTO_LL = 0, RAR_PROTO_LL128 = 1, RAR_PROTO_SIMPLE = 2 } rar_proto_t;

/* Element types.  bfloat16 partial sums are rounded to bfloat16 (nearest,
 * ties to even) after every ring hop; int32 wraps modulo 2^32. */
typedef enum { RAR_INT32 = 0, RAR_FLOAT32 = 1, RAR_BFLOAT16 = 2 } rar_dtype_t;

/* Reduction operators [C23 "RunWorkColl 与 Template Dispatch": the kernel is
 * specialised on its RedOp; C12 "源码步骤三": the owner's fused final step
 * applies the post-op].  With acc the partial from the previous rank and x
 * the rank's own input, one hop computes
 *   RAR_SUM   acc + x           RAR_PROD  acc * x (int32: low 32 bits)
 *   RAR_MAX   x if x > acc      RAR_MIN   x if x < acc   (else acc, bits kept)
 *   RAR_AVG   acc + x; the owner divides its final sum by N (int32:
 *             truncating toward zero) before writing and forwarding it.
 *   RAR_PREMULSUM  acc + s_r * x: rank r's input is first multiplied by
 *             the rank's scalar s_r and rounded to the payload type (int32:
 *             low 32 bits) where it enters the fold; only through the
 *             *_premul entry points, which take the scalars.  (The pages do
 *             not describe PreMulSum; this is the reading.)
 * Floating results round to the payload type after every hop. */
typedef enum { RAR_SUM = 0, RAR_PROD = 1, RAR_MAX = 2, RAR_MIN = 3, RAR_AVG = 4,
               RAR_PREMULSUM = 5 } rar_redop_t;

typedef struct rar_comm* rar_comm_t;

/* Performance knobs; none of them changes any result bit. */
typedef struct {
  int lanes_per_channel; /* workgroups that split each channel's slices; each
                            lane owns its own head/tail counters. 0 = auto   */
  int waves_per_lane;    /* 64-thread waves per workgroup (1..8). 0 = auto   */
  int spin_timeout_us;   /* watchdog for every device-side wait, in
                            microseconds. 0 = 10 s                        */
  int debug_flags;       /* test hooks, 0 in normal use.  Bit 0: receivers
                            never publish head credit (the pages' "drop recv
                            head" fault), so senders stall after exactly
                            NCCL_STEPS slots and the watchdog ends the launch
                            with RAR_ABORTED [C23 "状态机故障注入"].  Bit 1:
                            record a timeline (rar_comm_read_trace).  Bit 2:
                            LL flags wrap at 0x100 instead of 2^32 [C23 "LL：
                            Data 与 Flag 同 Line" test mode]; the slot
                            cleanup that makes a wrap safe then runs every
                            128 steps instead of every 2^31            */
  int launch_mode;       /* 0: cooperative launch, the runtime guarantees that
                            every workgroup is resident (or fails the launch).
                            1: plain launch, shorter gaps between launches; the
                            grid still fits the device at once (checked), but
                            residency relies on no other kernel holding CUs;
                            the watchdog turns starvation into RAR_ABORTED  */
  int placement;         /* 0: the N ranks of each (channel, lane) pipeline
                            share one XCD, so their FIFO traffic stays in one
                            L2 and a slice is published without an L2
                            write-back (checked on the device every launch;
                            a pipeline found split falls back to the
                            agent-scope release).  1: spread the ranks over
                            different XCDs (every hop crosses L2s)         */
  int slices_per_chunk;  /* Simple: slices per chunk, 1, 2 (0 = default)
                            or 4 (needs chunk_steps 4).  Each slice moves
                            StepPerSlice = chunk_steps / slices FIFO steps
                            and every call still consumes chunk_steps steps;
                            smaller slices keep fewer FIFO bytes in flight,
                            fewer slices mean fewer dependent hops for small
                            messages.  Timing only: results are identical */
  int direct;            /* Simple only, bit mask of the direct variants
                            [C23 "发布顺序与 Fence", direct read/write].
                            Bit 0, direct write: the rank that completes a
                            chunk, and every rank that forwards it, writes it
                            straight into the next rank's receive buffer
                            instead of the FIFO (no send credit needed); the
                            final receive has nothing to copy.  Bit 1, direct
                            read: the loop's opening send moves nothing and
                            the next rank's first receive reads the raw input
                            from the sender's send buffer.  Steps still
                            advance on every connector.  Same results; bytes
                            of traffic (6N-4)M, (5N-4)M with bit 0, (6N-6)M
                            with bit 1, (5N-6)M with both.  Buffers of
                            different ranks must not overlap.              */
  int deal_works;        /* 0: the lanes of a channel split the lines of
                            every step.  1: they take the channel's works
                            in turn (work k of the channel runs whole on
                            lane k mod lanes_per_channel, over that lane's
                            own FIFO, which then holds the full buff_size).
                            A fused group of many small works is bound by
                            the latency of its dependent steps, not by
                            bytes: dealing the works divides the steps each
                            workgroup runs in sequence.  Timing only    */
  int strict_scope;      /* 0: to a receiver found on this XCD (placement 0),
                            Simple tails, LL lines and LL128 flags are
                            workgroup-scope stores into the L2 both sides
                            share, which relies on this GPU's L1 being
                            write-through to that L2 rather than on the
                            formal memory model.  1: every publication takes
                            the agent-scope path whatever the placement: a
                            release (L2 write-back) before Simple tails and
                            LL128 flags, agent-scope atomic stores for LL
                            lines and flags [C23 "发布顺序与 Fence": the
                            release before publishing].  The fallback should
                            the same-L2 behaviour change; same results,
                            slower                                       */
  int waves_by_size;     /* 0: every work of a launch runs on waves_per_lane
                            waves.  1: a work runs on as many waves as its
                            per-call data fills with full passes (Simple
                            4 KiB, LL 2 KiB, LL128 1,920 payload bytes per
                            wave and pass), at least 1 and at most
                            waves_per_lane, so the small pieces of a fused
                            group use fewer waves and RunWorkBatch fences
                            each change of the active wave count with a
                            barrier [C23 "RunWorkBatch 与 Fused Work"].
                            Timing only                                  */
} rar_tuning_t;

#define RAR_DEBUG_DROP_RECV_HEAD 1
#define RAR_DEBUG_TRACE 2
#define RAR_DEBUG_LL_FLAG_WRAP8 4

/* Create a communicator: the ring, the active channels, the protocol and the
 * FIFOs for every (rank, channel).  Allocates N * popcount(mask) * buffSize
 * bytes of FIFO (rounded up per lane; lanes_per_channel times that with
 * deal_works) plus counters on the current HIP device and zeroes them.
 *
 *   nranks       2..64 virtual ranks
 *   ring_order   [nranks] user ranks listed along `next`; must be a
 *                permutation (any rotation names the same ring).  The ring
 *                index of a rank is its distance from rank 0 [C12 "ring index
 *                如何计算"; "Graph 如何变成完整 ring"].
 *   channel_mask active channels; bit c set = channel c runs.  Channels may be
 *                sparse; the n-th set bit is the n-th workgroup set
 *                [C23 "Kernel 如何把 Block 映射到 Channel"].  Must be nonzero.
 *   proto        RAR_PROTO_*.
 *   buff_size    FIFO bytes per (rank, channel); 0 = protocol default
 *                (Simple 4 MiB, LL 512 KiB, LL128 4915200).  Must be a
 *                multiple of 512 (Simple), 256 (LL) or 2048 (LL128), at most
 *                2 GiB.
 *   chunk_steps  Simple: FIFO steps per chunk, 2 or 4 (0 = 4).  A chunk of 8
 *                steps fills all slots and deadlocks the ring.  Ignored by LL
 *                and LL128, whose chunk is one step.
 *   tuning       NULL for defaults.
 * Errors: RAR_INVALID_ARGUMENT for any violation above or a NULL pointer;
 * RAR_UNSUPPORTED if the device cannot keep every workgroup resident;
 * RAR_HIP_ERROR if allocation fails. */
rar_result_t rar_comm_create(rar_comm_t* comm, int nranks, const int* ring_order,
                             uint64_t channel_mask, rar_proto_t proto, size_t buff_size,
                             int chunk_steps, const rar_tuning_t* tuning);

/* As rar_comm_create, with one ring per channel [C12 "GRAPH 重建：N=2 / N=3 /
 * N=4", "为什么 channels 会重复"]: ring_orders holds `nrings` rings of
 * `nranks` ranks each, one after the other, every one a permutation.
 * Channel id c runs ring (c mod nrings), so the base rings repeat over the
 * channels that follow them (with the six rings of four ranks and 12
 * channels, channels 6-11 run the rings of channels 0-5).  A channel's ring
 * sets both its neighbours and the order its elements are summed in, so the
 * result bits depend on it.  rar_comm_create(..., ring_order, ...) is
 * nrings = 1.
 * Errors: as rar_comm_create; RAR_INVALID_ARGUMENT if nrings is outside
 * [1, 64] or any ring is not a permutation (the message names the ring). */
rar_result_t rar_comm_create_rings(rar_comm_t* comm, int nranks, int nrings,
                                   const int* ring_orders, uint64_t channel_mask,
                                   rar_proto_t proto, size_t buff_size, int chunk_steps,
                                   const rar_tuning_t* tuning);

/* AllReduce of `count` elements over all virtual ranks [C12; C23 "Ring
 * AllReduce 到 Primitive"]: afterwards every recvbufs[r][i] holds the
 * reduction `op` over ranks of sendbufs[r][i], folded in ring order (the rank
 * after the chunk's owner starts, the owner combines last), identical on
 * every rank.
 *   sendbufs, recvbufs  host arrays of `nranks` device pointers, each aligned
 *                       to its element size (4 bytes for int32 and float32, 2
 *                       for bfloat16); 16-byte alignment is not needed
 *                       [C23 "LL128：15/16 Payload" stages misaligned user
 *                       data; here the hardware's unaligned vector accesses
 *                       serve it].  recvbufs[r] == sendbufs[r] runs in place;
 *                       no other two of the 2N buffers may overlap (checked
 *                       on the host: RAR_INVALID_ARGUMENT, nothing queued).
 *   count               elements per rank; 0 launches nothing, leaves the
 *                       FIFO steps untouched and does not look at the pointers.
 * Inside rar_group_start/rar_group_end the call is queued instead of launched.
 * Errors: RAR_INVALID_ARGUMENT (NULL or misaligned pointer, bad enum),
 * RAR_UNSUPPORTED (a group mixing dtypes or operators; under stream capture,
 * a cooperative communicator or a plan too large to travel inline),
 * RAR_ABORTED (poisoned communicator), RAR_HIP_ERROR (launch failed). */
rar_result_t rar_allreduce(rar_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                           size_t count, rar_dtype_t dtype, rar_redop_t op, void* stream);

/* As rar_allreduce with RAR_PREMULSUM: scalars is a host array of `nranks`
 * elements of `dtype` (bfloat16 as its 16-bit pattern), copied at call time;
 * rank r's input is scaled by scalars[r].  Inside a group every call brings
 * its own scalars.  Errors: as rar_allreduce; RAR_INVALID_ARGUMENT if
 * scalars is NULL (count 0 aside). */
rar_result_t rar_allreduce_premul(rar_comm_t comm, const void* const* sendbufs,
                                  void* const* recvbufs, size_t count, rar_dtype_t dtype,
                                  const void* scalars, void* stream);

/* Fused works [C23 "RunWorkBatch 与 Fused Work"]: AllReduces queued between
 * start and end run as one launch; their elements are laid end to end and cut
 * into one contiguous range per channel, each channel executing its pieces in
 * call order from work batches staged in LDS.  All queued calls must share
 * one dtype.  The pointer arrays are copied when queued.  Errors as above;
 * rar_group_end with nothing queued is a no-op. */
rar_result_t rar_group_start(rar_comm_t comm);
rar_result_t rar_group_end(rar_comm_t comm, void* stream);
/* Close an open group without launching it: the queued calls are dropped
 * and nothing reaches the device or the FIFO steps.  For callers whose
 * queueing failed halfway (the pages' group brackets [C2 "1 communicator":
 * ncclGroupStart/End around the per-rank calls] leave no half-built group
 * behind).  A communicator without an open group is left as it is. */
rar_result_t rar_group_discard(rar_comm_t comm);

/* Release the communicator's FIFOs, counters and launch-plan memory.  The
 * pages' clean-up order ends with destroying the communicator, after the
 * collectives that use it and the buffers they touch are done with
 * [C2 "4 User Buffer Registration", the ncclCommDestroy step]: destroy after
 * the stream has passed the last call, and after every HIP
 * graph that captured a launch on this communicator has been destroyed or
 * will not be replayed again (a replay would use freed memory).  NULL is a
 * no-op. */
rar_result_t rar_comm_destroy(rar_comm_t comm);

/* The collective call with its communicator set-up folded in: the
 * single-process set-up that builds one communicator for all ranks at once
 * [C2 "1 communicator": ncclCommInitAll] followed by the stream-ordered
 * AllReduce call (send and receive buffers, count, type, operator, stream)
 * [C2 "2 CUDA stream": ncclAllReduce(d_in, d_out, count, ncclFloat, ncclSum,
 * comm, stream)], with the ring, protocol, channels, buffer size and chunk
 * steps as arguments instead of tuner choices.  It creates (and caches, keyed
 * by every argument that shapes the FIFOs) a communicator on first use, then
 * runs rar_allreduce.  The mask is the nchannels lowest bits.  Creation
 * allocates and initialises device memory, which a stream capture does not
 * allow: make the first call with a given shape outside any capture.  The
 * cached communicators use the cooperative launch, so under capture this
 * entry point fails with RAR_UNSUPPORTED.  Buffers are checked before
 * anything touches the device: NULL, misaligned or overlapping buffers of
 * different ranks give RAR_INVALID_ARGUMENT.  A cached communicator may be
 * used from several threads and streams: calls on it are serialised by a
 * lock, and a call on another stream than the previous one first makes its
 * stream wait for the previous launch (hipStreamWaitEvent), since both
 * share one set of FIFOs and step counters.  Errors as for rar_comm_create
 * and rar_allreduce. */
rar_result_t ring_allreduce(const void* const* sendbufs, void* const* recvbufs, int nranks,
                            size_t count, rar_dtype_t dtype, rar_redop_t op,
                            const int* ring_order, rar_proto_t proto, int nchannels,
                            size_t buff_size, int chunk_steps, void* stream);

/* Destroy every communicator that ring_allreduce has cached, on every
 * device: the clean-up step that ends the pages' communicator life cycle,
 * after the collectives that used it are done [C2 "4 User Buffer
 * Registration", the ncclCommDestroy step].  Each one's last launch is waited
 * for (hipEventSynchronize on the event ring_allreduce records after it)
 * before its FIFOs, counters and plan memory are freed; the next
 * ring_allreduce of that shape builds a fresh communicator.  Use it to give
 * the device memory back (a 64 MiB Simple shape at 12 channels holds 192 MiB
 * of FIFOs), or after ring_allreduce returned RAR_ABORTED: a communicator
 * whose launch hit the wait watchdog refuses every later call until it is
 * destroyed.  Must not run while another thread is inside ring_allreduce,
 * nor while a HIP graph that captured a ring_allreduce launch may still be
 * replayed (the replay would use freed memory).  With nothing cached it
 * touches no device.  RAR_HIP_ERROR if a wait or a free fails (the
 * communicators not yet freed stay cached). */
rar_result_t ring_allreduce_cache_release(void);

/* For callers that cannot allocate device memory (code that runs under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * ring_allreduce with the same arguments and the same results, bit for bit,
 * that keeps no communicator.  Its device state (FIFOs, step counters, abort
 * words, workgroup map, ring table) lives in one static device array of
 * 64 MiB per GPU, which the library holds from its first use on that GPU
 * until the process ends.  Each call lays the state out afresh (a small
 * set-up kernel clears what must start at zero, then the ring kernel runs),
 * so no call depends on an earlier one; the call makes no hipMalloc,
 * hipFree or memset and copies nothing to the device.  Shapes whose state
 * exceeds 64 MiB (N * nchannels * buff_size for the FIFOs, plus under 1 MiB)
 * fail with RAR_INVALID_ARGUMENT, and a launch plan larger than the 3,584
 * bytes that travel inside the kernel arguments with RAR_UNSUPPORTED.
 * Every call on one GPU shares that GPU's array: calls that can overlap in
 * time on one GPU (other streams, other threads) race and corrupt each
 * other; issue them in order on one stream.  A cooperative launch, or a
 * plain one while the stream is being captured (the grid fits the device at
 * once, checked).  The wait watchdog still bounds every wait, but with no
 * host-mapped word it cannot report an abort: the call's outputs are then
 * undefined.  Errors as for ring_allreduce. */
rar_result_t ring_allreduce_noalloc(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                    size_t count, rar_dtype_t dtype, rar_redop_t op,
                                    const int* ring_order, rar_proto_t proto, int nchannels,
                                    size_t buff_size, int chunk_steps, void* stream);

/* One-shot AllReduce [C2 "5 Symmetric Memory", "6.1 LSA": with every rank's
 * buffer reachable by plain loads, one kernel finishes the reduction in one
 * hop instead of the ring's 2(N-1)].  Afterwards every recvbufs[r][i] holds
 * the fold of sendbufs[0..N-1][i] with `op` in user-rank order (rank 0
 * first): fp32 rounded per operation, bf16 accumulated in fp32 and rounded to
 * nearest-even bf16 once, int32 wrapping; RAR_AVG divides the sum by N at the
 * end; identical on every rank.  Each element is folded once
 * and stored to all N receive buffers, so the launch reads N*count and writes
 * N*count elements.  Needs no communicator and allocates nothing; one kernel
 * launch on `stream`, stream-ordered.
 *   sendbufs, recvbufs  host arrays of `nranks` (2..64) device pointers, each
 *                       aligned to its element size, copied at call time.  recvbufs[r] ==
 *                       sendbufs[r] runs in place; no other two buffers may
 *                       overlap (checked).
 *   count               elements per rank; 0 launches nothing and does not
 *                       look at the pointers.
 *   tuning              NULL for defaults; launch shape only, no result bit
 *                       depends on it.
 * Errors: RAR_INVALID_ARGUMENT for a bad count of ranks, dtype, tuning, NULL
 * or misaligned or overlapping buffers, an unknown op; RAR_HIP_ERROR if the
 * launch fails. */
typedef struct {
  int32_t workgroups; /* 0 = auto (enough for one pass, at most 2048)            */
  int32_t waves;      /* waves per workgroup, 0 = auto (4), at most 8            */
  int32_t unroll;     /* 16-byte vectors in flight per thread and input:
                         0 = auto (2), 1, 2 or 4                               */
  int32_t pad;
} rar_oneshot_tuning_t;

rar_result_t rar_oneshot_allreduce(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                   size_t count, rar_dtype_t dtype, rar_redop_t op,
                                   const rar_oneshot_tuning_t* tuning, void* stream);

/* As rar_oneshot_allreduce with RAR_PREMULSUM: scalars is a host array of
 * `nranks` elements of `dtype`; each input is scaled by its rank's scalar in
 * the fp32 (int32) accumulator, then summed in rank order. */
rar_result_t rar_oneshot_allreduce_premul(const void* const* sendbufs, void* const* recvbufs,
                                          int nranks, size_t count, rar_dtype_t dtype,
                                          const void* scalars, const rar_oneshot_tuning_t* tuning,
                                          void* stream);

/* Watchdog status: RAR_ABORTED if a launch on this communicator timed out in
 * a wait, else RAR_SUCCESS.  Does not synchronize; reflects launches the
 * device has finished. */
rar_result_t rar_comm_get_async_error(rar_comm_t comm);

/* Hang triage [C23 "排障树"]: synchronizes the device, then writes for every
 * connector lane (receiving rank r, dense channel n, lane p) two values at
 * out[((r*C+n)*P+p)*2]: tail (producer step; for LL/LL128 only updated at the
 * end of a launch) and head (consumer step).  `cap` is the number of int64
 * slots available; *written receives the number used. */
rar_result_t rar_comm_query_state(rar_comm_t comm, int64_t* out, size_t cap, size_t* written);

/* Timeline of the last launch, recorded when tuning.debug_flags has
 * RAR_DEBUG_TRACE: one record per Simple slice or LL/LL128 step of every
 * workgroup, at most 4096 per workgroup.  Times are 100 MHz ticks of the
 * device clock.  Synchronizes the device.  op: 0 send, 1 recvReduceSend,
 * 2 recvReduceCopySend, 3 recvCopySend, 4 recv [C12 steps one to five]. */
typedef struct {
  int32_t rank, channel_id, lane, op;
  int32_t chunk;         /* ring-position chunk index of the call          */
  uint32_t nelem;        /* elements of the unit over all lanes            */
  uint64_t t_begin;      /* start of the unit's wait                       */
  uint32_t wait_ticks;   /* until the workgroup passed its wait             */
  uint32_t data_ticks;   /* moving data until the workgroup's last barrier  */
  uint64_t recv_step;    /* receive step at the start of the unit (low bits)*/
  int32_t waves;         /* waves that moved the unit's data (its work's)   */
  int32_t pad;
} rar_trace_rec_t;
rar_result_t rar_comm_read_trace(rar_comm_t comm, rar_trace_rec_t* out, size_t cap,
                                 size_t* written);

/* Geometry of a communicator: active channels C, lanes per channel P, waves
 * per lane W, workgroups in the grid G (including idle padding). */
rar_result_t rar_comm_shape(rar_comm_t comm, int* nchannels, int* lanes, int* waves, int* grid);

/* The communicator's rings as GRAPH lines, each followed by that channel's
 * geometry [C12 "Graph 如何变成完整 ring": the ring a channel runs is
 * recomputed from the connector graph; "GRAPH 重建：N=2 / N=3 / N=4": one
 * line per channel].  For every active channel, in channel id order:
 *   "Channel cc/CC : r0 r1 ... r(N-1)\n"   as rar_graph_text, then
 *   "  lanes P, waves W, FIFO B B per connection, S B per lane and step,
 *    XCD per lane: x ...\n"
 * where x is the XCD of the lane's workgroups, or x0/x1/... (rank order)
 * when its ranks run on different XCDs.  Text and sizes as rar_graph_text.
 * RAR_INVALID_ARGUMENT: comm NULL, or buf too small (only *len set). */
rar_result_t rar_comm_graph_text(rar_comm_t comm, char* buf, size_t cap, size_t* len);

/* ---- host planner, exposed for testing (no device needed) ------------------ */

/* Ring index, prev and next of every user rank, as rar_comm_create computes
 * them.  Errors: RAR_INVALID_ARGUMENT if ring_order is not a permutation. */
rar_result_t rar_ring_info(int nranks, const int* ring_order, int* index, int* prev, int* next);

/* GRAPH lines of a ring layout, without a communicator [C12 "Graph 如何变成完整
 * ring": each ring is rebuilt from the connector graph by walking next from
 * rank 0 N times, which must return to rank 0 having met every rank once;
 * C12 "GRAPH 重建：N=2 / N=3 / N=4" for the lines].  One line per set bit c
 * of channel_mask, in increasing c:
 *   "Channel cc/CC : r0 r1 ... r(N-1)\n"
 * with cc = c and CC = the highest set bit + 1 (two digits each), and the
 * ring channel c runs (ring c mod nrings of ring_orders, nrings rows of
 * nranks ints, as rar_comm_create_rings) listed from rank 0 along next.
 * The text goes to buf with a terminating NUL; *len (may be NULL) receives
 * its length without the NUL.  buf NULL with cap 0 only reports the length.
 * RAR_INVALID_ARGUMENT: nranks outside [2, 64], nrings outside [1, 64],
 * NULL ring_orders, an empty mask, a ring that is not a permutation of the
 * ranks (its walk would not loop back), or a buf too small (only *len set). */
rar_result_t rar_graph_text(int nranks, int nrings, const int* ring_orders, uint64_t channel_mask,
                            char* buf, size_t cap, size_t* len);

typedef struct {
  int32_t channel;    /* dense channel index n                        */
  int32_t channel_id; /* n-th set bit of the mask                     */
  int32_t work;       /* position of the collective in the launch     */
  int32_t pad;
  int64_t grid_offset;   /* first element of the piece in that collective */
  int64_t channel_count; /* elements of the piece                         */
  int64_t chunk_count;   /* protocol maximum chunk, in elements           */
} rar_piece_t;

/* The channel split of a launch of `nworks` collectives of `counts[i]`
 * elements.  Writes at most `cap` pieces, returns the total in *npieces and
 * the protocol's chunk maximum (elements) in *chunk_max (may be NULL).
 * RAR_INVALID_ARGUMENT for a bad shape or dtype, nworks < 1, NULL counts or
 * npieces, a negative cap, or NULL pieces with cap > 0. */
rar_result_t rar_plan_pieces(int nranks, uint64_t channel_mask, rar_proto_t proto,
                             size_t buff_size, int chunk_steps, rar_dtype_t dtype, int nworks,
                             const size_t* counts, rar_piece_t* pieces, int cap, int* npieces,
                             int64_t* chunk_max);

/* Name of a result code, and the message of the last failing call on the
 * calling thread (empty if the last call succeeded), as the pages' ring
 * builder pairs its result code with a warning that says what failed
 * [C12 "Graph 如何变成完整 ring"].  Both return static or thread-local
 * storage owned by the library: valid until the thread's next call. */
const char* rar_get_error_string(rar_result_t r);
const char* rar_get_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* RAR_H */
