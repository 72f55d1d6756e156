/*
 * ring_sim.h -- CPU oracle for the N-rank ring AllReduce state machine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or execute this code: only the test suite, the smoke check of the
 * package entry module and the CPU-baseline leg of the benchmark use it.  It
 * shares no code, header, table or constant with the HIP implementation.
 *
 * What it models (sources are two public course pages on NCCL):
 *   [C12] "NCCL 专家课程 12：Ring AllReduce 逐步推导、真实 Ring 与 Channel 并行"
 *         (Ring AllReduce step by step, real rings and channel parallelism)
 *   [C23] "NCCL 专家课程 23：Device Kernel、Primitives、Step/Credit 与 LL Flag"
 *         (Device kernel, primitives, step/credit and the LL flag)
 *
 * Every function is plain, sequential and slow on purpose.  All values are
 * handled as raw bytes; arithmetic on floating payloads is done in binary64
 * and rounded to the payload type after every hop.
 */
#ifndef RING_SIM_H
#define RING_SIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Protocol / datatype codes used by this oracle (its own numbering). */
enum { ORC_PROTO_LL = 0, ORC_PROTO_LL128 = 1, ORC_PROTO_SIMPLE = 2 };
enum { ORC_INT32 = 0, ORC_FLOAT32 = 1, ORC_BFLOAT16 = 2 };

/* Primitive kinds of one ring loop [C12 "源码步骤一..五"; C23 "Ring AllReduce 到 Primitive"]. */
enum {
  ORC_OP_SEND = 0,                  /* send own input chunk                          */
  ORC_OP_RECV_REDUCE_SEND = 1,      /* recv partial, add own input, forward         */
  ORC_OP_RECV_REDUCE_COPY_SEND = 2, /* final add, write output, forward (fused)     */
  ORC_OP_RECV_COPY_SEND = 3,        /* recv final chunk, write output, forward      */
  ORC_OP_RECV = 4                   /* recv final chunk, write output               */
};

/* Options of orc_allreduce (bit flags). */
enum {
  ORC_OPT_DROP_RECV_HEAD = 1, /* fault hook: receivers never publish head           */
  ORC_OPT_DIRECT = 2,         /* Simple only: the all-gather half writes straight into
                                 the next rank's receive buffer instead of its FIFO
                                 [C23 "发布顺序与 Fence", direct read/write]        */
  ORC_OPT_LL_WRAP8 = 4,       /* LL flags wrap at 0x100 (test mode) instead of 2^32 */
  ORC_OPT_DIRECT_READ = 16,   /* Simple only: the first receive of every loop reads the
                                 previous rank's send buffer in place, and the loop's
                                 opening send moves no data [C23 "发布顺序与 Fence",
                                 direct read/write]                                   */
  ORC_OPT_RED_SHIFT = 8       /* bits 8..11: the reduction operator, ORC_RED_*     */
};

/* Reduction operators [C23 "RunWorkColl 与 Template Dispatch": the kernel is
 * specialised on a RedOp; C12 "源码步骤三": the fused final step applies the
 * post-op].  acc is the partial received from the previous rank, x the
 * rank's own input:
 *   SUM  acc + x                  PROD  acc * x
 *   MAX  x if x > acc, else acc   MIN   x if x < acc, else acc
 *   AVG  acc + x at every hop; the owner's final value is divided by N
 *        (the post-op) before it is written and forwarded.
 * Floating results round to the payload type after every operation; int32
 * wraps modulo 2^32 and AVG divides the wrapped signed sum, truncating. */
enum { ORC_RED_SUM = 0, ORC_RED_PROD = 1, ORC_RED_MAX = 2, ORC_RED_MIN = 3, ORC_RED_AVG = 4,
       ORC_RED_PREMULSUM = 5 };

/* Return codes. */
enum { ORC_OK = 0, ORC_DEADLOCK = 1, ORC_INVALID = 2, ORC_CORRUPT = 3 };

/* Ring set-up [C12 "ring index 如何计算", "Graph 如何变成完整 ring"].
 * ring_order lists user ranks along the `next` direction.  Outputs are indexed
 * by user rank.  Returns ORC_INVALID when ring_order is not a permutation. */
int orc_ring_setup(int nranks, const int* ring_order, int* index, int* prev, int* next);

/* The 2N-1 primitive calls of one loop for the rank at ring index `ring_index`
 * [C12 "Schedule 生成器的断言"].  ops/chunks must hold 2N-1 entries.
 * Chunks are in ring-position coordinates. */
int orc_ring_schedule(int nranks, int ring_index, int* ops, int* chunks);

/* Geometry of one launch.  For each active channel (dense index 0..C-1) the
 * pieces (work, gridOffset, channelCount, chunkCount) in execution order.
 * Returns the number of pieces written (<= max_pieces) or -1 on bad input.
 * chunk_max_out receives the per-protocol maximum chunk in elements. */
typedef struct {
  int32_t channel;     /* dense channel index n                          */
  int32_t channel_id;  /* n-th set bit of the mask                       */
  int32_t work;        /* index of the collective in the group           */
  int32_t pad;
  int64_t grid_offset; /* element offset inside that collective's buffer */
  int64_t channel_count;
  int64_t chunk_count;
} orc_piece;

int orc_geometry(int nranks, uint64_t channel_mask, int proto, size_t buff_size, int chunk_steps,
                 int dtype, int nworks, const size_t* counts, orc_piece* pieces, int max_pieces,
                 int64_t* chunk_max_out);

/* One recorded primitive call (for schedule/geometry checks). */
typedef struct {
  int32_t rank, channel_id, work, op;
  int32_t chunk, loop;
  int64_t offset, nelem;
} orc_call;

typedef struct {
  int64_t send_ops[64];       /* per user rank: primitive calls that send    */
  int64_t recv_ops[64];       /* per user rank: primitive calls that receive */
  int64_t payload_sent[64];   /* per user rank: payload bytes sent           */
  int64_t wire_sent[64];      /* per user rank: FIFO bytes written (lines);
                                 direct sends write none                    */
  int64_t units_run;          /* slices / steps executed in total            */
  int64_t calls_recorded;     /* entries written to the call log             */
  int32_t deadlock_rank, deadlock_channel;
  int64_t deadlock_send_step, deadlock_recv_step;
} orc_stats;

/* Run the whole collective (or fused group of collectives sharing one dtype).
 *   sendbufs / recvbufs : [nworks * nranks] host pointers, index work*nranks+rank
 *                          (a recv pointer equal to the send pointer = in place)
 *   slots               : FIFO slots per connector (NCCL_STEPS, normally 8)
 *   sched               : 0 = round robin, each agent runs until it blocks
 *                          1 = seeded random choice of agent, one unit at a time
 *                          2 = channel-parallel: channels share no connector or
 *                              output element, so `seed` threads (0 = the
 *                              hardware's count, at most one per channel) run
 *                              whole channels, each with the round-robin
 *                              schedule; call_log must be NULL
 *   options             : ORC_OPT_* bits
 *   call_log            : optional, records every primitive call (may be NULL)
 */
int orc_allreduce(int nranks, const int* ring_order, uint64_t channel_mask, int proto,
                  size_t buff_size, int chunk_steps, int dtype, int nworks, const size_t* counts,
                  const void* const* sendbufs, void* const* recvbufs, int slots, int sched,
                  uint64_t seed, int options, orc_stats* stats, orc_call* call_log,
                  int64_t call_log_cap);

/* Same, with one ring per channel [C12 "GRAPH 重建", "为什么 channels 会重复"]:
 * ring_orders holds nrings rings of nranks ranks each; channel id c runs ring
 * c mod nrings (the base rings duplicated onto the following channels). */
int orc_allreduce_rings(int nranks, int nrings, const int* ring_orders, uint64_t channel_mask,
                        int proto, size_t buff_size, int chunk_steps, int dtype, int nworks,
                        const size_t* counts, const void* const* sendbufs, void* const* recvbufs,
                        int slots, int sched, uint64_t seed, int options, orc_stats* stats,
                        orc_call* call_log, int64_t call_log_cap);

/* Single-connector fault model [C23 "状态机故障注入"]: a producer streams
 * `nsteps` tagged steps through one connector of `slots` slots while a
 * consumer drains it.  Faults:
 *   0 none
 *   1 drop_recv_head        (Simple)  consumer never publishes head
 *   2 tail_before_payload   (Simple)  producer publishes tail before payload
 *   3 ll_flag2_missing      (LL)      second flag of each line never written
 *   4 ll_constant_flag      (LL)      flag is a constant instead of step+1
 *   5 ll128_flag_missing    (LL128)   flag word never written
 *   6 ll128_flag_before_data(LL128)   flag word written before the data words
 * Outcome: ORC_OK (all steps delivered intact), ORC_DEADLOCK (neither side can
 * move), ORC_CORRUPT (consumer accepted data that is not the step's payload).
 * *steps_done = steps the producer completed; *consumed = steps the consumer
 * accepted; *bad_step = first corrupted step (or -1). */
int orc_stream_fault(int proto, int fault, int slots, int nsteps, int64_t* steps_done,
                     int64_t* consumed, int64_t* bad_step);

/* PreMulSum (READING: the pages do not describe it): as orc_allreduce_rings
 * with the sum, where every rank's own input is first multiplied by that
 * rank's scalar and rounded to the payload type (int32: low 32 bits) at the
 * point it enters the fold -- the loop's opening send, recvReduceSend, the
 * fused final step, and (direct read) the raw input read from the previous
 * rank's send buffer, which takes the previous rank's scalar.
 *   scalars  [nworks * nranks] elements of the payload type (raw bytes), index
 *            work*nranks + rank.
 * The options' operator bits are ignored. */
int orc_allreduce_premul(int nranks, int nrings, const int* ring_orders, uint64_t channel_mask,
                         int proto, size_t buff_size, int chunk_steps, int dtype, int nworks,
                         const size_t* counts, const void* const* sendbufs, void* const* recvbufs,
                         const void* scalars, int slots, int sched, uint64_t seed, int options,
                         orc_stats* stats, orc_call* call_log, int64_t call_log_cap);

/* LL flag generations on one connector [C23 "LL：Data 与 Flag 同 Line": a test
 * mode makes the flag wrap at 0x100; at cleanup steps the sender writes the
 * rest of the slot with the current generation].  A producer streams `nsteps`
 * steps; step k carries lines_of[k mod nsizes] lines (1..cap) into slot
 * k mod slots, which holds `cap` lines and starts zeroed.  Line flags are
 * (k+1) mod 2^flag_bits (flag_bits 8 or 32).  With `cleanup`, the last
 * `slots` steps of each half of the flag period also stamp lines [n, cap) of
 * their slot with their flag.  The consumer is eager: it takes each line of
 * its step as soon as both flags equal its generation -- possibly before the
 * producer has written that line -- and checks the payload; the producer
 * writes one line at a time and waits for head credit per step.
 * Returns ORC_OK, ORC_CORRUPT (*bad_step = first step that took a stale line)
 * or ORC_INVALID. */
int orc_ll_wrap(int flag_bits, int cleanup, int slots, int cap, int nsizes, const int* lines_of,
                int nsteps, int64_t* bad_step);

/* Round a binary64 value to bfloat16 (round to nearest, ties to even,
 * subnormals kept, overflow to infinity).  Exposed for pinning. */
uint16_t orc_bf16_round(double v);

#ifdef __cplusplus
}
#endif
#endif
