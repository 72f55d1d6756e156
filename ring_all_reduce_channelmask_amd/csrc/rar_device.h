// rar_device.h -- layouts shared by the host planner and the gfx950 kernel.
//
// Everything the kernel reads lives in device memory in the structures below.
// Sizes are fixed and 16-byte multiples so that one wave can copy them into
// LDS in 16-byte packs.
#pragma once

#include <stdint.h>

namespace rar {

constexpr int kSteps = 8;            // NCCL_STEPS: FIFO slots per connector
constexpr int kSlicesPerChunk = 2;   // Simple default: slices per chunk (StepPerSlice = chunkSteps/2)
constexpr int kMaxRanks = 64;
constexpr int kMaxChannels = 64;     // channelMask is 64 bits
constexpr int kMaxLanes = 16;
constexpr int kMaxWaves = 8;         // 512 threads: keeps the kernel free of register spills
constexpr int kWaveSize = 64;
constexpr int kBatchWorks = 16;      // 16 works x 64 B = a 1024-byte batch
constexpr uint32_t kIdleWg = 0xFFFFFFFFu;

enum Proto : int32_t { kLL = 0, kLL128 = 1, kSimple = 2 };
enum Dtype : int32_t { kInt32 = 0, kFloat32 = 1, kBFloat16 = 2 };
enum Red : int32_t { kRedSum = 0, kRedProd = 1, kRedMax = 2, kRedMin = 3, kRedAvg = 4, kRedPreMulSum = 5 };
constexpr int kNumRed = 6;

// Arguments of the one-shot kernel (by value: at most 64 ranks' pointers).
struct OneshotArgs {
  const void* src[kMaxRanks];  // send buffer of every rank
  void* dst[kMaxRanks];        // receive buffer of every rank
  int64_t nvec;                // whole 16-byte vectors per rank
  int64_t vec_per_block;       // contiguous vectors folded by one workgroup
  int32_t nranks;
  int32_t tail;                // elements after the last whole vector
  uint32_t scalar[kMaxRanks];  // PreMulSum: each rank's scalar bits (bf16 in the low half)
};

// One (collective, channel) piece: what ncclDevWorkColl carries for runRing.
struct alignas(16) DevWork {
  int64_t grid_offset;    // first element of the piece in its collective
  int64_t channel_count;  // elements of the piece
  int64_t chunk_count;    // protocol maximum chunk (elements); the tail loop shrinks it
  uint32_t buf_index;     // collective index into the pointer table
  uint16_t n_waves;       // waves that move data for this work
  uint16_t flags;
  uint32_t pad[6];
};
static_assert(sizeof(DevWork) == 64, "DevWork must be 64 bytes");

// Header of a work batch: works are the set bits of offset_bitset, counted
// from offset_base in the work array.  next_jump chains the next batch of
// the same channel (0 = end of the chain; batch 0 is a sentinel).
struct alignas(16) DevBatch {
  uint32_t next_jump;
  uint32_t offset_base;
  uint64_t offset_bitset;
};
static_assert(sizeof(DevBatch) == 16, "DevBatch must be 16 bytes");

// Head/tail counters of one connector lane, each on its own 128-byte line.
struct alignas(128) Counter {
  uint64_t value;
  uint64_t pad[15];
};
struct ConnCounters {
  Counter tail;  // producer progress, written by the sending lane of prev(r)
  Counter head;  // consumer progress, written by the receiving lane of r
};
static_assert(sizeof(ConnCounters) == 256, "counter layout");

// One traced primitive unit (a Simple slice or an LL/LL128 step), written by
// thread 0 of a workgroup when tracing is on.  Times are s_memrealtime ticks
// (100 MHz).
struct alignas(16) TraceRec {
  uint64_t t_begin;     // before the unit's wait
  uint32_t wait_ticks;  // waiting for tail / credit (until the first barrier)
  uint32_t data_ticks;  // moving data, line polls included, until the last barrier
  uint32_t recv_step;   // low bits of the receive step at the unit
  uint16_t op, chunk;
  uint32_t nelem;       // elements of the unit (all lanes together)
  uint32_t waves;       // waves that moved data for the unit's work
};
static_assert(sizeof(TraceRec) == 32, "trace record layout");

// Per-rank ring position, as setupChannel computes it.
struct alignas(16) DevRank {
  int32_t index;  // ring distance from rank 0
  int32_t prev;
  int32_t next;
  int32_t pad;
};

// Communicator hot fields (copied into LDS by one wave at kernel entry).
struct alignas(16) DevCommHot {
  int32_t n_ranks;
  int32_t n_channels;   // popcount(mask)
  int32_t n_lanes;      // workgroups per (rank, channel)
  int32_t proto;
  int64_t buff_size;    // FIFO bytes per (rank, channel) as requested
  int64_t step_bytes;   // buff_size / kSteps: one slot of the channel
  int64_t lane_step_bytes;  // one slot of one lane's own FIFO (>= step_bytes / n_lanes)
  int64_t lane_buff_bytes;  // kSteps * lane_step_bytes
  int32_t chunk_steps;  // Simple
  int32_t step_per_slice;      // Simple: chunk_steps / slices_per_chunk
  int32_t slices_per_chunk;    // Simple: 2 (default), 1 or 4; timing only
  int32_t direct;              // Simple: direct all-gather (next rank's receive buffer)
  uint64_t channel_mask;
  uint8_t* fifo;               // lane FIFO of (r, n, p) at ((r * C + n) * P + p) * lane_buff_bytes
  ConnCounters* counters;      // ((r * C + n) * P + p)
  uint32_t* abort_flag;        // device word, nonzero = stop
  uint32_t* abort_host;        // host-mapped word, mirrors abort_flag for the host
  uint64_t spin_timeout_ticks; // s_memrealtime ticks (100 MHz)
  int32_t debug_flags;         // bit 0: receivers never publish head (fault test)
                               // bit 1: record a TraceRec per unit
  int32_t trace_cap;           // records per workgroup
  TraceRec* trace;             // [grid][trace_cap]
  uint32_t* trace_count;       // [grid] records written by the last launch
  uint64_t* placement;         // [grid] launch count << 8 | XCC id, written at kernel entry
  const uint32_t* wg_peer;     // [grid] -> workgroup that receives from this one
  uint32_t ll_flag_mask;       // LL flag period - 1 (0xFFFFFFFF, or 0xFF in the wrap test mode)
  int32_t deal_works;          // 1: work k of a channel runs whole on lane k mod n_lanes
  int32_t strict_scope;        // 1: publish at agent scope with the release even to a
                               // receiver on this XCD (the placement check is ignored)
  int32_t pad_hot[3];
};
static_assert(sizeof(DevCommHot) % 16 == 0, "hot fields are copied in 16-byte packs");

// ranks[c][r]: rank r's place on the ring that channel id c runs.  With
// several base rings, channel id c runs ring c mod nrings, so the rings repeat
// over the channels that follow them.
struct alignas(16) DevComm {
  DevCommHot hot;
  DevRank ranks[kMaxChannels][kMaxRanks];
};

// The workgroup map in closed form.  The dispatcher hands block g to XCD
// g mod 8, so the map puts the N ranks of one (channel, lane) pipeline on one
// XCD: XCD x takes pipelines q = x, x + 8, x + 16, ... (q = n * lanes + lane),
// and its k-th workgroup is rank k mod N of pipeline x + 8 * (k / N).  Slots
// past the last pipeline stay idle.  The host planner builds the map from
// these, and the no-alloc entry point builds it on the device.
__host__ __device__ inline uint32_t wg_grid_size(int nranks, int pipes) {
  return 8u * (uint32_t)nranks * (uint32_t)((pipes + 7) / 8);
}
__host__ __device__ inline uint32_t wg_entry(uint32_t g, int nranks, int n_lanes, int pipes) {
  const uint32_t x = g % 8u, k = g / 8u;
  const uint32_t q = x + 8u * (k / (uint32_t)nranks), r = k % (uint32_t)nranks;
  if (q >= (uint32_t)pipes) return 0xFFFFFFFFu;
  return r | ((q / (uint32_t)n_lanes) << 8) | ((q % (uint32_t)n_lanes) << 16);
}
// The workgroup of rank `rank` in the pipeline of workgroup g.
__host__ __device__ inline uint32_t wg_of_rank(uint32_t g, int nranks, int rank) {
  const uint32_t x = g % 8u, k = g / 8u;
  return ((k / (uint32_t)nranks) * (uint32_t)nranks + (uint32_t)rank) * 8u + x;
}

// Bytes of launch plan that travel inside the kernel arguments.  A plan that
// fits (every single collective up to 16 channels and 8 ranks, small groups)
// needs no upload before the launch, and a captured launch stays valid for
// every replay of its graph.
constexpr int kInlinePlanBytes = 3584;

// Kernel arguments (by value).  The launch plan is one block of bytes, either
// `plan` below (inline_plan = 1) or device memory at `arena`; the offsets
// locate its tables inside it:
//   batches      DevBatch[]  (batch 0 is a sentinel)
//   works        DevWork[]
//   ptrs         void*[(buf_index * N + rank) * 2 + {0 send, 1 recv}]
//   first_batch  uint32[64]  first batch of each channel id (0 = none)
//   scalars      uint32[buf_index * N + rank]  PreMulSum scalar bits (bf16 in the low half)
struct alignas(16) KernelArgs {
  const DevComm* comm;
  const uint32_t* wg_map;  // [grid] rank | n << 8 | lane << 16, or kIdleWg
  const uint8_t* arena;    // the plan in device memory when it is not inline
  uint32_t off_batches, off_works, off_ptrs, off_first, off_scalars;
  uint32_t inline_plan;
  alignas(16) uint8_t plan[kInlinePlanBytes];
};
static_assert(sizeof(KernelArgs) <= 4096, "kernel arguments are limited to 4 KiB");

}  // namespace rar
