// noalloc.hip -- ring_allreduce_noalloc: ring_allreduce for callers that
// cannot allocate device memory.
//
// ring_allreduce keeps a communicator per shape, whose FIFOs, step counters,
// workgroup map and abort words it allocates on first use.  Here the same
// state lives in one static device array per GPU, `scratch`, which the
// library holds from the moment it is loaded on a device until the process
// ends.  Every call lays its state out from the start of the array again:
// a small set-up kernel writes the communicator fields, the ring table and
// the workgroup map, and zeroes the step counters, the abort words and the
// placement slots (and, for LL and LL128, whose lines carry their step in
// flags, the FIFO bytes the call uses); then the ring kernel runs on that
// state with the launch plan inside its arguments.  No hipMalloc, hipFree,
// hipMemset or copy: two kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "capi_internal.h"

namespace {

// 64 MiB: the FIFOs of, e.g., 4 ranks x 4 channels at the 512 KiB LL buffer
// (8 MiB), 4 ranks x 12 channels at a 1 MiB Simple buffer (48 MiB), or 8
// ranks x 16 channels at a 256 KiB Simple buffer (32 MiB), plus the rest of
// the state (under 1 MiB for those shapes).
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
// `scratch` as seen from the host is a stand-in for the array, not its
// device address: the address is looked up once per device, with that device
// current, and only this pointer reaches kernels.
uint8_t* g_scratch_ptr[kMaxDevices] = {};

rar_result_t scratch_for(int dev, uint8_t** out) {
  if (dev < 0 || dev >= kMaxDevices) return rar::set_error(RAR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return rar::set_error(RAR_HIP_ERROR, std::string("hipGetSymbolAddress(scratch) failed: ") +
                                               hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return RAR_SUCCESS;
}

// What the set-up kernel writes; read through the kernel-argument segment
// (the ring tables are indexed by thread, which a by-value copy would move
// to private memory).
struct SetupArgs {
  rar::DevCommHot hot;          // communicator fields, pointers into the array
  rar::DevComm* comm;
  uint8_t* counters;            // counter_bytes, zeroed
  int64_t counter_bytes;
  uint8_t* abort_words;         // 256 bytes, zeroed
  uint64_t* placement;          // [grid], zeroed
  uint32_t* wg_map;             // [grid]
  uint32_t* wg_peer;            // [grid]
  uint8_t* fifo;                // fifo_zero_bytes from here are zeroed
  int64_t fifo_zero_bytes;
  int32_t grid, nranks, n_channels, n_lanes;
  int32_t index[rar::kMaxRanks], prev[rar::kMaxRanks], next[rar::kMaxRanks];
};

__global__ void __launch_bounds__(256) noalloc_setup_kernel(SetupArgs) {
  const SetupArgs& a = *(const SetupArgs*)__builtin_amdgcn_kernarg_segment_ptr();
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  const uint4 zero = {0, 0, 0, 0};
  if (tid == 0) a.comm->hot = a.hot;
  // ring table: every active channel runs the one ring (channel ids 0..C-1)
  for (int64_t i = tid; i < (int64_t)a.n_channels * a.nranks; i += nthr) {
    const int n = (int)(i / a.nranks), r = (int)(i % a.nranks);
    rar::DevRank d;
    d.index = a.index[r];
    d.prev = a.prev[r];
    d.next = a.next[r];
    d.pad = 0;
    a.comm->ranks[n][r] = d;
  }
  for (int64_t i = tid; i < a.counter_bytes / 16; i += nthr) reinterpret_cast<uint4*>(a.counters)[i] = zero;
  for (int64_t i = tid; i < 256 / 16; i += nthr) reinterpret_cast<uint4*>(a.abort_words)[i] = zero;
  const int pipes = a.n_channels * a.n_lanes;
  for (int64_t g = tid; g < a.grid; g += nthr) {
    const uint32_t m = rar::wg_entry((uint32_t)g, a.nranks, a.n_lanes, pipes);
    a.placement[g] = 0;
    a.wg_map[g] = m;
    a.wg_peer[g] = m == rar::kIdleWg ? (uint32_t)g : rar::wg_of_rank((uint32_t)g, a.nranks, a.next[m & 0xFFu]);
  }
  for (int64_t i = tid; i < a.fifo_zero_bytes / 16; i += nthr) reinterpret_cast<uint4*>(a.fifo)[i] = zero;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace

extern "C" rar_result_t ring_allreduce_noalloc(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                               size_t count, rar_dtype_t dtype, rar_redop_t op,
                                               const int* ring_order, rar_proto_t proto, int nchannels,
                                               size_t buff_size, int chunk_steps, void* stream) {
  rar::clear_error();
  uint64_t mask = 0;
  rar::RingInfo ring;
  if (rar_result_t r = rar::check_ring_call(sendbufs, recvbufs, nranks, count, dtype, op, ring_order, proto,
                                            nchannels, &buff_size, &chunk_steps, &mask, &ring))
    return r;
  if (count == 0) return RAR_SUCCESS;  // nothing to move: no launch
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
#define NA_HIP(expr)                                                                                 \
  do {                                                                                               \
    const hipError_t e_ = (expr);                                                                    \
    if (e_ != hipSuccess)                                                                            \
      return rar::set_error(RAR_HIP_ERROR, std::string(#expr) + " failed: " + hipGetErrorString(e_)); \
  } while (0)
  int dev = 0, cus = 0;
  NA_HIP(hipGetDevice(&dev));
  NA_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));

  // The shape ring_allreduce's communicator takes with default tuning, so
  // both entry points run the same kernel on the same geometry.
  const int C = nchannels;
  const int P = rar::auto_lanes(nranks, C, cus);
  const int W = (int)proto == rar::kLL ? 4 : 8;
  const int pipes = C * P;
  const int64_t grid = rar::wg_grid_size(nranks, pipes);
  const int64_t lane_step = rar::lane_step_bytes(proto, buff_size, P);
  const size_t lanes_total = (size_t)nranks * C * P;
  const size_t fifo_bytes = lanes_total * rar::kSteps * (size_t)lane_step;

  // Layout of the array: communicator, counters, abort words, placement,
  // workgroup map and receivers, FIFOs; every table 256-byte aligned.
  const size_t off_comm = 0;
  const size_t off_counters = align_up(off_comm + sizeof(rar::DevComm), 256);
  const size_t off_abort = align_up(off_counters + lanes_total * sizeof(rar::ConnCounters), 256);
  const size_t off_placement = align_up(off_abort + 256, 256);
  const size_t off_wgmap = align_up(off_placement + (size_t)grid * sizeof(uint64_t), 256);
  const size_t off_wgpeer = align_up(off_wgmap + (size_t)grid * sizeof(uint32_t), 256);
  const size_t off_fifo = align_up(off_wgpeer + (size_t)grid * sizeof(uint32_t), 256);
  const size_t need = off_fifo + fifo_bytes;
  if (need > kScratchBytes)
    return rar::set_error(RAR_INVALID_ARGUMENT,
                          "this shape needs " + std::to_string(need) + " bytes of device state; the no-alloc "
                          "entry point has " + std::to_string(kScratchBytes) +
                          " (lower buff_size, nchannels or nranks, or use ring_allreduce)");

  // The launch plan travels inside the kernel arguments: nothing to upload.
  rar::QueuedCall q;
  for (int r = 0; r < nranks; ++r) q.send.push_back(const_cast<void*>(sendbufs[r]));
  q.recv.assign(recvbufs, recvbufs + nranks);
  q.count = count;
  q.dtype = dtype;
  q.red = op;
  std::vector<rar::QueuedCall> calls;
  calls.push_back(std::move(q));
  const rar::PlanBlock pb = rar::build_plan_block(calls, nranks, mask, proto, buff_size, chunk_steps, C, W);
  if (pb.bytes.empty()) return RAR_SUCCESS;
  if (pb.bytes.size() > (size_t)rar::kInlinePlanBytes)
    return rar::set_error(RAR_UNSUPPORTED, "the launch plan of " + std::to_string(pb.bytes.size()) +
                                               " bytes exceeds the " + std::to_string(rar::kInlinePlanBytes) +
                                               " bytes that travel inside the kernel arguments; use fewer "
                                               "channels or ranks, or ring_allreduce");

  const void* fn = rar::get_kernel(dtype, proto, op);
  if (!fn) return rar::set_error(RAR_INTERNAL_ERROR, "no kernel for this dtype/protocol/operator");
  // every workgroup must be resident at once: the ranks wait on each other
  int per_cu = 0;
  NA_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, W * rar::kWaveSize, 0));
  if ((int64_t)per_cu * cus < grid)
    return rar::set_error(RAR_UNSUPPORTED, "grid of " + std::to_string(grid) +
                                               " workgroups cannot be co-resident; use fewer channels or ranks");

  uint8_t* base = nullptr;
  if (rar_result_t r = scratch_for(dev, &base)) return r;

  SetupArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  rar::DevCommHot& h = sa.hot;
  h.n_ranks = nranks;
  h.n_channels = C;
  h.n_lanes = P;
  h.proto = proto;
  h.buff_size = (int64_t)buff_size;
  h.step_bytes = (int64_t)buff_size / rar::kSteps;
  h.lane_step_bytes = lane_step;
  h.lane_buff_bytes = lane_step * rar::kSteps;
  h.chunk_steps = chunk_steps;
  h.slices_per_chunk = rar::kSlicesPerChunk;
  h.step_per_slice = (int)proto == rar::kSimple ? chunk_steps / rar::kSlicesPerChunk : 1;
  h.direct = 0;
  h.deal_works = 0;
  h.channel_mask = mask;
  h.fifo = base + off_fifo;
  h.counters = reinterpret_cast<rar::ConnCounters*>(base + off_counters);
  // no host-mapped word can exist without an allocation: the watchdog's
  // mirror is a second device word
  h.abort_flag = reinterpret_cast<uint32_t*>(base + off_abort);
  h.abort_host = reinterpret_cast<uint32_t*>(base + off_abort + 128);
  h.spin_timeout_ticks = 10000000ull * 100ull;  // 10 s of the 100 MHz clock
  h.debug_flags = 0;
  h.trace_cap = 0;
  h.trace = nullptr;
  h.trace_count = nullptr;
  h.placement = reinterpret_cast<uint64_t*>(base + off_placement);
  h.wg_peer = reinterpret_cast<const uint32_t*>(base + off_wgpeer);
  h.ll_flag_mask = 0xFFFFFFFFu;
  sa.comm = reinterpret_cast<rar::DevComm*>(base + off_comm);
  sa.counters = base + off_counters;
  sa.counter_bytes = (int64_t)(lanes_total * sizeof(rar::ConnCounters));
  sa.abort_words = base + off_abort;
  sa.placement = reinterpret_cast<uint64_t*>(base + off_placement);
  sa.wg_map = reinterpret_cast<uint32_t*>(base + off_wgmap);
  sa.wg_peer = reinterpret_cast<uint32_t*>(base + off_wgpeer);
  sa.fifo = base + off_fifo;
  // LL and LL128 lines carry their step in flags, and every call starts its
  // steps from 0 again: lines a previous call left behind must not match
  sa.fifo_zero_bytes = (int)proto == rar::kSimple ? 0 : (int64_t)fifo_bytes;
  sa.grid = (int32_t)grid;
  sa.nranks = nranks;
  sa.n_channels = C;
  sa.n_lanes = P;
  for (int r = 0; r < nranks; ++r) {
    sa.index[r] = ring.index[r];
    sa.prev[r] = ring.prev[r];
    sa.next[r] = ring.next[r];
  }
  const int64_t setup_work = std::max<int64_t>({sa.fifo_zero_bytes / 16, sa.counter_bytes / 16, grid,
                                                (int64_t)C * nranks});
  const unsigned setup_blocks = (unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, (setup_work + 255) / 256));
  void* sparams[] = {&sa};
  NA_HIP(hipLaunchKernel(reinterpret_cast<const void*>(noalloc_setup_kernel), dim3(setup_blocks), dim3(256),
                         sparams, 0, hs));

  rar::KernelArgs args;
  std::memset(&args, 0, offsetof(rar::KernelArgs, plan));
  args.comm = sa.comm;
  args.wg_map = sa.wg_map;
  args.arena = nullptr;
  args.off_batches = pb.off_batches;
  args.off_works = pb.off_works;
  args.off_ptrs = pb.off_ptrs;
  args.off_first = pb.off_first;
  args.off_scalars = pb.off_scalars;
  args.inline_plan = 1;
  std::memcpy(args.plan, pb.bytes.data(), pb.bytes.size());
  void* params[] = {&args};
  // A cooperative launch, as ring_allreduce's communicators use; under
  // stream capture, where a cooperative launch cannot be recorded, a plain
  // one (the grid fits the device at once, checked above).
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  NA_HIP(hipStreamIsCapturing(hs, &capture));
  if (capture == hipStreamCaptureStatusNone)
    NA_HIP(hipLaunchCooperativeKernel(fn, dim3((unsigned)grid), dim3(W * rar::kWaveSize), params, 0, hs));
  else
    NA_HIP(hipLaunchKernel(fn, dim3((unsigned)grid), dim3(W * rar::kWaveSize), params, 0, hs));
#undef NA_HIP
  return RAR_SUCCESS;
}
