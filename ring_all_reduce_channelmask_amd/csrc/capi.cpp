// capi.cpp -- the C ABI declared in include/rar.h.
//
// A communicator owns, on one HIP device: the FIFOs of every (rank, channel),
// the head/tail counters of every connector lane, the abort words, the
// workgroup map and placement table, and an arena for launch plans too large
// to travel inside the kernel arguments (work batches, works, buffer
// pointers, scalars).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "capi_internal.h"

namespace rar {
const void* get_ring_kernel_i32(int proto, int red);
const void* get_ring_kernel_f32(int proto, int red);
const void* get_ring_kernel_bf16(int proto, int red);
const void* get_oneshot_kernel(int dtype, int red, int unroll);

// The ring kernel for (payload type, protocol, reduction operator).
const void* get_kernel(int dtype, int proto, int red) {
  switch (dtype) {
    case kInt32: return get_ring_kernel_i32(proto, red);
    case kFloat32: return get_ring_kernel_f32(proto, red);
    case kBFloat16: return get_ring_kernel_bf16(proto, red);
  }
  return nullptr;
}
}  // namespace rar

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace rar {
rar_result_t set_error(rar_result_t r, const std::string& msg) {
  g_last_error = msg;
  return r;
}
void clear_error() { g_last_error.clear(); }
}  // namespace rar

namespace {

using rar::QueuedCall;
using rar::check_dtype;
using rar::check_op;
using rar::check_rank_buffers;
rar_result_t fail(rar_result_t r, const std::string& msg) { return rar::set_error(r, msg); }

// Copy a text result out: *len (if given) gets its length without the NUL;
// with buf NULL and cap 0 the call only reports the length.
rar_result_t put_text(const std::string& text, char* buf, size_t cap, size_t* len) {
  if (len) *len = text.size();
  if (!buf && cap == 0) return RAR_SUCCESS;
  if (!buf || cap < text.size() + 1)
    return fail(RAR_INVALID_ARGUMENT, "text buffer holds " + std::to_string(cap) + " bytes, " +
                                          std::to_string(text.size() + 1) + " needed");
  std::memcpy(buf, text.c_str(), text.size() + 1);
  return RAR_SUCCESS;
}

#define RAR_HIP(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess)                                                                  \
      return fail(RAR_HIP_ERROR, std::string(#expr) + " failed: " + hipGetErrorString(e_)); \
  } while (0)

// Scalar bits of rank r from a host array of payload-type elements.
uint32_t scalar_bits(const void* scalars, int dtype, int r) {
  if (dtype == RAR_BFLOAT16) return reinterpret_cast<const uint16_t*>(scalars)[r];
  return reinterpret_cast<const uint32_t*>(scalars)[r];
}

}  // namespace

struct rar_comm {
  int device = 0;
  int nranks = 0;
  std::vector<int> order;             // nrings * nranks, ring after ring
  int nrings = 1;
  uint64_t mask = 0;
  int C = 0, P = 0, W = 0, grid = 0;
  int proto = 0;
  size_t buff = 0;
  int chunk_steps = 4;
  uint64_t timeout_ticks = 0;
  rar::DevComm* d_comm = nullptr;
  uint8_t* d_fifo = nullptr;
  rar::ConnCounters* d_counters = nullptr;
  uint32_t* d_abort = nullptr;
  uint32_t* h_abort = nullptr;
  uint32_t* d_abort_host = nullptr;
  uint32_t* d_wgmap = nullptr;
  std::vector<uint32_t> wgmap;
  int launch_mode = 0;
  int debug_flags = 0;
  rar::WaveSizing sizing;  // per-work wave counts (waves_by_size)
  rar::TraceRec* d_trace = nullptr;
  uint64_t* d_placement = nullptr;
  uint32_t* d_wg_peer = nullptr;
  uint32_t* d_trace_count = nullptr;
  uint8_t* d_arena = nullptr;
  size_t arena_cap = 0;
  uint8_t* h_stage = nullptr;
  size_t stage_cap = 0;
  std::vector<uint8_t> last_upload;
  // The launch plan of the previous launch and the calls it was built for
  // (count, dtype, operator, pointers, scalars of each): a launch that
  // repeats them reuses the plan instead of splitting, encoding and laying
  // it out again.
  std::vector<uint64_t> plan_key;
  rar::PlanBlock plan_cached;
  hipEvent_t upload_done = nullptr;
  bool upload_pending = false;
  bool in_group = false;
  std::vector<QueuedCall> queue;
  // ring_allreduce's cached communicators: callers may reach one from
  // several threads and streams, so its calls are serialised here, and a
  // call on a new stream waits for the previous launch (last_done).
  std::mutex call_mu;
  hipEvent_t last_done = nullptr;
  hipStream_t last_stream = nullptr;
  bool has_last = false;
};

namespace rar {

rar_result_t check_dtype(int dtype) {
  if (dtype != RAR_INT32 && dtype != RAR_FLOAT32 && dtype != RAR_BFLOAT16)
    return set_error(RAR_INVALID_ARGUMENT, "unknown dtype");
  return RAR_SUCCESS;
}

rar_result_t check_op(int op) {
  if (op < RAR_SUM || op > RAR_AVG) {
    if (op == RAR_PREMULSUM)
      return set_error(RAR_INVALID_ARGUMENT, "RAR_PREMULSUM needs scalars: use the *_premul entry point");
    return set_error(RAR_INVALID_ARGUMENT, "unknown reduction operator");
  }
  return RAR_SUCCESS;
}

// Buffers of one collective: none NULL, each aligned to its element size,
// and no two of the 2N buffers overlapping, except that a rank's receive
// buffer may be its own send buffer (in place).  The direct variants write
// into the next rank's receive buffer and read the previous rank's send
// buffer, so an overlap between ranks would corrupt an input before it is
// read.  Host-side only: no device call.
rar_result_t check_rank_buffers(int nranks, const void* const* sendbufs, void* const* recvbufs,
                                size_t count, int dtype) {
  if (!sendbufs || !recvbufs) return set_error(RAR_INVALID_ARGUMENT, "sendbufs/recvbufs is NULL");
  const size_t es = (size_t)rar::elem_size(dtype);
  if (count > (SIZE_MAX / 2) / es) return set_error(RAR_INVALID_ARGUMENT, "count too large");
  const uintptr_t bytes = count * es;
  std::vector<std::pair<uintptr_t, int>> ranges;
  ranges.reserve(2 * (size_t)nranks);
  for (int r = 0; r < nranks; ++r) {
    if (!sendbufs[r] || !recvbufs[r])
      return set_error(RAR_INVALID_ARGUMENT, "buffer of rank " + std::to_string(r) + " is NULL");
    const uintptr_t s = reinterpret_cast<uintptr_t>(sendbufs[r]);
    const uintptr_t d = reinterpret_cast<uintptr_t>(recvbufs[r]);
    if ((s | d) & (es - 1))
      return set_error(RAR_INVALID_ARGUMENT,
                  "buffer of rank " + std::to_string(r) + " is not aligned to its element size");
    ranges.push_back({s, r});
    if (d != s) ranges.push_back({d, r});
  }
  // sorted by start: two ranges overlap iff a start lies inside its predecessor
  std::sort(ranges.begin(), ranges.end());
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].first - ranges[i - 1].first < bytes)
      return set_error(RAR_INVALID_ARGUMENT, "buffers of ranks " + std::to_string(ranges[i - 1].second) + " and " +
                                            std::to_string(ranges[i].second) + " overlap");
  return RAR_SUCCESS;
}


PlanBlock build_plan_block(const std::vector<QueuedCall>& calls, int nranks, uint64_t mask, int proto,
                           size_t buff, int chunk_steps, int n_channels, int n_waves,
                           const WaveSizing& sizing) {
  PlanBlock out;
  const int64_t es = elem_size(calls.front().dtype);
  std::vector<size_t> counts;
  for (const QueuedCall& q : calls) counts.push_back(q.count);
  const std::vector<Piece> pieces = split_channels(mask, proto, buff, chunk_steps, es, counts);
  if (pieces.empty()) return out;  // nothing to move
  WaveSizing sz = sizing;
  sz.es = es;  // the launch's payload type
  const BatchPlan plan = encode_batches(pieces, n_channels, n_waves, sz);
  auto align_to = [](size_t v, size_t a) { return (v + a - 1) / a * a; };
  const size_t off_batches = 0;
  const size_t off_works = align_to(off_batches + plan.batches.size() * sizeof(DevBatch), 64);
  const size_t off_ptrs = align_to(off_works + plan.works.size() * sizeof(DevWork), 64);
  const size_t nptrs = calls.size() * (size_t)nranks * 2;
  const size_t off_scalars = align_to(off_ptrs + nptrs * sizeof(void*), 64);
  const size_t nscalars = calls.size() * (size_t)nranks;
  const size_t off_first = align_to(off_scalars + nscalars * sizeof(uint32_t), 64);
  const size_t total = align_to(off_first + plan.first_batch.size() * sizeof(uint32_t), 64);
  out.bytes.assign(total, 0);
  uint8_t* b = out.bytes.data();
  std::memcpy(b + off_batches, plan.batches.data(), plan.batches.size() * sizeof(DevBatch));
  std::memcpy(b + off_works, plan.works.data(), plan.works.size() * sizeof(DevWork));
  void** ptrs = reinterpret_cast<void**>(b + off_ptrs);
  for (size_t w = 0; w < calls.size(); ++w)
    for (int r = 0; r < nranks; ++r) {
      ptrs[(w * nranks + r) * 2] = calls[w].send[r];
      ptrs[(w * nranks + r) * 2 + 1] = calls[w].recv[r];
    }
  uint32_t* scal = reinterpret_cast<uint32_t*>(b + off_scalars);
  for (size_t w = 0; w < calls.size(); ++w)
    for (int r = 0; r < nranks && !calls[w].scalars.empty(); ++r) scal[w * nranks + r] = calls[w].scalars[r];
  std::memcpy(b + off_first, plan.first_batch.data(), plan.first_batch.size() * sizeof(uint32_t));
  out.off_batches = (uint32_t)off_batches;
  out.off_works = (uint32_t)off_works;
  out.off_ptrs = (uint32_t)off_ptrs;
  out.off_scalars = (uint32_t)off_scalars;
  out.off_first = (uint32_t)off_first;
  return out;
}

rar_result_t check_ring_call(const void* const* sendbufs, void* const* recvbufs, int nranks,
                             size_t count, int dtype, int op, const int* ring_order, int proto,
                             int nchannels, size_t* buff_size, int* chunk_steps, uint64_t* mask,
                             RingInfo* ring) {
  if (nchannels < 1 || nchannels > 64) return set_error(RAR_INVALID_ARGUMENT, "nchannels must be in [1, 64]");
  if (nranks < 2 || nranks > 64 || !ring_order)
    return set_error(RAR_INVALID_ARGUMENT, "nranks must be in [2, 64] with a ring_order");
  *mask = nchannels == 64 ? ~0ull : ((1ull << nchannels) - 1);
  if (*buff_size == 0) *buff_size = default_buff_size(proto);
  if (*chunk_steps == 0) *chunk_steps = 4;
  std::string err;
  if (!check_shape(nranks, *mask, proto, *buff_size, *chunk_steps, &err))
    return set_error(RAR_INVALID_ARGUMENT, err);
  if (!build_ring(nranks, ring_order, ring, &err)) return set_error(RAR_INVALID_ARGUMENT, err);
  if (rar_result_t r = check_dtype(dtype)) return r;
  if (rar_result_t r = check_op(op)) return r;
  if (count == 0) return RAR_SUCCESS;  // the pointers are not looked at
  if (count > (size_t(1) << 40)) return set_error(RAR_INVALID_ARGUMENT, "count too large");
  return check_rank_buffers(nranks, sendbufs, recvbufs, count, dtype);
}

}  // namespace rar

namespace {

void release(rar_comm* c) {
  if (!c) return;
  if (c->upload_done) (void)hipEventDestroy(c->upload_done);
  if (c->last_done) (void)hipEventDestroy(c->last_done);
  if (c->h_stage) (void)hipHostFree(c->h_stage);
  if (c->h_abort) (void)hipHostFree(c->h_abort);
  (void)hipFree(c->d_arena);
  (void)hipFree(c->d_trace);
  (void)hipFree(c->d_placement);
  (void)hipFree(c->d_wg_peer);
  (void)hipFree(c->d_trace_count);
  (void)hipFree(c->d_wgmap);
  (void)hipFree(c->d_abort);
  (void)hipFree(c->d_counters);
  (void)hipFree(c->d_fifo);
  (void)hipFree(c->d_comm);
  delete c;
}

// Copy the launch description into the device arena (skipped when it is
// byte-identical to the previous launch's) and launch the kernel.
// Everything a launch plan depends on besides the communicator's shape.
void plan_key(const std::vector<QueuedCall>& calls, std::vector<uint64_t>* key) {
  key->clear();
  key->push_back(calls.size());
  key->push_back((uint64_t)calls.front().dtype << 32 | (uint32_t)calls.front().red);
  for (const QueuedCall& q : calls) {
    key->push_back(q.count);
    key->push_back(q.scalars.size());
    for (uint32_t v : q.scalars) key->push_back(v);
    for (void* p : q.send) key->push_back(reinterpret_cast<uintptr_t>(p));
    for (void* p : q.recv) key->push_back(reinterpret_cast<uintptr_t>(p));
  }
}

rar_result_t launch(rar_comm* c, const std::vector<QueuedCall>& calls, hipStream_t stream) {
  const int dtype = calls.front().dtype;
  std::vector<uint64_t> key;
  plan_key(calls, &key);
  if (key != c->plan_key) {
    c->plan_cached = rar::build_plan_block(calls, c->nranks, c->mask, c->proto, c->buff, c->chunk_steps, c->C,
                                           c->W, c->sizing);
    c->plan_key.swap(key);
  }
  const rar::PlanBlock& pb = c->plan_cached;
  if (pb.bytes.empty()) return RAR_SUCCESS;  // nothing to move: no launch, no step advance
  if (__atomic_load_n(c->h_abort, __ATOMIC_ACQUIRE))
    return fail(RAR_ABORTED, "a previous launch on this communicator hit the wait watchdog");
  const std::vector<uint8_t>& bytes = pb.bytes;
  const size_t total = bytes.size();

  rar::KernelArgs args;
  std::memset(&args, 0, offsetof(rar::KernelArgs, plan));
  args.comm = c->d_comm;
  args.wg_map = c->d_wgmap;
  args.off_batches = pb.off_batches;
  args.off_works = pb.off_works;
  args.off_ptrs = pb.off_ptrs;
  args.off_first = pb.off_first;
  args.off_scalars = pb.off_scalars;
  // Under stream capture the launch becomes a graph node whose arguments are
  // copied at capture time: the plan must travel inline, and the launch must
  // be a plain one.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  RAR_HIP(hipStreamIsCapturing(stream, &capture));
  const bool capturing = capture != hipStreamCaptureStatusNone;
  if (capturing && c->launch_mode == 0)
    return fail(RAR_UNSUPPORTED, "a cooperative launch cannot be captured: use launch_mode 1");
  if (total <= (size_t)rar::kInlinePlanBytes) {
    args.inline_plan = 1;
    std::memcpy(args.plan, bytes.data(), total);
  } else if (capturing) {
    return fail(RAR_UNSUPPORTED, "a launch plan of " + std::to_string(total) +
                                     " bytes exceeds the " + std::to_string(rar::kInlinePlanBytes) +
                                     " bytes a captured launch carries inline");
  } else if (bytes != c->last_upload) {
    if (total > c->arena_cap) {
      RAR_HIP(hipDeviceSynchronize());  // the old arena may still be read by a running launch
      (void)hipFree(c->d_arena);
      c->d_arena = nullptr;
      c->arena_cap = 0;
      RAR_HIP(hipMalloc(&c->d_arena, total * 2));
      c->arena_cap = total * 2;
      c->last_upload.clear();
    }
    if (c->upload_pending) RAR_HIP(hipEventSynchronize(c->upload_done));
    c->upload_pending = false;
    if (total > c->stage_cap) {
      if (c->h_stage) RAR_HIP(hipHostFree(c->h_stage));
      c->h_stage = nullptr;
      c->stage_cap = 0;
      RAR_HIP(hipHostMalloc(reinterpret_cast<void**>(&c->h_stage), total * 2, hipHostMallocDefault));
      c->stage_cap = total * 2;
    }
    std::memcpy(c->h_stage, bytes.data(), total);
    RAR_HIP(hipMemcpyAsync(c->d_arena, c->h_stage, total, hipMemcpyHostToDevice, stream));
    RAR_HIP(hipEventRecord(c->upload_done, stream));
    c->upload_pending = true;
    c->last_upload = bytes;
  }

  if (!args.inline_plan) args.arena = c->d_arena;
  void* params[] = {&args};
  const void* fn = rar::get_kernel(dtype, c->proto, calls.front().red);
  if (!fn) return fail(RAR_INTERNAL_ERROR, "no kernel for this dtype/protocol/operator");
  if (c->launch_mode == 0)
    RAR_HIP(hipLaunchCooperativeKernel(fn, dim3(c->grid), dim3(c->W * rar::kWaveSize), params, 0, stream));
  else
    RAR_HIP(hipLaunchKernel(fn, dim3(c->grid), dim3(c->W * rar::kWaveSize), params, 0, stream));
  return RAR_SUCCESS;
}

std::mutex g_cache_mu;
std::map<std::vector<int64_t>, rar_comm*> g_cache;

}  // namespace

extern "C" {

const char* rar_get_error_string(rar_result_t r) {
  switch (r) {
    case RAR_SUCCESS: return "success";
    case RAR_INVALID_ARGUMENT: return "invalid argument";
    case RAR_UNSUPPORTED: return "unsupported";
    case RAR_HIP_ERROR: return "HIP runtime error";
    case RAR_INTERNAL_ERROR: return "internal error";
    case RAR_ABORTED: return "aborted by the wait watchdog";
  }
  return "unknown result code";
}

const char* rar_get_last_error(void) { return g_last_error.c_str(); }

rar_result_t rar_ring_info(int nranks, const int* ring_order, int* index, int* prev, int* next) {
  g_last_error.clear();
  rar::RingInfo ring;
  std::string err;
  if (!rar::build_ring(nranks, ring_order, &ring, &err)) return fail(RAR_INVALID_ARGUMENT, err);
  for (int r = 0; r < nranks; ++r) {
    if (index) index[r] = ring.index[r];
    if (prev) prev[r] = ring.prev[r];
    if (next) next[r] = ring.next[r];
  }
  return RAR_SUCCESS;
}

rar_result_t rar_plan_pieces(int nranks, uint64_t channel_mask, rar_proto_t proto, size_t buff_size,
                             int chunk_steps, rar_dtype_t dtype, int nworks, const size_t* counts,
                             rar_piece_t* pieces, int cap, int* npieces, int64_t* chunk_max) {
  g_last_error.clear();
  if (buff_size == 0) buff_size = rar::default_buff_size(proto);
  if (chunk_steps == 0) chunk_steps = 4;
  std::string err;
  if (!rar::check_shape(nranks, channel_mask, proto, buff_size, chunk_steps, &err))
    return fail(RAR_INVALID_ARGUMENT, err);
  if (rar_result_t r = check_dtype(dtype)) return r;
  if (nworks < 1 || !counts || !npieces) return fail(RAR_INVALID_ARGUMENT, "bad work list");
  if (cap < 0 || (cap > 0 && !pieces)) return fail(RAR_INVALID_ARGUMENT, "bad piece buffer");
  std::vector<size_t> cv(counts, counts + nworks);
  const int64_t es = rar::elem_size(dtype);
  const std::vector<rar::Piece> ps = rar::split_channels(channel_mask, proto, buff_size, chunk_steps, es, cv);
  *npieces = (int)ps.size();
  if (chunk_max) *chunk_max = rar::chunk_max_elems(proto, buff_size, chunk_steps, es);
  for (int i = 0; i < (int)ps.size() && i < cap; ++i) {
    pieces[i].channel = ps[i].channel;
    pieces[i].channel_id = ps[i].channel_id;
    pieces[i].work = ps[i].work;
    pieces[i].pad = 0;
    pieces[i].grid_offset = ps[i].grid_offset;
    pieces[i].channel_count = ps[i].channel_count;
    pieces[i].chunk_count = ps[i].chunk_count;
  }
  return RAR_SUCCESS;
}

rar_result_t rar_comm_create(rar_comm_t* out, int nranks, const int* ring_order, uint64_t channel_mask,
                             rar_proto_t proto, size_t buff_size, int chunk_steps,
                             const rar_tuning_t* tuning) {
  return rar_comm_create_rings(out, nranks, 1, ring_order, channel_mask, proto, buff_size, chunk_steps,
                               tuning);
}

rar_result_t rar_comm_create_rings(rar_comm_t* out, int nranks, int nrings, const int* ring_orders,
                                   uint64_t channel_mask, rar_proto_t proto, size_t buff_size,
                                   int chunk_steps, const rar_tuning_t* tuning) {
  g_last_error.clear();
  if (!out) return fail(RAR_INVALID_ARGUMENT, "comm is NULL");
  *out = nullptr;
  if (buff_size == 0) buff_size = rar::default_buff_size(proto);
  if (chunk_steps == 0) chunk_steps = 4;
  std::string err;
  if (!rar::check_shape(nranks, channel_mask, proto, buff_size, chunk_steps, &err))
    return fail(RAR_INVALID_ARGUMENT, err);
  if (nrings < 1 || nrings > rar::kMaxChannels)
    return fail(RAR_INVALID_ARGUMENT, "nrings must be in [1, 64]");
  if (!ring_orders) return fail(RAR_INVALID_ARGUMENT, "ring_order is NULL");
  std::vector<rar::RingInfo> rings(nrings);
  for (int k = 0; k < nrings; ++k)
    if (!rar::build_ring(nranks, ring_orders + (size_t)k * nranks, &rings[k], &err))
      return fail(RAR_INVALID_ARGUMENT, "ring " + std::to_string(k) + ": " + err);
  rar_tuning_t tune{};
  if (tuning) tune = *tuning;
  if (tune.lanes_per_channel < 0 || tune.lanes_per_channel > rar::kMaxLanes)
    return fail(RAR_INVALID_ARGUMENT, "lanes_per_channel must be in [0, 16]");
  if (tune.waves_per_lane < 0 || tune.waves_per_lane > rar::kMaxWaves)
    return fail(RAR_INVALID_ARGUMENT, "waves_per_lane must be in [0, 8]");
  if (tune.spin_timeout_us < 0) return fail(RAR_INVALID_ARGUMENT, "spin_timeout_us is negative");
  if (tune.launch_mode != 0 && tune.launch_mode != 1)
    return fail(RAR_INVALID_ARGUMENT, "launch_mode must be 0 or 1");
  if (tune.debug_flags & ~7) return fail(RAR_INVALID_ARGUMENT, "unknown debug_flags bits");
  if (tune.placement != 0 && tune.placement != 1)
    return fail(RAR_INVALID_ARGUMENT, "placement must be 0 or 1");
  if (tune.slices_per_chunk < 0 || tune.slices_per_chunk > 4 || tune.slices_per_chunk == 3)
    return fail(RAR_INVALID_ARGUMENT, "slices_per_chunk must be 0, 1, 2 or 4");
  if (tune.slices_per_chunk == 4 && (int)proto == rar::kSimple && chunk_steps != 4)
    return fail(RAR_INVALID_ARGUMENT, "4 slices per chunk need chunk_steps 4");
  if (tune.direct < 0 || tune.direct > 3)
    return fail(RAR_INVALID_ARGUMENT, "direct must be 0..3 (bit 0 write, bit 1 read)");
  if (tune.direct && (int)proto != rar::kSimple)
    return fail(RAR_UNSUPPORTED, "the direct variant exists for the Simple protocol only");
  if (tune.deal_works != 0 && tune.deal_works != 1)
    return fail(RAR_INVALID_ARGUMENT, "deal_works must be 0 or 1");
  if (tune.strict_scope != 0 && tune.strict_scope != 1)
    return fail(RAR_INVALID_ARGUMENT, "strict_scope must be 0 or 1");
  if (tune.waves_by_size != 0 && tune.waves_by_size != 1)
    return fail(RAR_INVALID_ARGUMENT, "waves_by_size must be 0 or 1");

  int dev = 0;
  RAR_HIP(hipGetDevice(&dev));
  int cus = 0, coop = 0;
  RAR_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  RAR_HIP(hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev));
  if (!coop) return fail(RAR_UNSUPPORTED, "device has no cooperative launch");

  rar_comm* c = new rar_comm();
  c->device = dev;
  c->nranks = nranks;
  c->order.assign(ring_orders, ring_orders + (size_t)nrings * nranks);
  c->nrings = nrings;
  c->mask = channel_mask;
  c->C = __builtin_popcountll(channel_mask);
  c->proto = proto;
  c->buff = buff_size;
  c->chunk_steps = chunk_steps;
  c->P = tune.lanes_per_channel ? tune.lanes_per_channel : rar::auto_lanes(nranks, c->C, cus);
  c->W = tune.waves_per_lane ? tune.waves_per_lane : ((int)proto == rar::kLL ? 4 : 8);
  const uint64_t timeout_us = tune.spin_timeout_us ? (uint64_t)tune.spin_timeout_us : 10000000ull;
  c->timeout_ticks = timeout_us * 100ull;  // s_memrealtime runs at 100 MHz
  const std::vector<uint32_t> wg = rar::make_wg_map(nranks, c->C, c->P, tune.placement == 1);
  c->grid = (int)wg.size();
  c->wgmap = wg;
  c->launch_mode = tune.launch_mode;
  c->debug_flags = tune.debug_flags;
  c->sizing.on = tune.waves_by_size != 0;
  c->sizing.nranks = nranks;
  c->sizing.proto = proto;
  c->sizing.split_lanes = tune.deal_works ? 1 : c->P;

  // every workgroup must be resident at once: the ranks wait on each other
  for (int k = 0; k < 3 * rar::kNumRed; ++k) {
    const int dt = k / rar::kNumRed, red = k % rar::kNumRed;
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, rar::get_kernel(dt, proto, red),
                                                                c->W * rar::kWaveSize, 0);
    if (e != hipSuccess) {
      release(c);
      return fail(RAR_HIP_ERROR, std::string("occupancy query failed: ") + hipGetErrorString(e));
    }
    if ((int64_t)per_cu * cus < c->grid) {
      const int g = c->grid;
      release(c);
      return fail(RAR_UNSUPPORTED, "grid of " + std::to_string(g) +
                                       " workgroups cannot be co-resident; lower lanes or waves");
    }
  }

  auto guard = [&](hipError_t e, const char* what) -> rar_result_t {
    if (e == hipSuccess) return RAR_SUCCESS;
    release(c);
    return fail(RAR_HIP_ERROR, std::string(what) + " failed: " + hipGetErrorString(e));
  };
  // dealt works run whole on one lane: every lane FIFO holds the full buffer
  const int64_t lane_step = rar::lane_step_bytes(proto, buff_size, tune.deal_works ? 1 : c->P);
  const size_t fifo_bytes = (size_t)nranks * c->C * c->P * rar::kSteps * (size_t)lane_step;
  const size_t counter_bytes = (size_t)nranks * c->C * c->P * sizeof(rar::ConnCounters);
  rar_result_t r;
  if ((r = guard(hipMalloc(&c->d_fifo, fifo_bytes), "hipMalloc(fifo)"))) return r;
  if ((r = guard(hipMalloc(&c->d_counters, counter_bytes), "hipMalloc(counters)"))) return r;
  if ((r = guard(hipMalloc(&c->d_abort, 256), "hipMalloc(abort)"))) return r;
  if ((r = guard(hipMalloc(&c->d_wgmap, wg.size() * sizeof(uint32_t)), "hipMalloc(wgmap)"))) return r;
  if ((r = guard(hipMalloc(&c->d_comm, sizeof(rar::DevComm)), "hipMalloc(comm)"))) return r;
  // wg_peer[g]: the workgroup that receives from workgroup g (same dense
  // channel and lane, the next rank on that channel's ring)
  std::vector<uint32_t> wg_of((size_t)nranks * c->C * c->P, 0);
  for (size_t g = 0; g < wg.size(); ++g)
    if (wg[g] != rar::kIdleWg) {
      const uint32_t m = wg[g];
      wg_of[((size_t)(m & 0xFF) * c->C + ((m >> 8) & 0xFF)) * c->P + ((m >> 16) & 0xFF)] = (uint32_t)g;
    }
  std::vector<int> channel_ids;
  for (int id = 0; id < rar::kMaxChannels; ++id)
    if ((channel_mask >> id) & 1) channel_ids.push_back(id);
  std::vector<uint32_t> wg_peer(wg.size(), 0);
  for (size_t g = 0; g < wg.size(); ++g) {
    wg_peer[g] = (uint32_t)g;
    if (wg[g] == rar::kIdleWg) continue;
    const uint32_t m = wg[g];
    const int rank = (int)(m & 0xFF), n = (int)((m >> 8) & 0xFF), lane = (int)((m >> 16) & 0xFF);
    const int next = rings[channel_ids[n] % nrings].next[rank];
    wg_peer[g] = wg_of[((size_t)next * c->C + n) * c->P + lane];
  }
  if ((r = guard(hipMalloc(&c->d_placement, wg.size() * sizeof(uint64_t)), "hipMalloc(placement)"))) return r;
  if ((r = guard(hipMemset(c->d_placement, 0, wg.size() * sizeof(uint64_t)), "hipMemset(placement)"))) return r;
  if ((r = guard(hipMalloc(&c->d_wg_peer, wg_peer.size() * sizeof(uint32_t)), "hipMalloc(wg_peer)"))) return r;
  if ((r = guard(hipMemcpy(c->d_wg_peer, wg_peer.data(), wg_peer.size() * sizeof(uint32_t),
                           hipMemcpyHostToDevice),
                 "hipMemcpy(wg_peer)")))
    return r;
  constexpr int kTraceCap = 4096;
  if (tune.debug_flags & 2) {
    if ((r = guard(hipMalloc(&c->d_trace, (size_t)c->grid * kTraceCap * sizeof(rar::TraceRec)),
                   "hipMalloc(trace)")))
      return r;
    if ((r = guard(hipMalloc(&c->d_trace_count, (size_t)c->grid * sizeof(uint32_t)), "hipMalloc(trace count)")))
      return r;
    if ((r = guard(hipMemset(c->d_trace_count, 0, (size_t)c->grid * sizeof(uint32_t)), "hipMemset(trace)")))
      return r;
  }
  if ((r = guard(hipHostMalloc(reinterpret_cast<void**>(&c->h_abort), 256, hipHostMallocMapped),
                 "hipHostMalloc(abort)")))
    return r;
  std::memset(c->h_abort, 0, 256);
  if ((r = guard(hipHostGetDevicePointer(reinterpret_cast<void**>(&c->d_abort_host), c->h_abort, 0),
                 "hipHostGetDevicePointer")))
    return r;
  if ((r = guard(hipEventCreateWithFlags(&c->upload_done, hipEventDisableTiming), "hipEventCreate")))
    return r;
  if ((r = guard(hipMemset(c->d_fifo, 0, fifo_bytes), "hipMemset(fifo)"))) return r;
  if ((r = guard(hipMemset(c->d_counters, 0, counter_bytes), "hipMemset(counters)"))) return r;
  if ((r = guard(hipMemset(c->d_abort, 0, 256), "hipMemset(abort)"))) return r;
  if ((r = guard(hipMemcpy(c->d_wgmap, wg.data(), wg.size() * sizeof(uint32_t), hipMemcpyHostToDevice),
                 "hipMemcpy(wgmap)")))
    return r;
  // 64 KiB of ring tables: built on the heap, not the stack
  std::unique_ptr<rar::DevComm> hcp(new rar::DevComm());
  rar::DevComm& hc = *hcp;
  std::memset(&hc, 0, sizeof(hc));
  hc.hot.n_ranks = nranks;
  hc.hot.n_channels = c->C;
  hc.hot.n_lanes = c->P;
  hc.hot.proto = proto;
  hc.hot.buff_size = (int64_t)buff_size;
  hc.hot.step_bytes = (int64_t)buff_size / rar::kSteps;
  hc.hot.lane_step_bytes = lane_step;
  hc.hot.lane_buff_bytes = lane_step * rar::kSteps;
  hc.hot.chunk_steps = chunk_steps;
  const int spc = tune.slices_per_chunk ? tune.slices_per_chunk : rar::kSlicesPerChunk;
  hc.hot.slices_per_chunk = spc;
  hc.hot.direct = tune.direct;
  hc.hot.deal_works = tune.deal_works;
  hc.hot.strict_scope = tune.strict_scope;
  hc.hot.step_per_slice = (int)proto == rar::kSimple ? chunk_steps / spc : 1;
  hc.hot.channel_mask = channel_mask;
  hc.hot.fifo = c->d_fifo;
  hc.hot.counters = c->d_counters;
  hc.hot.abort_flag = c->d_abort;
  hc.hot.abort_host = c->d_abort_host;
  hc.hot.spin_timeout_ticks = c->timeout_ticks;
  hc.hot.debug_flags = tune.debug_flags;
  hc.hot.trace_cap = (tune.debug_flags & 2) ? kTraceCap : 0;
  hc.hot.trace = c->d_trace;
  hc.hot.trace_count = c->d_trace_count;
  hc.hot.placement = c->d_placement;
  hc.hot.wg_peer = c->d_wg_peer;
  hc.hot.ll_flag_mask = (tune.debug_flags & RAR_DEBUG_LL_FLAG_WRAP8) ? 0xFFu : 0xFFFFFFFFu;
  for (int id = 0; id < rar::kMaxChannels; ++id) {
    if (!((channel_mask >> id) & 1)) continue;
    const rar::RingInfo& ring = rings[id % nrings];
    for (int i = 0; i < nranks; ++i) {
      hc.ranks[id][i].index = ring.index[i];
      hc.ranks[id][i].prev = ring.prev[i];
      hc.ranks[id][i].next = ring.next[i];
    }
  }
  if ((r = guard(hipMemcpy(c->d_comm, &hc, sizeof(hc), hipMemcpyHostToDevice), "hipMemcpy(comm)")))
    return r;
  if ((r = guard(hipDeviceSynchronize(), "hipDeviceSynchronize"))) return r;
  *out = c;
  return RAR_SUCCESS;
}

rar_result_t rar_comm_destroy(rar_comm_t c) {
  g_last_error.clear();
  if (!c) return RAR_SUCCESS;
  {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    for (auto it = g_cache.begin(); it != g_cache.end(); ++it)
      if (it->second == c) {
        g_cache.erase(it);
        break;
      }
  }
  release(c);
  return RAR_SUCCESS;
}

static rar_result_t allreduce_impl(rar_comm_t c, const void* const* sendbufs, void* const* recvbufs,
                           size_t count, rar_dtype_t dtype, int op, const void* scalars, void* stream) {
  if (!c) return fail(RAR_INVALID_ARGUMENT, "comm is NULL");
  if (rar_result_t r = check_dtype(dtype)) return r;
  if (op == RAR_PREMULSUM) {
    if (!scalars) return fail(RAR_INVALID_ARGUMENT, "scalars is NULL");
  } else if (rar_result_t r = check_op(op)) {
    return r;
  }
  if (c->in_group && !c->queue.empty() && (c->queue.front().dtype != dtype || c->queue.front().red != op))
    return fail(RAR_UNSUPPORTED, "all AllReduces of a group must share one dtype and operator");
  // nothing to move: no launch, no step advance, pointers are not looked at
  if (count == 0) return RAR_SUCCESS;
  if (count > (size_t(1) << 40)) return fail(RAR_INVALID_ARGUMENT, "count too large");
  if (rar_result_t r = check_rank_buffers(c->nranks, sendbufs, recvbufs, count, dtype)) return r;
  QueuedCall q;
  for (int r = 0; r < c->nranks; ++r) q.send.push_back(const_cast<void*>(sendbufs[r]));
  q.recv.assign(recvbufs, recvbufs + c->nranks);
  q.count = count;
  q.dtype = dtype;
  q.red = op;
  if (op == RAR_PREMULSUM)
    for (int r = 0; r < c->nranks; ++r) q.scalars.push_back(scalar_bits(scalars, dtype, r));
  if (c->in_group) {
    c->queue.push_back(std::move(q));
    return RAR_SUCCESS;
  }
  std::vector<QueuedCall> one;
  one.push_back(std::move(q));
  return launch(c, one, reinterpret_cast<hipStream_t>(stream));
}

rar_result_t rar_allreduce(rar_comm_t c, const void* const* sendbufs, void* const* recvbufs,
                           size_t count, rar_dtype_t dtype, rar_redop_t op, void* stream) {
  g_last_error.clear();
  return allreduce_impl(c, sendbufs, recvbufs, count, dtype, op, nullptr, stream);
}

rar_result_t rar_allreduce_premul(rar_comm_t c, const void* const* sendbufs, void* const* recvbufs,
                                  size_t count, rar_dtype_t dtype, const void* scalars, void* stream) {
  g_last_error.clear();
  return allreduce_impl(c, sendbufs, recvbufs, count, dtype, RAR_PREMULSUM, scalars, stream);
}

rar_result_t rar_group_start(rar_comm_t c) {
  g_last_error.clear();
  if (!c) return fail(RAR_INVALID_ARGUMENT, "comm is NULL");
  if (c->in_group) return fail(RAR_INVALID_ARGUMENT, "group already open");
  c->in_group = true;
  c->queue.clear();
  return RAR_SUCCESS;
}

rar_result_t rar_group_discard(rar_comm_t c) {
  g_last_error.clear();
  if (!c) return fail(RAR_INVALID_ARGUMENT, "comm is NULL");
  c->in_group = false;
  c->queue.clear();
  return RAR_SUCCESS;
}

rar_result_t rar_group_end(rar_comm_t c, void* stream) {
  g_last_error.clear();
  if (!c) return fail(RAR_INVALID_ARGUMENT, "comm is NULL");
  if (!c->in_group) return fail(RAR_INVALID_ARGUMENT, "no open group");
  c->in_group = false;
  std::vector<QueuedCall> calls;
  calls.swap(c->queue);
  if (calls.empty()) return RAR_SUCCESS;
  return launch(c, calls, reinterpret_cast<hipStream_t>(stream));
}

rar_result_t ring_allreduce(const void* const* sendbufs, void* const* recvbufs, int nranks, size_t count,
                            rar_dtype_t dtype, rar_redop_t op, const int* ring_order, rar_proto_t proto,
                            int nchannels, size_t buff_size, int chunk_steps, void* stream) {
  g_last_error.clear();
  // every argument is checked on the host before the device is touched
  uint64_t mask = 0;
  rar::RingInfo ring;
  if (rar_result_t r = rar::check_ring_call(sendbufs, recvbufs, nranks, count, dtype, op, ring_order, proto,
                                            nchannels, &buff_size, &chunk_steps, &mask, &ring))
    return r;
  if (count == 0) return RAR_SUCCESS;  // nothing to move: no launch, pointers not looked at
  int dev = 0;
  RAR_HIP(hipGetDevice(&dev));
  std::vector<int64_t> key = {dev, nranks, (int64_t)mask, (int64_t)proto, (int64_t)buff_size, chunk_steps};
  key.insert(key.end(), ring_order, ring_order + nranks);
  rar_comm* c = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_cache_mu);
    auto it = g_cache.find(key);
    if (it != g_cache.end()) c = it->second;
  }
  if (!c) {
    rar_result_t r = rar_comm_create(&c, nranks, ring_order, mask, proto, buff_size, chunk_steps, nullptr);
    if (r != RAR_SUCCESS) return r;
    rar_comm* extra = nullptr;
    {
      std::lock_guard<std::mutex> lk(g_cache_mu);
      auto it = g_cache.find(key);
      if (it == g_cache.end()) {
        g_cache[key] = c;
      } else {
        // another thread cached the same shape meanwhile: use that one
        extra = c;
        c = it->second;
      }
    }
    if (extra) release(extra);
  }
  // One set of FIFOs and step counters serves every caller of this shape:
  // launches must follow each other.  Same stream: stream order does it.
  // Another stream: that stream first waits for the previous launch.
  std::lock_guard<std::mutex> lk(c->call_mu);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  if (!c->last_done) RAR_HIP(hipEventCreateWithFlags(&c->last_done, hipEventDisableTiming));
  if (c->has_last && c->last_stream != hs) RAR_HIP(hipStreamWaitEvent(hs, c->last_done, 0));
  const rar_result_t r = rar_allreduce(c, sendbufs, recvbufs, count, dtype, op, stream);
  if (r != RAR_SUCCESS) return r;
  RAR_HIP(hipEventRecord(c->last_done, hs));
  c->last_stream = hs;
  c->has_last = true;
  return RAR_SUCCESS;
}

rar_result_t ring_allreduce_cache_release(void) {
  g_last_error.clear();
  std::lock_guard<std::mutex> lk(g_cache_mu);
  if (g_cache.empty()) return RAR_SUCCESS;  // nothing cached: no device call
  int cur = 0;
  RAR_HIP(hipGetDevice(&cur));
  rar_result_t res = RAR_SUCCESS;
  while (!g_cache.empty()) {
    auto it = g_cache.begin();
    rar_comm* c = it->second;
    // wait for its last launch and free it with its own device current
    hipError_t e = hipSetDevice(c->device);
    if (e == hipSuccess && c->has_last) {
      std::lock_guard<std::mutex> call_lk(c->call_mu);
      e = hipEventSynchronize(c->last_done);
    }
    if (e != hipSuccess) {
      res = fail(RAR_HIP_ERROR, std::string("waiting for a cached communicator's last launch failed: ") +
                                    hipGetErrorString(e));
      break;
    }
    g_cache.erase(it);
    release(c);
  }
  (void)hipSetDevice(cur);
  return res;
}

static rar_result_t oneshot_impl(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                 size_t count, rar_dtype_t dtype, int op, const void* scalars,
                                 const rar_oneshot_tuning_t* tuning, void* stream) {
  if (nranks < 2 || nranks > rar::kMaxRanks) return fail(RAR_INVALID_ARGUMENT, "nranks must be in [2, 64]");
  if (rar_result_t r = check_dtype(dtype)) return r;
  if (op == RAR_PREMULSUM) {
    if (!scalars) return fail(RAR_INVALID_ARGUMENT, "scalars is NULL");
  } else if (rar_result_t r = check_op(op)) {
    return r;
  }
  rar_oneshot_tuning_t tune{0, 0, 0, 0};
  if (tuning) tune = *tuning;
  if (tune.workgroups < 0 || tune.workgroups > 65536)
    return fail(RAR_INVALID_ARGUMENT, "workgroups must be in [0, 65536]");
  if (tune.waves < 0 || tune.waves > 8) return fail(RAR_INVALID_ARGUMENT, "waves must be in [0, 8]");
  if (tune.unroll != 0 && tune.unroll != 1 && tune.unroll != 2 && tune.unroll != 4)
    return fail(RAR_INVALID_ARGUMENT, "unroll must be 0, 1, 2 or 4");
  if (count == 0) return RAR_SUCCESS;  // nothing to move: no launch, pointers not inspected
  if (rar_result_t r = check_rank_buffers(nranks, sendbufs, recvbufs, count, dtype)) return r;
  const size_t es = (size_t)rar::elem_size(dtype);

  rar::OneshotArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int r = 0; r < nranks; ++r) {
    a.src[r] = sendbufs[r];
    a.dst[r] = recvbufs[r];
    a.scalar[r] = op == RAR_PREMULSUM ? scalar_bits(scalars, dtype, r) : 0;
  }
  const int64_t vec = 16 / (int64_t)es;
  a.nranks = nranks;
  a.nvec = (int64_t)(count / vec);
  a.tail = (int32_t)(count % vec);
  const int threads = 64 * (tune.waves ? tune.waves : 4);
  const int unroll = tune.unroll ? tune.unroll : 2;
  const int64_t per_pass = (int64_t)threads * unroll;
  int64_t blocks = tune.workgroups ? tune.workgroups : std::min<int64_t>((a.nvec + per_pass - 1) / per_pass, 2048);
  if (blocks < 1) blocks = 1;
  a.vec_per_block = std::max<int64_t>(1, (a.nvec + blocks - 1) / blocks);
  blocks = std::max<int64_t>(1, (a.nvec + a.vec_per_block - 1) / a.vec_per_block);
  void* params[] = {&a};
  RAR_HIP(hipLaunchKernel(rar::get_oneshot_kernel(dtype, op, unroll), dim3((unsigned)blocks), dim3(threads),
                          params, 0, reinterpret_cast<hipStream_t>(stream)));
  return RAR_SUCCESS;
}

rar_result_t rar_oneshot_allreduce(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                   size_t count, rar_dtype_t dtype, rar_redop_t op,
                                   const rar_oneshot_tuning_t* tuning, void* stream) {
  g_last_error.clear();
  return oneshot_impl(sendbufs, recvbufs, nranks, count, dtype, op, nullptr, tuning, stream);
}

rar_result_t rar_oneshot_allreduce_premul(const void* const* sendbufs, void* const* recvbufs, int nranks,
                                          size_t count, rar_dtype_t dtype, const void* scalars,
                                          const rar_oneshot_tuning_t* tuning, void* stream) {
  g_last_error.clear();
  return oneshot_impl(sendbufs, recvbufs, nranks, count, dtype, RAR_PREMULSUM, scalars, tuning, stream);
}

rar_result_t rar_comm_get_async_error(rar_comm_t c) {
  if (!c) return fail(RAR_INVALID_ARGUMENT, "comm is NULL");
  return __atomic_load_n(c->h_abort, __ATOMIC_ACQUIRE) ? RAR_ABORTED : RAR_SUCCESS;
}

rar_result_t rar_comm_query_state(rar_comm_t c, int64_t* out, size_t cap, size_t* written) {
  g_last_error.clear();
  if (!c || !out || !written) return fail(RAR_INVALID_ARGUMENT, "NULL argument");
  RAR_HIP(hipDeviceSynchronize());
  const size_t lanes = (size_t)c->nranks * c->C * c->P;
  std::vector<rar::ConnCounters> h(lanes);
  RAR_HIP(hipMemcpy(h.data(), c->d_counters, lanes * sizeof(rar::ConnCounters), hipMemcpyDeviceToHost));
  size_t k = 0;
  for (size_t i = 0; i < lanes && k + 2 <= cap; ++i) {
    out[k++] = (int64_t)h[i].tail.value;
    out[k++] = (int64_t)h[i].head.value;
  }
  *written = k;
  return RAR_SUCCESS;
}

rar_result_t rar_comm_read_trace(rar_comm_t c, rar_trace_rec_t* out, size_t cap, size_t* written) {
  g_last_error.clear();
  if (!c || !written || (cap && !out)) return fail(RAR_INVALID_ARGUMENT, "NULL argument");
  *written = 0;
  if (!(c->debug_flags & 2)) return fail(RAR_INVALID_ARGUMENT, "communicator created without tracing");
  RAR_HIP(hipDeviceSynchronize());
  std::vector<uint32_t> counts(c->grid);
  RAR_HIP(hipMemcpy(counts.data(), c->d_trace_count, counts.size() * sizeof(uint32_t), hipMemcpyDeviceToHost));
  std::vector<int> ids;
  for (int b = 0; b < rar::kMaxChannels; ++b)
    if ((c->mask >> b) & 1ull) ids.push_back(b);
  const int cap_per_wg = 4096;
  std::vector<rar::TraceRec> buf;
  size_t k = 0;
  for (int g = 0; g < c->grid && k < cap; ++g) {
    const uint32_t m = c->wgmap[g];
    if (m == rar::kIdleWg || counts[g] == 0) continue;
    const uint32_t n_rec = std::min<uint32_t>(counts[g], cap_per_wg);
    buf.resize(n_rec);
    RAR_HIP(hipMemcpy(buf.data(), c->d_trace + (size_t)g * cap_per_wg, n_rec * sizeof(rar::TraceRec),
                      hipMemcpyDeviceToHost));
    for (uint32_t i = 0; i < n_rec && k < cap; ++i, ++k) {
      rar_trace_rec_t& o = out[k];
      o.rank = (int32_t)(m & 0xFF);
      o.channel_id = ids[(m >> 8) & 0xFF];
      o.lane = (int32_t)((m >> 16) & 0xFF);
      o.op = buf[i].op;
      o.chunk = buf[i].chunk;
      o.nelem = buf[i].nelem;
      o.t_begin = buf[i].t_begin;
      o.wait_ticks = buf[i].wait_ticks;
      o.data_ticks = buf[i].data_ticks;
      o.recv_step = buf[i].recv_step;
      o.waves = (int32_t)buf[i].waves;
      o.pad = 0;
    }
  }
  *written = k;
  return RAR_SUCCESS;
}

rar_result_t rar_graph_text(int nranks, int nrings, const int* ring_orders, uint64_t channel_mask,
                            char* buf, size_t cap, size_t* len) {
  g_last_error.clear();
  std::vector<std::string> lines;
  std::string err;
  if (!rar::graph_lines(nranks, nrings, ring_orders, channel_mask, &lines, &err))
    return fail(RAR_INVALID_ARGUMENT, err);
  std::string text;
  for (const std::string& l : lines) text += l + "\n";
  return put_text(text, buf, cap, len);
}

rar_result_t rar_comm_graph_text(rar_comm_t c, char* buf, size_t cap, size_t* len) {
  g_last_error.clear();
  if (!c) return fail(RAR_INVALID_ARGUMENT, "comm is NULL");
  std::vector<std::string> lines;
  std::string err;
  if (!rar::graph_lines(c->nranks, c->nrings, c->order.data(), c->mask, &lines, &err))
    return fail(RAR_INTERNAL_ERROR, err);
  // XCD of every (channel, lane, rank) workgroup: block g of the grid runs on
  // XCD g mod 8 (the dispatcher deals workgroups to the XCDs in turn)
  std::vector<int> xcd((size_t)c->C * c->P * c->nranks, -1);
  for (size_t g = 0; g < c->wgmap.size(); ++g) {
    const uint32_t m = c->wgmap[g];
    if (m == rar::kIdleWg) continue;
    const int r = (int)(m & 0xFF), n = (int)((m >> 8) & 0xFF), lane = (int)(m >> 16);
    xcd[((size_t)n * c->P + lane) * c->nranks + r] = (int)(g % 8);
  }
  const int64_t lane_step = rar::lane_step_bytes(c->proto, c->buff, c->sizing.split_lanes);
  std::string text;
  for (int n = 0; n < (int)lines.size(); ++n) {
    text += lines[n] + "\n";
    char head[160];
    snprintf(head, sizeof head, "  lanes %d, waves %d, FIFO %zu B per connection, %lld B per lane and step, XCD per lane:",
             c->P, c->W, c->buff, (long long)lane_step);
    text += head;
    for (int lane = 0; lane < c->P; ++lane) {
      const int* x = &xcd[((size_t)n * c->P + lane) * c->nranks];
      const bool one = std::all_of(x, x + c->nranks, [&](int v) { return v == x[0]; });
      text += " " + std::to_string(x[0]);
      if (!one)
        for (int r = 1; r < c->nranks; ++r) text += "/" + std::to_string(x[r]);
    }
    text += "\n";
  }
  return put_text(text, buf, cap, len);
}

rar_result_t rar_comm_shape(rar_comm_t c, int* nchannels, int* lanes, int* waves, int* grid) {
  if (!c) return fail(RAR_INVALID_ARGUMENT, "comm is NULL");
  if (nchannels) *nchannels = c->C;
  if (lanes) *lanes = c->P;
  if (waves) *waves = c->W;
  if (grid) *grid = c->grid;
  return RAR_SUCCESS;
}

}  // extern "C"
