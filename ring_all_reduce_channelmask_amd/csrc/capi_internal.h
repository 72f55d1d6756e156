// capi_internal.h -- pieces of the C ABI shared by its two source files:
// capi.cpp (communicators, groups, the one-shot) and noalloc.hip (the entry
// point whose device state lives in a static array).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "plan.h"
#include "rar.h"
#include "rar_device.h"

namespace rar {

// The last failure's message on the calling thread (rar_get_last_error).
rar_result_t set_error(rar_result_t r, const std::string& msg);
void clear_error();

rar_result_t check_dtype(int dtype);
rar_result_t check_op(int op);
// NULL, element alignment and cross-rank overlap of one collective's 2N
// buffers; host-side only.
rar_result_t check_rank_buffers(int nranks, const void* const* sendbufs, void* const* recvbufs,
                                size_t count, int dtype);

// The ring kernel for (payload type, protocol, reduction operator).
const void* get_kernel(int dtype, int proto, int red);

// One collective of a launch, as queued by rar_allreduce.
struct QueuedCall {
  std::vector<void*> send, recv;
  size_t count;
  int dtype;
  int red;
  std::vector<uint32_t> scalars;  // PreMulSum: one scalar per rank (payload bits)
};

// A launch plan laid out as one block of bytes with 64-byte aligned tables
// (batches, works, buffer pointers, PreMulSum scalars, first batch per
// channel id), and the offsets KernelArgs carries.  Empty `bytes` when the
// launch moves nothing.
struct PlanBlock {
  std::vector<uint8_t> bytes;
  uint32_t off_batches = 0, off_works = 0, off_ptrs = 0, off_scalars = 0, off_first = 0;
};
PlanBlock build_plan_block(const std::vector<QueuedCall>& calls, int nranks, uint64_t mask, int proto,
                           size_t buff, int chunk_steps, int n_channels, int n_waves,
                           const WaveSizing& sizing = WaveSizing());

// The arguments shared by ring_allreduce and ring_allreduce_noalloc, checked
// on the host in the same order by both: on success the channel mask, the
// buffer size and chunk steps with defaults filled in, and the ring.
rar_result_t check_ring_call(const void* const* sendbufs, void* const* recvbufs, int nranks,
                             size_t count, int dtype, int op, const int* ring_order, int proto,
                             int nchannels, size_t* buff_size, int* chunk_steps, uint64_t* mask,
                             RingInfo* ring);

}  // namespace rar
