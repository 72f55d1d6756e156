// ring_kernel.h -- the ring AllReduce device path for gfx950 (MI355X, wave64).
//
// Device templates only; ring_kernel_{i32,f32,bf16}.hip instantiate them.
//
// One cooperative launch runs every virtual rank.  Workgroup = (rank r, dense
// channel n, lane p).  The lanes of a channel split every slice (Simple) or
// step (LL, LL128) into contiguous parts, each with its own head/tail
// counters, so they run as independent pipelines of identical geometry.
//
// Structure follows the two NCCL course pages:
//   [C23] "NCCL 专家课程 23：Device Kernel、Primitives、Step/Credit 与 LL Flag"
//   [C12] "NCCL 专家课程 12：Ring AllReduce 逐步推导、真实 Ring 与 Channel 并行"
// Memory ordering uses HIP's scoped atomics: agent scope (all XCDs of this
// GPU) is the widest observer set, since every rank lives on this device.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <type_traits>

#include "rar_device.h"

namespace rar {
namespace {

enum Op : int { kOpSend = 0, kOpRecvReduceSend, kOpRecvReduceCopySend, kOpRecvCopySend, kOpRecv };

__device__ __forceinline__ int64_t div_up(int64_t a, int64_t b) { return (a + b - 1) / b; }
__device__ __forceinline__ int64_t align_up(int64_t a, int64_t b) { return div_up(a, b) * b; }
__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// ---------------------------------------------------------------- addressing
// Every FIFO, counter and user buffer lives in device (or host-mapped)
// memory.  Their pointers reach the kernel as generic pointers, which would
// compile to FLAT instructions; FLAT accesses may complete out of order with
// LDS and scalar traffic, so the compiler must wait for everything
// outstanding before using any of their results.  Accessing them through
// the global address space gives GLOBAL instructions whose completions are
// counted in order: loads stay in flight while earlier results are used.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* G(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// A value that is the same on every lane of the wave, moved to a scalar
// register so that the compiler knows it is uniform.
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------- ordering
__device__ __forceinline__ uint64_t load_relaxed(const uint64_t* p) {
  return __hip_atomic_load(G(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_relaxed(uint64_t* p, uint64_t v) {
  __hip_atomic_store(G(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A relaxed store at workgroup scope: a plain vector store, which lands in
// this XCD's L2 like any store but is not written through at agent scope.  A
// reader on the same XCD (same L2) sees it through its agent-scope loads; a
// reader on another XCD may not, so callers use it only where the placement
// handshake found the receiver on this XCD.
__device__ __forceinline__ void store_relaxed_xcd(uint64_t* p, uint64_t v) {
  __hip_atomic_store(G(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void acquire_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ void release_fence() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
// The XCD (and so the L2) this wave runs on.
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xFu;
}
// Wait until every memory operation this wave issued has completed, so that
// a barrier that follows also covers this wave's payload stores.  The FIFO
// and user pointers are generic, so their accesses are FLAT instructions,
// which count in both vmcnt and lgkmcnt: wait for both.
__device__ __forceinline__ void drain_vmem() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------- arithmetic
// A 16-byte vector is four 32-bit words; each word holds one fp32 / int32 or
// two bf16.  The kernel is specialised on the payload type and the reduction
// operator [C23 "RunWorkColl 与 Template Dispatch"].  red(acc, x) combines
// the partial from the previous rank with the own input:
//   sum / avg  acc + x          prod  acc * x
//   max        x if x > acc     min   x if x < acc   (else acc, bits kept)
// bf16 sums and products are formed in fp32 (exact for two bf16 operands)
// and rounded to nearest-even bf16 per hop; int32 wraps.  avg's post-op
// divides the owner's final sum by N, rounded once [C12 "源码步骤三"].
// Rounding to bf16 uses gfx950's conversion instruction (v_cvt_pk_bf16_f32,
// round to nearest, ties to even; a NaN stays a quiet NaN with its high
// payload bits), two results per instruction where a word holds two
// elements.  On MI355X it agrees bit for bit, on all 2^32 fp32 inputs, with
// the integer form of the rule: (u + 0x7fff + ((u >> 16) & 1)) >> 16 for
// non-NaN u, ((u >> 16) | 0x40) for NaN.  Measured against that integer form:
// bf16 8 ranks 437.0 -> 431.0 us, the fused bf16 LL group 22.2 -> 21.4 us.
typedef float f2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// lo -> bits 0..15, hi -> bits 16..31
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{lo, hi}, bf2_t));
}

template <int R>
__device__ __forceinline__ float red_f(float a, float b) {
  if constexpr (R == kRedProd) return a * b;
  else if constexpr (R == kRedMax) return b > a ? b : a;
  else if constexpr (R == kRedMin) return b < a ? b : a;
  else return a + b;
}

// PreMulSum: a rank's own input is multiplied by the rank's scalar, rounded
// to the payload type, where it enters the fold; the fold is the sum's.
template <int R>
struct TyF32 {
  using S = uint32_t;
  static constexpr bool kPost = R == kRedAvg;
  static constexpr bool kPre = R == kRedPreMulSum;
  static __device__ __forceinline__ uint32_t pre_word(uint32_t x, uint32_t s) {
    return __float_as_uint(__uint_as_float(x) * __uint_as_float(s));
  }
  static __device__ __forceinline__ S pre_elem(S x, uint32_t s) { return pre_word(x, s); }
  static __device__ __forceinline__ uint32_t red_word(uint32_t a, uint32_t b) {
    return __float_as_uint(red_f<R>(__uint_as_float(a), __uint_as_float(b)));
  }
  static __device__ __forceinline__ S red_elem(S a, S b) { return red_word(a, b); }
  static __device__ __forceinline__ uint32_t post_word(uint32_t a, int n) {
    return __float_as_uint(__uint_as_float(a) / (float)n);  // IEEE division, nearest-even
  }
  static __device__ __forceinline__ S post_elem(S a, int n) { return post_word(a, n); }
};
template <int R>
struct TyI32 {
  using S = uint32_t;
  static constexpr bool kPost = R == kRedAvg;
  static constexpr bool kPre = R == kRedPreMulSum;
  static __device__ __forceinline__ uint32_t pre_word(uint32_t x, uint32_t s) { return x * s; }
  static __device__ __forceinline__ S pre_elem(S x, uint32_t s) { return x * s; }
  static __device__ __forceinline__ uint32_t red_word(uint32_t a, uint32_t b) {
    if constexpr (R == kRedProd) return a * b;  // low 32 bits
    else if constexpr (R == kRedMax) return (int32_t)b > (int32_t)a ? b : a;
    else if constexpr (R == kRedMin) return (int32_t)b < (int32_t)a ? b : a;
    else return a + b;
  }
  static __device__ __forceinline__ S red_elem(S a, S b) { return red_word(a, b); }
  static __device__ __forceinline__ uint32_t post_word(uint32_t a, int n) {
    return (uint32_t)((int32_t)a / n);  // truncates toward zero
  }
  static __device__ __forceinline__ S post_elem(S a, int n) { return post_word(a, n); }
};
template <int R>
struct TyBF16 {
  using S = uint16_t;
  static constexpr bool kPost = R == kRedAvg;
  static constexpr bool kPre = R == kRedPreMulSum;
  // bf16 x bf16 is exact in fp32: one rounding, to bf16
  static __device__ __forceinline__ uint16_t pre_elem(uint16_t x, uint32_t s) {
    return (uint16_t)bf16_rne(__uint_as_float((uint32_t)x << 16) * __uint_as_float(s << 16));
  }
  static __device__ __forceinline__ uint32_t pre_word(uint32_t x, uint32_t s) {
    const float fs = __uint_as_float(s << 16);
    return bf16x2_rne(__uint_as_float(x << 16) * fs, __uint_as_float(x & 0xffff0000u) * fs);
  }
  static __device__ __forceinline__ uint32_t red_half(uint32_t a, uint32_t b) {  // bf16 in the low 16 bits
    const float fa = __uint_as_float(a << 16), fb = __uint_as_float(b << 16);
    if constexpr (R == kRedMax) return fb > fa ? b : a;
    else if constexpr (R == kRedMin) return fb < fa ? b : a;
    else return bf16_rne(red_f<R>(fa, fb));
  }
  static __device__ __forceinline__ uint16_t red_elem(uint16_t a, uint16_t b) {
    return (uint16_t)red_half(a, b);
  }
  static __device__ __forceinline__ uint32_t red_word(uint32_t a, uint32_t b) {
    if constexpr (R == kRedSum || R == kRedAvg || R == kRedPreMulSum || R == kRedProd) {
      const float alo = __uint_as_float(a << 16), ahi = __uint_as_float(a & 0xffff0000u);
      const float blo = __uint_as_float(b << 16), bhi = __uint_as_float(b & 0xffff0000u);
      return bf16x2_rne(red_f<R>(alo, blo), red_f<R>(ahi, bhi));
    } else {
      return (red_half(a & 0xffffu, b & 0xffffu) & 0xffffu) | (red_half(a >> 16, b >> 16) << 16);
    }
  }
  static __device__ __forceinline__ uint16_t post_elem(uint16_t a, int n) {
    return (uint16_t)bf16_rne(__uint_as_float((uint32_t)a << 16) / (float)n);
  }
  static __device__ __forceinline__ uint32_t post_word(uint32_t a, int n) {
    return bf16x2_rne(__uint_as_float(a << 16) / (float)n, __uint_as_float(a & 0xffff0000u) / (float)n);
  }
};

template <class Ty>
__device__ __forceinline__ uint64_t red8(uint64_t a, uint64_t b) {
  return (uint64_t)Ty::red_word((uint32_t)a, (uint32_t)b) |
         ((uint64_t)Ty::red_word((uint32_t)(a >> 32), (uint32_t)(b >> 32)) << 32);
}
template <class Ty>
__device__ __forceinline__ uint64_t pre8(uint64_t a, uint32_t s) {
  return (uint64_t)Ty::pre_word((uint32_t)a, s) | ((uint64_t)Ty::pre_word((uint32_t)(a >> 32), s) << 32);
}
template <class Ty>
__device__ __forceinline__ uint64_t post8(uint64_t a, int n) {
  return (uint64_t)Ty::post_word((uint32_t)a, n) | ((uint64_t)Ty::post_word((uint32_t)(a >> 32), n) << 32);
}

template <int OP> struct OpTraits {
  static constexpr bool kRecv = OP != kOpSend;
  static constexpr bool kSend = OP != kOpRecv;
  static constexpr bool kSrc = OP == kOpSend || OP == kOpRecvReduceSend || OP == kOpRecvReduceCopySend;
  static constexpr bool kDst = OP == kOpRecvReduceCopySend || OP == kOpRecvCopySend || OP == kOpRecv;
};

// ---------------------------------------------------------------- LDS state
struct alignas(16) Shmem {
  DevCommHot comm;
  DevBatch batch;
  DevWork works[kBatchWorks];
  int32_t slot_bit[kBatchWorks];
  int32_t channel_id;
  int32_t n_works;
  int32_t abort;
  int32_t local_send;
  uint32_t first_batch;  // the channel's first work batch
  DevRank me;            // this rank's place on the channel's ring
};

// Per-thread view of the workgroup's channel (values are uniform).
struct Ctx {
  Shmem* sh;
  void* const* ptrs;
  int tid, nthreads, workers;
  int rank, next, prev, nranks, ring_index, lane, nlanes, sps, spc;
  // this workgroup's part of every step: part split_lane of split_lanes
  // (the lane of nlanes, or the whole step when the works are dealt)
  int split_lane, split_lanes;
  bool direct;       // Simple: all-gather half straight into the next rank's receive buffer
  bool direct_read;  // Simple: the loop's first receive reads the previous rank's send buffer
  uint32_t s_own, s_prev;  // PreMulSum scalars of this rank and the previous one (current work)
  int64_t step_bytes;       // channel slot: sets the slice geometry
  int64_t lane_step_bytes;  // this lane's slot in its own FIFO
  uint8_t* recv_fifo;
  uint8_t* send_fifo;
  uint64_t* recv_tail;
  uint64_t* recv_head;
  uint64_t* send_tail;
  uint64_t* send_head;
  uint64_t recv_step, send_step;
  // last values read of the receive tail and the send head (the pages'
  // connStepCache): a wait that the cached value already satisfies loads nothing
  uint64_t tail_cache, head_cache;
  uint32_t* abort_flag;
  uint32_t* abort_host;
  uint64_t timeout;
  bool drop_head;  // fault test: never publish head credit
  uint32_t ll_mask;  // LL flag period - 1: 2^32 - 1, or 0xFF in the wrap test mode
  uint8_t* stage;    // LL128: per-wave LDS tiles for the user <-> line layout change
  const uint32_t* scalars;  // PreMulSum: [buf_index * N + rank] scalar bits
  bool aborted;
  // The receiving workgroup of the send connector shares this workgroup's L2:
  // payload stores that have completed (vmcnt drained) are already visible to
  // it, so publishing needs no L2 write-back.
  bool local_send;
  // tracing (thread 0 only)
  TraceRec* trace;
  uint32_t trace_n, trace_cap;
};

__device__ __forceinline__ uint64_t now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// Thread 0 appends one record when tracing is on (trace != nullptr).
__device__ __forceinline__ void trace_unit(Ctx& cx, int op, int chunk, int64_t nelem,
                                           uint64_t step, uint64_t t0, uint64_t t1, uint64_t t2) {
  if (cx.trace && cx.tid == 0 && cx.trace_n < cx.trace_cap) {
    TraceRec r;
    r.t_begin = t0;
    r.wait_ticks = (uint32_t)(t1 - t0);
    r.data_ticks = (uint32_t)(t2 - t1);
    r.recv_step = (uint32_t)step;
    r.op = (uint16_t)op;
    r.chunk = (uint16_t)chunk;
    r.nelem = (uint32_t)nelem;
    r.waves = (uint32_t)(cx.workers / kWaveSize);
    cx.trace[cx.trace_n++] = r;
  }
}

// ---------------------------------------------------------------- waits
// Every wait is bounded [C23 "Simple 的 Credit 与 Step": the wait loop checks
// abort]: after `timeout` ticks of the 100 MHz clock the waiter raises the
// communicator's abort word and every other waiter leaves on seeing it.
__device__ void raise_abort(Ctx& cx) {
  __hip_atomic_store(G(cx.abort_flag), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(G(cx.abort_host), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ bool should_stop(Ctx& cx, uint64_t t0) {
  if (__hip_atomic_load(G(cx.abort_flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) return true;
  if (__builtin_amdgcn_s_memrealtime() - t0 > cx.timeout) {
    raise_abort(cx);
    return true;
  }
  return false;
}

// Spin until *p >= want (relaxed reads; the caller issues any acquire fence).
// `cache` keeps the last value read [C23 "Simple 的 Credit 与 Step": the wait
// loop reloads connStepCache only while it is short of the desired step].
__device__ bool wait_cached(const uint64_t* p, uint64_t want, uint64_t& cache, Ctx& cx) {
  if (cache >= want) return true;
  cache = load_relaxed(p);
  if (cache >= want) return true;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t it = 1;; ++it) {
    __builtin_amdgcn_s_sleep(1);
    cache = load_relaxed(p);
    if (cache >= want) return true;
    if ((it & 31u) == 0 && should_stop(cx, t0)) return false;
  }
}

__device__ __forceinline__ bool wait_geq(const uint64_t* p, uint64_t want, Ctx& cx) {
  uint64_t cache = 0;
  return wait_cached(p, want, cache, cx);
}

// Sender credit [C23 "Simple 的 Credit 与 Step"]: head + NCCL_STEPS >= step + n.
__device__ __forceinline__ bool wait_credit(Ctx& cx, uint64_t n) {
  const uint64_t need = cx.send_step + n;
  return need <= (uint64_t)kSteps ? true : wait_cached(cx.send_head, need - kSteps, cx.head_cache, cx);
}

// ---------------------------------------------------------------- Simple
// Loads in flight per thread and per source in reduceCopy (16-byte vectors;
// bf16, whose per-element widening needs more registers, keeps fewer), and
// whether the user buffers (each read once, written once) and the FIFO slots
// are accessed with the non-temporal hint, so that streaming user data does
// not push the FIFO slots (re-read moments later on the same XCD) out of L2.
// Measured on MI355X at 64 MiB x 4 ranks: user-buffer hint on, FIFO hint off.
// Vectors in flight, fp32 64 MiB x 4 ranks: 4 -> 212.0 us, 8 -> 207.5, 12 ->
// 213.0 (a larger remainder after the last whole block), 16 -> 205.0; int32
// 128 MiB x 8 ranks: 835.5 / 833.3 / 839.5 / 831.7 us; bf16 64 MiB x 8 ranks:
// 8 -> 425.4 us against 431.0 with 4 and 431.4 with 16 (with the hardware
// bf16 rounding).  16 keeps 2 waves per SIMD, as 4 did (218-222 registers).
// Performance only.
#ifndef RAR_UNROLL
#define RAR_UNROLL 16
#endif
#ifndef RAR_UNROLL_BF16
#define RAR_UNROLL_BF16 8
#endif
#ifndef RAR_NT_USER
#define RAR_NT_USER 1
#endif
#ifndef RAR_NT_FIFO
#define RAR_NT_FIFO 0
#endif
// Direct variants: the chunk written into the next rank's receive buffer is
// read back by that rank one hop later, like a FIFO slot.
#ifndef RAR_NT_DIRECT
#define RAR_NT_DIRECT 0
#endif

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

template <class Ty>
__device__ __forceinline__ v4u red16(v4u a, v4u b) {
  v4u r;
  r.x = Ty::red_word(a.x, b.x);
  r.y = Ty::red_word(a.y, b.y);
  r.z = Ty::red_word(a.z, b.z);
  r.w = Ty::red_word(a.w, b.w);
  return r;
}
template <class Ty>
__device__ __forceinline__ v4u pre16(v4u a, uint32_t s) {
  v4u r;
  r.x = Ty::pre_word(a.x, s);
  r.y = Ty::pre_word(a.y, s);
  r.z = Ty::pre_word(a.z, s);
  r.w = Ty::pre_word(a.w, s);
  return r;
}
template <class Ty>
__device__ __forceinline__ v4u post16(v4u a, int n) {
  v4u r;
  r.x = Ty::post_word(a.x, n);
  r.y = Ty::post_word(a.y, n);
  r.z = Ty::post_word(a.z, n);
  r.w = Ty::post_word(a.w, n);
  return r;
}
// User buffers need only element alignment [C23 "LL128：15/16 Payload": a
// misaligned user buffer takes a staging path there].  gfx950 serves
// unaligned global loads and stores in hardware (the target runs in
// unaligned access mode), so user data is read and written through an
// under-aligned 16-byte type: the same dwordx4 instructions as the aligned
// case, split by the memory system where they cross a cache line.  FIFO
// slots stay 16-byte aligned.
typedef uint32_t v4u_user __attribute__((ext_vector_type(4), aligned(2)));
typedef uint64_t u64_user __attribute__((aligned(2)));
typedef __attribute__((address_space(1))) v4u_user g_v4u_user;
typedef __attribute__((address_space(1))) u64_user g_u64_user;
typedef __attribute__((address_space(1))) v4u g_v4u;

// Vector i of a buffer: kUser = element-aligned user buffer, else a FIFO
// slot.  The pointer types are spelled out here (an alignment attribute on a
// typedef does not survive a template argument).
template <bool kNt, bool kUser>
__device__ __forceinline__ v4u ldv(const void* base, int64_t i) {
  if constexpr (kUser) {
    const g_v4u_user* p = (const g_v4u_user*)base + i;
    if constexpr (kNt) return __builtin_nontemporal_load(p);
    else return *p;
  } else {
    const g_v4u* p = (const g_v4u*)base + i;
    if constexpr (kNt) return __builtin_nontemporal_load(p);
    else return *p;
  }
}
template <bool kNt, bool kUser>
__device__ __forceinline__ void stv(void* base, int64_t i, v4u v) {
  if constexpr (kUser) {
    g_v4u_user* p = (g_v4u_user*)base + i;
    const v4u_user w = v;
    if constexpr (kNt) __builtin_nontemporal_store(w, p);
    else *p = w;
  } else {
    g_v4u* p = (g_v4u*)base + i;
    if constexpr (kNt) __builtin_nontemporal_store(v, p);
    else *p = v;
  }
}

// reduceCopy over n elements with 16-byte vectors, kUnroll in flight per
// thread and source; consecutive threads touch consecutive 16-byte vectors.
// The call that combines a partial with the own input and writes the output
// is the owner's final step, which also applies the post-op (divisor n_post).
// `fin` / `fout` are FIFO slots, or user buffers in the direct variants
// (kUserIn / kUserOut), which then take the user-buffer access hint.
// PreMulSum scales the own input by s_own and, when `fin` is the previous
// rank's raw input (kRawIn, direct read), that by s_in.
template <class Ty, bool kRecv, bool kSrc, bool kDst, bool kSend, bool kUserIn = false,
          bool kUserOut = false, bool kRawIn = false>
__device__ __forceinline__ void reduce_copy(const typename Ty::S* fin, const typename Ty::S* src,
                                            typename Ty::S* dst, typename Ty::S* fout, int64_t n,
                                            int tid, int nthr, int n_post, uint32_t s_own = 0,
                                            uint32_t s_in = 0) {
  using S = typename Ty::S;
  constexpr bool kPost = kRecv && kSrc && kDst && Ty::kPost;
  constexpr bool kPreOwn = kSrc && Ty::kPre;
  constexpr bool kPreIn = kRecv && kRawIn && Ty::kPre;
  constexpr int kVec = 16 / sizeof(S);
  constexpr int kUnroll = sizeof(S) == 2 ? RAR_UNROLL_BF16 : RAR_UNROLL;
  constexpr bool kNu = RAR_NT_USER != 0;
  constexpr bool kNi = kUserIn ? RAR_NT_DIRECT != 0 : RAR_NT_FIFO != 0;
  constexpr bool kNo = kUserOut ? RAR_NT_DIRECT != 0 : RAR_NT_FIFO != 0;
  // The unrolled loop runs on wave-uniform indices (scalar registers, so it
  // branches per wave): block ib covers ib + lane + u * nthr for every lane.
  const int64_t nv = uni64(n / kVec);
  const int nth = __builtin_amdgcn_readfirstlane(nthr);
  const int lane = tid & 63;
  const int64_t istep = (int64_t)kUnroll * nth;
  auto full = [&](int64_t ib) { return ib + 63 + (int64_t)(kUnroll - 1) * nth < nv; };
  auto load = [&](int64_t ib, v4u* a, v4u* b) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (kRecv) a[u] = ldv<kNi, kUserIn>(fin, ib + lane + (int64_t)u * nth);
      if (kSrc) b[u] = ldv<kNu, true>(src, ib + lane + (int64_t)u * nth);
    }
  };
  auto reduce_store = [&](int64_t ib, v4u* a, v4u* b) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if constexpr (kPreOwn) b[u] = pre16<Ty>(b[u], s_own);
      if constexpr (kPreIn) a[u] = pre16<Ty>(a[u], s_in);
      v4u r = (kRecv && kSrc) ? red16<Ty>(a[u], b[u]) : (kRecv ? a[u] : b[u]);
      if constexpr (kPost) r = post16<Ty>(r, n_post);
      if (kDst) stv<kNu, true>(dst, ib + lane + (int64_t)u * nth, r);
      if (kSend) stv<kNo, kUserOut>(fout, ib + lane + (int64_t)u * nth, r);
    }
  };
  int64_t ib = __builtin_amdgcn_readfirstlane(tid - lane);
  for (; full(ib); ib += istep) {
    v4u a[kUnroll], b[kUnroll];
    load(ib, a, b);
    reduce_store(ib, a, b);
  }
  int64_t i = ib + lane;
  for (; i < nv; i += nthr) {
    v4u a = {0, 0, 0, 0}, b = a;
    if (kRecv) a = ldv<kNi, kUserIn>(fin, i);
    if (kSrc) b = ldv<kNu, true>(src, i);
    if constexpr (kPreOwn) b = pre16<Ty>(b, s_own);
    if constexpr (kPreIn) a = pre16<Ty>(a, s_in);
    v4u r = (kRecv && kSrc) ? red16<Ty>(a, b) : (kRecv ? a : b);
    if constexpr (kPost) r = post16<Ty>(r, n_post);
    if (kDst) stv<kNu, true>(dst, i, r);
    if (kSend) stv<kNo, kUserOut>(fout, i, r);
  }
  for (int64_t e = nv * kVec + tid; e < n; e += nthr) {
    S a = 0, b = 0;
    if (kRecv) a = G(fin)[e];
    if (kSrc) b = G(src)[e];
    if constexpr (kPreOwn) b = Ty::pre_elem(b, s_own);
    if constexpr (kPreIn) a = Ty::pre_elem(a, s_in);
    S r = (kRecv && kSrc) ? Ty::red_elem(a, b) : (kRecv ? a : b);
    if constexpr (kPost) r = Ty::post_elem(r, n_post);
    if (kDst) G(dst)[e] = r;
    if (kSend) G(fout)[e] = r;
  }
}

// One Simple primitive call: SlicePerChunk slices; each slice waits (role
// threads of wave 0), moves data (all workers), then publishes (role thread
// of the last wave) [C23 "Primitive API 是模板组合", "Simple 的线程角色",
// "发布顺序与 Fence", "Slice Size"].  Empty slices still wait and post.
template <class Ty, int OP>
__device__ void simple_call(Ctx& cx, const typename Ty::S* src, typename Ty::S* dst,
                            typename Ty::S* next_dst, const typename Ty::S* prev_src, bool raw,
                            int64_t nelem, int chunk) {
  using S = typename Ty::S;
  using O = OpTraits<OP>;
  // Direct variants [C23 "发布顺序与 Fence"]: the final value goes straight
  // into the next rank's receive buffer (no FIFO slot: no credit wait), and
  // the all-gather receivers find their data in their own receive buffer.
  // With the direct read the loop's opening send moves nothing and the next
  // rank's first receive (`raw`) reads the raw input from this rank's send
  // buffer (prev_src on its side).  Steps, waits and posts are unchanged.
  const bool direct_send = cx.direct && (OP == kOpRecvReduceCopySend || OP == kOpRecvCopySend);
  const bool skip_send = cx.direct_read && OP == kOpSend;
  const bool read_prev = cx.direct_read && raw;
  constexpr int kVec = 16 / sizeof(S);
  const int sps = cx.sps;
  const int64_t step_elems = cx.step_bytes / (int64_t)sizeof(S);
  const int spc = cx.spc;
  int64_t slice = div_up(nelem, 16 * spc) * 16;
  const int64_t floor_slice = step_elems * sps / 32;
  if (slice < floor_slice) slice = floor_slice;
  for (int s = 0; s < spc; ++s) {
    const int64_t s_off = (int64_t)s * slice;
    const int64_t s_n = clamp64(nelem - s_off, 0, slice);
    // this lane's part of the slice, in whole 128-byte cache lines, so every
    // lane's stream starts on a line boundary (measured at 64 MiB over 10
    // lanes: 214 -> 212 us against 16-byte parts)
    constexpr int64_t kLine = 128 / sizeof(S);
    const int64_t part = kLine * div_up(div_up(s_n, kLine), cx.split_lanes);
    const int64_t lo = clamp64((int64_t)cx.split_lane * part, 0, s_n);
    const int64_t hi = clamp64(lo + part, 0, s_n);
    const uint64_t t0 = cx.trace ? now_ticks() : 0;
    const uint64_t step0 = cx.recv_step;
    // wait roles (lanes 0 and 1 of wave 0): the receiver needs
    // tail >= step + StepPerSlice, the sender head + NCCL_STEPS >= step + StepPerSlice
    if (cx.tid < 2) {
      bool ok = true;
      if (cx.tid == 0 && O::kRecv) ok = wait_cached(cx.recv_tail, cx.recv_step + sps, cx.tail_cache, cx);
      if (cx.tid == 1 && O::kSend && !direct_send && !skip_send) ok = wait_credit(cx, sps);
      acquire_fence();
      if (!ok) cx.sh->abort = 1;
    }
    __syncthreads();
    if (cx.sh->abort) {
      cx.aborted = true;
      return;
    }
    const uint64_t t1 = cx.trace ? now_ticks() : 0;
    if (cx.tid < cx.workers && hi > lo && !skip_send) {
      const S* fin = reinterpret_cast<const S*>(cx.recv_fifo + (cx.recv_step % kSteps) * cx.lane_step_bytes);
      S* fout = reinterpret_cast<S*>(cx.send_fifo + (cx.send_step % kSteps) * cx.lane_step_bytes);
      const int64_t e0 = s_off + lo;
      if (read_prev && OP == kOpRecvReduceSend) {
        // previous rank's raw input + own input -> FIFO
        reduce_copy<Ty, true, true, false, true, true, false, true>(prev_src + e0, src + e0, dst + e0, fout,
                                                                    hi - lo, cx.tid, cx.workers, cx.nranks,
                                                                    cx.s_own, cx.s_prev);
      } else if (read_prev && OP == kOpRecvReduceCopySend) {
        // two ranks: previous rank's raw input + own input -> own output, forwarded
        if (cx.direct)
          reduce_copy<Ty, true, true, true, true, true, true, true>(prev_src + e0, src + e0, dst + e0,
                                                                    next_dst + e0, hi - lo, cx.tid,
                                                                    cx.workers, cx.nranks, cx.s_own,
                                                                    cx.s_prev);
        else
          reduce_copy<Ty, true, true, true, true, true, false, true>(prev_src + e0, src + e0, dst + e0, fout,
                                                                     hi - lo, cx.tid, cx.workers, cx.nranks,
                                                                     cx.s_own, cx.s_prev);
      } else if (!cx.direct || OP == kOpSend || OP == kOpRecvReduceSend) {
        reduce_copy<Ty, O::kRecv, O::kSrc, O::kDst, O::kSend>(fin, src + e0, dst + e0, fout, hi - lo,
                                                               cx.tid, cx.workers, cx.nranks, cx.s_own);
      } else if (OP == kOpRecvReduceCopySend) {
        // FIFO partial + own input -> own output and the next rank's output
        reduce_copy<Ty, true, true, true, true, false, true>(fin, src + e0, dst + e0, next_dst + e0,
                                                             hi - lo, cx.tid, cx.workers, cx.nranks,
                                                             cx.s_own);
      } else if (OP == kOpRecvCopySend) {
        // already in the own output (written by prev) -> the next rank's output
        reduce_copy<Ty, true, false, false, true, true, true>(dst + e0, src + e0, dst + e0,
                                                              next_dst + e0, hi - lo, cx.tid,
                                                              cx.workers, cx.nranks);
      }
      // direct recv: the data is already in place
    }
    drain_vmem();
    __syncthreads();
    if (cx.trace) trace_unit(cx, OP, chunk, s_n, step0, t0, t1, now_ticks());
    if (O::kRecv) cx.recv_step += sps;
    if (O::kSend) cx.send_step += sps;
    // post roles (the last two lanes).  Every wave drained its memory
    // operations before the barrier, so the slice's FIFO reads are complete
    // (head needs nothing more) and its payload stores sit in this XCD's L2;
    // a receiver on another XCD additionally needs them written back.
    if (cx.tid == cx.nthreads - 2 && O::kRecv && !cx.drop_head) store_relaxed(cx.recv_head, cx.recv_step);
    if (cx.tid == cx.nthreads - 1 && O::kSend) {
      // to a receiver on this XCD the tail, like the payload before it, only
      // has to reach the shared L2: a workgroup-scope store
      if (cx.local_send) {
        store_relaxed_xcd(cx.send_tail, cx.send_step);
      } else {
        if (!skip_send) release_fence();
        store_relaxed(cx.send_tail, cx.send_step);
      }
    }
  }
}

// ---------------------------------------------------------------- LL
// 16-byte line: {data1, flag1, data2, flag2}, flags = step+1 [C23 "LL：Data
// 与 Flag 同 Line"].  Each half is one 64-bit atomic access, so a half whose
// flag matches carries that step's data and no fence is needed on either
// side.  Every worker thread checks the sender credit itself (cached, so
// usually without a load) and keeps kLlUnroll lines in flight.
constexpr int kLlUnroll = 4;

// LL cleanup [C23 "LL：Data 与 Flag 同 Line": when the flag period is about
// to wrap, the sender stamps the rest of the slot with the current flag].
// Cleanup steps are the last NCCL_STEPS steps of each half of the flag
// period, so each slot is restamped at least once per half period and no
// line keeps a generation that could come round again (nor the zero of a
// never-written line, which flag 0 would match).
__device__ __forceinline__ bool ll_cleanup_step(uint64_t step, uint32_t mask) {
  const uint64_t half = ((uint64_t)mask + 1) >> 1;
  return ((step + 1) & (half - 1)) >= half - kSteps;
}

__device__ __forceinline__ bool ll_ready(uint64_t a, uint64_t b, uint32_t flag) {
  return (uint32_t)(a >> 32) == flag && (uint32_t)(b >> 32) == flag;
}

// Reload a line until both flags carry `flag`.
__device__ bool ll_wait_line(const uint64_t* line, uint32_t flag, uint64_t& a, uint64_t& b, Ctx& cx) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (uint32_t it = 1;; ++it) {
    a = load_relaxed(line);
    b = load_relaxed(line + 1);
    if (ll_ready(a, b, flag)) return true;
    if ((it & 63u) == 0 && should_stop(cx, t0)) return false;
  }
}

template <class S>
__device__ __forceinline__ uint64_t load_bytes8(const uint8_t* p, int64_t valid) {
  if (valid >= 8) return *(const g_u64_user*)p;
  uint64_t v = 0;
  for (int64_t b = 0; b < valid; b += sizeof(S))
    v |= (uint64_t)(*G(reinterpret_cast<const S*>(p + b))) << (8 * b);
  return v;
}
template <class S>
__device__ __forceinline__ void store_bytes8(uint8_t* p, uint64_t v, int64_t valid) {
  if (valid >= 8) {
    *(g_u64_user*)p = v;
    return;
  }
  for (int64_t b = 0; b < valid; b += sizeof(S)) *G(reinterpret_cast<S*>(p + b)) = (S)(v >> (8 * b));
}

template <class Ty, int OP>
__device__ void ll_call(Ctx& cx, const typename Ty::S* src, typename Ty::S* dst, int64_t nelem,
                        int chunk) {
  using S = typename Ty::S;
  using O = OpTraits<OP>;
  constexpr int U = kLlUnroll;
  const int64_t nbytes = nelem * (int64_t)sizeof(S);
  const int64_t nlines = div_up(nbytes, 8);
  const int64_t part = div_up(nlines, cx.split_lanes);
  const int64_t lo = clamp64((int64_t)cx.split_lane * part, 0, nlines);
  const int64_t hi = clamp64(lo + part, 0, nlines);
  const uint64_t t0 = cx.trace ? now_ticks() : 0;
  const uint64_t step0 = cx.recv_step;
  bool ok = true;
  const bool worker = cx.tid < cx.workers;
  // a cleanup step writes the whole slot, so it needs the credit even with no lines
  const bool cleanup = O::kSend && ll_cleanup_step(cx.send_step, cx.ll_mask);
  if (O::kSend && worker && (lo < hi || cleanup)) ok = wait_credit(cx, 1);
  const uint64_t t1 = cx.trace ? now_ticks() : 0;
  const uint32_t rflag = (uint32_t)(cx.recv_step + 1) & cx.ll_mask;
  const uint32_t sflag = (uint32_t)(cx.send_step + 1) & cx.ll_mask;
  // line j of the step sits at line j - lo of this lane's slot
  const uint64_t* rl = reinterpret_cast<const uint64_t*>(cx.recv_fifo + (cx.recv_step % kSteps) * cx.lane_step_bytes) - 2 * lo;
  uint64_t* sl = reinterpret_cast<uint64_t*>(cx.send_fifo + (cx.send_step % kSteps) * cx.lane_step_bytes) - 2 * lo;
  const uint8_t* sb = reinterpret_cast<const uint8_t*>(src);
  uint8_t* db = reinterpret_cast<uint8_t*>(dst);
  if (worker && ok) {
    const int64_t stride = cx.workers;
    for (int64_t j0 = lo + cx.tid; j0 < hi && ok; j0 += (int64_t)U * stride) {
      uint64_t a[U], b[U], own[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = j0 + (int64_t)u * stride;
        a[u] = b[u] = own[u] = 0;
        if (j < hi) {
          if (O::kRecv) {
            a[u] = load_relaxed(rl + 2 * j);
            b[u] = load_relaxed(rl + 2 * j + 1);
          }
          if (O::kSrc) {
            own[u] = load_bytes8<S>(sb + 8 * j, nbytes - 8 * j);
            if constexpr (Ty::kPre) own[u] = pre8<Ty>(own[u], cx.s_own);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = j0 + (int64_t)u * stride;
        if (O::kRecv && j < hi && !ll_ready(a[u], b[u], rflag))
          ok = ok && ll_wait_line(rl + 2 * j, rflag, a[u], b[u], cx);
      }
      if (!ok) break;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = j0 + (int64_t)u * stride;
        if (j >= hi) continue;
        const uint64_t in = (a[u] & 0xffffffffull) | (b[u] << 32);
        uint64_t v = (O::kRecv && O::kSrc) ? red8<Ty>(in, own[u]) : (O::kRecv ? in : own[u]);
        if constexpr (OP == kOpRecvReduceCopySend && Ty::kPost) v = post8<Ty>(v, cx.nranks);
        if (O::kDst) store_bytes8<S>(db + 8 * j, v, nbytes - 8 * j);
        if (O::kSend) {
          // to a receiver on this XCD at workgroup scope: the half-lines merge
          // in the shared L2 instead of each being written through as an
          // 8-byte partial write (measured at 64 MiB over 12 channels: 1100
          // -> 643 us; no change at 512 KiB, which is latency-bound)
          const uint64_t h0 = (v & 0xffffffffull) | ((uint64_t)sflag << 32);
          const uint64_t h1 = (v >> 32) | ((uint64_t)sflag << 32);
          if (cx.local_send) {
            store_relaxed_xcd(sl + 2 * j, h0);
            store_relaxed_xcd(sl + 2 * j + 1, h1);
          } else {
            store_relaxed(sl + 2 * j, h0);
            store_relaxed(sl + 2 * j + 1, h1);
          }
        }
      }
    }
  }
  if (cleanup && worker && ok) {
    // lines [hi - lo, cap) of this lane's slot take the current flag; they
    // complete before the barrier, ahead of any later write to the slot
    const int64_t cap = cx.lane_step_bytes / 16;
    const uint64_t stamp = (uint64_t)sflag << 32;
    for (int64_t p = hi - lo + cx.tid; p < cap; p += cx.workers) {
      store_relaxed(sl + 2 * (lo + p), stamp);
      store_relaxed(sl + 2 * (lo + p) + 1, stamp);
    }
    drain_vmem();
  }
  if (!ok) cx.sh->abort = 1;
  // Every line value was consumed before this barrier, so every line read of
  // the step has completed: the slot can be handed back.
  __syncthreads();
  if (cx.sh->abort) {
    cx.aborted = true;
    return;
  }
  if (cx.trace) trace_unit(cx, OP, chunk, nelem, step0, t0, t1, now_ticks());
  if (O::kRecv) cx.recv_step += 1;
  if (O::kSend) cx.send_step += 1;
  if (O::kRecv && cx.tid == cx.nthreads - 1 && !cx.drop_head) store_relaxed(cx.recv_head, cx.recv_step);
}

// ---------------------------------------------------------------- LL128
// 128-byte line = 16 words: words 0..14 payload, word 15 = step+1 [C23
// "LL128：15/16 Payload"].  A wave covers 8 lines per pass, 8 lanes per line,
// 16 bytes per lane; lane 7 of each line holds word 14 and the flag word.
// Sender: every wave stores the data words of its lines, drains (plus an L2
// write-back when the receiver is on another XCD), then stores the flag words
// (at workgroup scope to a receiver on this XCD).  Receiver: each wave waits
// for one flag per group of lines it is about to read (the flags follow all
// of those lines' data) and reads the lines with agent-coherent loads.
// Groups of 8 lines in flight per wave: 4 for 4-byte payloads, 3 for bf16,
// whose operators need more registers (measured at 64 MiB against 2 groups:
// fp32 -2 %, int32 -2 %, bf16 -2 %; bf16 with 4 spills more and is slower).
#ifndef RAR_LL128_UNROLL
#define RAR_LL128_UNROLL 4
#endif
#ifndef RAR_LL128_UNROLL_BF16
#define RAR_LL128_UNROLL_BF16 3
#endif
// Word 3 of a raw buffer resource on gfx9 (untyped access), and the cache
// policy bit of an agent-coherent load (sc1).
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kCpolSc1 = 16;
template <class S>
constexpr int ll128_unroll() {
  return sizeof(S) == 2 ? RAR_LL128_UNROLL_BF16 : RAR_LL128_UNROLL;
}

// Wait until every vector memory operation this wave has issued has
// completed (stores: reached L2).  The asm is also a compiler barrier: no
// memory access moves across it.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Orders this wave's LDS accesses around a hand-off between its lanes.  The
// fences cover LDS only ("local"): a fence over all address spaces would also
// wait for the wave's outstanding global stores.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

template <class S>
__device__ __forceinline__ v4u load_bytes16(const uint8_t* p, int64_t valid, int64_t cap) {
  // 8-byte aligned source; `cap` = 16 or 8 bytes owned by the lane
  uint64_t lo = 0, hi = 0;
  if (valid > 0) lo = load_bytes8<S>(p, valid);
  if (cap > 8 && valid > 8) hi = load_bytes8<S>(p + 8, valid - 8);
  v4u r = {(uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi, (uint32_t)(hi >> 32)};
  return r;
}
template <class S>
__device__ __forceinline__ void store_bytes16(uint8_t* p, v4u v, int64_t valid, int64_t cap) {
  if (valid > 0) store_bytes8<S>(p, (uint64_t)v.x | ((uint64_t)v.y << 32), valid);
  if (cap > 8 && valid > 8) store_bytes8<S>(p + 8, (uint64_t)v.z | ((uint64_t)v.w << 32), valid - 8);
}

template <class Ty, int OP>
__device__ void ll128_call(Ctx& cx, const typename Ty::S* src, typename Ty::S* dst, int64_t nelem,
                           int chunk) {
  using S = typename Ty::S;
  using O = OpTraits<OP>;
  constexpr int U = ll128_unroll<S>();
  // the share's bounds and the wave index are the same on every lane of a
  // wave: held in scalar registers, the loops below branch per wave rather
  // than through lane masks
  const int64_t nbytes = uni64(nelem * (int64_t)sizeof(S));
  const int64_t nlines = div_up(nbytes, 120);
  // lanes take an even number of lines, so every group of 8 lines starts
  // 16-byte aligned in the user buffer (120 x 2 = 15 x 16)
  const int64_t part = 2 * div_up(nlines, 2 * (int64_t)cx.split_lanes);
  const int64_t lo = uni64(clamp64((int64_t)cx.split_lane * part, 0, nlines));
  const int64_t hi = uni64(clamp64(lo + part, 0, nlines));
  const uint64_t t0 = cx.trace ? now_ticks() : 0;
  const uint64_t step0 = cx.recv_step;
  const int wave = __builtin_amdgcn_readfirstlane(cx.tid >> 6), lid = cx.tid & 63;
  const int nw = __builtin_amdgcn_readfirstlane(cx.workers >> 6);
  const int sub = lid >> 3;  // line within the wave's group of 8
  const int k = lid & 7;     // 16-byte segment of the line

  const int64_t first = lo + (int64_t)wave * 8, stride = (int64_t)nw * 8;
  const bool active = wave < nw && first < hi;
  bool ok = true;
  if (O::kSend && active) ok = wait_credit(cx, 1);
  const uint64_t t1 = cx.trace ? now_ticks() : 0;
  const uint64_t rflag = cx.recv_step + 1, sflag = cx.send_step + 1;
  // line j of the step sits at line j - lo of this lane's slot
  const uint64_t* rl = reinterpret_cast<const uint64_t*>(cx.recv_fifo + (cx.recv_step % kSteps) * cx.lane_step_bytes) - 16 * lo;
  uint64_t* sl = reinterpret_cast<uint64_t*>(cx.send_fifo + (cx.send_step % kSteps) * cx.lane_step_bytes) - 16 * lo;
  const uint8_t* sb = reinterpret_cast<const uint8_t*>(src);
  uint8_t* db = reinterpret_cast<uint8_t*>(dst);
  // The receive slot as a buffer resource: its FIFO words are read with
  // agent-coherent (sc1) loads, like the flag words, so they read the L2 the
  // sender wrote and need no L1 invalidation first.
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      cx.recv_fifo + (cx.recv_step % kSteps) * cx.lane_step_bytes, 0, (int)cx.lane_step_bytes,
      kRawBufferWord3);
  // every lane of a wave read the same words: a wave-uniform answer, so
  // the loops below compile to scalar branches
  ok = __builtin_amdgcn_readfirstlane(ok ? 1 : 0) != 0;
  if (active && ok) {
    // A wave moves groups of 8 lines: 960 payload bytes, 1 KiB of FIFO.
    // User data goes through an LDS tile [C23 "LL128：15/16 Payload" stages
    // user data through shared memory]: 60 lanes load or store 16
    // contiguous user bytes each, and the tile is read or written in
    // line layout (lane (line, segment), 16 bytes, 8 in the last segment).
    // Every lane then stores its 16 FIFO bytes with one instruction; the
    // flag word gets a placeholder 0 that never matches a flag, and the
    // real flag follows after the drain below.
    constexpr bool kNu = RAR_NT_USER != 0;
    uint8_t* stage = cx.stage + (int64_t)wave * U * 1024;
    const int64_t ub = 16 * (int64_t)lid;  // this lane's 16 bytes of a group, user layout
    const bool ulane = lid < 60;
    const v4u zero = {0, 0, 0, 0};
    // The FIFO words (in) and user bytes (x) of U groups of 8 lines, group u
    // starting at line g + u * stride.  whole(g): all U groups are full
    // lines inside the step and the chunk.
    auto whole = [&](int64_t g) {
      const int64_t last_end = g + (int64_t)(U - 1) * stride + 8;
      return last_end <= hi && 120 * last_end <= nbytes;
    };
    // this lane's 16 bytes of line j of the receive slot
    auto fifo_load = [&](int64_t j) -> v4u {
      return __builtin_amdgcn_raw_buffer_load_b128(rsrc, (uint32_t)(128 * (j - lo) + 16 * k), 0, kCpolSc1);
    };
    auto load_whole = [&](int64_t g, v4u* in, v4u* x) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = g + (int64_t)u * stride + sub;
        in[u] = zero;
        if (O::kRecv) {
          // lane 7's upper half is the line's flag word: process() drops
          // it (a zeroing here would wait for the load)
          in[u] = fifo_load(j);
        }
      }
      // lanes 60..63 hold no user bytes of a group: they repeat lane 0's
      // load (in bounds) so that no load needs a branch around it
#pragma unroll
      for (int u = 0; u < U; ++u)
        x[u] = O::kSrc ? ldv<kNu, true>(sb + 120 * (g + (int64_t)u * stride) + (ulane ? ub : 0), 0) : zero;
    };
    auto load_part = [&](int64_t g, v4u* in, v4u* x) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t gs = g + (int64_t)u * stride;  // first line of group u
        const int64_t ge = gs + 8 < hi ? gs + 8 : hi;
        const int64_t gend = 120 * ge < nbytes ? 120 * ge : nbytes;
        const int64_t gvalid = gs < hi ? gend - 120 * gs : 0;  // payload bytes of the group
        const int64_t j = gs + sub;
        in[u] = zero;
        x[u] = zero;
        if (O::kRecv && j < hi) {
          in[u] = fifo_load(j);
          if (k == 7) in[u].z = in[u].w = 0;
        }
        if (O::kSrc && ulane) {
          if (ub + 16 <= gvalid) x[u] = ldv<kNu, true>(sb + 120 * gs + ub, 0);
          else if (ub < gvalid) x[u] = load_bytes16<S>(sb + 120 * gs + ub, gvalid - ub, 16);
        }
      }
    };
    // Reduce and store the U groups at g whose loads are in `in` and `x`;
    // kWhole: every group is whole (known at compile time: no bounds
    // checks around the stores).
    auto process = [&](auto kWhole, int64_t g, const v4u* in, const v4u* x) {
      v4u own[U];
#pragma unroll
      for (int u = 0; u < U; ++u) own[u] = zero;
      if (O::kSrc) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (ulane) *reinterpret_cast<v4u*>(stage + u * 1024 + ub) = x[u];
        wave_sync();
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint8_t* q = stage + u * 1024 + 120 * sub + 16 * k;
          const uint64_t w0 = *reinterpret_cast<const uint64_t*>(q);
          const uint64_t w1 = k < 7 ? *reinterpret_cast<const uint64_t*>(q + 8) : 0;
          own[u].x = (uint32_t)w0;
          own[u].y = (uint32_t)(w0 >> 32);
          own[u].z = (uint32_t)w1;
          own[u].w = (uint32_t)(w1 >> 32);
          if constexpr (Ty::kPre) own[u] = pre16<Ty>(own[u], cx.s_own);
        }
        wave_sync();  // the tile is read before it is written again
      }
      v4u v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        v[u] = (O::kRecv && O::kSrc) ? red16<Ty>(in[u], own[u]) : (O::kRecv ? in[u] : own[u]);
        if constexpr (OP == kOpRecvReduceCopySend && Ty::kPost) v[u] = post16<Ty>(v[u], cx.nranks);
        if (k == 7) v[u].z = v[u].w = 0;  // flag placeholder
        const int64_t j = g + (int64_t)u * stride + sub;
        if (O::kSend && (kWhole || j < hi)) *G(reinterpret_cast<v4u*>(sl + 16 * j + 2 * k)) = v[u];
      }
      if (O::kDst) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          uint8_t* q = stage + u * 1024 + 120 * sub + 16 * k;
          *reinterpret_cast<uint64_t*>(q) = (uint64_t)v[u].x | ((uint64_t)v[u].y << 32);
          if (k < 7) *reinterpret_cast<uint64_t*>(q + 8) = (uint64_t)v[u].z | ((uint64_t)v[u].w << 32);
        }
        wave_sync();
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (!ulane) continue;
          const int64_t gs = g + (int64_t)u * stride;
          const v4u y = *reinterpret_cast<const v4u*>(stage + u * 1024 + ub);
          if (kWhole) {
            stv<kNu, true>(db + 120 * gs + ub, 0, y);
            continue;
          }
          const int64_t ge = gs + 8 < hi ? gs + 8 : hi;
          const int64_t gend = 120 * ge < nbytes ? 120 * ge : nbytes;
          const int64_t gvalid = gs < hi ? gend - 120 * gs : 0;
          if (ub + 16 <= gvalid) stv<kNu, true>(db + 120 * gs + ub, 0, y);
          else if (ub < gvalid) store_bytes16<S>(db + 120 * gs + ub, y, gvalid - ub, 16);
        }
        wave_sync();
      }
    };
    // Whole groups run software-pipelined: the next iteration's loads are
    // issued before this iteration's stores, so they are in flight while
    // this iteration computes and stores.  Two register sets take turns
    // (no copies between them, which would wait for the loads); the last
    // whole iteration is peeled (nothing to prefetch).  The partial groups
    // at the end of a share follow unpipelined.
    const std::integral_constant<bool, true> kW{};
    const std::integral_constant<bool, false> kP{};
    const int64_t gstep = (int64_t)U * stride;
    // Flags to a receiver on this XCD go out while the step is still
    // being written: after an iteration's data stores, the wave waits for
    // every vector memory operation it has outstanding (those stores and
    // the next iteration's loads) and then stores that iteration's flags.
    // A flag thus lands in L2 after its line's data, and soon enough to
    // merge with the line while it is still there (a flag stored after
    // the whole step found most half-lines written back already, and they
    // went to memory twice).  Other flags, and every flag to a receiver on
    // another XCD, follow the drain at the end of the step.
    const bool early = O::kSend && __builtin_amdgcn_readfirstlane(cx.local_send ? 1 : 0) != 0;
    // pub and g0 pass through readfirstlane when they advance: they are
    // the same on every lane, but they merge right after the per-lane
    // flag stores, and without it the compiler keeps them per lane and
    // runs the loop on lane masks (measured: 3 % slower at 64 MiB)
    int64_t pub = first;  // first group whose flags are not out
    // flags of the iteration at g, once its data stores have retired
    auto publish = [&](int64_t g) {
      if (!early) return;
      wait_vmem();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t j = g + (int64_t)u * stride + sub;
        if (k == 7) store_relaxed_xcd(sl + 16 * j + 15, sflag);
      }
      pub = uni64(g + gstep);
    };
    // Receive group by group: before a wave loads the lines of an
    // iteration it waits for the flag of the iteration's first line.  The
    // sender stores an iteration's flags only after all of that
    // iteration's data stores have completed (the rest of the step's
    // flags after the step's drain), so one flag stands for every line of
    // the iteration.  The next iteration's flag is loaded one iteration
    // ahead: a sender that is ahead costs no extra round trip.  Measured
    // against wave 0 polling every flag of the step before any wave reads
    // (then one acquire and a barrier): 276 -> 245 us at 64 MiB, the
    // receivers no longer wait for whole steps of their senders.
    constexpr bool kGroupRecv = O::kRecv;
    auto wait_line = [&](int64_t j) -> bool {
      if constexpr (!kGroupRecv) return true;
      const uint64_t tp = __builtin_amdgcn_s_memrealtime();
      for (uint32_t it = 1;; ++it) {
        if (uni64(load_relaxed(rl + 16 * j + 15)) == rflag) break;
        __builtin_amdgcn_s_sleep(1);
        if ((it & 15u) == 0 && __builtin_amdgcn_readfirstlane(should_stop(cx, tp) ? 1 : 0) != 0)
          return false;
      }
      asm volatile("" ::: "memory");  // the lines' loads stay after the flag
      return true;
    };
    auto ready = [&](int64_t j, uint64_t seen) -> bool {
      if constexpr (!kGroupRecv) return true;
      if (uni64(seen) == rflag) {
        asm volatile("" ::: "memory");
        return true;
      }
      return wait_line(j);
    };
    auto peek = [&](int64_t j) -> uint64_t {
      if constexpr (!kGroupRecv) return 0;
      return j < hi ? load_relaxed(rl + 16 * j + 15) : 0;
    };
    int64_t g0 = first;
    if (g0 < hi && whole(g0) && (ok = wait_line(g0))) {
      v4u inA[U], xA[U], inB[U], xB[U];
      load_whole(g0, inA, xA);
      uint64_t seen = peek(g0 + gstep);
      for (;;) {
        if (!(g0 + gstep < hi && whole(g0 + gstep))) {
          process(kW, g0, inA, xA);
          publish(g0);
          g0 = uni64(g0 + gstep);
          break;
        }
        if (!(ok = ready(g0 + gstep, seen))) break;
        load_whole(g0 + gstep, inB, xB);
        seen = peek(g0 + 2 * gstep);
        process(kW, g0, inA, xA);
        publish(g0);
        g0 = uni64(g0 + gstep);
        if (!(g0 + gstep < hi && whole(g0 + gstep))) {
          process(kW, g0, inB, xB);
          publish(g0);
          g0 = uni64(g0 + gstep);
          break;
        }
        if (!(ok = ready(g0 + gstep, seen))) break;
        load_whole(g0 + gstep, inA, xA);
        seen = peek(g0 + 2 * gstep);
        process(kW, g0, inB, xB);
        publish(g0);
        g0 = uni64(g0 + gstep);
      }
    }
    for (; ok && g0 < hi; g0 = uni64(g0 + gstep)) {
      if (!(ok = wait_line(g0))) break;
      v4u in[U], x[U];
      load_part(g0, in, x);
      process(kP, g0, in, x);
    }
    if (O::kSend && ok) {
      // data words before flag words: drained into this L2, and written
      // back when the receiver runs on another XCD
      drain_vmem();
      if (!cx.local_send) release_fence();
      for (int64_t g = pub; g < hi; g += stride) {
        const int64_t j = g + sub;
        // to a receiver on this XCD the flag goes out at workgroup scope: it
        // merges into the line in L2 instead of being written through as
        // a partial line (measured: 472 -> 332 us at 64 MiB, partial
        // memory-side writes from 24 % to 6 %)
        if (j < hi && k == 7) {
          if (cx.local_send) store_relaxed_xcd(sl + 16 * j + 15, sflag);
          else store_relaxed(sl + 16 * j + 15, sflag);
        }
      }
    }
  }
  if (!ok) cx.sh->abort = 1;
  // every data word of the step was consumed before this barrier
  __syncthreads();
  if (cx.sh->abort) {
    cx.aborted = true;
    return;
  }
  if (cx.trace) trace_unit(cx, OP, chunk, nelem, step0, t0, t1, now_ticks());
  if (O::kRecv) cx.recv_step += 1;
  if (O::kSend) cx.send_step += 1;
  if (O::kRecv && cx.tid == cx.nthreads - 1 && !cx.drop_head) store_relaxed(cx.recv_head, cx.recv_step);
}

// ---------------------------------------------------------------- runRing
template <class Ty, int PROTO, int OP>
__device__ __forceinline__ void prim(Ctx& cx, const typename Ty::S* sendbuf, typename Ty::S* recvbuf,
                                     typename Ty::S* next_recvbuf, const typename Ty::S* prev_sendbuf,
                                     bool raw, int64_t base, int64_t cc, int64_t rem, int chunk) {
  const int64_t chunk_off = (int64_t)chunk * cc;
  const int64_t nelem = clamp64(rem - chunk_off, 0, cc);
  const int64_t off = base + chunk_off;
  if (PROTO == kSimple)
    simple_call<Ty, OP>(cx, sendbuf + off, recvbuf + off, next_recvbuf + off, prev_sendbuf + off, raw,
                        nelem, chunk);
  else if (PROTO == kLL)
    ll_call<Ty, OP>(cx, sendbuf + off, recvbuf + off, nelem, chunk);
  else
    ll128_call<Ty, OP>(cx, sendbuf + off, recvbuf + off, nelem, chunk);
}

// runRing [C12 "runRing 的数据切分" and steps one to five; C23 "Ring
// AllReduce 到 Primitive"]: loops of N chunks; the tail loop shrinks the
// chunk to alignUp(divUp(rem, N), 16 bytes); per loop the 2N-1 calls with
// chunk indices in ring-position coordinates.
template <class Ty, int PROTO>
__device__ __forceinline__ void run_ring(Ctx& cx, const DevWork& w) {
  using S = typename Ty::S;
  constexpr int kVec = 16 / sizeof(S);
  const int N = cx.nranks, ix = cx.ring_index;
  void* const* ptrs = cx.ptrs;
  const S* sendbuf = reinterpret_cast<const S*>(G(ptrs)[((int64_t)w.buf_index * N + cx.rank) * 2]);
  S* recvbuf = reinterpret_cast<S*>(G(ptrs)[((int64_t)w.buf_index * N + cx.rank) * 2 + 1]);
  S* next_recvbuf = reinterpret_cast<S*>(G(ptrs)[((int64_t)w.buf_index * N + cx.next) * 2 + 1]);
  const S* prev_sendbuf = reinterpret_cast<const S*>(G(ptrs)[((int64_t)w.buf_index * N + cx.prev) * 2]);
  if constexpr (Ty::kPre) {
    cx.s_own = G(cx.scalars)[(int64_t)w.buf_index * N + cx.rank];
    cx.s_prev = G(cx.scalars)[(int64_t)w.buf_index * N + cx.prev];
  }
  int workers = (int)w.n_waves * kWaveSize;
  cx.workers = workers < cx.nthreads ? workers : cx.nthreads;
  const int64_t loop_count = (int64_t)N * w.chunk_count;
  for (int64_t eo = 0; eo < w.channel_count; eo += loop_count) {
    const int64_t rem = w.channel_count - eo;
    const int64_t cc = rem < loop_count ? align_up(div_up(rem, N), kVec) : w.chunk_count;
    const int64_t base = w.grid_offset + eo;
    auto mod = [N](int x) { return ((x % N) + N) % N; };
    // the call right after the opening send receives that send's raw input
    prim<Ty, PROTO, kOpSend>(cx, sendbuf, recvbuf, next_recvbuf, prev_sendbuf, false, base, cc, rem,
                             mod(ix - 1));
    for (int j = 2; j < N && !cx.aborted; ++j)
      prim<Ty, PROTO, kOpRecvReduceSend>(cx, sendbuf, recvbuf, next_recvbuf, prev_sendbuf, j == 2,
                                         base, cc, rem, mod(ix - j));
    if (cx.aborted) return;
    prim<Ty, PROTO, kOpRecvReduceCopySend>(cx, sendbuf, recvbuf, next_recvbuf, prev_sendbuf, N == 2,
                                           base, cc, rem, ix);
    for (int j = 1; j < N - 1 && !cx.aborted; ++j)
      prim<Ty, PROTO, kOpRecvCopySend>(cx, sendbuf, recvbuf, next_recvbuf, prev_sendbuf, false, base,
                                       cc, rem, mod(ix - j));
    if (cx.aborted) return;
    prim<Ty, PROTO, kOpRecv>(cx, sendbuf, recvbuf, next_recvbuf, prev_sendbuf, false, base, cc, rem,
                             mod(ix + 1));
    if (cx.aborted) return;
  }
}

// ---------------------------------------------------------------- staging
// Copy `bytes` (multiple of 16) with one wave in 16-byte packs.
__device__ __forceinline__ void copy16(void* dst, const void* src, int bytes, int lid) {
  uint4* d = reinterpret_cast<uint4*>(dst);
  const uint4* s = reinterpret_cast<const uint4*>(src);
  for (int i = lid; i < bytes / 16; i += kWaveSize) d[i] = s[i];
}

// Load batch `b` into LDS with one wave [C23 "前两个 Warp 与 Work Loader"]:
// the k-th set bit of offset_bitset names the k-th work (found through an LDS
// scratch table), then 64 lanes x 16 bytes move up to 16 works of 64 bytes.
// The tables of a launch plan (see KernelArgs).
struct Plan {
  const DevBatch* batches;
  const DevWork* works;
  void* const* ptrs;
  const uint32_t* first_batch;
  const uint32_t* scalars;
};

__device__ void load_batch(Shmem& sh, const Plan& a, uint32_t b, int lid) {
  const DevBatch hdr = a.batches[b];
  const uint64_t bits = hdr.offset_bitset;
  if (lid == 0) {
    sh.batch = hdr;
    sh.n_works = __popcll(bits);
  }
  if ((bits >> lid) & 1ull) sh.slot_bit[__popcll(bits & ((1ull << lid) - 1ull))] = lid;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const int nw = __popcll(bits);
  const int k = lid >> 2, pack = lid & 3;
  if (k < nw) {
    const uint4* src = reinterpret_cast<const uint4*>(a.works + hdr.offset_base + sh.slot_bit[k]) + pack;
    reinterpret_cast<uint4*>(&sh.works[k])[pack] = *src;
  }
}

}  // namespace

// ---------------------------------------------------------------- entry
// LL128 workgroups are small (4 waves in the measured shape) and the protocol
// wants many of them: capping its registers at three waves per SIMD lets three
// such workgroups share a CU (fp32 and int32, with 4 groups of lines in flight,
// then spill 4 registers per lane, 12 for avg and PreMulSum; bf16 with 3
// groups spills none).  Measured at 64 MiB: this beats a two-waves-per-SIMD
// cap with 6 or 8 groups in flight and fewer workgroups (254-288 us against
// 246 us).
template <class Ty, int PROTO>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(PROTO == kLL128 ? 3 : 1)))
ring_allreduce_kernel(KernelArgs args) {
  __shared__ Shmem sh;
  __shared__ __attribute__((aligned(16))) uint8_t
      stage[PROTO == kLL128 ? kMaxWaves * ll128_unroll<typename Ty::S>() * 1024 : 16];
  const DevComm* comm = args.comm;
  // Startup is a chain of dependent loads, so the independent ones go out
  // together: the workgroup map and the channel mask here, the ring position,
  // step counters, channel batch and placement check below, between the same
  // two barriers.
  const uint32_t m = args.wg_map[blockIdx.x];
  const uint64_t mask = comm->hot.channel_mask;
  if (m == kIdleWg) return;
  // An inline plan is read where the dispatch put it, in the kernel-argument
  // segment (global memory), through that segment's base pointer.  Taking
  // the address of the parameter itself would let the compiler hand out a
  // private copy, which global loads cannot reach.
  const uint8_t* kernargs = (const uint8_t*)__builtin_amdgcn_kernarg_segment_ptr();
  const uint8_t* plan_base = args.inline_plan ? kernargs + offsetof(KernelArgs, plan) : args.arena;
  Plan plan;
  plan.batches = reinterpret_cast<const DevBatch*>(plan_base + args.off_batches);
  plan.works = reinterpret_cast<const DevWork*>(plan_base + args.off_works);
  plan.ptrs = reinterpret_cast<void* const*>(plan_base + args.off_ptrs);
  plan.first_batch = reinterpret_cast<const uint32_t*>(plan_base + args.off_first);
  plan.scalars = reinterpret_cast<const uint32_t*>(plan_base + args.off_scalars);
  const int tid = threadIdx.x, nthreads = blockDim.x;
  const int wave = tid >> 6, lid = tid & 63, nwaves = nthreads >> 6;
  const int rank = (int)(m & 0xFFu), n = (int)((m >> 8) & 0xFFu), lane = (int)((m >> 16) & 0xFFu);
  // Placement handshake, first half: one lane publishes this workgroup's XCD
  // with its launch count (each workgroup's own slot holds the count, so a
  // launch replayed from a captured graph counts as well).  The second half,
  // below, reads what the receiving workgroup published; both publish at
  // entry, so that read rarely has to wait.
  const int hs_wave = nwaves - 1;
  const bool hs_lane = wave == hs_wave && lid == 0;
  uint64_t epoch = 0;
  uint32_t my_xcc = 0, peer_wg = 0;
  if (hs_lane) {
    uint64_t* slot = &comm->hot.placement[blockIdx.x];
    peer_wg = comm->hot.wg_peer[blockIdx.x];
    my_xcc = xcc_id();
    epoch = (load_relaxed(slot) >> 8) + 1;
    store_relaxed(slot, (epoch << 8) | my_xcc);
  }
  // Block -> channel [C23 "Kernel 如何把 Block 映射到 Channel"]: the lanes of
  // wave 0 scan the 64 mask bits; the dense index n picks the n-th set bit.
  if (wave == 0) {
    if (lid == 0) {
      sh.channel_id = -1;
      sh.abort = 0;
      sh.local_send = 0;
    }
    // the lane of the channel id also fetches what depends on it alone
    if (((mask >> lid) & 1ull) && __popcll(mask & ((1ull << lid) - 1ull)) == n) {
      sh.channel_id = lid;
      sh.first_batch = plan.first_batch[lid];
      sh.me = comm->ranks[lid][rank];
    }
  }
  __syncthreads();
  if (sh.channel_id < 0) return;  // n beyond popcount(mask): not a channel of this launch
  const int C = __popcll(mask);
  const int nlanes = comm->hot.n_lanes;
  // Staging [C23 "前两个 Warp 与 Work Loader"]: wave 0 copies the
  // communicator hot fields, another wave the channel's first work batch.
  const uint32_t first = sh.first_batch;
  if (wave == 0) copy16(&sh.comm, &comm->hot, (int)sizeof(DevCommHot), lid);
  const int loader = nwaves > 1 ? 1 : 0;
  if (wave == loader) {
    if (first != 0) {
      load_batch(sh, plan, first, lid);
    } else if (lid == 0) {
      sh.n_works = 0;
      sh.batch = DevBatch{0, 0, 0};
    }
  }
  // step counters, read from global memory by every thread
  const DevRank me = sh.me;
  ConnCounters* rc = comm->hot.counters + ((int64_t)rank * C + n) * nlanes + lane;
  ConnCounters* sc = comm->hot.counters + ((int64_t)me.next * C + n) * nlanes + lane;
  // Steps persist across launches: this workgroup alone writes its receive
  // head and its send tail, so they hold where it stopped last time.
  const uint64_t recv_step0 = load_relaxed(&rc->head.value);
  const uint64_t send_step0 = load_relaxed(&sc->tail.value);
  // Placement handshake, second half: same XCD as the receiver = same L2 =
  // the cheap publication path; anything else takes the agent-scope release.
  // The dispatcher is not trusted: the check runs every launch.
  if (hs_lane) {
    const uint64_t* peer = &comm->hot.placement[peer_wg];
    const uint64_t timeout = comm->hot.spin_timeout_ticks;
    const uint32_t* abort_flag = comm->hot.abort_flag;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    uint64_t v = load_relaxed(peer);
    bool ok = true;
    for (uint32_t it = 1; v < (epoch << 8); ++it) {
      __builtin_amdgcn_s_sleep(1);
      v = load_relaxed(peer);
      if ((it & 31u) == 0 && v < (epoch << 8) &&
          (__hip_atomic_load(G(abort_flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ||
           __builtin_amdgcn_s_memrealtime() - t0 > timeout)) {
        ok = false;
        break;
      }
    }
    if (ok) {
      // strict scope: every publication takes the agent-scope path
      sh.local_send = (v & 0xFFu) == my_xcc && !comm->hot.strict_scope;
    } else {
      // the receiving workgroup never arrived (or another waiter gave up):
      // raise the communicator's abort word, as every bounded wait does
      __hip_atomic_store(G(comm->hot.abort_flag), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(G(comm->hot.abort_host), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      sh.abort = 1;
    }
  }
  __syncthreads();

  Ctx cx;
  cx.sh = &sh;
  cx.ptrs = plan.ptrs;
  cx.tid = tid;
  cx.nthreads = nthreads;
  cx.workers = nthreads;
  cx.rank = rank;
  cx.nranks = sh.comm.n_ranks;
  cx.ring_index = me.index;
  cx.next = me.next;
  cx.direct = (sh.comm.direct & 1) != 0;
  cx.direct_read = (sh.comm.direct & 2) != 0;
  cx.prev = me.prev;
  cx.lane = lane;
  cx.nlanes = nlanes;
  const bool deal = sh.comm.deal_works != 0;
  cx.split_lane = deal ? 0 : lane;
  cx.split_lanes = deal ? 1 : cx.nlanes;
  cx.sps = sh.comm.step_per_slice;
  cx.spc = sh.comm.slices_per_chunk;
  cx.step_bytes = sh.comm.step_bytes;
  cx.lane_step_bytes = sh.comm.lane_step_bytes;
  // each lane of a connector has its own FIFO of kSteps slots
  cx.recv_fifo = sh.comm.fifo + (((int64_t)rank * C + n) * cx.nlanes + lane) * sh.comm.lane_buff_bytes;
  cx.send_fifo = sh.comm.fifo + (((int64_t)me.next * C + n) * cx.nlanes + lane) * sh.comm.lane_buff_bytes;
  cx.recv_tail = &rc->tail.value;
  cx.recv_head = &rc->head.value;
  cx.send_tail = &sc->tail.value;
  cx.send_head = &sc->head.value;
  cx.recv_step = recv_step0;
  cx.send_step = send_step0;
  cx.tail_cache = 0;
  cx.head_cache = 0;
  cx.abort_flag = sh.comm.abort_flag;
  cx.abort_host = sh.comm.abort_host;
  cx.timeout = sh.comm.spin_timeout_ticks;
  cx.drop_head = (sh.comm.debug_flags & 1) != 0;
  cx.ll_mask = sh.comm.ll_flag_mask;
  cx.scalars = plan.scalars;
  cx.s_own = cx.s_prev = 0;
  cx.stage = stage;
  cx.aborted = false;
  cx.trace = (sh.comm.debug_flags & 2) ? sh.comm.trace + (int64_t)blockIdx.x * sh.comm.trace_cap : nullptr;
  cx.trace_n = 0;
  cx.trace_cap = (uint32_t)sh.comm.trace_cap;
  cx.local_send = sh.local_send != 0;
  if (sh.abort) return;

  // RunWorkBatch [C23 "RunWorkBatch 与 Fused Work"]: the works of a batch run
  // in order; a change of active waves between two works the workgroup runs
  // is fenced by a barrier; next_jump chains the channel's next batch.  With
  // dealt works, the k-th work of the channel (counted over all its batches)
  // runs on lane k mod n_lanes only, and the other lanes step over it.
  uint32_t b = first;
  int dealt = 0;         // with dealt works: the lane that runs the batch's first work
  int prev_waves = -1;   // active waves of the previous work this workgroup ran
  while (b != 0) {
    const int nworks = sh.n_works;
    // every work of the batch, or (dealt) this lane's first one and then
    // every n_lanes-th
    int w0 = 0, wstep = 1;
    if (deal) {
      w0 = lane - dealt;
      if (w0 < 0) w0 += cx.nlanes;
      wstep = cx.nlanes;
      dealt = (dealt + nworks) % cx.nlanes;
    }
    for (int w = w0; w < nworks; w += wstep) {
      const int nw = sh.works[w].n_waves;
      if (prev_waves >= 0 && nw != prev_waves) __syncthreads();
      prev_waves = nw;
      run_ring<Ty, PROTO>(cx, sh.works[w]);
      if (cx.aborted) break;
    }
    if (cx.aborted) break;
    b = sh.batch.next_jump;
    __syncthreads();
    if (b != 0 && wave == loader) load_batch(sh, plan, b, lid);
    __syncthreads();
  }
  // LL and LL128 publish no tail while running; record the sender step.
  if (PROTO != kSimple && tid == 0 && !cx.aborted) store_relaxed(cx.send_tail, cx.send_step);
  if (cx.trace && tid == 0) sh.comm.trace_count[blockIdx.x] = cx.trace_n;
}

// Kernel table of one payload type: [operator][protocol].  Each payload type
// is instantiated in its own translation unit so the library builds in
// parallel.
template <template <int> class Ty>
const void* ring_kernel_table(int proto, int red) {
  using KernelFn = void (*)(KernelArgs);
  static const KernelFn table[kNumRed][3] = {
      {ring_allreduce_kernel<Ty<kRedSum>, kLL>, ring_allreduce_kernel<Ty<kRedSum>, kLL128>,
       ring_allreduce_kernel<Ty<kRedSum>, kSimple>},
      {ring_allreduce_kernel<Ty<kRedProd>, kLL>, ring_allreduce_kernel<Ty<kRedProd>, kLL128>,
       ring_allreduce_kernel<Ty<kRedProd>, kSimple>},
      {ring_allreduce_kernel<Ty<kRedMax>, kLL>, ring_allreduce_kernel<Ty<kRedMax>, kLL128>,
       ring_allreduce_kernel<Ty<kRedMax>, kSimple>},
      {ring_allreduce_kernel<Ty<kRedMin>, kLL>, ring_allreduce_kernel<Ty<kRedMin>, kLL128>,
       ring_allreduce_kernel<Ty<kRedMin>, kSimple>},
      {ring_allreduce_kernel<Ty<kRedAvg>, kLL>, ring_allreduce_kernel<Ty<kRedAvg>, kLL128>,
       ring_allreduce_kernel<Ty<kRedAvg>, kSimple>},
      {ring_allreduce_kernel<Ty<kRedPreMulSum>, kLL>, ring_allreduce_kernel<Ty<kRedPreMulSum>, kLL128>,
       ring_allreduce_kernel<Ty<kRedPreMulSum>, kSimple>},
  };
  if (proto < 0 || proto > 2 || red < 0 || red >= kNumRed) return nullptr;
  return reinterpret_cast<const void*>(table[red][proto]);
}

}  // namespace rar
