// oneshot_kernel.hip -- the one-shot AllReduce for gfx950 (MI355X, wave64).
//
// With every rank's buffer reachable by plain loads, the reduction finishes
// in one hop: each element is loaded from all N inputs, folded in registers
// and stored [C2 "5 Symmetric Memory", "6.1 LSA"; the notes list the one-shot
// AllReduce among the abilities symmetric memory unlocks].  All N virtual
// ranks live in this GPU's HBM, so the N identical folds of an element are
// done once and the result is stored to all N receive buffers: each input is
// read once and each output written once, 2*N*M bytes in all, the least any
// AllReduce can move.
//
// Fold order is fixed so every rank holds the same bits: user rank 0 first,
// then ranks 1 .. N-1 in turn.  fp32 rounds per operation; bf16 is widened to
// fp32, accumulated, and rounded to nearest-even bf16 once; int32 wraps.
//
//   [C2] "cishoon.github.io/posts/ai-infra/nccl" (NCCL notes)
#include <hip/hip_runtime.h>

#include "rar_device.h"

namespace rar {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
// Buffers need only element alignment: gfx950 serves unaligned global
// loads and stores in hardware, so the under-aligned type compiles to the
// same dwordx4 accesses as an aligned one.
typedef uint32_t v4u_user __attribute__((ext_vector_type(4), aligned(2)));

__device__ __forceinline__ v4u ld_nt(const v4u_user* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(v4u_user* p, v4u v) { __builtin_nontemporal_store((v4u_user)v, p); }

__device__ __forceinline__ uint32_t bf16_round(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;  // quiet NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One step of the fold, acc <- acc (op) x, in fp32 [prod and sum round per
// operation; max / min keep acc unless x is strictly larger / smaller].
template <int R>
__device__ __forceinline__ float red_f(float a, float b) {
  if constexpr (R == kRedProd) return a * b;
  else if constexpr (R == kRedMax) return b > a ? b : a;
  else if constexpr (R == kRedMin) return b < a ? b : a;
  else return a + b;
}
template <int R>
__device__ __forceinline__ uint32_t red_i(uint32_t a, uint32_t b) {
  if constexpr (R == kRedProd) return a * b;  // low 32 bits
  else if constexpr (R == kRedMax) return (int32_t)b > (int32_t)a ? b : a;
  else if constexpr (R == kRedMin) return (int32_t)b < (int32_t)a ? b : a;
  else return a + b;  // wraps
}

// Accumulator of one 16-byte vector: fp32 and int32 fold the words as they
// are; bf16 widens each of the 8 elements to fp32 (exact) and rounds once in
// out().  avg divides the final sum by N there (int32: truncating).
// PreMulSum (R == kRedPreMulSum) scales every input by its rank's scalar
// `s` in the accumulator's precision, then sums; other operators ignore `s`.
template <int R>
__device__ __forceinline__ float pre_f(float x, float s) {
  return R == kRedPreMulSum ? x * s : x;
}

template <int R>
struct AccF32 {
  using S = uint32_t;
  float a[4];
  __device__ __forceinline__ void init(v4u x, uint32_t s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = pre_f<R>(__uint_as_float(x[i]), __uint_as_float(s));
  }
  __device__ __forceinline__ void add(v4u x, uint32_t s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = red_f<R>(a[i], pre_f<R>(__uint_as_float(x[i]), __uint_as_float(s)));
  }
  __device__ __forceinline__ v4u out(int n) const {
    v4u r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(R == kRedAvg ? a[i] / (float)n : a[i]);
    return r;
  }
  static __device__ __forceinline__ uint32_t elem_init(uint32_t x, uint32_t s) {
    return __float_as_uint(pre_f<R>(__uint_as_float(x), __uint_as_float(s)));
  }
  static __device__ __forceinline__ uint32_t elem_add(uint32_t acc, uint32_t x, uint32_t s) {
    return __float_as_uint(red_f<R>(__uint_as_float(acc), pre_f<R>(__uint_as_float(x), __uint_as_float(s))));
  }
  static __device__ __forceinline__ uint32_t elem_out(uint32_t acc, int n) {
    return R == kRedAvg ? __float_as_uint(__uint_as_float(acc) / (float)n) : acc;
  }
};
template <int R>
struct AccI32 {
  using S = uint32_t;
  v4u a;
  static __device__ __forceinline__ uint32_t pre(uint32_t x, uint32_t s) {
    return R == kRedPreMulSum ? x * s : x;  // low 32 bits
  }
  __device__ __forceinline__ void init(v4u x, uint32_t s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = pre(x[i], s);
  }
  __device__ __forceinline__ void add(v4u x, uint32_t s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = red_i<R>(a[i], pre(x[i], s));
  }
  __device__ __forceinline__ v4u out(int n) const {
    if constexpr (R != kRedAvg) return a;
    v4u r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)((int32_t)a[i] / n);
    return r;
  }
  static __device__ __forceinline__ uint32_t elem_init(uint32_t x, uint32_t s) { return pre(x, s); }
  static __device__ __forceinline__ uint32_t elem_add(uint32_t acc, uint32_t x, uint32_t s) {
    return red_i<R>(acc, pre(x, s));
  }
  static __device__ __forceinline__ uint32_t elem_out(uint32_t acc, int n) {
    return R == kRedAvg ? (uint32_t)((int32_t)acc / n) : acc;
  }
};
template <int R>
struct AccBF16 {
  using S = uint16_t;
  float lo[4], hi[4];  // element 2i in the low half of word i, 2i+1 in the high half
  __device__ __forceinline__ void init(v4u x, uint32_t s) {
    const float fs = __uint_as_float(s << 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = pre_f<R>(__uint_as_float(x[i] << 16), fs);
      hi[i] = pre_f<R>(__uint_as_float(x[i] & 0xffff0000u), fs);
    }
  }
  __device__ __forceinline__ void add(v4u x, uint32_t s) {
    const float fs = __uint_as_float(s << 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo[i] = red_f<R>(lo[i], pre_f<R>(__uint_as_float(x[i] << 16), fs));
      hi[i] = red_f<R>(hi[i], pre_f<R>(__uint_as_float(x[i] & 0xffff0000u), fs));
    }
  }
  __device__ __forceinline__ v4u out(int n) const {
    v4u r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float l = R == kRedAvg ? lo[i] / (float)n : lo[i];
      const float h = R == kRedAvg ? hi[i] / (float)n : hi[i];
      r[i] = bf16_round(l) | (bf16_round(h) << 16);
    }
    return r;
  }
  static __device__ __forceinline__ uint32_t elem_init(uint16_t x, uint32_t s) {
    return __float_as_uint(pre_f<R>(__uint_as_float((uint32_t)x << 16), __uint_as_float(s << 16)));
  }
  static __device__ __forceinline__ uint32_t elem_add(uint32_t acc, uint16_t x, uint32_t s) {
    return __float_as_uint(
        red_f<R>(__uint_as_float(acc), pre_f<R>(__uint_as_float((uint32_t)x << 16), __uint_as_float(s << 16))));
  }
  static __device__ __forceinline__ uint16_t elem_out(uint32_t acc, int n) {
    const float f = __uint_as_float(acc);
    return (uint16_t)bf16_round(R == kRedAvg ? f / (float)n : f);
  }
};

// Inputs whose loads are issued together: 8 x U 16-byte vectors in flight
// per thread up to U = 2, 4 x 4 at U = 4 (no register spills at any U).
template <int U> constexpr int rank_batch() { return U >= 4 ? 4 : 8; }

// Workgroup b folds the contiguous vectors [b*per, (b+1)*per); inside it,
// consecutive threads take consecutive 16-byte vectors, U of them in flight
// per thread and input.  The ragged tail (< one vector per rank) is done
// element by element by the first workgroup.
template <class Acc, int U>
__global__ void __launch_bounds__(512) oneshot_kernel(OneshotArgs args) {
  constexpr int kRankBatch = rank_batch<U>();
  const int N = args.nranks;
  const int64_t per = args.vec_per_block;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < args.nvec ? lo + per : args.nvec;
  const int nthreads = blockDim.x;
  for (int64_t base = lo + threadIdx.x; base < hi; base += (int64_t)nthreads * U) {
    Acc acc[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) live[u] = base + (int64_t)u * nthreads < hi;
    for (int k0 = 0; k0 < N; k0 += kRankBatch) {
      v4u x[kRankBatch][U];
#pragma unroll
      for (int j = 0; j < kRankBatch; ++j) {
        if (k0 + j < N) {
          const v4u_user* src = reinterpret_cast<const v4u_user*>(args.src[k0 + j]);
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (live[u]) x[j][u] = ld_nt(src + base + (int64_t)u * nthreads);
        }
      }
#pragma unroll
      for (int j = 0; j < kRankBatch; ++j) {
        if (k0 + j < N) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (!live[u]) continue;
            if (k0 + j == 0) acc[u].init(x[j][u], args.scalar[0]);
            else acc[u].add(x[j][u], args.scalar[k0 + j]);
          }
        }
      }
    }
    v4u r[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (live[u]) r[u] = acc[u].out(N);
    for (int k = 0; k < N; ++k) {
      v4u_user* dst = reinterpret_cast<v4u_user*>(args.dst[k]);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (live[u]) st_nt(dst + base + (int64_t)u * nthreads, r[u]);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < args.tail) {
    using S = typename Acc::S;
    const int64_t e = args.nvec * (16 / (int64_t)sizeof(S)) + threadIdx.x;
    uint32_t a = Acc::elem_init(reinterpret_cast<const S*>(args.src[0])[e], args.scalar[0]);
    for (int k = 1; k < N; ++k) a = Acc::elem_add(a, reinterpret_cast<const S*>(args.src[k])[e], args.scalar[k]);
    const S v = (S)Acc::elem_out(a, N);
    for (int k = 0; k < N; ++k) reinterpret_cast<S*>(args.dst[k])[e] = v;
  }
}

template <class Acc>
const void* pick_unroll(int unroll) {
  switch (unroll) {
    case 1: return reinterpret_cast<const void*>(&oneshot_kernel<Acc, 1>);
    case 4: return reinterpret_cast<const void*>(&oneshot_kernel<Acc, 4>);
    default: return reinterpret_cast<const void*>(&oneshot_kernel<Acc, 2>);
  }
}

template <template <int> class Acc>
const void* pick(int red, int unroll) {
  switch (red) {
    case kRedSum: return pick_unroll<Acc<kRedSum>>(unroll);
    case kRedProd: return pick_unroll<Acc<kRedProd>>(unroll);
    case kRedMax: return pick_unroll<Acc<kRedMax>>(unroll);
    case kRedMin: return pick_unroll<Acc<kRedMin>>(unroll);
    case kRedAvg: return pick_unroll<Acc<kRedAvg>>(unroll);
    case kRedPreMulSum: return pick_unroll<Acc<kRedPreMulSum>>(unroll);
  }
  return nullptr;
}

}  // namespace

const void* get_oneshot_kernel(int dtype, int red, int unroll) {
  switch (dtype) {
    case kInt32: return pick<AccI32>(red, unroll);
    case kFloat32: return pick<AccF32>(red, unroll);
    case kBFloat16: return pick<AccBF16>(red, unroll);
  }
  return nullptr;
}

}  // namespace rar
