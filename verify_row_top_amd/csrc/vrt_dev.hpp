// Device building blocks for the gfx950 kernels: counter-based uniforms, the
// ranking exponential, wave64 reductions and scans, bf16 unpacking, sort keys.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace vrt {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11). Each round multiplies
// words 0 and 2 by the two Philox constants, swaps the halves into place and
// mixes the round key; the key advances by the Weyl constants between rounds.
struct U4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 philox10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo_a = 0xD2511F53u * c.x;
    const uint32_t hi_a = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo_b = 0xCD9E8D57u * c.z;
    const uint32_t hi_b = __umulhi(0xCD9E8D57u, c.z);
    c = U4{hi_b ^ c.y ^ k0, lo_b, hi_a ^ c.w ^ k1, lo_a};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

enum : uint32_t { kPurposeProbe = 1, kPurposeTest = 2, kPurposeFinal = 3 };

// u in [0, 1 - 2^-24]: the top 24 bits of the first output word.
__device__ __forceinline__ float uniform24(uint64_t seed, uint32_t idx, uint32_t b, uint32_t step,
                                           uint32_t purpose) {
  const U4 o = philox10(U4{idx, b, step, purpose}, (uint32_t)seed, (uint32_t)(seed >> 32));
  return (float)(o.x >> 8) * 5.9604644775390625e-08f;  // exact
}

// ---------------------------------------------------------------------------
// Ranking exponential: a fixed recipe so that draft ranking is reproducible
// bit for bit on any IEEE machine (no contraction; every step correctly rounded).
// Cody-Waite reduction by ln 2 split in two parts, e^r by its degree-7 Taylor
// polynomial evaluated with fma, exact scaling by 2^k. Inputs below -80 give 0.
__device__ __forceinline__ float exp_rank(float x) {
  if (!(x >= -80.0f)) return 0.0f;
  const float k = __builtin_rintf(x * 1.44269504f);
  float r = __builtin_fmaf(-k, 0.693145751953125f, x);
  r = __builtin_fmaf(-k, 1.428606765330187e-06f, r);
  // coefficients 1/7!, 1/6!, ..., 1/1!, 1/0!, each the correctly rounded fp32 quotient
  float p = __builtin_fmaf(1.0f / 5040.0f, r, 1.0f / 720.0f);
  p = __builtin_fmaf(p, r, 1.0f / 120.0f);
  p = __builtin_fmaf(p, r, 1.0f / 24.0f);
  p = __builtin_fmaf(p, r, 1.0f / 6.0f);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)k);
}

// exp((x - M)/T) to about 1e-7 relative (dense rows): the fp64 exponent is split into
// an fp32 head and a tail, e^a = e^head (1 + tail); -inf and NaN give 0.
__device__ __forceinline__ double dense_tempered(float x, float M, double invT) {
  if (!(x > -INFINITY)) return 0.0;
  const double a = ((double)x - (double)M) * invT;
  const float h = (float)a;
  const float t = (float)(a - (double)h);
  return (double)expf(h) * (1.0 + (double)t);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Orders LDS accesses between the lanes of one wave (no block barrier: usable
// after the other waves of the block have exited).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// ---------------------------------------------------------------------------
// 16-byte streaming load with the non-temporal hint: data read once is not kept
// in the caches (measured ~10% more HBM read bandwidth for row streams).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint64_t u64x2_t __attribute__((ext_vector_type(2)));

// Device-coherent (every XCD) 32-bit store and load, for words that blocks of one
// launch hand to each other: the store is written through the XCD's L2 and the load
// does not take a possibly stale L2 copy, so neither side needs an L2 write-back or
// invalidate fence. The writer waits for its stores (wait_stores) before it signals.
__device__ __forceinline__ void st_dev(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(float* p, float v) { st_dev((int*)p, __float_as_int(v)); }
__device__ __forceinline__ int ld_dev(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) { return __int_as_float(ld_dev((const int*)p)); }
__device__ __forceinline__ void st_dev64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_dev64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0); }
__device__ __forceinline__ uint4 load_nt(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// ---------------------------------------------------------------------------
// bf16 <-> fp32 and order-preserving keys
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Monotone map of an fp32 value to uint32 (NaN maps to 0, below -inf).
__device__ __forceinline__ uint32_t ord32(float f) {
  if (f != f) return 0u;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord32(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// Support key: larger is better; value descending, then token id ascending.
__device__ __forceinline__ uint64_t sup_key(float v, uint32_t id) {
  return ((uint64_t)ord32(v) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ uint32_t sup_key_id(uint64_t k) { return 0xFFFFFFFFu - (uint32_t)k; }
__device__ __forceinline__ float sup_key_val(uint64_t k) { return unord32((uint32_t)(k >> 32)); }

// Node key: path score descending (non-negative fp32 bits are ordered), then
// creation index ascending.
__device__ __forceinline__ uint64_t node_key(float score, uint32_t cidx) {
  return ((uint64_t)__float_as_uint(score) << 32) | (uint64_t)(0xFFFFFFFFu - cidx);
}

// ---------------------------------------------------------------------------
// In-LDS bitonic sort of n (a power of two) 64-bit keys into descending order,
// by all threads of the block.
__device__ inline void bitonic_desc(uint64_t* a, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < (n >> 1); t += blockDim.x) {
        const int i = ((t & ~(j - 1)) << 1) | (t & (j - 1));
        const int p = i | j;
        const uint64_t x = a[i], y = a[p];
        const bool desc = ((i & k) == 0);
        if (desc ? (x < y) : (x > y)) {
          a[i] = y;
          a[p] = x;
        }
      }
      __syncthreads();
    }
  }
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1, so array
// indices are constants before any optimisation runs.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------
// Lane exchanges: the value of lane (lane ^ LJ). Distances 1 and 2 are one DPP quad
// permutation; 4 and 8 compose two DPP mirrors (reversal within 8 lanes, within 16)
// with a quad reversal; 16 and 32 use gfx950's row/half swaps plus a select.
__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const uint32_t lo = __shfl((uint32_t)v, src, kWave);
  const uint32_t hi = __shfl((uint32_t)(v >> 32), src, kWave);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint32_t shfl32(uint32_t v, int src) { return (uint32_t)__shfl((int)v, src, kWave); }
__device__ __forceinline__ uint64_t shflk(uint64_t v, int src) { return shfl64(v, src); }
__device__ __forceinline__ uint32_t shflk(uint32_t v, int src) { return shfl32(v, src); }

template <int LJ>
__device__ __forceinline__ uint32_t xchg32(uint32_t v) {
  if constexpr (LJ == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);  // quad [1,0,3,2]
  } else if constexpr (LJ == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);  // quad [2,3,0,1]
  } else if constexpr (LJ == 4) {
    const int t = __builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true);  // lane ^ 7
    return (uint32_t)__builtin_amdgcn_mov_dpp(t, 0x1B, 0xF, 0xF, true);     // then ^ 3
  } else if constexpr (LJ == 8) {
    const int t = __builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true);  // lane ^ 15
    return (uint32_t)__builtin_amdgcn_mov_dpp(t, 0x141, 0xF, 0xF, true);    // then ^ 7
  } else if constexpr (LJ == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane_id() & 16) ? r[0] : r[1];
  } else {
    static_assert(LJ == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane_id() & 32) ? r[0] : r[1];
  }
}
template <int LJ>
__device__ __forceinline__ uint32_t xchg(uint32_t v) { return xchg32<LJ>(v); }
template <int LJ>
__device__ __forceinline__ uint64_t xchg(uint64_t v) {
  return ((uint64_t)xchg32<LJ>((uint32_t)(v >> 32)) << 32) | xchg32<LJ>((uint32_t)v);
}

template <int LJ>
__device__ __forceinline__ float xchg(float v) { return __uint_as_float(xchg32<LJ>(__float_as_uint(v))); }
template <int LJ>
__device__ __forceinline__ int xchg(int v) { return (int)xchg32<LJ>((uint32_t)v); }
template <int LJ>
__device__ __forceinline__ double xchg(double v) {
  return __longlong_as_double((long long)xchg<LJ>((uint64_t)__double_as_longlong(v)));
}

// ---------------------------------------------------------------------------
// wave64 reductions by xor butterflies over lane exchanges: every lane ends with the
// same value, and for a sum the combination order is the aligned pairwise tree over
// lanes.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, xchg<1>(v));
  v = op(v, xchg<2>(v));
  v = op(v, xchg<4>(v));
  v = op(v, xchg<8>(v));
  v = op(v, xchg<16>(v));
  v = op(v, xchg<32>(v));
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
  return wave_reduce(v, [](T x, T y) { return x + y; });
}
__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}
__device__ __forceinline__ int wave_sum_i(int v) { return wave_sum(v); }

// Inclusive prefix sum over lanes: shifts by 1, 2, 4, 8 inside each row of 16 lanes
// (DPP row_shr, zero fill), then the row totals broadcast into the following rows
// (DPP row_bcast15 into rows 1 and 3, row_bcast31 into rows 2 and 3).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_fill0(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_fill0(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = dpp_fill0<CTRL, ROWS>((uint32_t)u), hi = dpp_fill0<CTRL, ROWS>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_fill0(float v) {
  return __uint_as_float(dpp_fill0<CTRL, ROWS>(__float_as_uint(v)));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_fill0(int v) { return (int)dpp_fill0<CTRL, ROWS>((uint32_t)v); }

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  v = v + dpp_fill0<0x111, 0xF>(v);
  v = v + dpp_fill0<0x112, 0xF>(v);
  v = v + dpp_fill0<0x114, 0xF>(v);
  v = v + dpp_fill0<0x118, 0xF>(v);
  v = v + dpp_fill0<0x142, 0xA>(v);
  v = v + dpp_fill0<0x143, 0xC>(v);
  return v;
}

// ---------------------------------------------------------------------------
// Sorted key lists held in a wave's registers: PL keys per lane, position
// p = lane*PL + s, 64*PL keys. Bitonic networks run on them with in-lane swaps and
// lane exchanges only (no LDS, no barriers).
//
// One compare-exchange stage: partner q = p ^ J; pairs inside blocks with
// (p & SIZE) == 0 are ordered descending, the others ascending.
template <int PL, int SIZE, int J, typename K>
__device__ __forceinline__ void bitonic_stage(K (&k)[PL], int lane) {
  if constexpr (J < PL) {
    static_for<PL>([&](auto s) {
      constexpr int t = s ^ J;
      if constexpr (s < t) {
        const bool desc = ((lane * PL + s) & SIZE) == 0;
        const K x = k[s], y = k[t];
        const K hi = x > y ? x : y, lo = x > y ? y : x;
        k[s] = desc ? hi : lo;
        k[t] = desc ? lo : hi;
      }
    });
  } else {
    constexpr int LJ = J / PL;
    static_for<PL>([&](auto s) {
      const K x = k[s];
      const K y = xchg<LJ>(x);
      const bool desc = ((lane * PL + s) & SIZE) == 0;
      const bool lower = (lane & LJ) == 0;
      const K hi = x > y ? x : y, lo = x > y ? y : x;
      k[s] = (lower == desc) ? hi : lo;
    });
  }
}

template <int PL, int SIZE, int J, typename K>
__device__ __forceinline__ void bitonic_stages(K (&k)[PL], int lane) {
  bitonic_stage<PL, SIZE, J>(k, lane);
  if constexpr (J > 1) bitonic_stages<PL, SIZE, J / 2>(k, lane);
}

template <int PL, int SIZE, typename K>
__device__ __forceinline__ void bitonic_sort_from(K (&k)[PL], int lane) {
  bitonic_stages<PL, SIZE, SIZE / 2>(k, lane);
  if constexpr (SIZE < PL * kWave) bitonic_sort_from<PL, SIZE * 2>(k, lane);
}

// Sort the wave list descending.
template <int PL, typename K>
__device__ __forceinline__ void wave_sort_desc(K (&k)[PL]) {
  bitonic_sort_from<PL, 2>(k, lane_id());
}

// top <- the 64*PL largest of top and add, both sorted descending; result sorted
// descending. (max of top[p] and add[last - p] is a bitonic sequence holding the
// largest half; one bitonic merge orders it.)
template <int PL, typename K>
__device__ __forceinline__ void wave_merge_top(K (&top)[PL], const K (&add)[PL]) {
  const int lane = lane_id();
  static_for<PL>([&](auto s) {
    const K r = shflk(add[PL - 1 - s], kWave - 1 - lane);
    top[s] = top[s] > r ? top[s] : r;
  });
  bitonic_stages<PL, 2 * PL * kWave, PL * kWave / 2>(top, lane);
}

__host__ __device__ inline int next_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

}  // namespace vrt
