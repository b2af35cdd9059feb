// Device helpers shared by the libhsla kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsla {

constexpr int kWave = 64;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Loads through an explicit address space.  A pointer whose address space
// the compiler cannot infer (one chosen between two buffers, or one that may
// point to LDS or to global memory) becomes a flat access, which counts on
// both the vector-memory and the LDS counters: every later LDS access then
// waits for it, and so for every global load issued before it.
template <typename T>
__device__ __forceinline__ T ld_global(const void* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}
// The same load marked non-temporal: for data read once per step (gathered
// K/V pages), so that it does not displace what the next kernels reuse.
template <typename T>
__device__ __forceinline__ T ld_global_nt(const void* p) {
  return __builtin_nontemporal_load((const __attribute__((address_space(1))) T*)(p));
}
template <typename T>
__device__ __forceinline__ T ld_lds(const void* p) {
  return *(const __attribute__((address_space(3))) T*)(p);
}

// ---------------------------------------------------------------------------
// Storage formats.  bf16 values are carried as raw 16-bit patterns; a bf16
// widens to fp32 exactly by placing its bits in the upper half.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

struct KvBf16 {
  static constexpr int kBytes = 2;
};
struct KvF32 {
  static constexpr int kBytes = 4;
};

// Eight consecutive channels of one row, widened to fp32.
template <typename KV>
struct Row8;

template <>
struct Row8<KvBf16> {
  uint4 raw;  // 8 bf16
  __device__ __forceinline__ void load(const void* p) { raw = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void load_nt(const void* p) {
    raw = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(p)));
  }
  __device__ __forceinline__ void zero() { raw = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void to_f32(float (&f)[8]) const {
    f[0] = bf16_lo(raw.x); f[1] = bf16_hi(raw.x);
    f[2] = bf16_lo(raw.y); f[3] = bf16_hi(raw.y);
    f[4] = bf16_lo(raw.z); f[5] = bf16_hi(raw.z);
    f[6] = bf16_lo(raw.w); f[7] = bf16_hi(raw.w);
  }
};

template <>
struct Row8<KvF32> {
  float4 a, b;
  __device__ __forceinline__ void load(const void* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void load_nt(const void* p) {
    const auto* q = (const __attribute__((address_space(1))) u32x4*)(p);
    a = __builtin_bit_cast(float4, __builtin_nontemporal_load(q));
    b = __builtin_bit_cast(float4, __builtin_nontemporal_load(q + 1));
  }
  __device__ __forceinline__ void zero() {
    a = make_float4(0.f, 0.f, 0.f, 0.f);
    b = a;
  }
  __device__ __forceinline__ void to_f32(float (&f)[8]) const {
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
};

// ---------------------------------------------------------------------------
// Cross-lane reductions inside a DPP row (16 lanes) through data-parallel
// primitives: quad xor 1, quad xor 2, half-row mirror, row mirror.  After
// reduce_rowN every lane of its N-lane group holds the group's sum.
// ---------------------------------------------------------------------------
// Every pattern used here reads a lane of the same row, so bound_ctrl never
// applies; with it set the compiler folds the move into the consuming VALU op.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// The values of lane l and lane l ^ OFF, as (a, b).  Which of the two is
// lane l's own value is fixed per OFF but not exposed: callers combine a and
// b symmetrically (sum, max, or a pairing that is the same for every
// variable), so they do not depend on it.  OFF 8 uses DPP row_ror:8; 16 and
// 32 use the gfx950 permlane swaps; no LDS traffic.
template <int OFF>
__device__ __forceinline__ void lane_pair(float x, float& a, float& b) {
  if constexpr (OFF == 8) {
    a = x;
    b = dpp_f<0x128>(x);
  } else if constexpr (OFF == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else if constexpr (OFF == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
  } else {
    a = x;
    b = __shfl_xor(x, OFF);
  }
}

template <int OFF>
__device__ __forceinline__ float pair_sum(float x) {
  float a, b;
  lane_pair<OFF>(x, a, b);
  return a + b;
}

template <int N>
__device__ __forceinline__ float reduce_sum_lanes(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "group size");
  if constexpr (N >= 2) v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (N >= 16) v += dpp_f<0x140>(v); // row_mirror
  if constexpr (N >= 32) v = pair_sum<16>(v);
  return v;
}

// Wavefront-wide reductions without LDS: DPP within rows, permlane swaps
// across rows.  Every lane ends with the result.
__device__ __forceinline__ float wave_sum(float v) {
  v = reduce_sum_lanes<16>(v);
  v = pair_sum<16>(v);
  return pair_sum<32>(v);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  float a, b;
  lane_pair<16>(v, a, b);
  v = fmaxf(a, b);
  lane_pair<32>(v, a, b);
  return fmaxf(a, b);
}

__device__ __forceinline__ float fast_exp(float x) {
  // exp(x) = 2^(x log2 e); v_exp_f32 is exact to ~1 ulp on its argument.
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Its inverse.
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Candidate blocks of a sequence of T tokens: blocks intersecting
// [num_sink, T - window), i.e. [lo, lo + count).
struct CandRange {
  int lo;
  int count;
};
__host__ __device__ __forceinline__ CandRange candidate_range(int T, int B, int ns, int W) {
  CandRange r;
  r.lo = ns / B;
  const int hi_tok = T - W;
  if (hi_tok <= ns) {
    r.count = 0;
  } else {
    r.count = ceil_div(hi_tok, B) - r.lo;
  }
  return r;
}

}  // namespace hsla
