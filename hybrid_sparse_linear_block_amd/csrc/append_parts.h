// Pieces of the token append ("SPLA: Block Sparse Plus Linear Attention for
// Long Context Modeling", section "Recurrence") shared by the stand-alone
// append kernel and the decode kernel that takes the append in with its
// state readout: element access in either storage format, and the
// statistics of a block the new token completes.
#pragma once

#include "common.h"

namespace hsla {

template <typename KV>
__device__ __forceinline__ float kv_elem(const void* p, size_t i) {
  if constexpr (KV::kBytes == 2) {
    return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

template <typename KV>
__device__ __forceinline__ void kv_put(void* p, size_t i, const void* src, size_t j) {
  if constexpr (KV::kBytes == 2) {
    reinterpret_cast<uint16_t*>(p)[i] = reinterpret_cast<const uint16_t*>(src)[j];
  } else {
    reinterpret_cast<float*>(p)[i] = reinterpret_cast<const float*>(src)[j];
  }
}

// Four consecutive elements widened to fp32.
template <typename KV>
__device__ __forceinline__ float4 kv_load4(const void* p, size_t i) {
  if constexpr (KV::kBytes == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + i);
    return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
  } else {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
  }
}

// LDS of filled_block_stats for NT threads and head dim D.
template <int NT, int D>
struct BlockStatsLds {
  float part[NT / (D / 8) * D];
  float mean[D];
};

// Statistics of the block the new token fills (SPLA, section "Principled
// Block Selection via Taylor Expansion": the mean and the per-channel
// variance of the block's keys): rows [0, B) of
// the page-head tile at row0 of k_pages, row `last` taken from k_new at
// nbase (its page write may not have landed).  NT threads = D/8 channel
// groups x (NT / (D/8)) row groups; each thread loads its rows as
// 8-channel vectors, four rows in flight, and the partial sums meet in LDS.
// The second pass re-reads the rows (cache hits) for the squared deviations
// from the mean.  Every thread of the workgroup must call it.
template <typename KV, int D, int NT>
__device__ __forceinline__ void filled_block_stats(const void* k_pages, const void* k_new, size_t row0, int last, size_t nbase,
                                   int B, float* mean_out, float* var_out, BlockStatsLds<NT, D>& s) {
  constexpr int CG = D / 8;      // channel groups of 8
  constexpr int RG = NT / CG;    // row groups
  const int tid = threadIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;
  auto load_row = [&](int r, float (&x)[8]) __attribute__((always_inline)) {
    Row8<KV> row;
    if (r == last)
      row.load(reinterpret_cast<const char*>(k_new) + (nbase + cg * 8) * KV::kBytes);
    else
      row.load(reinterpret_cast<const char*>(k_pages) + ((row0 + r) * D + cg * 8) * KV::kBytes);
    row.to_f32(x);
  };
  auto pass = [&](bool second) __attribute__((always_inline)) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float mu[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) mu[j] = second ? s.mean[cg * 8 + j] : 0.f;
    for (int r0 = rg; r0 < B; r0 += 4 * RG) {
      float x[4][8];
#pragma unroll
      for (int u = 0; u < 4; ++u) load_row(min(r0 + u * RG, B - 1), x[u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = r0 + u * RG < B ? 1.f : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float dl = x[u][j] - mu[j];
          acc[j] = fmaf(w, second ? dl * dl : x[u][j], acc[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) s.part[rg * D + cg * 8 + j] = acc[j];
    __syncthreads();
    float t = 0.f;
    if (tid < D)
      for (int r = 0; r < RG; ++r) t += s.part[r * D + tid];
    return t;
  };
  const float sum = pass(false);
  if (tid < D) s.mean[tid] = sum / static_cast<float>(B);
  __syncthreads();
  const float m2 = pass(true);
  if (tid < D) {
    mean_out[tid] = s.mean[tid];
    var_out[tid] = m2 / static_cast<float>(B);
  }
}

// The block a new token completes: rows [0, B) of the page-head tiles at
// row0 of the key and value pages, row `last` (the new token) read from
// k_new / v_new at nbase instead, since its page write may not have landed.
struct CompletedBlock {
  const void* k_pages;
  const void* v_pages;
  const void* k_new;
  const void* v_new;
  size_t row0;
  size_t nbase;
  int last;
  int B;
};

template <typename KV, int D>
__device__ __forceinline__ const char* block_row(const void* pages, const void* nw, const CompletedBlock& cb, int j) {
  return j == cb.last ? reinterpret_cast<const char*>(nw) + cb.nbase * KV::kBytes
                      : reinterpret_cast<const char*>(pages) + (cb.row0 + j) * D * KV::kBytes;
}

// Staging of a completed block's rows in LDS for the fold: up to 64 rows of
// keys and values per stage, within kFoldStageBytes.
constexpr int kFoldStageBytes = 32768;

template <typename KV, int D>
struct FoldStage {
  static constexpr int kRowBytes = D * KV::kBytes;
  static constexpr int kFit = kFoldStageBytes / (2 * kRowBytes);
  static constexpr int kRows = kFit < 64 ? kFit : 64;   // rows per stage
  static constexpr int kVec = kRowBytes / 16;           // 16-byte vectors per row
};

// Rows [j0, j0 + n) of the block's keys and then values into LDS (`lds`:
// keys [kRows][D], values [kRows][D], in kv_dtype), every load issued before
// the first LDS store.  NT threads, 16-byte vectors.
template <typename KV, int D, int NT>
__device__ __forceinline__ void stage_block_rows(const CompletedBlock& cb, int j0, int n, uint4* lds) {
  using F = FoldStage<KV, D>;
  constexpr int PER = (2 * F::kRows * F::kVec + NT - 1) / NT;
  const int per_kv = n * F::kVec;
  // every slot loads (past the rows: the last one again), so that buf stays
  // in registers (a native vector type: HIP's uint4 is a union, which keeps
  // the array on the stack)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 buf[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int idx = min(static_cast<int>(threadIdx.x) + p * NT, 2 * per_kv - 1);
    const int kv = idx < per_kv ? 0 : 1;
    const int rem = idx - kv * per_kv;
    const int j = rem / F::kVec;
    const int c16 = rem % F::kVec;
    const char* row = kv ? block_row<KV, D>(cb.v_pages, cb.v_new, cb, j0 + j)
                         : block_row<KV, D>(cb.k_pages, cb.k_new, cb, j0 + j);
    buf[p] = reinterpret_cast<const u32x4*>(row)[c16];
  }
  // slots past the rows store the last row's vector again: the same value
  // to the same place as its own thread
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int idx = min(static_cast<int>(threadIdx.x) + p * NT, 2 * per_kv - 1);
    const int kv = idx < per_kv ? 0 : 1;
    const int rem = idx - kv * per_kv;
    reinterpret_cast<u32x4*>(lds)[kv * F::kRows * F::kVec + rem] = buf[p];
  }
}

// The linear state takes a block's tokens when the block completes (tokens
// of the incomplete last block always lie inside the window, so they are
// exact and never enter the linear part).  This adds the completed block to
// one workgroup's rows: rows r_first + RG i (i < NR), columns 4 col4 ..
// 4 col4 + 3 of S (srow) gain sum_j k_j[r] v_j[c]; the thread's z row
// (zrow >= 0) gains sum_j k_j[zrow] and its sv channel (svcol >= 0) sum_j
// v_j[svcol].  The block is staged through `lds` (kFoldStageBytes) and every
// sum runs in row order, then is added once.  Every thread of the
// workgroup must call it.
template <typename KV, int D, int NT, int NR, int RG>
__device__ __forceinline__ void fold_completed_block(const CompletedBlock& cb, uint4* lds, float4 (&srow)[NR], int r_first, int col4,
                                     int zrow, float& z, int svcol, float& sv) {
  using F = FoldStage<KV, D>;
  float4 acc[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  float zacc = 0.f, svacc = 0.f;
  const char* ks = reinterpret_cast<const char*>(lds);
  const char* vs = ks + F::kRows * F::kRowBytes;
  for (int j0 = 0; j0 < cb.B; j0 += F::kRows) {
    const int n = min(F::kRows, cb.B - j0);
    if (j0 > 0) __syncthreads();   // the previous stage is consumed
    stage_block_rows<KV, D, NT>(cb, j0, n, lds);
    __syncthreads();
    for (int j = 0; j < n; ++j) {
      const float4 v = kv_load4<KV>(vs + j * F::kRowBytes, col4 * 4);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const float kr = kv_elem<KV>(ks + j * F::kRowBytes, r_first + i * RG);
        acc[i].x = fmaf(kr, v.x, acc[i].x);
        acc[i].y = fmaf(kr, v.y, acc[i].y);
        acc[i].z = fmaf(kr, v.z, acc[i].z);
        acc[i].w = fmaf(kr, v.w, acc[i].w);
      }
    }
    if (zrow >= 0)
      for (int j = 0; j < n; ++j) zacc += kv_elem<KV>(ks + j * F::kRowBytes, zrow);
    if (svcol >= 0)
      for (int j = 0; j < n; ++j) svacc += kv_elem<KV>(vs + j * F::kRowBytes, svcol);
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    srow[i].x += acc[i].x;
    srow[i].y += acc[i].y;
    srow[i].z += acc[i].z;
    srow[i].w += acc[i].w;
  }
  z += zacc;
  sv += svacc;
}

}  // namespace hsla
