// Append of one decoded token ("SPLA: Block Sparse Plus Linear Attention for
// Long Context Modeling", section "Recurrence"): the token's key and value go
// into their page slot, the global linear state takes the rank-1 update
// S += k v^T, z += k, sv += v, and when the token completes its block the
// block's mean / variance statistics are computed.
//
// Grid: (row chunks of S, sequence x kv head); a chunk is RPW rows (more rows
// per workgroup for large batches).  Every load of a workgroup's rows is
// issued before any update.  Row chunk 0 also writes the page slot, z, sv,
// the new length, and -- when the token fills its block -- the block's
// statistics: the whole workgroup reads the block's rows as 16-byte vectors
// (the new token's row from k_new, since its page write may not have landed)
// and reduces per channel through LDS, mean first, then the variance around
// it.
#include "common.h"
#include "internal.h"

namespace hsla {

namespace {

constexpr int kThreads = 256;

struct AppendParams {
  void* k_pages;
  void* v_pages;
  float* blk_mean;
  float* blk_var;
  const int32_t* block_table;
  float* S;
  float* z;
  float* sv;
  const void* k_new;
  const void* v_new;
  const int32_t* seq_lens_before;
  int32_t* seq_lens_after;
  int Hkv, B, max_blocks, max_seq_len;
};

template <typename KV>
__device__ __forceinline__ float elem(const void* p, size_t i) {
  if constexpr (KV::kBytes == 2) {
    return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
  } else {
    return reinterpret_cast<const float*>(p)[i];
  }
}

template <typename KV>
__device__ __forceinline__ void put(void* p, size_t i, const void* src, size_t j) {
  if constexpr (KV::kBytes == 2) {
    reinterpret_cast<uint16_t*>(p)[i] = reinterpret_cast<const uint16_t*>(src)[j];
  } else {
    reinterpret_cast<float*>(p)[i] = reinterpret_cast<const float*>(src)[j];
  }
}

// Four consecutive elements widened to fp32.
template <typename KV>
__device__ __forceinline__ float4 load4(const void* p, size_t i) {
  if constexpr (KV::kBytes == 2) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + i);
    return make_float4(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y));
  } else {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
  }
}

// Statistics of the block the new token fills: rows [0, B) of the page-head
// tile at row0, row `last` taken from k_new.  256 threads = D/8 channel
// groups x (256 / (D/8)) row groups; each thread loads its rows as 8-channel
// vectors, four rows in flight, and the partial sums meet in LDS (`part`:
// [row groups][D], `mean_s`: [D]).  The second pass re-reads the rows
// (cache hits) for the squared deviations from the mean.
template <typename KV, int D>
__device__ void filled_block_stats(const AppendParams& P, size_t row0, int last, size_t nbase, size_t out_off,
                                   float* part, float* mean_s) {
  constexpr int CG = D / 8;              // channel groups of 8
  constexpr int RG = kThreads / CG;      // row groups
  const int tid = threadIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;
  const int B = P.B;
  auto load_row = [&](int r, float (&x)[8]) __attribute__((always_inline)) {
    Row8<KV> row;
    if (r == last)
      row.load(reinterpret_cast<const char*>(P.k_new) + (nbase + cg * 8) * KV::kBytes);
    else
      row.load(reinterpret_cast<const char*>(P.k_pages) + ((row0 + r) * D + cg * 8) * KV::kBytes);
    row.to_f32(x);
  };
  auto pass = [&](bool second) __attribute__((always_inline)) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float mu[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) mu[j] = second ? mean_s[cg * 8 + j] : 0.f;
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
    for (int j = 0; j < 8; ++j) part[rg * D + cg * 8 + j] = acc[j];
    __syncthreads();
    float t = 0.f;
    if (tid < D)
      for (int r = 0; r < RG; ++r) t += part[r * D + tid];
    return t;
  };
  const float sum = pass(false);
  if (tid < D) mean_s[tid] = sum / static_cast<float>(B);
  __syncthreads();
  const float m2 = pass(true);
  if (tid < D) {
    P.blk_mean[out_off + tid] = mean_s[tid];
    P.blk_var[out_off + tid] = m2 / static_cast<float>(B);
  }
}

template <typename KV, int D, int RPW>
__global__ __launch_bounds__(kThreads) void k_append(AppendParams P) {
  constexpr int C4 = D / 4;
  constexpr int ITEMS = RPW * C4 / kThreads;   // float4 of S per thread
  static_assert(RPW * C4 % kThreads == 0, "whole items per thread");
  const int pair = blockIdx.y;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int rc = blockIdx.x;
  const int tid = threadIdx.x;
  const int T = min(max(P.seq_lens_before[b], 0), P.max_seq_len - 1);  // new token's position
  const size_t nbase = static_cast<size_t>(pair) * D;

  // Rank-1 update of rows [rc*RPW, rc*RPW + RPW) of S: loads first.
  float* Sp = P.S + static_cast<size_t>(pair) * D * D;
  float4 sv4[ITEMS], v4[ITEMS];
  float kr[ITEMS];
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int idx = tid + i * kThreads;
    const int r = rc * RPW + idx / C4;
    const int c4 = idx % C4;
    sv4[i] = *reinterpret_cast<const float4*>(Sp + static_cast<size_t>(r) * D + c4 * 4);
    v4[i] = load4<KV>(P.v_new, nbase + c4 * 4);
    kr[i] = elem<KV>(P.k_new, nbase + r);
  }
#pragma unroll
  for (int i = 0; i < ITEMS; ++i) {
    const int idx = tid + i * kThreads;
    const int r = rc * RPW + idx / C4;
    const int c4 = idx % C4;
    float4 s = sv4[i];
    s.x = fmaf(kr[i], v4[i].x, s.x);
    s.y = fmaf(kr[i], v4[i].y, s.y);
    s.z = fmaf(kr[i], v4[i].z, s.z);
    s.w = fmaf(kr[i], v4[i].w, s.w);
    *reinterpret_cast<float4*>(Sp + static_cast<size_t>(r) * D + c4 * 4) = s;
  }
  if (rc != 0) return;

  const int B = P.B;
  const int blk = T / B;
  const size_t page = static_cast<size_t>(P.block_table[static_cast<size_t>(b) * P.max_blocks + blk]);
  const size_t row0 = (page * P.Hkv + g) * B;  // first row of this page-head tile
  if (tid < D) {
    const int c = tid;
    P.z[nbase + c] += elem<KV>(P.k_new, nbase + c);
    P.sv[nbase + c] += elem<KV>(P.v_new, nbase + c);
    put<KV>(P.k_pages, (row0 + T % B) * D + c, P.k_new, nbase + c);
    put<KV>(P.v_pages, (row0 + T % B) * D + c, P.v_new, nbase + c);
  }
  if ((T + 1) % B == 0) {   // uniform: the token completes block blk
    __shared__ float part[kThreads / (D / 8) * D];
    __shared__ float mean_s[D];
    filled_block_stats<KV, D>(P, row0, T % B, nbase, (page * P.Hkv + g) * D, part, mean_s);
  }
  if (g == 0 && tid == 0 && P.seq_lens_after) P.seq_lens_after[b] = T + 1;
}

template <typename KV, int D, int RPW>
hipError_t launch_rows(const Problem& p, const AppendParams& P, hipStream_t s) {
  dim3 grid(D / RPW, p.batch * p.Hkv);
  hipLaunchKernelGGL((k_append<KV, D, RPW>), grid, dim3(kThreads), 0, s, P);
  return launch_status("k_append");
}

// Rows of S per workgroup: 16 for small batches (enough workgroups to spread
// the update), all of S for large ones.
template <typename KV, int D>
hipError_t launch_t(const Problem& p, const AppendParams& P, hipStream_t s) {
  const long pairs = static_cast<long>(p.batch) * p.Hkv;
  if (pairs * (D / 16) <= 1024) return launch_rows<KV, D, 16>(p, P, s);
  if (pairs * (D / 32) <= 1024) return launch_rows<KV, D, 32>(p, P, s);
  return launch_rows<KV, D, D>(p, P, s);
}

}  // namespace

hipError_t launch_append(const Problem& p, const AppendArgs& a, hipStream_t s) {
  AppendParams P{};
  P.k_pages = a.k_pages;
  P.v_pages = a.v_pages;
  P.blk_mean = a.blk_mean;
  P.blk_var = a.blk_var;
  P.block_table = a.block_table;
  P.S = a.S;
  P.z = a.z;
  P.sv = a.sv;
  P.k_new = a.k_new;
  P.v_new = a.v_new;
  P.seq_lens_before = a.seq_lens_before;
  P.seq_lens_after = a.seq_lens_after;
  P.Hkv = p.Hkv;
  P.B = p.B;
  P.max_blocks = p.max_blocks;
  P.max_seq_len = p.max_seq_len;
  if (p.bf16) return p.D == 64 ? launch_t<KvBf16, 64>(p, P, s) : launch_t<KvBf16, 128>(p, P, s);
  return p.D == 64 ? launch_t<KvF32, 64>(p, P, s) : launch_t<KvF32, 128>(p, P, s);
}

}  // namespace hsla
