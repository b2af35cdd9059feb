// Append of one decoded token ("SPLA: Block Sparse Plus Linear Attention for
// Long Context Modeling", section "Recurrence"): the token's key and value go
// into their page slot, the global linear state takes the rank-1 update
// S += k v^T, z += k, sv += v, and when the token completes its block the
// block's mean / variance statistics are computed.
//
// Grid: (row chunks of S, sequence x kv head).  Row chunk 0 also writes the
// page slot, z, sv, the filled block's statistics and the new length.
#include "common.h"
#include "internal.h"

namespace hsla {

namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;  // rows of S per workgroup

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

template <typename KV, int D>
__global__ __launch_bounds__(kThreads) void k_append(AppendParams P) {
  const int pair = blockIdx.y;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int rc = blockIdx.x;
  const int tid = threadIdx.x;
  const int T = min(max(P.seq_lens_before[b], 0), P.max_seq_len - 1);  // new token's position
  const size_t nbase = static_cast<size_t>(pair) * D;

  // Rank-1 update of rows [rc*kRows, rc*kRows + kRows) of S.
  constexpr int C4 = D / 4;
  float* Sp = P.S + static_cast<size_t>(pair) * D * D;
  for (int idx = tid; idx < kRows * C4; idx += kThreads) {
    const int r = rc * kRows + idx / C4;
    const int c4 = idx % C4;
    const float kr = elem<KV>(P.k_new, nbase + r);
    float4* sp = reinterpret_cast<float4*>(Sp + static_cast<size_t>(r) * D + c4 * 4);
    float4 s = *sp;
    s.x = fmaf(kr, elem<KV>(P.v_new, nbase + c4 * 4 + 0), s.x);
    s.y = fmaf(kr, elem<KV>(P.v_new, nbase + c4 * 4 + 1), s.y);
    s.z = fmaf(kr, elem<KV>(P.v_new, nbase + c4 * 4 + 2), s.z);
    s.w = fmaf(kr, elem<KV>(P.v_new, nbase + c4 * 4 + 3), s.w);
    *sp = s;
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
    if ((T + 1) % B == 0) {
      // Tokens [blk*B, T]; the last one is the new key itself.
      const int last = T % B;
      float s = 0.f;
      for (int t = 0; t < last; ++t) s += elem<KV>(P.k_pages, (row0 + t) * D + c);
      s += elem<KV>(P.k_new, nbase + c);
      const float mu = s / static_cast<float>(B);
      float q = 0.f;
      for (int t = 0; t < last; ++t) {
        const float dlt = elem<KV>(P.k_pages, (row0 + t) * D + c) - mu;
        q = fmaf(dlt, dlt, q);
      }
      const float dn = elem<KV>(P.k_new, nbase + c) - mu;
      q = fmaf(dn, dn, q);
      P.blk_mean[(page * P.Hkv + g) * D + c] = mu;
      P.blk_var[(page * P.Hkv + g) * D + c] = q / static_cast<float>(B);
    }
  }
  if (g == 0 && tid == 0 && P.seq_lens_after) P.seq_lens_after[b] = T + 1;
}

template <typename KV, int D>
hipError_t launch_t(const Problem& p, const AppendParams& P, hipStream_t s) {
  dim3 grid(D / kRows, p.batch * p.Hkv);
  hipLaunchKernelGGL((k_append<KV, D>), grid, dim3(kThreads), 0, s, P);
  return launch_status("k_append");
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
