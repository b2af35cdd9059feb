// Append of one decoded token ("SPLA: Block Sparse Plus Linear Attention for
// Long Context Modeling", section "Recurrence"): the token's key and value go
// into their page slot and the length grows by one.  The linear state takes
// whole blocks: when the token completes its block, the block's tokens are
// added (S += K_b^T V_b, z += sum k, sv += sum v) and the block's mean /
// variance statistics are computed.  Until then the incomplete block's
// tokens sit inside the window, where attention is exact, so the linear part
// never needs them; folding them in at completion gives the same outputs as
// a per-token update while the per-step work shrinks to one row write.
//
// A chunk of Q tokens (the multi-query form) goes in two launches around
// the chunk's attention: the first writes the Q page slots (and each query
// row's length for the decode), the second, once every query has read the
// state as it stood before the chunk, folds the block the chunk completed (at
// most one, Q <= B) and sets the new length.
//
// Grid: (row chunks of 32 rows of S + 1, sequence x kv head).  Row chunk 0
// writes the page slots and the new length; on a completing step every chunk
// stages the block through LDS and adds it to its rows of S and z (chunk 0
// also to sv), while the extra workgroup computes the block's statistics
// (it reads the block's rows as 16-byte vectors and reduces per channel
// through LDS, mean first, then the variance around it).
#include "append_parts.h"
#include "internal.h"

namespace hsla {

namespace {

constexpr int kThreads = 256;
constexpr int kFoldRows = 32;   // rows of S per workgroup

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
  int32_t* row_lens;   // chunk writes: each query row's length [batch x count] (or null)
  int Hkv, B, max_blocks, max_seq_len;
  int count;           // tokens per sequence: 1, or the chunk length
  int mode;            // kWriteRows | kFold
  int state_all;       // a per-token state: every appended token enters S, z and sv at once
};
constexpr int kWriteRows = kAppendWriteRows;
constexpr int kFold = kAppendFold;

template <typename KV, int D>
__global__ __launch_bounds__(kThreads) void k_append(AppendParams P) {
  constexpr int C4 = D / 4;                 // float4 columns per row
  constexpr int RG = kThreads / C4;         // row groups
  constexpr int NR = kFoldRows / RG;        // rows per thread
  static_assert(kFoldRows % RG == 0, "rows per workgroup");
  const int pair = blockIdx.y;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int rc = blockIdx.x;
  const int tid = threadIdx.x;
  const int Q = P.count;
  const int T0 = min(max(P.seq_lens_before[b], 0), P.max_seq_len - Q);  // first new token's position
  const size_t nbase = static_cast<size_t>(pair) * D;   // the pair's state rows
  const int B = P.B;
  const int32_t* bt = P.block_table + static_cast<size_t>(b) * P.max_blocks;
  // new token i of the pair: k_new / v_new row ((b Q + i) Hkv + g)
  auto new_row = [&](int i) { return ((static_cast<size_t>(b) * Q + i) * P.Hkv + g) * D; };
  if (rc == 0) {
    if (P.mode & kWriteRows) {
      for (int i = 0; i < Q; ++i) {
        const int t = T0 + i;
        const size_t r = (static_cast<size_t>(bt[t / B]) * P.Hkv + g) * B + t % B;
        if (tid < D) {
          kv_put<KV>(P.k_pages, r * D + tid, P.k_new, new_row(i) + tid);
          kv_put<KV>(P.v_pages, r * D + tid, P.v_new, new_row(i) + tid);
        }
      }
      if (P.row_lens && g == 0 && tid < Q) P.row_lens[static_cast<size_t>(b) * Q + tid] = T0 + 1 + tid;
    }
    if ((P.mode & kFold) && g == 0 && tid == 0 && P.seq_lens_after) P.seq_lens_after[b] = T0 + Q;
  }
  if (!(P.mode & kFold)) return;
  if (P.state_all && rc < D / kFoldRows) {
    // A per-token state (one token per call: the chunk form refuses this
    // state): row chunk rc adds k_r v^T to its rows of S, k_r to z, and
    // chunk 0 adds v to sv.  No block is folded later.
    const int col4 = tid % C4;
    const int r_first = rc * kFoldRows + tid / C4;
    float* Sp = P.S + static_cast<size_t>(pair) * D * D;
    const float4 vv = kv_load4<KV>(P.v_new, new_row(0) + col4 * 4);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int r = r_first + i * RG;
      const float kr = kv_elem<KV>(P.k_new, new_row(0) + r);
      float4* sp = reinterpret_cast<float4*>(Sp + static_cast<size_t>(r) * D + col4 * 4);
      float4 s = *sp;
      s.x = fmaf(kr, vv.x, s.x);
      s.y = fmaf(kr, vv.y, s.y);
      s.z = fmaf(kr, vv.z, s.z);
      s.w = fmaf(kr, vv.w, s.w);
      *sp = s;
    }
    if (tid < kFoldRows) P.z[nbase + rc * kFoldRows + tid] += kv_elem<KV>(P.k_new, new_row(0) + rc * kFoldRows + tid);
    if (rc == 0 && tid < D) P.sv[nbase + tid] += kv_elem<KV>(P.v_new, new_row(0) + tid);
    return;
  }
  const int ic = B - 1 - T0 % B;   // the new token that completes a block, if ic < Q
  if (ic >= Q) return;              // uniform: no block completes
  const int T = T0 + ic;
  const size_t page = static_cast<size_t>(bt[T / B]);
  const size_t row0 = (page * P.Hkv + g) * B;  // first row of this page-head tile
  __shared__ uint4 lds[kFoldStageBytes / 16];   // block stage, or the statistics' sums
  if (rc == D / kFoldRows) {      // the statistics workgroup
    const size_t so = (page * P.Hkv + g) * D;
    filled_block_stats<KV, D, kThreads>(P.k_pages, P.k_new, row0, T % B, new_row(ic), B, P.blk_mean + so, P.blk_var + so,
                                        *reinterpret_cast<BlockStatsLds<kThreads, D>*>(lds));
    return;
  }
  const CompletedBlock cb{P.k_pages, P.v_pages, P.k_new, P.v_new, row0, new_row(ic), T % B, B};
  const int col4 = tid % C4;
  const int r_first = rc * kFoldRows + tid / C4;
  float* Sp = P.S + static_cast<size_t>(pair) * D * D;
  float4 srow[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i)
    srow[i] = *reinterpret_cast<const float4*>(Sp + static_cast<size_t>(r_first + i * RG) * D + col4 * 4);
  const int zrow = tid < kFoldRows ? rc * kFoldRows + tid : -1;
  const int svcol = rc == 0 && tid < D ? tid : -1;
  float z = zrow >= 0 ? P.z[nbase + zrow] : 0.f;
  float sv = svcol >= 0 ? P.sv[nbase + svcol] : 0.f;
  fold_completed_block<KV, D, kThreads, NR, RG>(cb, lds, srow, r_first, col4, zrow, z, svcol, sv);
#pragma unroll
  for (int i = 0; i < NR; ++i)
    *reinterpret_cast<float4*>(Sp + static_cast<size_t>(r_first + i * RG) * D + col4 * 4) = srow[i];
  if (zrow >= 0) P.z[nbase + zrow] = z;
  if (svcol >= 0) P.sv[nbase + svcol] = sv;
}

template <typename KV, int D>
hipError_t launch_t(const Problem& p, const AppendParams& P, hipStream_t s) {
  dim3 grid(D / kFoldRows + 1, p.batch * p.Hkv);   // row chunks + the statistics workgroup
  hipLaunchKernelGGL((k_append<KV, D>), grid, dim3(kThreads), 0, s, P);
  return launch_status("k_append");
}

}  // namespace

hipError_t launch_append(const Problem& p, const AppendArgs& a, hipStream_t s, int count, int mode,
                         int32_t* row_lens) {
  AppendParams P{};
  P.count = count;
  P.mode = mode;
  P.row_lens = row_lens;
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
  P.state_all = p.state_all;
  if (p.bf16) return p.D == 64 ? launch_t<KvBf16, 64>(p, P, s) : launch_t<KvBf16, 128>(p, P, s);
  return p.D == 64 ? launch_t<KvF32, 64>(p, P, s) : launch_t<KvF32, 128>(p, P, s);
}

}  // namespace hsla
