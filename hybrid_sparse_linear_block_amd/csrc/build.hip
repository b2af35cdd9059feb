// Prefill build of the block statistics and the global linear state
// ("SPLA: Block Sparse Plus Linear Attention for Long Context Modeling",
// TL;DR / Abstract: selection from block statistics, residual linear
// attention from a compact state; "SLAKE ..." abstract: first-order Taylor
// kernel, whose state is S = sum_t k_t v_t^T, z = sum_t k_t, sv = sum_t v_t,
// here over the tokens of complete blocks).
//
// k_build_*: one workgroup per (sequence, kv head, chunk of tokens).  Tiles of
// the chunk are staged in LDS; the workgroup writes the statistics of every
// full block in the chunk and a chunk partial of S, z, sv to the workspace.
// For bf16 keys/values the d x d contraction K^T V runs on MFMA
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation, exact bf16 products); tiles are
// stored channel-major in LDS so that each lane's MFMA operand (4 consecutive
// tokens of one channel) is one 8-byte LDS read.  fp32 keys/values use fp32
// FMAs on VALU.
// k_build_reduce: sums the chunk partials in chunk order (deterministic).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace hsla {

namespace {

constexpr int kThreads = 256;
constexpr int kPad = 8;  // bf16 elements of padding per LDS row

struct BuildParams {
  const void* k_pages;
  const void* v_pages;
  float* blk_mean;
  float* blk_var;
  const int32_t* block_table;
  float* S;
  float* z;
  float* sv;
  const int32_t* seq_lens;
  float* ws;
  int Hkv, B, max_blocks, max_seq_len, chunk, nchunk;
  int state_all;   // the state takes every token, not only those of complete blocks
  size_t part_stride;
};

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int clamp_len(int T, int max_len) { return min(max(T, 0), max_len); }
__device__ __forceinline__ int full_blocks_len(int T, int B) { return T - T % B; }
// Tokens the state is built over: those of complete blocks, or all of them.
__device__ __forceinline__ int state_len(const BuildParams& P, int b) {
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  return P.state_all ? T : full_blocks_len(T, P.B);
}

// ---------------------------------------------------------------------------
// bf16: MFMA
// ---------------------------------------------------------------------------
// One workgroup per (sequence, kv head, chunk of tokens); tiles of 64 tokens.
// Thread task = 8 tokens x 8 channels of K or V (eight 16-byte row loads of
// one page); the 8 x 8 block is transposed in registers and stored
// channel-major in LDS.  Lanes take the token groups fastest, so that the
// 16 lanes of one 16-byte LDS store hit 16 distinct bank quads (with the
// channel groups fastest, lanes 8 channels apart share banks: 8-way
// conflicts that dominated the kernel), while each global load still reads
// whole 128-byte lines.  The layout serves two readers:
//   * the MFMA operands (8 consecutive tokens of one channel) are single
//     16-byte LDS reads: S += K^T V with v_mfma_f32_32x32x16_bf16, wave
//     (wi, wj) owning a D/2 x D/2 quarter of S;
//   * thread c < D reads channel c of K as contiguous vectors for the block
//     statistics (two-pass within the tile, combined across the tiles of a
//     block larger than 64 tokens by the pairwise update of Chan et al.) and
//     threads D..2D-1 sum V for sv.
// The chunk's block-table entries are staged in LDS once; every load is
// unconditional (rows past the end are read from a mapped page and zeroed),
// and three tiles are in flight while one is processed.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kTile = 64;           // tokens per tile
constexpr int kMaxChunkBlocks = 256;  // block-table entries staged per chunk

template <int D>
__global__ __launch_bounds__(kThreads, 2) void k_build_bf16(BuildParams P) {
  constexpr int LD = kTile + kPad;                 // LDS row length (bf16)
  constexpr int TASKS = (kTile / 8) * (D / 8) * 2;
  static_assert(TASKS % kThreads == 0 || kThreads % TASKS == 0, "whole tasks per thread");
  constexpr int TPT = TASKS >= kThreads ? TASKS / kThreads : 1;   // tasks per thread
  constexpr bool kPartial = TASKS < kThreads;      // D = 64: waves 2, 3 have no load task
  constexpr int TI = D / 64;                       // 32x32 tiles per wave, each dim
  __shared__ __attribute__((aligned(16))) uint16_t Kt[D * LD];   // [D][LD] channel-major
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * LD];
  __shared__ int32_t pages[kMaxChunkBlocks];

  const int pair = blockIdx.y;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int chunk = blockIdx.x;
  // the state holds the tokens of complete blocks (the incomplete last
  // block's tokens lie inside the window and are attended exactly), or
  // every token when the caller keeps a per-token state
  const int T = state_len(P, b);
  const int c_begin = chunk * P.chunk;
  const int c_end = min(c_begin + P.chunk, T);
  if (c_begin >= c_end) {
    // still write a zero partial so that the reduction reads defined data
    float* part = P.ws + (static_cast<size_t>(pair) * P.nchunk + chunk) * P.part_stride;
    for (int i = threadIdx.x; i < D * D + 2 * D; i += kThreads) part[i] = 0.f;
    return;
  }
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int B = P.B;
  const int blk0 = c_begin / B;                             // chunks start on block boundaries
  const int nblk = ceil_div(c_end - c_begin, B);            // blocks touched by the chunk
  const int32_t* bt = P.block_table + static_cast<size_t>(b) * P.max_blocks;
  for (int i = tid; i < nblk; i += kThreads) pages[i] = bt[blk0 + i];
  __syncthreads();

  f32x16_t acc[TI][TI];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  float csum = 0.f;                   // z (threads < D) or sv (threads D..2D-1) partial
  float run_mean = 0.f, run_m2 = 0.f; // statistics of a block spanning tiles (B > 64)
  int run_n = 0;

  const char* kbase = reinterpret_cast<const char*>(P.k_pages);
  const char* vbase = reinterpret_cast<const char*>(P.v_pages);
  struct TileRegs {
    uint4 w[TPT][8];
  };
  auto load_tile = [&](int tile0, TileRegs& x) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int task = tid + u * kThreads;
      if (kPartial && task >= TASKS) break;
      const int tensor = task / ((kTile / 8) * (D / 8));
      const int rem = task % ((kTile / 8) * (D / 8));
      const int tg = rem % (kTile / 8);
      const int cg = rem / (kTile / 8);
      // first token of the group, clamped to the last group that holds a
      // token (a multiple of 8, so the 8 rows stay inside one page)
      const int t8 = min(tile0 + tg * 8, (c_end - 1) & ~7);
      const int page = pages[(t8 - c_begin) / B];
      const int row0 = t8 % B;                                 // 8 | B: the group is in one page
      const char* base = (tensor ? vbase : kbase) +
                         (((static_cast<size_t>(page) * P.Hkv + g) * B + row0) * D + cg * 8) * 2;
#pragma unroll
      for (int r = 0; r < 8; ++r) x.w[u][r] = *reinterpret_cast<const uint4*>(base + r * D * 2);
    }
  };
  auto store_tile = [&](int tile0, const TileRegs& x) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int task = tid + u * kThreads;
      if (kPartial && task >= TASKS) break;
      const int tensor = task / ((kTile / 8) * (D / 8));
      const int rem = task % ((kTile / 8) * (D / 8));
      const int tg = rem % (kTile / 8);
      const int cg = rem / (kTile / 8);
      uint16_t* dst = tensor ? Vt : Kt;
      uint32_t w[8][4];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const bool live = tile0 + tg * 8 + r < c_end;   // rows past the end enter as zero
        w[r][0] = live ? x.w[u][r].x : 0u;
        w[r][1] = live ? x.w[u][r].y : 0u;
        w[r][2] = live ? x.w[u][r].z : 0u;
        w[r][3] = live ? x.w[u][r].w : 0u;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t a = w[2 * j][c / 2];
          const uint32_t bb = w[2 * j + 1][c / 2];
          o[j] = (c & 1) ? __builtin_amdgcn_perm(bb, a, 0x07060302u) : __builtin_amdgcn_perm(bb, a, 0x05040100u);
        }
        *reinterpret_cast<uint4*>(dst + (cg * 8 + c) * LD + tg * 8) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  };

  // Three tiles in flight.  The loop runs a multiple of three tiles so that
  // every buffer is named statically (no load stays in flight across a
  // branch); tiles past the chunk end load clamped rows and contribute zero.
  const int ntile = ceil_div(c_end - c_begin, kTile);
  const int nrun = ceil_div(ntile, 3) * 3;
  TileRegs r0, r1, r2;
  load_tile(c_begin, r0);
  load_tile(c_begin + kTile, r1);
  load_tile(c_begin + 2 * kTile, r2);
  auto tile_step = [&](int it, TileRegs& buf) __attribute__((always_inline)) {
    const int tile0 = c_begin + it * kTile;
    __syncthreads();   // the previous tile's LDS reads are done
    store_tile(tile0, buf);
    __syncthreads();
    load_tile(tile0 + 3 * kTile, buf);   // refill the buffer just stored

    // ---- sums of K and V per channel; block statistics of K
    if (tid < 2 * D) {
      const uint16_t* row = tid < D ? Kt + tid * LD : Vt + (tid - D) * LD;
      uint4 q[kTile / 8];
#pragma unroll
      for (int v = 0; v < kTile / 8; ++v) q[v] = *reinterpret_cast<const uint4*>(row + v * 8);
      auto xt = [&](int t) -> float {   // token t of the tile (t is a constant after unrolling)
        const uint4 w = q[t / 8];
        const uint32_t u = (t % 8) / 2 == 0 ? w.x : (t % 8) / 2 == 1 ? w.y : (t % 8) / 2 == 2 ? w.z : w.w;
        return (t % 2) ? bf16_hi(u) : bf16_lo(u);
      };
#pragma unroll
      for (int t = 0; t < kTile; ++t) csum += xt(t);
      if (tid < D) {
        auto stats = [&](auto seg_c) __attribute__((always_inline)) {
          constexpr int SEG = decltype(seg_c)::value;   // tokens of one block inside the tile
#pragma unroll
          for (int s0 = 0; s0 < kTile; s0 += SEG) {
            const int blk = (tile0 + s0) / B;
            float sm = 0.f;
#pragma unroll
            for (int t = 0; t < SEG; ++t) sm += xt(s0 + t);
            const float mu = sm / static_cast<float>(SEG);
            float m2 = 0.f;
#pragma unroll
            for (int t = 0; t < SEG; ++t) {
              const float dlt = xt(s0 + t) - mu;
              m2 = fmaf(dlt, dlt, m2);
            }
            // fold the segment into its block (a new block starts the run)
            if (run_n == 0) {
              run_mean = mu;
              run_m2 = m2;
            } else {
              const float n_a = static_cast<float>(run_n);
              const float n_b = static_cast<float>(SEG);
              const float dl = mu - run_mean;
              run_mean = run_mean + dl * (n_b / (n_a + n_b));
              run_m2 = run_m2 + m2 + dl * dl * (n_a * n_b / (n_a + n_b));
            }
            run_n += SEG;
            if (run_n == B) {   // the block is complete
              // only blocks that end inside the chunk (c_end <= T): the
              // padding tiles past the chunk reach blocks whose pages are
              // not staged
              if ((blk + 1) * B <= c_end) {
                const size_t off = (static_cast<size_t>(pages[blk - blk0]) * P.Hkv + g) * D + tid;
                P.blk_mean[off] = run_mean;
                P.blk_var[off] = run_m2 / static_cast<float>(B);
              }
              run_n = 0;
            }
          }
        };
        if (B == 16)
          stats(std::integral_constant<int, 16>{});
        else if (B == 32)
          stats(std::integral_constant<int, 32>{});
        else
          stats(std::integral_constant<int, kTile>{});
      }
    }

    // ---- S += K^T V over the tile
    const int rbase = (wave / 2) * TI * 32;
    const int cbase = (wave % 2) * TI * 32;
    const int kl = (lane / 32) * 8;
#pragma unroll
    for (int k0 = 0; k0 < kTile; k0 += 16) {
      bf16x8_t a[TI], bv[TI];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        a[i] = *reinterpret_cast<const bf16x8_t*>(Kt + (rbase + i * 32 + lane % 32) * LD + k0 + kl);
        bv[i] = *reinterpret_cast<const bf16x8_t*>(Vt + (cbase + i * 32 + lane % 32) * LD + k0 + kl);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], bv[j], acc[i][j], 0, 0, 0);
    }
  };
  for (int it = 0; it < nrun; it += 3) {
    tile_step(it, r0);
    tile_step(it + 1, r1);
    tile_step(it + 2, r2);
  }

  // Chunk partial: S (D*D), z (D), sv (D).
  float* part = P.ws + (static_cast<size_t>(pair) * P.nchunk + chunk) * P.part_stride;
  const int rbase = (wave / 2) * TI * 32;
  const int cbase = (wave % 2) * TI * 32;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = rbase + i * 32 + (r / 4) * 8 + (lane / 32) * 4 + (r % 4);
        const int col = cbase + j * 32 + lane % 32;
        part[row * D + col] = acc[i][j][r];
      }
  if (tid < 2 * D) part[D * D + tid] = csum;
}

// ---------------------------------------------------------------------------
// fp32: VALU
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void k_build_f32(BuildParams P) {
  constexpr int TT = 32;
  constexpr int MT = D / 16;  // 16x16 threads, each owns an MT x MT block of S
  __shared__ float Ks[TT][D];
  __shared__ float Vs[TT][D];
  const int pair = blockIdx.y;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int chunk = blockIdx.x;
  // the state holds the tokens of complete blocks (the incomplete last
  // block's tokens lie inside the window and are attended exactly), or
  // every token when the caller keeps a per-token state
  const int T = state_len(P, b);
  const int c_begin = chunk * P.chunk;
  const int c_end = min(c_begin + P.chunk, T);
  const int tid = threadIdx.x;
  const int ti = tid / 16;
  const int tj = tid % 16;
  const int32_t* bt = P.block_table + static_cast<size_t>(b) * P.max_blocks;
  const int B = P.B;
  float acc[MT][MT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[i][j] = 0.f;
  float csum = 0.f;
  const float* kp = reinterpret_cast<const float*>(P.k_pages);
  const float* vp = reinterpret_cast<const float*>(P.v_pages);

  for (int tile0 = c_begin; tile0 < c_end; tile0 += TT) {
    __syncthreads();
    for (int idx = tid; idx < TT * D / 4; idx += kThreads) {
      const int t = idx / (D / 4);
      const int c4 = idx % (D / 4);
      const int tok = tile0 + t;
      float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
      if (tok < c_end) {
        const size_t row = (static_cast<size_t>(bt[tok / B]) * P.Hkv + g) * B + (tok % B);
        kv = *reinterpret_cast<const float4*>(kp + row * D + c4 * 4);
        vv = *reinterpret_cast<const float4*>(vp + row * D + c4 * 4);
      }
      *reinterpret_cast<float4*>(&Ks[t][c4 * 4]) = kv;
      *reinterpret_cast<float4*>(&Vs[t][c4 * 4]) = vv;
    }
    __syncthreads();
    if (tid < 2 * D) {
      const int c = tid % D;
      if (tid < D) {
        for (int t = 0; t < TT; ++t) csum += Ks[t][c];
      } else {
        for (int t = 0; t < TT; ++t) csum += Vs[t][c];
      }
    }
    for (int t = 0; t < TT; ++t) {
      float kr[MT], vr[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        kr[i] = Ks[t][ti * MT + i];
        vr[i] = Vs[t][tj * MT + i];
      }
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[i][j] = fmaf(kr[i], vr[j], acc[i][j]);
    }
  }
  float* part = P.ws + (static_cast<size_t>(pair) * P.nchunk + chunk) * P.part_stride;
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < MT; ++j) part[(ti * MT + i) * D + tj * MT + j] = acc[i][j];
  if (tid < 2 * D) part[D * D + tid] = csum;
}

// Statistics of every full block, one workgroup per (block, sequence, kv
// head), one thread per channel (fp32 keys).
template <int D>
__global__ __launch_bounds__(D) void k_block_stats_f32(BuildParams P) {
  const int pair = blockIdx.y;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int blk = blockIdx.x;
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const int B = P.B;
  if ((blk + 1) * B > T) return;
  const int c = threadIdx.x;
  const size_t page = static_cast<size_t>(P.block_table[static_cast<size_t>(b) * P.max_blocks + blk]);
  const float* rows = reinterpret_cast<const float*>(P.k_pages) + (page * P.Hkv + g) * B * D + c;
  float s = 0.f;
  for (int t = 0; t < B; ++t) s += rows[static_cast<size_t>(t) * D];
  const float mu = s / static_cast<float>(B);
  float q = 0.f;
  for (int t = 0; t < B; ++t) {
    const float dlt = rows[static_cast<size_t>(t) * D] - mu;
    q = fmaf(dlt, dlt, q);
  }
  P.blk_mean[(page * P.Hkv + g) * D + c] = mu;
  P.blk_var[(page * P.Hkv + g) * D + c] = q / static_cast<float>(B);
}

// Sum of the chunk partials, in chunk order.
template <int D>
__global__ __launch_bounds__(kThreads) void k_build_reduce(BuildParams P) {
  const int pair = blockIdx.y;
  const int e4 = blockIdx.x * kThreads + threadIdx.x;   // float4 index
  constexpr int N4 = (D * D + 2 * D) / 4;
  if (e4 >= N4) return;
  const float* src = P.ws + static_cast<size_t>(pair) * P.nchunk * P.part_stride + e4 * 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  // eight partials in flight, summed in chunk order
  constexpr int U = 8;
  for (int c0 = 0; c0 < P.nchunk; c0 += U) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = c0 + u < P.nchunk ? *reinterpret_cast<const float4*>(src + static_cast<size_t>(c0 + u) * P.part_stride)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      s.x += v[u].x;
      s.y += v[u].y;
      s.z += v[u].z;
      s.w += v[u].w;
    }
  }
  const int e = e4 * 4;
  float* dst;
  if (e < D * D) {
    dst = P.S + static_cast<size_t>(pair) * D * D + e;
  } else if (e < D * D + D) {
    dst = P.z + static_cast<size_t>(pair) * D + (e - D * D);
  } else {
    dst = P.sv + static_cast<size_t>(pair) * D + (e - D * D - D);
  }
  *reinterpret_cast<float4*>(dst) = s;
}

template <int D>
hipError_t launch_d(const Problem& p, const BuildLayout& L, const BuildParams& P, hipStream_t s) {
  hipError_t e;
  if (p.bf16) {
    dim3 grid(L.nchunk, p.batch * p.Hkv);
    hipLaunchKernelGGL((k_build_bf16<D>), grid, dim3(kThreads), 0, s, P);
    e = launch_status("k_build_bf16");
  } else {
    dim3 grid(L.nchunk, p.batch * p.Hkv);
    hipLaunchKernelGGL((k_build_f32<D>), grid, dim3(kThreads), 0, s, P);
    e = launch_status("k_build_f32");
    if (e != hipSuccess) return e;
    dim3 sgrid(std::max(1, p.nblk_max), p.batch * p.Hkv);
    hipLaunchKernelGGL((k_block_stats_f32<D>), sgrid, dim3(D), 0, s, P);
    e = launch_status("k_block_stats_f32");
  }
  if (e != hipSuccess) return e;
  constexpr int N4 = (D * D + 2 * D) / 4;
  dim3 rgrid(ceil_div(N4, kThreads), p.batch * p.Hkv);
  hipLaunchKernelGGL((k_build_reduce<D>), rgrid, dim3(kThreads), 0, s, P);
  return launch_status("k_build_reduce");
}

}  // namespace

BuildLayout build_layout(const Problem& p) {
  BuildLayout L{};
  L.tile = p.bf16 ? kTile : 32;
  const long pairs = static_cast<long>(p.batch) * p.Hkv;
  // About two workgroups per CU (512); chunks are whole blocks and whole
  // tiles, at most 4096 tokens and at most kMaxChunkBlocks blocks.
  const long want = (pairs * p.max_seq_len) / 512;
  const long unit = std::max<long>(L.tile, p.B);
  const long cap = std::min<long>(4096, static_cast<long>(kMaxChunkBlocks) * p.B);
  long chunk = unit;
  while (chunk * 2 <= want && chunk * 2 <= cap) chunk *= 2;
  L.chunk = static_cast<int>(chunk);
  L.nchunk = ceil_div(p.max_seq_len, L.chunk);
  L.part_stride = static_cast<size_t>(p.D) * p.D + 2 * p.D;
  L.total = sizeof(float) * static_cast<size_t>(pairs) * L.nchunk * L.part_stride;
  return L;
}

hipError_t launch_build(const Problem& p, const BuildLayout& L, const BuildArgs& a, hipStream_t s) {
  BuildParams P{};
  P.k_pages = a.k_pages;
  P.v_pages = a.v_pages;
  P.blk_mean = a.blk_mean;
  P.blk_var = a.blk_var;
  P.block_table = a.block_table;
  P.S = a.S;
  P.z = a.z;
  P.sv = a.sv;
  P.seq_lens = a.seq_lens;
  P.ws = a.ws;
  P.Hkv = p.Hkv;
  P.B = p.B;
  P.max_blocks = p.max_blocks;
  P.max_seq_len = p.max_seq_len;
  P.chunk = L.chunk;
  P.nchunk = L.nchunk;
  P.state_all = p.state_all;
  P.part_stride = L.part_stride;
  return p.D == 64 ? launch_d<64>(p, L, P, s) : launch_d<128>(p, L, P, s);
}

}  // namespace hsla
