// Prefill build of the block statistics and the global linear state
// ("SPLA: Block Sparse Plus Linear Attention for Long Context Modeling",
// TL;DR / Abstract: selection from block statistics, residual linear
// attention from a compact state; "SLAKE ..." abstract: first-order Taylor
// kernel, whose state is S = sum_t k_t v_t^T, z = sum_t k_t, sv = sum_t v_t).
//
// k_build_*: one workgroup per (sequence, kv head, chunk of tokens).  Tiles of
// the chunk are staged in LDS; the workgroup writes the statistics of every
// full block in the chunk and a chunk partial of S, z, sv to the workspace.
// For bf16 keys/values the d x d contraction K^T V runs on MFMA
// (v_mfma_f32_32x32x8_bf16, fp32 accumulation, exact bf16 products); tiles are
// stored channel-major in LDS so that each lane's MFMA operand (4 consecutive
// tokens of one channel) is one 8-byte LDS read.  fp32 keys/values use fp32
// FMAs on VALU.
// k_build_reduce: sums the chunk partials in chunk order (deterministic).
#include <algorithm>

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
  size_t part_stride;
};

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int clamp_len(int T, int max_len) { return min(max(T, 0), max_len); }

// Statistics of the full blocks inside a staged tile, channel c, values
// fetched through get(t) for tile-relative token t.  Two passes: mean, then
// the population variance around it.
template <typename Get>
__device__ __forceinline__ void tile_block_stats(const BuildParams& P, int b, int g, int D, int c,
                                                 int tile0, int TT, int T, Get get) {
  const int B = P.B;
  const int32_t* bt = P.block_table + static_cast<size_t>(b) * P.max_blocks;
  for (int t0 = 0; t0 < TT; t0 += B) {
    const int blk = (tile0 + t0) / B;
    if ((blk + 1) * B > T) break;
    float s = 0.f;
    for (int t = 0; t < B; ++t) s += get(t0 + t);
    const float mu = s / static_cast<float>(B);
    float q = 0.f;
    for (int t = 0; t < B; ++t) {
      const float dlt = get(t0 + t) - mu;
      q = fmaf(dlt, dlt, q);
    }
    const size_t off = (static_cast<size_t>(bt[blk]) * P.Hkv + g) * D + c;
    P.blk_mean[off] = mu;
    P.blk_var[off] = q / static_cast<float>(B);
  }
}

// ---------------------------------------------------------------------------
// bf16: MFMA
// ---------------------------------------------------------------------------
template <int D, int TT>
__global__ __launch_bounds__(kThreads) void k_build_bf16(BuildParams P) {
  constexpr int LD = TT + kPad;                    // LDS row length (bf16)
  constexpr int TASKS = (TT / 8) * (D / 8) * 2;    // 8x8 sub-tiles of K and V
  constexpr int TPT = (TASKS + kThreads - 1) / kThreads;
  constexpr int TI = D / 64;                       // 32x32 tiles per wave, each dim
  extern __shared__ uint16_t lds[];
  uint16_t* Kt = lds;                              // [D][LD] channel-major
  uint16_t* Vt = lds + D * LD;

  const int pair = blockIdx.y;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int chunk = blockIdx.x;
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const int c_begin = chunk * P.chunk;
  const int c_end = min(c_begin + P.chunk, T);
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int32_t* bt = P.block_table + static_cast<size_t>(b) * P.max_blocks;
  const int B = P.B;

  f32x16_t acc[TI][TI];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  float csum = 0.f;  // z (threads < D) or sv (threads D..2D-1) partial

  uint4 buf[TPT][8];
  auto load_tile = [&](int tile0) {
#pragma unroll
    for (int x = 0; x < TPT; ++x) {
      const int task = tid + x * kThreads;
      if (task < TASKS) {
        const int tensor = task / ((TT / 8) * (D / 8));
        const int rem = task % ((TT / 8) * (D / 8));
        const int tg = rem / (D / 8);
        const int cg = rem % (D / 8);
        const char* base = reinterpret_cast<const char*>(tensor ? P.v_pages : P.k_pages);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int t = tile0 + tg * 8 + r;
          if (t < c_end) {
            const size_t row = (static_cast<size_t>(bt[t / B]) * P.Hkv + g) * B + (t % B);
            buf[x][r] = *reinterpret_cast<const uint4*>(base + (row * D + cg * 8) * 2);
          } else {
            buf[x][r] = make_uint4(0, 0, 0, 0);
          }
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int x = 0; x < TPT; ++x) {
      const int task = tid + x * kThreads;
      if (task < TASKS) {
        const int tensor = task / ((TT / 8) * (D / 8));
        const int rem = task % ((TT / 8) * (D / 8));
        const int tg = rem / (D / 8);
        const int cg = rem % (D / 8);
        uint16_t* dst = tensor ? Vt : Kt;
        const uint32_t* w = reinterpret_cast<const uint32_t*>(buf[x]);  // [r][4]
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          uint32_t o[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t a = w[(2 * j) * 4 + c / 2];
            const uint32_t bb = w[(2 * j + 1) * 4 + c / 2];
            o[j] = (c & 1) ? ((a >> 16) | (bb & 0xffff0000u)) : ((a & 0xffffu) | (bb << 16));
          }
          *reinterpret_cast<uint4*>(dst + (cg * 8 + c) * LD + tg * 8) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      }
    }
  };

  if (c_begin < c_end) load_tile(c_begin);
  for (int tile0 = c_begin; tile0 < c_end; tile0 += TT) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (tile0 + TT < c_end) load_tile(tile0 + TT);

    // Per-channel sums and the statistics of full blocks.
    if (tid < 2 * D) {
      const uint16_t* row = (tid < D ? Kt + tid * LD : Vt + (tid - D) * LD);
      for (int t = 0; t < TT; t += 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(row + t);
        csum += bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) +
                bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
      }
      if (tid < D) {
        tile_block_stats(P, b, g, D, tid, tile0, TT, T, [&](int t) {
          return __uint_as_float(static_cast<uint32_t>(row[t]) << 16);
        });
      }
    }

    // S += K^T V over the tile: wave (wi, wj) owns rows wi*TI*32.. and
    // columns wj*TI*32.. of S.
    const int rbase = (wave / 2) * TI * 32;
    const int cbase = (wave % 2) * TI * 32;
    const int kl = (lane / 32) * 4;
#pragma unroll 2
    for (int k0 = 0; k0 < TT; k0 += 8) {
      short4_t a[TI], bv[TI];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        a[i] = *reinterpret_cast<const short4_t*>(Kt + (rbase + i * 32 + lane % 32) * LD + k0 + kl);
        bv[i] = *reinterpret_cast<const short4_t*>(Vt + (cbase + i * 32 + lane % 32) * LD + k0 + kl);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a[i], bv[j], acc[i][j], 0, 0, 0);
    }
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
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
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
  for (int c = 0; c < P.nchunk; ++c) {
    const float4 v = *reinterpret_cast<const float4*>(src + static_cast<size_t>(c) * P.part_stride);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
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

template <int D, int TT>
hipError_t launch_bf16(const Problem& p, const BuildLayout& L, const BuildParams& P, hipStream_t s) {
  const size_t lds = static_cast<size_t>(2) * D * (TT + kPad) * sizeof(uint16_t);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_build_bf16<D, TT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  dim3 grid(L.nchunk, p.batch * p.Hkv);
  hipLaunchKernelGGL((k_build_bf16<D, TT>), grid, dim3(kThreads), lds, s, P);
  return launch_status("k_build_bf16");
}

template <int D>
hipError_t launch_d(const Problem& p, const BuildLayout& L, const BuildParams& P, hipStream_t s) {
  hipError_t e;
  if (p.bf16) {
    switch (L.tile) {
      case 64: e = launch_bf16<D, 64>(p, L, P, s); break;
      case 128: e = launch_bf16<D, 128>(p, L, P, s); break;
      case 256: e = launch_bf16<D, 256>(p, L, P, s); break;
      default: return hipErrorInvalidValue;
    }
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
  L.tile = p.bf16 ? std::max(64, p.B) : 32;
  const long pairs = static_cast<long>(p.batch) * p.Hkv;
  // Aim for >= 256 workgroups; chunks of at most 4096 tokens.
  long want = (pairs * p.max_seq_len) / 256;
  long chunk = L.tile;
  while (chunk * 2 <= want && chunk * 2 <= 4096) chunk *= 2;
  if (chunk < L.tile) chunk = L.tile;
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
  P.part_stride = L.part_stride;
  return p.D == 64 ? launch_d<64>(p, L, P, s) : launch_d<128>(p, L, P, s);
}

}  // namespace hsla
