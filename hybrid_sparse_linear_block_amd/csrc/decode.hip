// Decode step of hybrid sparse-plus-linear attention on gfx950.
//
// Four kernels, all enqueued on the caller's stream:
//   1. k_score_readout  per (sequence, kv head): block scores of the candidate
//      blocks for the G query heads of the group, read from the per-block
//      mean / variance statistics ("SPLA: Block Sparse Plus Linear Attention
//      for Long Context Modeling", section "Principled Block Selection via
//      Taylor Expansion"), and, in the same launch, the readout of the global
//      linear state S^T q, q.z for those heads ("Residual Linear Attention
//      (RLA)").
//   2. k_select         one wavefront per query head: radix select of the
//      top-k candidates (score desc, index asc), ascending index output, and
//      the per-(sequence, kv head) union of the group's exact blocks (sinks,
//      window and selected blocks) with a per-block mask of the heads that
//      selected it (SPLA Figure 1(a)).
//   3. k_attend         split-K over the union: each page is read once per kv
//      head and serves every query head that needs it; online softmax for
//      the exact part plus the first-order-Taylor sums sum(1+s)v, sum(1+s)
//      of the exact tokens, which are subtracted from the global state
//      (SPLA Abstract, "global minus selected").
//   4. k_merge          log-sum-exp combination of the splits and the
//      residual linear part into the normalised output.
#include <math.h>

#include <algorithm>

#include <type_traits>
#include <utility>

#include "common.h"
#include "internal.h"

namespace hsla {

namespace {

constexpr int kThreads = 256;
constexpr float kNegInf = -INFINITY;
constexpr int kScoreChunk = 64;  // candidates per scoring workgroup
constexpr int kRoRows = 16;      // rows of S per readout workgroup
constexpr int kUnit = 64;        // tokens per attention work unit
constexpr int kUnitsPerWg = 8;   // attention work units per workgroup

struct DecodeParams {
  const void* k_pages;
  const void* v_pages;
  const float* blk_mean;
  const float* blk_var;
  const int32_t* block_table;
  const float* S;
  const float* z;
  const float* sv;
  const void* q;
  const int32_t* seq_lens;
  float* out;
  int32_t* sel_idx;
  float* scores;
  float* ro;
  float* roz;
  int32_t* ulist;
  int32_t* upage;
  int32_t* ucount;
  float* part;
  int Hq, Hkv, B, top_k, ns, W, linear_tail;
  int max_blocks, max_seq_len, nc_max, nblk_max;
  int score_wgs, ro_wgs;
  int umax, bps, max_split, pstride;
  int keys_staged;
  float sigma;
};

__device__ __forceinline__ int clamp_len(int T, int max_len) { return min(max(T, 1), max_len); }

// Query of one head, 8 channels per lane.
template <typename KV>
struct QReg;

template <>
struct QReg<KvBf16> {
  uint32_t w[4];
  __device__ __forceinline__ void load(const void* p) {
    const uint4 r = *reinterpret_cast<const uint4*>(p);
    w[0] = r.x; w[1] = r.y; w[2] = r.z; w[3] = r.w;
  }
  __device__ __forceinline__ float dot(const Row8<KvBf16>& k) const {
    float d = 0.f;
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[0]), __builtin_bit_cast(bf16x2_t, k.raw.x), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[1]), __builtin_bit_cast(bf16x2_t, k.raw.y), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[2]), __builtin_bit_cast(bf16x2_t, k.raw.z), d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[3]), __builtin_bit_cast(bf16x2_t, k.raw.w), d, false);
    return d;
  }
  __device__ __forceinline__ void to_f32(float (&f)[8]) const {
    f[0] = bf16_lo(w[0]); f[1] = bf16_hi(w[0]); f[2] = bf16_lo(w[1]); f[3] = bf16_hi(w[1]);
    f[4] = bf16_lo(w[2]); f[5] = bf16_hi(w[2]); f[6] = bf16_lo(w[3]); f[7] = bf16_hi(w[3]);
  }
};

template <>
struct QReg<KvF32> {
  float f[8];
  __device__ __forceinline__ void load(const void* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ __forceinline__ float dot(const Row8<KvF32>& k) const {
    float d = f[0] * k.a.x;
    d = fmaf(f[1], k.a.y, d); d = fmaf(f[2], k.a.z, d); d = fmaf(f[3], k.a.w, d);
    d = fmaf(f[4], k.b.x, d); d = fmaf(f[5], k.b.y, d); d = fmaf(f[6], k.b.z, d); d = fmaf(f[7], k.b.w, d);
    return d;
  }
  __device__ __forceinline__ void to_f32(float (&o)[8]) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f[i];
  }
};

template <typename KV>
__device__ __forceinline__ float q_elem(const void* q, size_t idx) {
  if constexpr (KV::kBytes == 2) {
    const uint16_t u = reinterpret_cast<const uint16_t*>(q)[idx];
    return __uint_as_float(static_cast<uint32_t>(u) << 16);
  } else {
    return reinterpret_cast<const float*>(q)[idx];
  }
}

// ---------------------------------------------------------------------------
// 1. Block scores + global-state readout
// ---------------------------------------------------------------------------
template <typename KV, int D, int G>
__device__ __forceinline__ void score_part(const DecodeParams& P, int b, int g, int T, int chunk) {
  constexpr int LPT = D / 8;            // lanes per candidate (8 channels each)
  constexpr int CPP = kThreads / LPT;   // candidates per pass
  constexpr int NIT = kScoreChunk / CPP;
  static_assert(G <= LPT, "one writer lane per head");
  const CandRange cr = candidate_range(T, P.B, P.ns, P.W);
  const int nc = min(cr.count, P.nc_max);
  const int c_begin = chunk * kScoreChunk;
  if (c_begin >= nc) return;
  const int tid = threadIdx.x;
  const int lig = tid % LPT;
  const int slot = tid / LPT;
  const int32_t* bt = P.block_table + static_cast<size_t>(b) * P.max_blocks;

  // Issue every load of the chunk before any arithmetic: page ids, then the
  // statistics rows, then the queries.
  int page[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int c = c_begin + slot + it * CPP;
    const int pg = bt[cr.lo + min(c, nc - 1)];
    page[it] = (c < nc) ? pg : -1;
  }
  float4 m0[NIT], m1[NIT], v0[NIT], v1[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {   // unconditional loads; unused slots read page 0
    const size_t off = (static_cast<size_t>(max(page[it], 0)) * P.Hkv + g) * D + lig * 8;
    m0[it] = *reinterpret_cast<const float4*>(P.blk_mean + off);
    m1[it] = *reinterpret_cast<const float4*>(P.blk_mean + off + 4);
    v0[it] = *reinterpret_cast<const float4*>(P.blk_var + off);
    v1[it] = *reinterpret_cast<const float4*>(P.blk_var + off + 4);
  }
  // sigma q and (sigma^2 / 2) q^2: the score is then two plain dot products.
  float qs[G][8], qq[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    QReg<KV> qr;
    qr.load(reinterpret_cast<const char*>(P.q) +
            ((static_cast<size_t>(b) * P.Hq + g * G + h) * D + lig * 8) * KV::kBytes);
    float qf[8];
    qr.to_f32(qf);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qs[h][i] = P.sigma * qf[i];
      qq[h][i] = 0.5f * qs[h][i] * qs[h][i];
    }
  }
  const int hsel = lig % G;   // the head whose score this lane finishes
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const float mu[8] = {m0[it].x, m0[it].y, m0[it].z, m0[it].w, m1[it].x, m1[it].y, m1[it].z, m1[it].w};
    const float va[8] = {v0[it].x, v0[it].y, v0[it].z, v0[it].w, v1[it].x, v1[it].y, v1[it].z, v1[it].w};
    float d1 = 0.f, d2 = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.f, c = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a = fmaf(qs[h][i], mu[i], a);
        c = fmaf(qq[h][i], va[i], c);
      }
      a = reduce_sum_lanes<LPT>(a);
      c = reduce_sum_lanes<LPT>(c);
      d1 = (h == hsel) ? a : d1;
      d2 = (h == hsel) ? c : d2;
    }
    const int cidx = c_begin + slot + it * CPP;
    if (lig < G && page[it] >= 0) {
      // log(1 + x) via the hardware logarithm: x >= 0, absolute error ~1e-7.
      P.scores[(static_cast<size_t>(b) * P.Hq + g * G + lig) * P.nc_max + cidx] = d1 + __logf(1.f + d2);
    }
  }
}

template <typename KV, int D, int G>
__device__ __forceinline__ void readout_part(const DecodeParams& P, int b, int g, int rc) {
  constexpr int C4 = D / 4;            // float4 columns per row
  constexpr int RG = kThreads / C4;    // row groups
  constexpr int NR = kRoRows / RG;     // rows per thread
  static_assert(kRoRows % RG == 0, "rows per readout workgroup");
  __shared__ float red[kThreads / kWave][C4][G][4];
  const int tid = threadIdx.x;
  const int col4 = tid % C4;
  const int rg = tid / C4;
  const int pair = b * P.Hkv + g;
  const int r0 = rc * kRoRows;
  const float* Sp = P.S + static_cast<size_t>(pair) * D * D;
  const size_t qbase = (static_cast<size_t>(b) * P.Hq + g * G) * D;

  float4 srow[NR];
  float qv[NR][G];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int r = r0 + rg + i * RG;
    srow[i] = *reinterpret_cast<const float4*>(Sp + static_cast<size_t>(r) * D + col4 * 4);
#pragma unroll
    for (int h = 0; h < G; ++h) qv[i][h] = q_elem<KV>(P.q, qbase + static_cast<size_t>(h) * D + r);
  }
  float acc[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.f;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      acc[h][0] = fmaf(qv[i][h], srow[i].x, acc[h][0]);
      acc[h][1] = fmaf(qv[i][h], srow[i].y, acc[h][1]);
      acc[h][2] = fmaf(qv[i][h], srow[i].z, acc[h][2]);
      acc[h][3] = fmaf(qv[i][h], srow[i].w, acc[h][3]);
    }
  }
  // Row groups inside a wavefront sit C4 lanes apart.
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (C4 <= 16) acc[h][j] = pair_sum<16>(acc[h][j]);
      acc[h][j] = pair_sum<32>(acc[h][j]);
    }
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  if (lane < C4) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][lane][h][j] = acc[h][j];
  }
  __syncthreads();
  float* ro = P.ro + (static_cast<size_t>(pair) * P.ro_wgs + rc) * G * D;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int c = idx % D;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) v += red[w][c / 4][h][c % 4];
    ro[idx] = v;
  }
  if (tid < G) {
    const int h = tid;
    const float* zp = P.z + static_cast<size_t>(pair) * D + r0;
    float zr[kRoRows], qr[kRoRows];
#pragma unroll
    for (int r = 0; r < kRoRows; ++r) {
      zr[r] = zp[r];
      qr[r] = q_elem<KV>(P.q, qbase + static_cast<size_t>(h) * D + r0 + r);
    }
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < kRoRows; ++r) v = fmaf(qr[r], zr[r], v);
    P.roz[(static_cast<size_t>(pair) * P.ro_wgs + rc) * G + h] = v;
  }
}

template <typename KV, int D, int G>
__global__ __launch_bounds__(kThreads) void k_score_readout(DecodeParams P) {
  const int pair = blockIdx.y;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int x = blockIdx.x;
  if (x < P.score_wgs) {
    const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
    score_part<KV, D, G>(P, b, g, T, x);
  } else {
    readout_part<KV, D, G>(P, b, g, x - P.score_wgs);
  }
}

// ---------------------------------------------------------------------------
// 2. Top-k selection and union of the group's exact blocks
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off)));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), off)));
  return v;
}
__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// Union of the group's exact blocks, ascending: blocks below the candidates
// (sinks), candidates that some head selected or that hold sink or window
// tokens, and blocks past the candidates (window).  Entry = block index |
// (mask of the heads that selected it) << 20; the block's page goes to upage.
template <int G>
__device__ __forceinline__ void build_union(const DecodeParams& P, int pair, int b, int T, const CandRange& cr,
                                            int nc, int nwords, const uint64_t* sel_bits, int lane, int hh) {
  if (hh != 0) return;
  const int nb = min(ceil_div(T, P.B), P.nblk_max);
  const int win0 = T - P.W;
  int cnt = 0;
  int32_t* ul = P.ulist + static_cast<size_t>(pair) * P.umax;
  int32_t* up = P.upage + static_cast<size_t>(pair) * P.umax;
  const int32_t* bt = P.block_table + static_cast<size_t>(b) * P.max_blocks;
  for (int base = 0; base < nb; base += kWave) {
    const int j = base + lane;
    bool inc = false;
    int hm = 0;
    if (j < nb) {
      if (nc == 0 || j < cr.lo || j >= cr.lo + nc) {
        inc = true;
      } else {
        const int c = j - cr.lo;
#pragma unroll
        for (int x = 0; x < G; ++x)
          hm |= static_cast<int>((sel_bits[static_cast<size_t>(x) * nwords + (c >> 6)] >> (c & 63)) & 1ull) << x;
        const bool overlap = (j * P.B < P.ns) || ((j + 1) * P.B > win0);
        inc = hm != 0 || overlap;
      }
    }
    const uint64_t im = __ballot(inc);
    const int pos = cnt + __popcll(im & lanes_below(lane));
    if (inc && pos < P.umax) {
      ul[pos] = j | (hm << 20);
      up[pos] = bt[j];
    }
    cnt += __popcll(im);
  }
  if (lane == 0) P.ucount[pair] = min(cnt, P.umax);
}

template <int G>
__global__ __launch_bounds__(kWave * G) void k_select_generic(DecodeParams P) {
  // Dynamic LDS: per-head selection bitmaps [G][nwords] (uint64), then, when
  // they fit, the per-head order keys [G][nc_max] (uint32).
  extern __shared__ uint64_t dyn_lds[];
  __shared__ uint32_t hist[G][256];
  const int pair = blockIdx.x;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const CandRange cr = candidate_range(T, P.B, P.ns, P.W);
  const int nc = min(cr.count, P.nc_max);
  const int nwords = (P.nc_max + 63) / 64;
  const int hh = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int h = g * G + hh;
  const int k = P.top_k;
  const float* sc = P.scores + (static_cast<size_t>(b) * P.Hq + h) * P.nc_max;
  uint64_t* bits = dyn_lds + static_cast<size_t>(hh) * nwords;
  const bool staged = P.keys_staged != 0;
  uint32_t* keys = reinterpret_cast<uint32_t*>(dyn_lds + static_cast<size_t>(G) * nwords) +
                   static_cast<size_t>(hh) * P.nc_max;
  if (staged) {
#pragma unroll 4
    for (int i = lane; i < nc; i += kWave) keys[i] = f32_order_key(sc[i]);
  }
  __syncthreads();
  auto key_at = [&](int i) -> uint32_t { return staged ? keys[i] : f32_order_key(sc[i]); };

  const bool take_all = k >= nc;
  const bool take_none = (k <= 0) || (nc == 0);
  // Threshold key (order key of the k-th best score) and how many of the
  // candidates equal to it are taken (lowest indices first).
  uint32_t prefix = 0, mask = 0;
  int rem = k;
  int shift = 0;
  if (!take_all && !take_none) {
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    for (int i = lane; i < nc; i += kWave) {
      const uint32_t key = key_at(i);
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    const uint32_t diff = kmin ^ kmax;
    shift = diff ? 32 - __clz(static_cast<int>(diff)) : 0;   // low bits that still vary
    mask = (shift == 32) ? 0u : ~((1u << shift) - 1u);
    prefix = kmax & mask;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const bool active = shift > 0;
    uint32_t dmask = 0;
    if (active) {
      const int nb = min(8, shift);
      shift -= nb;
      dmask = (1u << nb) - 1u;
    }
    __syncthreads();
    if (active)
      for (int j = lane; j < 256; j += kWave) hist[hh][j] = 0u;
    __syncthreads();
    if (active) {
      for (int i = lane; i < nc; i += kWave) {
        const uint32_t key = key_at(i);
        if ((key & mask) == prefix) atomicAdd(&hist[hh][(key >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    if (active) {
      const uint32_t c0 = hist[hh][4 * lane], c1 = hist[hh][4 * lane + 1];
      const uint32_t c2 = hist[hh][4 * lane + 2], c3 = hist[hh][4 * lane + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      uint32_t suffix = mine;   // keys whose digit >= 4*lane
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = static_cast<uint32_t>(__shfl_down(static_cast<int>(suffix), off));
        if (lane + off < kWave) suffix += t;
      }
      const uint32_t above = suffix - mine;   // keys whose digit > 4*lane + 3
      const bool here = above < static_cast<uint32_t>(rem) && static_cast<uint32_t>(rem) <= suffix;
      int digit = 0, rem_here = rem;
      if (here) {
        uint32_t acc = above;
        const uint32_t cs[4] = {c0, c1, c2, c3};
        for (int j = 3; j >= 0; --j) {
          if (acc + cs[j] >= static_cast<uint32_t>(rem)) {
            digit = 4 * lane + j;
            rem_here = rem - static_cast<int>(acc);
            break;
          }
          acc += cs[j];
        }
      }
      const uint64_t hm = __ballot(here);
      const int src = __ffsll(static_cast<unsigned long long>(hm)) - 1;
      digit = __shfl(digit, src);
      rem = __shfl(rem_here, src);
      prefix |= static_cast<uint32_t>(digit) << shift;
      mask |= dmask << shift;
    }
  }
  const uint32_t thr = prefix;

  // Ascending output and per-head selection bitmap.
  int nsel = 0, neq = 0;
  int32_t* out = P.sel_idx ? P.sel_idx + (static_cast<size_t>(b) * P.Hq + h) * k : nullptr;
  for (int base = 0; base < nwords * 64; base += 64) {
    const int i = base + lane;
    const bool valid = i < nc;
    const uint32_t key = valid ? key_at(i) : 0u;
    bool sel;
    if (take_none) {
      sel = false;
    } else if (take_all) {
      sel = valid;
    } else {
      const bool eq = valid && key == thr;
      const uint64_t eqm = __ballot(eq);
      const int eqrank = neq + __popcll(eqm & lanes_below(lane));
      sel = valid && (key > thr || (eq && eqrank < rem));
      neq += __popcll(eqm);
    }
    const uint64_t sm = __ballot(sel);
    const int pos = nsel + __popcll(sm & lanes_below(lane));
    if (sel && out && pos < k) out[pos] = cr.lo + i;
    nsel += __popcll(sm);
    if (lane == 0) bits[base / 64] = sm;
  }
  if (out)
    for (int j = nsel + lane; j < k; j += kWave) out[j] = -1;
  __syncthreads();

  build_union<G>(P, pair, b, T, cr, nc, nwords, dyn_lds, lane, hh);
}

// Inclusive prefix sum over the 64 lanes of a wavefront (DPP row shifts,
// then row broadcasts 15 and 31 across rows).
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
  auto add = [](uint32_t x, int y) { return x + static_cast<uint32_t>(y); };
  v = add(v, __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xf, 0xf, true));   // row_shr:1
  v = add(v, __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xf, 0xf, true));   // row_shr:2
  v = add(v, __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xf, 0xf, true));   // row_shr:4
  v = add(v, __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xf, 0xf, true));   // row_shr:8
  v = add(v, __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = add(v, __builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xc, 0xf, false));  // row_bcast:31
  return v;
}

// Top-k with the order keys of one head held in registers: lane l holds
// candidates l, l + 64, ..., l + 64 (KPL - 1).  A radix select over the
// 32-bit order keys (8-bit digits, skipping the bits every key shares) finds
// the k-th largest key with a histogram private to the wavefront, so no
// workgroup barrier is needed until the union step.
template <int G, int KPL>
__global__ __launch_bounds__(kWave * G) void k_select(DecodeParams P) {
  extern __shared__ uint64_t dyn_lds[];   // [G][nwords] selection bitmaps
  __shared__ __attribute__((aligned(16))) uint32_t hist[G][256];
  const int pair = blockIdx.x;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const CandRange cr = candidate_range(T, P.B, P.ns, P.W);
  const int nc = min(cr.count, P.nc_max);
  const int nwords = (P.nc_max + 63) / 64;
  const int hh = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int h = g * G + hh;
  const int k = P.top_k;
  const float* sc = P.scores + (static_cast<size_t>(b) * P.Hq + h) * P.nc_max;
  uint64_t* bits = dyn_lds + static_cast<size_t>(hh) * nwords;

  uint32_t key[KPL];
  uint32_t valid = 0;   // bit j: slot j holds a candidate
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int c = lane + kWave * j;
    const float v = sc[min(c, max(nc - 1, 0))];
    key[j] = f32_order_key(v);
    valid |= (c < nc ? 1u : 0u) << j;
  }
  const bool take_all = k >= nc;
  const bool take_none = (k <= 0) || (nc == 0);
  uint32_t thr = 0;
  int rem = k;
  if (!take_all && !take_none) {
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      if ((valid >> j) & 1) {
        kmin = min(kmin, key[j]);
        kmax = max(kmax, key[j]);
      }
    }
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    const uint32_t diff = kmin ^ kmax;
    int shift = diff ? 32 - __clz(static_cast<int>(diff)) : 0;   // low bits that still vary
    uint32_t mask = (shift == 32) ? 0u : ~((1u << shift) - 1u);
    uint32_t prefix = kmax & mask;
    uint4* hrow = reinterpret_cast<uint4*>(&hist[hh][4 * lane]);
    while (shift > 0) {
      const int nb = min(8, shift);
      shift -= nb;
      const uint32_t dmask = (1u << nb) - 1u;
      *hrow = make_uint4(0, 0, 0, 0);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if (((valid >> j) & 1) && (key[j] & mask) == prefix) atomicAdd(&hist[hh][(key[j] >> shift) & dmask], 1u);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      const uint4 c4 = *hrow;
      const uint32_t mine = c4.x + c4.y + c4.z + c4.w;
      const uint32_t incl = wave_scan_incl(mine);
      const uint32_t total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1));
      const uint32_t suffix = total - incl + mine;   // keys whose digit >= 4 * lane
      const uint32_t above = suffix - mine;          // keys whose digit > 4 * lane + 3
      const bool here = above < static_cast<uint32_t>(rem) && static_cast<uint32_t>(rem) <= suffix;
      int digit = 0, rem_here = rem;
      if (here) {   // the crossing bin is one of this lane's four, scanned from the top
        uint32_t acc = above;
        bool found = false;
        const uint32_t cs[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          if (!found && acc + cs[j] >= static_cast<uint32_t>(rem)) {
            digit = 4 * lane + j;
            rem_here = rem - static_cast<int>(acc);
            found = true;
          }
          acc += cs[j];
        }
      }
      const uint64_t hm = __ballot(here);
      const int src = __ffsll(static_cast<unsigned long long>(hm)) - 1;
      digit = __builtin_amdgcn_readlane(digit, src);
      rem = __builtin_amdgcn_readlane(rem_here, src);
      prefix |= static_cast<uint32_t>(digit) << shift;
      mask |= dmask << shift;
    }
    thr = prefix;
  }

  // Ascending output and per-head selection bitmap.
  int nsel = 0, neq = 0;
  int32_t* out = P.sel_idx ? P.sel_idx + (static_cast<size_t>(b) * P.Hq + h) * k : nullptr;
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const bool vj = (valid >> j) & 1;
    bool sel;
    if (take_none) {
      sel = false;
    } else if (take_all) {
      sel = vj;
    } else {
      const bool eq = vj && key[j] == thr;
      const uint64_t eqm = __ballot(eq);
      const int eqrank = neq + __popcll(eqm & lanes_below(lane));
      sel = vj && (key[j] > thr || (eq && eqrank < rem));
      neq += __popcll(eqm);
    }
    const uint64_t sm = __ballot(sel);
    const int pos = nsel + __popcll(sm & lanes_below(lane));
    if (sel && out && pos < k) out[pos] = cr.lo + lane + kWave * j;
    nsel += __popcll(sm);
    if (lane == 0 && j < nwords) bits[j] = sm;
  }
  if (out)
    for (int j = nsel + lane; j < k; j += kWave) out[j] = -1;
  __syncthreads();
  build_union<G>(P, pair, b, T, cr, nc, nwords, dyn_lds, lane, hh);
}

// ---------------------------------------------------------------------------
// 3. Split-K exact attention over the union + exact tokens' linear sums
// ---------------------------------------------------------------------------
// A workgroup walks its split in units of 64 token rows (one block when B is
// 64, a slice of one when B is larger, several blocks when B is smaller).
// Each unit takes three passes:
//   dot      lanes form groups of D/8 lanes, each lane holding 8 channels of
//            one row (a 16-byte load for bf16); the group's dot product with
//            every active query head goes to LDS;
//   softmax  one wavefront per head takes the 64 scores at once (one row per
//            lane): running maximum, exponentials and the first-order weights
//            (1 + s) are computed once per row and published in LDS;
//   fma      every lane accumulates its 8 channels of p v and (1 + s) v.
// All lanes share one running maximum per head, so the final combine is a
// plain sum.  The next unit's rows are loaded into a second register buffer
// before the current unit's barriers, so they are in flight while it is
// processed.  For B >= 64 a unit lies in one page: its page, first token and
// selection mask are wavefront-uniform and each lane's row offset is fixed.
template <typename KV, int D, int G, bool BIG>
__global__ __launch_bounds__(kThreads, (G <= 4 ? 3 : 1)) void k_attend(DecodeParams P) {
  constexpr int LPT = D / 8;             // lanes per token row
  constexpr int NGRP = kThreads / LPT;   // token groups per workgroup
  constexpr int U = kUnit / NGRP;        // rows per group per unit
  constexpr int NW = kThreads / kWave;
  constexpr int kAll = (1 << G) - 1;
  static_assert(kUnit == kWave, "softmax pass maps one row to one lane");
  __shared__ float s_lds[G][kUnit];
  __shared__ float2 pw_lds[G][kUnit];
  __shared__ float scale_lds[G];
  __shared__ float red[NW][G][2 * D];
  __shared__ float mll[G][4];

  // Split s of a (sequence, kv head) takes union entries s, s + S, s + 2S, ...
  // (S = max_split), so window and sink blocks, which every head of the
  // group needs, spread over the splits instead of piling into the last one.
  // The count and the candidate entries are fetched in one round trip.
  const int pair = blockIdx.x / P.max_split;
  const int split = blockIdx.x % P.max_split;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int ent_at = split + lane * P.max_split;   // this lane's candidate entry
  const bool ent_in = lane < P.bps && ent_at < P.umax;
  const size_t ent_off = static_cast<size_t>(pair) * P.umax + (ent_in ? ent_at : 0);
  const int count = min(P.ucount[pair], P.umax);
  int my_ent = P.ulist[ent_off];
  int my_page = P.upage[ent_off];
  if (split >= count) return;
  const int ne = min(P.bps, ceil_div(count - split, P.max_split));
  if (!(ent_in && lane < ne)) {
    my_ent = 0;
    my_page = -1;
  }
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const int B = P.B;
  const int ns = P.ns;
  const int win0 = T - P.W;
  const int lig = tid % LPT;
  const int grp = tid / LPT;
  const int upb = BIG ? B / kUnit : 1;   // units per block
  const int epu = BIG ? 1 : kUnit / B;   // blocks per unit
  const int nu = BIG ? ne * upb : ceil_div(ne, epu);

  QReg<KV> qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h].load(reinterpret_cast<const char*>(P.q) +
               ((static_cast<size_t>(b) * P.Hq + g * G + h) * D + lig * 8) * KV::kBytes);

  float acc[G][8], lacc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = lacc[h][i] = 0.f;
  // Softmax state of the heads this wavefront owns (h % NW == wave): the
  // running maximum (uniform) and per-lane partial sums of p and 1 + s.
  constexpr int OWN = (G + NW - 1) / NW;   // heads owned per wavefront
  float m_run[OWN], l_lane[OWN], ld_lane[OWN];
#pragma unroll
  for (int o = 0; o < OWN; ++o) {
    m_run[o] = kNegInf;
    l_lane[o] = 0.f;
    ld_lane[o] = 0.f;
  }

  const char* kp = reinterpret_cast<const char*>(P.k_pages);
  const char* vp = reinterpret_cast<const char*>(P.v_pages);
  const size_t head_tile = static_cast<size_t>(B) * D * KV::kBytes;   // bytes of one (page, head) tile
  int lane_off[U];   // byte offset of this lane's row i inside a 64-row slice
#pragma unroll
  for (int i = 0; i < U; ++i) lane_off[i] = ((grp + NGRP * i) * D + lig * 8) * KV::kBytes;

  struct Unit {
    Row8<KV> k[U], v[U];
    int tok[U];    // token position of row i, or -1 when absent
    int fm;        // B >= 64: heads that selected the unit's block (uniform)
    int fmr[U];    // B < 64: heads that selected row i's block
    int active;    // heads any row of the unit needs (uniform)
  };
  // Issues the loads of unit u (any u: past the end it reads valid rows of
  // the split's first page and marks every row absent).
  auto fetch = [&](int u, Unit& x) __attribute__((always_inline)) {
    const bool live = u < nu;
    if constexpr (BIG) {
      const int e = live ? u / upb : 0;
      const int sub = live ? u - e * upb : 0;
      const int ent = __builtin_amdgcn_readlane(my_ent, e);
      const int page = max(__builtin_amdgcn_readlane(my_page, e), 0);
      const int t0 = (ent & 0xFFFFF) * B + sub * kUnit;
      const size_t base = (static_cast<size_t>(page) * P.Hkv + g) * head_tile +
                          static_cast<size_t>(sub) * kUnit * D * KV::kBytes;
      const bool ok = live && __builtin_amdgcn_readlane(my_page, e) >= 0;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int t = t0 + grp + NGRP * i;
        x.tok[i] = (ok && t < T) ? t : -1;
        x.k[i].load(kp + base + lane_off[i]);
        x.v[i].load(vp + base + lane_off[i]);
      }
      x.fm = (ent >> 20) & kAll;
      const bool sw = t0 < ns || t0 + kUnit > win0;
      x.active = ok ? (x.fm | (sw ? kAll : 0)) : 0;
    } else {
      int active = 0;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const int r = grp + NGRP * i;
        const int e = live ? u * epu + r / B : 0;
        const int row = r % B;
        const int ent = __shfl(my_ent, e & (kWave - 1));
        const int page = __shfl(my_page, e & (kWave - 1));
        const int t = (ent & 0xFFFFF) * B + row;
        const bool ok = live && e < ne && page >= 0 && t < T;
        x.tok[i] = ok ? t : -1;
        x.fmr[i] = (ent >> 20) & kAll;
        const size_t off = (((static_cast<size_t>(max(page, 0)) * P.Hkv + g) * B + row) * D + lig * 8) * KV::kBytes;
        x.k[i].load(kp + off);
        x.v[i].load(vp + off);
      }
      // Per-row selection masks differ across the unit; the unit's active set
      // is the union over its blocks.
      if (live) {
        for (int xx = 0; xx < epu; ++xx) {
          const int e = u * epu + xx;
          if (e < ne) {
            const int ent = __builtin_amdgcn_readlane(my_ent, e);
            const int t0 = (ent & 0xFFFFF) * B;
            const bool sw = t0 < ns || t0 + B > win0;
            active |= ((ent >> 20) & kAll) | (sw ? kAll : 0);
          }
        }
      }
      x.fm = 0;
      x.active = active;
    }
  };

  auto process = [&](Unit& x) __attribute__((always_inline)) {
    const int active = x.active;
    bool valid[U], vsw[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      valid[i] = x.tok[i] >= 0;
      vsw[i] = valid[i] && (x.tok[i] < ns || x.tok[i] >= win0);
    }
    // ---- dot pass: raw dot products (scaled in the softmax pass)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((active >> h) & 1)) continue;
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const float d = reduce_sum_lanes<LPT>(qr[h].dot(x.k[i]));
        bool inc;
        if constexpr (BIG) {
          inc = ((x.fm >> h) & 1) ? valid[i] : vsw[i];
        } else {
          inc = vsw[i] || (valid[i] && ((x.fmr[i] >> h) & 1));
        }
        if (lig == 0) s_lds[h][grp + NGRP * i] = inc ? d : kNegInf;
      }
    }
    __syncthreads();
    // ---- softmax pass: wavefront w owns heads w, w + NW, ...
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int h = wave + o * NW;
      if (h >= G || !((active >> h) & 1)) continue;
      const float sv = P.sigma * s_lds[h][lane];
      const bool inc = sv != kNegInf;
      const float mnew = fmaxf(m_run[o], wave_max(sv));
      const float c = (m_run[o] == kNegInf) ? 0.f : (mnew == m_run[o] ? 1.f : fast_exp(m_run[o] - mnew));
      const float pv = inc ? fast_exp(sv - mnew) : 0.f;
      const float wv = inc ? 1.f + sv : 0.f;
      pw_lds[h][lane] = make_float2(pv, wv);
      l_lane[o] = fmaf(l_lane[o], c, pv);
      ld_lane[o] += wv;
      m_run[o] = mnew;
      if (lane == 0) scale_lds[h] = c;
    }
    __syncthreads();
    // ---- fma pass
#pragma unroll
    for (int i = 0; i < U; ++i)
      if (!valid[i]) x.v[i].zero();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (!((active >> h) & 1)) continue;
      const float c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(scale_lds[h])));
      if (c != 1.f) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] *= c;
      }
#pragma unroll
      for (int i = 0; i < U; ++i) {
        const float2 pw = pw_lds[h][grp + NGRP * i];
        float vf[8];
        x.v[i].to_f32(vf);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          acc[h][j] = fmaf(pw.x, vf[j], acc[h][j]);
          lacc[h][j] = fmaf(pw.y, vf[j], lacc[h][j]);
        }
      }
    }
  };

  Unit ua, ub;
  fetch(0, ua);
  for (int u = 0; u < nu; u += 2) {
    fetch(u + 1, ub);
    process(ua);
    if (u + 1 >= nu) break;
    fetch(u + 2, ua);
    process(ub);
  }

  // ---- combine: plain sums over the groups of a wavefront, then over waves.
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (LPT <= 8) {
        acc[h][j] = pair_sum<8>(acc[h][j]);
        lacc[h][j] = pair_sum<8>(lacc[h][j]);
      }
      acc[h][j] = pair_sum<32>(pair_sum<16>(acc[h][j]));
      lacc[h][j] = pair_sum<32>(pair_sum<16>(lacc[h][j]));
    }
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        red[wave][h][lane * 8 + j] = acc[h][j];
        red[wave][h][D + lane * 8 + j] = lacc[h][j];
      }
  }
#pragma unroll
  for (int o = 0; o < OWN; ++o) {
    const int h = wave + o * NW;
    if (h < G) {
      const float lsum = wave_sum(l_lane[o]);
      const float ldsum = wave_sum(ld_lane[o]);
      if (lane == 0) {
        mll[h][0] = m_run[o];
        mll[h][1] = lsum;
        mll[h][2] = ldsum;
      }
    }
  }
  __syncthreads();
  float* outp = P.part + (static_cast<size_t>(pair) * P.max_split + split) * G * P.pstride;
  for (int idx = tid; idx < G * 2 * D; idx += kThreads) {
    const int h = idx / (2 * D);
    const int c = idx % (2 * D);
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += red[w][h][c];
    outp[static_cast<size_t>(h) * P.pstride + 4 + c] = v;
  }
  if (tid < G) {
    float* o = outp + static_cast<size_t>(tid) * P.pstride;
    o[0] = mll[tid][0];
    o[1] = mll[tid][1];
    o[2] = mll[tid][2];
    o[3] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// 4. Merge of the splits and the residual linear part
// ---------------------------------------------------------------------------
// One workgroup per (sequence, query head); NP = 256 / D lanes share a
// channel and walk the splits with a running maximum, then combine.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void k_merge(DecodeParams P) {
  constexpr int NP = kThreads / D;
  __shared__ float part_m[NP][D], part_num[NP][D], part_den[NP][D], part_lnum[NP][D], part_lden[NP][D];
  const int bh = blockIdx.x;
  const int b = bh / P.Hq;
  const int h = bh % P.Hq;
  const int g = h / G;
  const int hh = h % G;
  const int pair = b * P.Hkv + g;
  const int tid = threadIdx.x;
  const int c = tid % D;
  const int pp = tid / D;
  const int count = min(P.ucount[pair], P.umax);
  const int nsplit = min(count, P.max_split);   // split s holds entries s, s + max_split, ...
  const size_t sstride = static_cast<size_t>(G) * P.pstride;
  const float* pb = P.part + (static_cast<size_t>(pair) * P.max_split * G + hh) * P.pstride;

  float M = 0.f;   // the linear part is in unshifted units (log-scale 0)
  float num = 0.f, den = 0.f, lnum = 0.f, lden = 0.f;
  constexpr int NPC = 8;   // splits per lane whose loads are issued together
  for (int s0 = pp; s0 < nsplit; s0 += NP * NPC) {
    float ms[NPC], ls[NPC], lds[NPC], a[NPC], la[NPC];
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int sidx = min(s0 + i * NP, nsplit - 1);
      const float* ps = pb + sidx * sstride;
      ms[i] = ps[0];
      ls[i] = ps[1];
      lds[i] = ps[2];
      a[i] = ps[4 + c];
      la[i] = ps[4 + D + c];
    }
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      if (s0 + i * NP >= nsplit) break;
      lnum += la[i];
      lden += lds[i];
      if (ms[i] != kNegInf) {
        if (ms[i] > M) {
          const float r = __expf(M - ms[i]);
          num *= r;
          den *= r;
          M = ms[i];
        }
        const float f = __expf(ms[i] - M);
        num = fmaf(f, a[i], num);
        den = fmaf(f, ls[i], den);
      }
    }
  }
  part_m[pp][c] = M;
  part_num[pp][c] = num;
  part_den[pp][c] = den;
  part_lnum[pp][c] = lnum;
  part_lden[pp][c] = lden;
  __syncthreads();
  if (pp != 0) return;
#pragma unroll
  for (int x = 1; x < NP; ++x) M = fmaxf(M, part_m[x][c]);
  num = den = lnum = lden = 0.f;
#pragma unroll
  for (int x = 0; x < NP; ++x) {
    const float f = __expf(part_m[x][c] - M);
    num = fmaf(f, part_num[x][c], num);
    den = fmaf(f, part_den[x][c], den);
    lnum += part_lnum[x][c];
    lden += part_lden[x][c];
  }
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const CandRange cr = candidate_range(T, P.B, P.ns, P.W);
  if (P.linear_tail && P.top_k < min(cr.count, P.nc_max)) {
    float ro = 0.f, rz = 0.f;
#pragma unroll 8
    for (int rc = 0; rc < P.ro_wgs; ++rc) {
      ro += P.ro[((static_cast<size_t>(pair) * P.ro_wgs + rc) * G + hh) * D + c];
      rz += P.roz[(static_cast<size_t>(pair) * P.ro_wgs + rc) * G + hh];
    }
    const float num_u = P.sv[static_cast<size_t>(pair) * D + c] + P.sigma * ro - lnum;
    const float den_u = static_cast<float>(T) + P.sigma * rz - lden;
    const float em = __expf(-M);
    num = fmaf(em, num_u, num);
    den = fmaf(em, den_u, den);
  }
  P.out[(static_cast<size_t>(b) * P.Hq + h) * D + c] = num / den;
}

template <typename KV, int D, int G>
hipError_t launch_typed(const Problem& p, const DecodeLayout& L, const DecodeParams& P,
                        hipStream_t stream, RecordFn rec, void* ctx) {
  const int pairs = p.batch * p.Hkv;
  if (rec) rec(ctx, 0, "score_readout");
  {
    dim3 grid(L.score_wgs + L.ro_wgs, pairs);
    hipLaunchKernelGGL((k_score_readout<KV, D, G>), grid, dim3(kThreads), 0, stream, P);
    hipError_t e = launch_status("k_score_readout");
    if (e != hipSuccess) return e;
  }
  if (rec) rec(ctx, 1, "select");
  {
    const int nwords = (p.nc_max + 63) / 64;
    const size_t bits = static_cast<size_t>(G) * nwords * sizeof(uint64_t);
    const int kpl = ceil_div(std::max(p.nc_max, 1), kWave);
    auto go = [&](auto kernel, size_t lds) -> hipError_t {
      if (lds > 32 * 1024) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL(kernel, dim3(pairs), dim3(kWave * G), lds, stream, P);
      return launch_status("k_select");
    };
    hipError_t e;
    if (kpl <= 2) e = go(k_select<G, 2>, bits);
    else if (kpl <= 4) e = go(k_select<G, 4>, bits);
    else if (kpl <= 8) e = go(k_select<G, 8>, bits);
    else if (kpl <= 16) e = go(k_select<G, 16>, bits);
    else if (kpl <= 32) e = go(k_select<G, 32>, bits);
    else e = go(k_select_generic<G>, bits + (L.keys_staged ? static_cast<size_t>(G) * p.nc_max * sizeof(uint32_t) : 0));
    if (e != hipSuccess) return e;
  }
  if (rec) rec(ctx, 2, "attend");
  {
    if (p.B >= kUnit)
      hipLaunchKernelGGL((k_attend<KV, D, G, true>), dim3(pairs * L.max_split), dim3(kThreads), 0, stream, P);
    else
      hipLaunchKernelGGL((k_attend<KV, D, G, false>), dim3(pairs * L.max_split), dim3(kThreads), 0, stream, P);
    hipError_t e = launch_status("k_attend");
    if (e != hipSuccess) return e;
  }
  if (rec) rec(ctx, 3, "merge");
  {
    hipLaunchKernelGGL((k_merge<D, G>), dim3(p.batch * p.Hq), dim3(kThreads), 0, stream, P);
    hipError_t e = launch_status("k_merge");
    if (e != hipSuccess) return e;
  }
  if (rec) rec(ctx, 4, nullptr);
  return hipSuccess;
}

template <typename KV, int D>
hipError_t dispatch_g(const Problem& p, const DecodeLayout& L, const DecodeParams& P,
                      hipStream_t s, RecordFn rec, void* ctx) {
  switch (p.G) {
    case 1: return launch_typed<KV, D, 1>(p, L, P, s, rec, ctx);
    case 2: return launch_typed<KV, D, 2>(p, L, P, s, rec, ctx);
    case 4: return launch_typed<KV, D, 4>(p, L, P, s, rec, ctx);
    case 8: return launch_typed<KV, D, 8>(p, L, P, s, rec, ctx);
  }
  return hipErrorInvalidValue;
}

}  // namespace

static size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

DecodeLayout decode_layout(const Problem& p) {
  DecodeLayout L{};
  const int pairs = p.batch * p.Hkv;
  L.score_chunk = kScoreChunk;
  L.score_wgs = p.nc_max > 0 ? ceil_div(p.nc_max, L.score_chunk) : 0;
  L.ro_rows = kRoRows;
  L.ro_wgs = p.linear_tail ? p.D / L.ro_rows : 0;
  {
    const size_t bits = static_cast<size_t>(p.G) * ((p.nc_max + 63) / 64) * sizeof(uint64_t);
    const size_t keys = static_cast<size_t>(p.G) * p.nc_max * sizeof(uint32_t);
    L.keys_staged = (bits + keys) <= 96 * 1024 ? 1 : 0;
  }
  const int sink_blocks = p.ns / p.B;
  const long sel_blocks = std::min<long>(static_cast<long>(p.G) * p.top_k, p.nc_max);
  const long bound = static_cast<long>(sink_blocks) + sel_blocks + 2 + p.W / p.B + 1;
  L.umax = static_cast<int>(std::max<long>(1, std::min<long>(bound, p.nblk_max)));
  L.bps = std::max(1, kUnitsPerWg * kUnit / p.B);
  L.max_split = ceil_div(L.umax, L.bps);
  L.pstride = 2 * p.D + 4;
  size_t off = 0;
  L.off_scores = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(p.batch) * p.Hq * std::max(1, p.nc_max));
  L.off_ro = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(pairs) * std::max(1, L.ro_wgs) * p.G * p.D);
  L.off_roz = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(pairs) * std::max(1, L.ro_wgs) * p.G);
  L.off_union = off;
  off = align_up(off + sizeof(int32_t) * static_cast<size_t>(pairs) * L.umax);
  L.off_upage = off;
  off = align_up(off + sizeof(int32_t) * static_cast<size_t>(pairs) * L.umax);
  L.off_ucount = off;
  off = align_up(off + sizeof(int32_t) * static_cast<size_t>(pairs));
  L.off_part = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(pairs) * L.max_split * p.G * L.pstride);
  L.total = off;
  return L;
}

hipError_t launch_decode(const Problem& p, const DecodeLayout& L, const DecodeArgs& a,
                         hipStream_t stream, RecordFn rec, void* ctx) {
  DecodeParams P{};
  P.k_pages = a.k_pages;
  P.v_pages = a.v_pages;
  P.blk_mean = a.blk_mean;
  P.blk_var = a.blk_var;
  P.block_table = a.block_table;
  P.S = a.S;
  P.z = a.z;
  P.sv = a.sv;
  P.q = a.q;
  P.seq_lens = a.seq_lens;
  P.out = a.out;
  P.sel_idx = a.sel_idx;
  P.scores = reinterpret_cast<float*>(a.ws + L.off_scores);
  P.ro = reinterpret_cast<float*>(a.ws + L.off_ro);
  P.roz = reinterpret_cast<float*>(a.ws + L.off_roz);
  P.ulist = reinterpret_cast<int32_t*>(a.ws + L.off_union);
  P.upage = reinterpret_cast<int32_t*>(a.ws + L.off_upage);
  P.ucount = reinterpret_cast<int32_t*>(a.ws + L.off_ucount);
  P.part = reinterpret_cast<float*>(a.ws + L.off_part);
  P.Hq = p.Hq;
  P.Hkv = p.Hkv;
  P.B = p.B;
  P.top_k = p.top_k;
  P.ns = p.ns;
  P.W = p.W;
  P.linear_tail = p.linear_tail;
  P.max_blocks = p.max_blocks;
  P.max_seq_len = p.max_seq_len;
  P.nc_max = p.nc_max;
  P.nblk_max = p.nblk_max;
  P.score_wgs = L.score_wgs;
  P.ro_wgs = L.ro_wgs;
  P.keys_staged = L.keys_staged;
  P.umax = L.umax;
  P.bps = L.bps;
  P.max_split = L.max_split;
  P.pstride = L.pstride;
  P.sigma = p.sigma;
  if (p.bf16) {
    return p.D == 64 ? dispatch_g<KvBf16, 64>(p, L, P, stream, rec, ctx)
                     : dispatch_g<KvBf16, 128>(p, L, P, stream, rec, ctx);
  }
  return p.D == 64 ? dispatch_g<KvF32, 64>(p, L, P, stream, rec, ctx)
                   : dispatch_g<KvF32, 128>(p, L, P, stream, rec, ctx);
}

}  // namespace hsla
