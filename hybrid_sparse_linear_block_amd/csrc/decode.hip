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

#include "common.h"
#include "internal.h"

namespace hsla {

namespace {

constexpr int kThreads = 256;
constexpr float kNegInf = -INFINITY;

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
  int32_t* ucount;
  float* part;
  int Hq, Hkv, B, top_k, ns, W, linear_tail;
  int max_blocks, max_seq_len, nc_max, nblk_max;
  int score_chunk, score_wgs, ro_wgs, ro_rows;
  int umax, bps, max_split, pstride;
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
__device__ void score_part(const DecodeParams& P, int b, int g, int T, int chunk) {
  constexpr int LPT = D / 8;           // lanes per candidate (8 channels each)
  constexpr int CPP = kThreads / LPT;  // candidates per pass
  static_assert(G <= LPT, "one writer lane per head");
  const CandRange cr = candidate_range(T, P.B, P.ns, P.W);
  const int nc = min(cr.count, P.nc_max);
  const int c_begin = chunk * P.score_chunk;
  const int c_end = min(c_begin + P.score_chunk, nc);
  if (c_begin >= c_end) return;
  const int tid = threadIdx.x;
  const int lig = tid % LPT;
  const int slot = tid / LPT;

  float qf[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    QReg<KV> qr;
    qr.load(reinterpret_cast<const char*>(P.q) +
            ((static_cast<size_t>(b) * P.Hq + g * G + h) * D + lig * 8) * KV::kBytes);
    qr.to_f32(qf[h]);
  }
  const float sig = P.sigma;
  const float half_s2 = 0.5f * sig * sig;
  const int32_t* bt = P.block_table + static_cast<size_t>(b) * P.max_blocks;

  for (int c = c_begin + slot; c < c_end; c += CPP) {
    const int page = bt[cr.lo + c];
    const size_t off = (static_cast<size_t>(page) * P.Hkv + g) * D + lig * 8;
    const float4 m0 = *reinterpret_cast<const float4*>(P.blk_mean + off);
    const float4 m1 = *reinterpret_cast<const float4*>(P.blk_mean + off + 4);
    const float4 v0 = *reinterpret_cast<const float4*>(P.blk_var + off);
    const float4 v1 = *reinterpret_cast<const float4*>(P.blk_var + off + 4);
    const float mu[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    const float va[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float d1 = 0.f, d2 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        d1 = fmaf(qf[h][i], mu[i], d1);
        d2 = fmaf(qf[h][i] * va[i], qf[h][i], d2);
      }
      d1 = reduce_sum_lanes<LPT>(d1);
      d2 = reduce_sum_lanes<LPT>(d2);
      if (lig == h) {
        const float sc = sig * d1 + log1pf(half_s2 * d2);
        P.scores[(static_cast<size_t>(b) * P.Hq + g * G + h) * P.nc_max + c] = sc;
      }
    }
  }
}

template <typename KV, int D, int G>
__device__ void readout_part(const DecodeParams& P, int b, int g, int rc) {
  constexpr int C4 = D / 4;           // float4 columns per row
  constexpr int RG = kThreads / C4;   // row groups
  constexpr int RGW = kWave / C4;     // row groups per wavefront
  __shared__ float red[kThreads / kWave][C4][G][4];
  const int tid = threadIdx.x;
  const int col4 = tid % C4;
  const int rg = tid / C4;
  const int pair = b * P.Hkv + g;
  const int r0 = rc * P.ro_rows;
  const int r1 = min(r0 + P.ro_rows, D);
  const float* Sp = P.S + static_cast<size_t>(pair) * D * D;
  const size_t qbase = (static_cast<size_t>(b) * P.Hq + g * G) * D;

  float acc[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[h][j] = 0.f;

  for (int r = r0 + rg; r < r1; r += RG) {
    const float4 s = *reinterpret_cast<const float4*>(Sp + static_cast<size_t>(r) * D + col4 * 4);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float qv = q_elem<KV>(P.q, qbase + static_cast<size_t>(h) * D + r);
      acc[h][0] = fmaf(qv, s.x, acc[h][0]);
      acc[h][1] = fmaf(qv, s.y, acc[h][1]);
      acc[h][2] = fmaf(qv, s.z, acc[h][2]);
      acc[h][3] = fmaf(qv, s.w, acc[h][3]);
    }
  }
  // Row groups inside a wavefront sit C4 lanes apart.
#pragma unroll
  for (int off = C4; off < kWave; off <<= 1)
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[h][j] += __shfl_xor(acc[h][j], off);
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  if (lane < C4) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) red[wave][lane][h][j] = acc[h][j];
  }
  (void)RGW;
  __syncthreads();
  float* ro = P.ro + (static_cast<size_t>(pair) * P.ro_wgs + rc) * G * D;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int c = idx % D;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / kWave; ++w) s += red[w][c / 4][h][c % 4];
    ro[idx] = s;
  }
  if (tid < G) {
    const int h = tid;
    const float* zp = P.z + static_cast<size_t>(pair) * D;
    float s = 0.f;
    for (int r = r0; r < r1; ++r) s = fmaf(q_elem<KV>(P.q, qbase + static_cast<size_t>(h) * D + r), zp[r], s);
    P.roz[(static_cast<size_t>(pair) * P.ro_wgs + rc) * G + h] = s;
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

template <int G>
__global__ __launch_bounds__(kWave * G) void k_select(DecodeParams P) {
  extern __shared__ uint64_t sel_bits[];     // [G][nwords]
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
  uint64_t* bits = sel_bits + static_cast<size_t>(hh) * nwords;

  const bool take_all = k >= nc;
  const bool take_none = (k <= 0) || (nc == 0);
  // Threshold key (32-bit order key of the k-th best score) and how many of
  // the candidates equal to it are taken (lowest indices first).
  uint32_t prefix = 0, mask = 0;
  int rem = k;
  int shift = 0;
  if (!take_all && !take_none) {
    uint32_t kmin = 0xffffffffu, kmax = 0u;
    for (int i = lane; i < nc; i += kWave) {
      const uint32_t key = f32_order_key(sc[i]);
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    const uint32_t diff = kmin ^ kmax;
    shift = diff ? 32 - __clz(diff) : 0;          // low bits that still vary
    mask = (shift == 32) ? 0u : ~((1u << shift) - 1u);
    prefix = kmax & mask;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const bool active = shift > 0;
    int nb = 0;
    uint32_t dmask = 0;
    if (active) {
      nb = min(8, shift);
      shift -= nb;
      dmask = (1u << nb) - 1u;
    }
    __syncthreads();
    if (active)
      for (int j = lane; j < 256; j += kWave) hist[hh][j] = 0u;
    __syncthreads();
    if (active) {
      for (int i = lane; i < nc; i += kWave) {
        const uint32_t key = f32_order_key(sc[i]);
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
    bool sel = false;
    if (valid && !take_none) {
      if (take_all) {
        sel = true;
      } else {
        const uint32_t key = f32_order_key(sc[i]);
        const bool eq = key == thr;
        const uint64_t eqm = __ballot(eq);
        const int eqrank = neq + __popcll(eqm & lanes_below(lane));
        sel = key > thr || (eq && eqrank < rem);
      }
    }
    if (!take_all && !take_none) {
      // Keep the tie count in step across lanes (ballot from every lane).
      const uint32_t key = valid ? f32_order_key(sc[i]) : 0u;
      neq += __popcll(__ballot(valid && key == thr));
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

  // Union of the group's exact blocks, ascending: blocks below the
  // candidates (sinks), candidates that some head selected or that hold sink
  // or window tokens, and blocks past the candidates (window).
  if (hh == 0) {
    const int nb = min(ceil_div(T, P.B), P.nblk_max);
    const int win0 = T - P.W;
    int cnt = 0;
    int32_t* ul = P.ulist + static_cast<size_t>(pair) * P.umax;
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
      if (inc && pos < P.umax) ul[pos] = j | (hm << 20);
      cnt += __popcll(im);
    }
    if (lane == 0) P.ucount[pair] = min(cnt, P.umax);
  }
}

// ---------------------------------------------------------------------------
// 3. Split-K exact attention over the union + exact tokens' linear sums
// ---------------------------------------------------------------------------
template <typename KV, int D, int G>
__global__ __launch_bounds__(kThreads) void k_attend(DecodeParams P) {
  constexpr int LPT = D / 8;             // lanes per token row
  constexpr int NGRP = kThreads / LPT;   // token groups per workgroup
  constexpr int U = 4;                   // tokens per group per step
  __shared__ float red[kThreads / kWave][G][2 * D + 4];

  const int pair = blockIdx.x / P.max_split;
  const int split = blockIdx.x % P.max_split;
  const int count = min(P.ucount[pair], P.umax);
  const int e0 = split * P.bps;
  if (e0 >= count) return;
  const int e1 = min(e0 + P.bps, count);
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const int B = P.B;
  const int ns = P.ns;
  const int win0 = T - P.W;
  const float sig = P.sigma;
  const int tid = threadIdx.x;
  const int lig = tid % LPT;
  const int grp = tid / LPT;

  QReg<KV> qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h].load(reinterpret_cast<const char*>(P.q) +
               ((static_cast<size_t>(b) * P.Hq + g * G + h) * D + lig * 8) * KV::kBytes);

  float m[G], l[G], ld[G], acc[G][8], lacc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
    ld[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[h][i] = 0.f;
      lacc[h][i] = 0.f;
    }
  }

  const char* kp = reinterpret_cast<const char*>(P.k_pages);
  const char* vp = reinterpret_cast<const char*>(P.v_pages);
  const int32_t* bt = P.block_table + static_cast<size_t>(b) * P.max_blocks;
  const int32_t* ul = P.ulist + static_cast<size_t>(pair) * P.umax;
  constexpr int kAll = (1 << G) - 1;
  const int nblk = ceil_div(T, B);

  for (int e = e0; e < e1; ++e) {
    const int ent = ul[e];
    const int blk = ent & 0xFFFFF;
    if (blk >= nblk) continue;
    const int fmask = (ent >> 20) & kAll;
    const int t0 = blk * B;
    const bool sw = (t0 < ns) || (t0 + B > win0);
    const int active = fmask | (sw ? kAll : 0);
    const int page = bt[blk];
    const size_t row0 = (static_cast<size_t>(page) * P.Hkv + g) * B;
    for (int tt = 0; tt < B; tt += NGRP * U) {
      Row8<KV> kr[U], vr[U];
      int tok[U];
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = tt + grp + NGRP * u;
        tok[u] = t0 + r;
        valid[u] = (r < B) && (tok[u] < T);
        if (valid[u]) {
          const size_t off = ((row0 + r) * D + lig * 8) * KV::kBytes;
          kr[u].load(kp + off);
          vr[u].load(vp + off);
        } else {
          kr[u].zero();
          vr[u].zero();
        }
      }
      float vf[U][8];
#pragma unroll
      for (int u = 0; u < U; ++u) vr[u].to_f32(vf[u]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        if (!((active >> h) & 1)) continue;
        const bool full = (fmask >> h) & 1;
        float s[U];
        bool inc[U];
        float mx = kNegInf;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          s[u] = sig * reduce_sum_lanes<LPT>(qr[h].dot(kr[u]));
          inc[u] = valid[u] && (full || tok[u] < ns || tok[u] >= win0);
          if (inc[u]) mx = fmaxf(mx, s[u]);
        }
        const float mnew = fmaxf(m[h], mx);
        if (mnew > m[h]) {
          const float c = (m[h] == kNegInf) ? 0.f : fast_exp(m[h] - mnew);
          l[h] *= c;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[h][i] *= c;
          m[h] = mnew;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float p = inc[u] ? fast_exp(s[u] - m[h]) : 0.f;
          const float w = inc[u] ? 1.f + s[u] : 0.f;
          l[h] += p;
          ld[h] += w;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            acc[h][i] = fmaf(p, vf[u][i], acc[h][i]);
            lacc[h][i] = fmaf(w, vf[u][i], lacc[h][i]);
          }
        }
      }
    }
  }

  // Combine the token groups of each wavefront (they sit LPT lanes apart).
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
      const float mo = __shfl_xor(m[h], off);
      const float mn = fmaxf(m[h], mo);
      const float ca = (m[h] == kNegInf) ? 0.f : fast_exp(m[h] - mn);
      const float cb = (mo == kNegInf) ? 0.f : fast_exp(mo - mn);
      l[h] = l[h] * ca + __shfl_xor(l[h], off) * cb;
      ld[h] += __shfl_xor(ld[h], off);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc[h][i] = acc[h][i] * ca + __shfl_xor(acc[h][i], off) * cb;
        lacc[h][i] += __shfl_xor(lacc[h][i], off);
      }
      m[h] = mn;
    }
  }
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  if (lane < LPT) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        red[wave][h][lane * 8 + i] = acc[h][i];
        red[wave][h][D + lane * 8 + i] = lacc[h][i];
      }
      if (lane == 0) {
        red[wave][h][2 * D] = m[h];
        red[wave][h][2 * D + 1] = l[h];
        red[wave][h][2 * D + 2] = ld[h];
      }
    }
  }
  __syncthreads();
  constexpr int NW = kThreads / kWave;
  float* outp = P.part + (static_cast<size_t>(pair) * P.max_split + split) * G * P.pstride;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int c = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red[w][h][2 * D]);
    float a = 0.f, la = 0.f, ls = 0.f, lds = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = red[w][h][2 * D];
      const float f = (mw == kNegInf) ? 0.f : fast_exp(mw - M);
      a = fmaf(f, red[w][h][c], a);
      la += red[w][h][D + c];
      ls = fmaf(f, red[w][h][2 * D + 1], ls);
      lds += red[w][h][2 * D + 2];
    }
    float* o = outp + static_cast<size_t>(h) * P.pstride;
    o[4 + c] = a;
    o[4 + D + c] = la;
    if (c == 0) {
      o[0] = M;
      o[1] = ls;
      o[2] = lds;
      o[3] = 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// 4. Merge of the splits and the residual linear part
// ---------------------------------------------------------------------------
template <int D, int G>
__global__ __launch_bounds__(128) void k_merge(DecodeParams P) {
  const int bh = blockIdx.x;
  const int b = bh / P.Hq;
  const int h = bh % P.Hq;
  const int g = h / G;
  const int hh = h % G;
  const int pair = b * P.Hkv + g;
  const int c = threadIdx.x;
  if (c >= D) return;
  const int count = min(P.ucount[pair], P.umax);
  const int nsplit = ceil_div(count, P.bps);
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const size_t sstride = static_cast<size_t>(G) * P.pstride;
  const float* pb = P.part + (static_cast<size_t>(pair) * P.max_split * G + hh) * P.pstride;

  float M = 0.f;   // the linear part is in unshifted units (log-scale 0)
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pb[s * sstride]);
  float num = 0.f, den = 0.f, lnum = 0.f, lden = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float* ps = pb + s * sstride;
    const float ms = ps[0];
    const float f = (ms == kNegInf) ? 0.f : __expf(ms - M);
    num = fmaf(f, ps[4 + c], num);
    den = fmaf(f, ps[1], den);
    lnum += ps[4 + D + c];
    lden += ps[2];
  }
  const CandRange cr = candidate_range(T, P.B, P.ns, P.W);
  if (P.linear_tail && P.top_k < min(cr.count, P.nc_max)) {
    float ro = 0.f, rz = 0.f;
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
    const size_t lds = static_cast<size_t>(G) * nwords * sizeof(uint64_t);
    if (lds > 32 * 1024) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_select<G>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_select<G>), dim3(pairs), dim3(kWave * G), lds, stream, P);
    hipError_t e = launch_status("k_select");
    if (e != hipSuccess) return e;
  }
  if (rec) rec(ctx, 2, "attend");
  {
    hipLaunchKernelGGL((k_attend<KV, D, G>), dim3(pairs * L.max_split), dim3(kThreads), 0, stream, P);
    hipError_t e = launch_status("k_attend");
    if (e != hipSuccess) return e;
  }
  if (rec) rec(ctx, 3, "merge");
  {
    hipLaunchKernelGGL((k_merge<D, G>), dim3(p.batch * p.Hq), dim3(128), 0, stream, P);
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
  L.score_chunk = 64;
  L.score_wgs = p.nc_max > 0 ? ceil_div(p.nc_max, L.score_chunk) : 0;
  L.ro_rows = 16;
  L.ro_wgs = p.linear_tail ? p.D / L.ro_rows : 0;
  const int sink_blocks = p.ns / p.B;
  const long sel_blocks = std::min<long>(static_cast<long>(p.G) * p.top_k, p.nc_max);
  const long bound = static_cast<long>(sink_blocks) + sel_blocks + 2 + p.W / p.B + 1;
  L.umax = static_cast<int>(std::max<long>(1, std::min<long>(bound, p.nblk_max)));
  L.bps = std::max(1, 256 / p.B);
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
  P.score_chunk = L.score_chunk;
  P.score_wgs = L.score_wgs;
  P.ro_wgs = L.ro_wgs;
  P.ro_rows = L.ro_rows;
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
