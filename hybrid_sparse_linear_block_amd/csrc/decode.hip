// Decode step of hybrid sparse-plus-linear attention on gfx950.
//
// Up to four kernels, all enqueued on the caller's stream:
//   1. k_score_readout  per (sequence, kv head): block scores of the candidate
//      blocks for the G query heads of the group, read from the per-block
//      mean / variance statistics ("SPLA: Block Sparse Plus Linear Attention
//      for Long Context Modeling", section "Principled Block Selection via
//      Taylor Expansion"), and, in the same launch, the readout of the global
//      linear state S^T q, q.z for those heads ("Residual Linear Attention
//      (RLA)").
//   2. selection        top-k candidates per query head (score desc, index
//      asc), ascending index output, as a bitmap per head.  Up to 1024
//      candidates it runs inside the attention prologue (each wavefront one
//      head), and the grouped variant up to 512 candidates on the bf16 path;
//      beyond that in its own kernel (k_select / k_select_grouped).
//   3. k_attend         split-K over the union of the group's exact blocks
//      (sinks, window and selected blocks, SPLA Figure 1(a)), which each
//      workgroup builds from the bitmaps with a per-block mask of the heads
//      that selected it: each page is read once per kv head and serves every
//      query head that needs it; online softmax for the exact part plus the
//      first-order-Taylor sums sum(1+s)v, sum(1+s) of the exact tokens, which
//      are subtracted from the global state (SPLA Abstract, "global minus
//      selected").
//   4. k_merge          log-sum-exp combination of the splits and the
//      residual linear part into the normalised output.
//
// Multi-query form (qrows > 1): the batch counts query rows, row b being
// query b % qrows of sequence b / qrows at its own length; every stage runs
// per row, reading the sequence's block-table row and linear state.
#include <math.h>

#include <algorithm>

#include <type_traits>
#include <utility>

#include "append_parts.h"
#include "internal.h"

namespace hsla {

// Diagnostic build (HSLA_PHASE_TIMESTAMPS, libhsla_phases.so): thread 0 of
// every workgroup stamps the phases of the last launch of each decode kernel
// with s_memrealtime (a 100 MHz clock shared by the whole device).  Attention
// workgroups: 0 entry, 1 prologue loads staged, 2 + w selection done by
// wavefront w, 6 prologue done, 7 + w loop done by wavefront w, 11 partials
// written, 12 exit; scoring and merge workgroups: entry and exit.  The
// release build compiles none of it.
#ifdef HSLA_PHASE_TIMESTAMPS
__device__ uint64_t g_phase_attend[kPhaseAttendWgs][kPhaseSlots];
__device__ uint64_t g_phase_score[kPhaseScoreWgs][2];
__device__ uint64_t g_phase_merge[kPhaseMergeWgs][2];
#define HSLA_STAMP(slot)                                                         \
  do {                                                                           \
    if (threadIdx.x == 0 && blockIdx.x < kPhaseAttendWgs)                        \
      g_phase_attend[blockIdx.x][slot] = __builtin_amdgcn_s_memrealtime();       \
  } while (0)
#define HSLA_STAMP_WAVE(slot)                                                    \
  do {                                                                           \
    const uint64_t t_ = __builtin_amdgcn_s_memrealtime();                        \
    if (threadIdx.x % kWave == 0 && blockIdx.x < kPhaseAttendWgs)                \
      g_phase_attend[blockIdx.x][(slot) + threadIdx.x / kWave] = t_;             \
  } while (0)
// entry now, exit when the kernel returns
struct PhaseSpan {
  uint64_t (*arr)[2];
  size_t idx;
  __device__ PhaseSpan(uint64_t (*a)[2], size_t n, size_t i) : arr(a), idx(i < n ? i : n) {
    if (threadIdx.x == 0 && idx < n) arr[idx][0] = __builtin_amdgcn_s_memrealtime();
    if (idx >= n) arr = nullptr;
  }
  __device__ ~PhaseSpan() {
    if (threadIdx.x == 0 && arr) arr[idx][1] = __builtin_amdgcn_s_memrealtime();
  }
};
#else
#define HSLA_STAMP(slot) do {} while (0)
#define HSLA_STAMP_WAVE(slot) do {} while (0)
#endif

namespace {

constexpr int kThreads = 256;
constexpr float kNegInf = -INFINITY;
constexpr int kScoreChunk = 64;  // candidates per scoring workgroup
constexpr int kRoRows = 32;      // rows of S per readout workgroup
constexpr int kUnit = 64;        // tokens per attention work unit
// Attention workgroups per launch: one per compute unit of MI355X (256
// CUs), so that every CU carries the same number of splits.  With one slice
// in flight per wavefront this keeps 8-16 MB in flight, enough to saturate
// HBM; two workgroups per CU measured 2-3% slower (longer queues, and the
// younger workgroup of a CU starts its loop late).
constexpr int kAttendWgsTarget = 256;
constexpr int kCtrStride = 32;       // ints between two pairs' work counters (one 128-byte line each)
constexpr int kDoneSlot = 16;        // a pair's count of finished attention workgroups (fused merge)
// The last attention workgroup of a pair merges when the pair has at most
// this many splits.  Its tail (partial stores completing, the count, the
// partial loads: three round trips) costs about what the merge kernel does
// at 4 splits per pair, and wins where the merge kernel has many small
// workgroups of its own (one split per pair for large batches).
constexpr int kFusedMergeSplits = 2;
constexpr int kTokensPerSplit = 256;  // token-level variant: list entries per attention workgroup
constexpr int kTokenChunk = 256;      // token-level variant: candidate tokens per scoring workgroup
constexpr int kUnitSlices = 4;       // slices per dynamically claimed unit
constexpr int kMaxDynList = 2048;    // union entries a dynamic attention workgroup holds in LDS
constexpr int kDeadT0 = 1 << 30;     // first token of a slice whose rows are all invalid
constexpr int kFusedKplMax = 16;     // keys per lane of the selection fused into the attention prologue: 8 or 16
constexpr int kFusedKplGrouped = 8;  // keys per lane of the fused grouped selection
constexpr size_t kBtStageBytes = 8 * 1024;      // block-table row staged in LDS up to this size

// The token append taken in by the scoring / readout kernel
// (hsla_append_decode); k_new == nullptr: none.
struct DecodeAppend {
  void* k_pages;
  void* v_pages;
  float* blk_mean;
  float* blk_var;
  float* S;
  float* z;
  float* sv;
  const void* k_new;
  const void* v_new;
  const int32_t* lens_before;
  int32_t* lens_after;
};

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
  uint32_t* keys;   // block-score order keys [batch, Hq, sstride]
  float* ro;
  float* roz;
  uint64_t* bits;   // per-head selection bitmaps [batch, Hq, nwords]
  int32_t* ucount;
  int32_t* ctr;     // per-pair work counters (kCtrStride apart), dynamic attention only
  float* part;
  int Hq, Hkv, B, top_k, ns, W, linear_tail;
  int max_blocks, max_seq_len, nc_max, nblk_max;
  int score_wgs, ro_wgs;
  int umax, bps, max_split, pstride;
  int sstride, nwords, bt_staged;
  int dyn;          // attention workgroups of a pair claim its slices dynamically
  int fused_sel;    // per-head selection inside the attention prologue (no selection kernel)
  int fused_merge;  // the last attention workgroup of a pair merges its splits (no merge kernel)
  int tokens;       // token-level variant: candidates are single tokens, scored by their keys
  int qrows;        // query rows per sequence: 1, or the chunk length of the multi-query form
  int chunk;        // multi-query form: the state holds the whole blocks before the chunk
  int state_all;    // the caller's state holds every token (n = T)
  int bsel;         // candidate granularity: the block size, or 1 for the token-level variant
  int32_t* tlist;   // token-level variant: each pair's exact token list [pairs, umax] x (token | heads << 20, page)
  SelLayout sl;
  DecodeAppend app;
  float sigma;
};

__device__ __forceinline__ int clamp_len(int T, int max_len) { return min(max(T, 1), max_len); }

// Data handed between workgroups of one launch goes through agent-scope
// atomic stores and loads: each access is coherent across the XCDs' L2
// caches on its own, so no cache-wide release (an L2 writeback, which costs
// microseconds per workgroup) is needed.  A writer waits for its stores to
// complete (s_waitcnt) before it publishes a count; a reader issues its
// loads only after it has read that count, behind an agent-scope acquire
// fence.  This leans on gfx950's agent-scope cache policy (stores written
// through to the memory side that all XCDs share and acknowledged only
// there, loads that bypass the per-XCD caches), not on a release fence of
// the HIP memory model, whose L2 writeback per workgroup is the cost
// avoided.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<uint32_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
// Every store this thread issued has completed (vmcnt 0), with the
// compiler kept from moving memory operations across the wait.
__device__ __forceinline__ void stores_complete() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Position of the appended token (the append's own clamp).
__device__ __forceinline__ int append_pos(const DecodeParams& P, int b) {
  return min(max(P.app.lens_before[b], 0), P.max_seq_len - 1);
}

// Length of sequence b in the first decode kernel: with the append taken in,
// seq_lens is written by that same kernel, so the length comes from before.
__device__ __forceinline__ int first_kernel_len(const DecodeParams& P, int b) {
  return P.app.k_new ? append_pos(P, b) + 1 : clamp_len(P.seq_lens[b], P.max_seq_len);
}
// Multi-query form: row b is query b % qrows of sequence b / qrows, whose
// block-table row and linear state it reads.
__device__ __forceinline__ int seq_of(const DecodeParams& P, int b) { return b / P.qrows; }
__device__ __forceinline__ int state_pair(const DecodeParams& P, int pair) {
  return seq_of(P, pair / P.Hkv) * P.Hkv + pair % P.Hkv;
}
// Tokens the linear state holds for row b of length T: the whole blocks of
// T for a decode row; for query i of a chunk (T = T0 + 1 + i) the whole
// blocks of the T0 tokens before the chunk, since the chunk's blocks are
// folded in after it.  Every token from there to T is in the row's window
// (chunk length <= W - B + 1), so the exact part covers it.
__device__ __forceinline__ int state_tokens(const DecodeParams& P, int T, int b) {
  if (P.state_all) return T;   // a per-token state (never with the chunk form)
  const int t = P.chunk ? T - 1 - b % P.qrows : T;
  return t - t % P.B;
}

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
// The statistics rows of one chunk of kScoreChunk candidates: D/8 lanes
// share a candidate (8 channels each), a pass covers kThreads / (D/8)
// candidates.  page < 0 marks a slot past the candidates.
template <int D>
struct StatRows {
  static constexpr int LPT = D / 8;            // lanes per candidate
  static constexpr int CPP = kThreads / LPT;   // candidates per pass
  static constexpr int NIT = kScoreChunk / CPP;
  int page[NIT];
  float4 m0[NIT], m1[NIT], v0[NIT], v1[NIT];
};

// Issues the statistics loads of a chunk whose pages are set; unused slots
// read page 0.
template <int D>
__device__ __forceinline__ void stat_load(const DecodeParams& P, int g, StatRows<D>& r) {
  const int lig = threadIdx.x % StatRows<D>::LPT;
#pragma unroll
  for (int it = 0; it < StatRows<D>::NIT; ++it) {
    const size_t off = (static_cast<size_t>(max(r.page[it], 0)) * P.Hkv + g) * D + lig * 8;
    r.m0[it] = *reinterpret_cast<const float4*>(P.blk_mean + off);
    r.m1[it] = *reinterpret_cast<const float4*>(P.blk_mean + off + 4);
    r.v0[it] = *reinterpret_cast<const float4*>(P.blk_var + off);
    r.v1[it] = *reinterpret_cast<const float4*>(P.blk_var + off + 4);
  }
}

// sigma q of the pair's G heads, the lane's 8 channels.
template <typename KV, int D, int G>
__device__ __forceinline__ void score_query(const DecodeParams& P, int b, int g, float (&qs)[G][8]) {
  const int lig = threadIdx.x % (D / 8);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    QReg<KV> qr;
    qr.load(reinterpret_cast<const char*>(P.q) +
            ((static_cast<size_t>(b) * P.Hq + g * G + h) * D + lig * 8) * KV::kBytes);
    float qf[8];
    qr.to_f32(qf);
#pragma unroll
    for (int i = 0; i < 8; ++i) qs[h][i] = P.sigma * qf[i];
  }
}

// Group sums of P (a, c) pairs held in v[0 .. 2P) by each lane of an
// L-lane group, scattered: each exchange step pairs lanes whose bit L/2
// differs (row_mirror, row_half_mirror, then the quad swaps of 2 and 1);
// while more than one pair is held, the lane keeps half of them (the upper
// half when its bit is set) and adds what its partner sends of that half,
// afterwards both values are summed with the partner.  Lane lig ends with the
// sums of pair lig / (L / P0) (P0 the pairs at the start), one step per lane
// bit instead of a whole reduction per value.
template <int L, int P>
__device__ __forceinline__ void pair_sums_scatter(const float* v, int lig, float& a, float& c) {
  if constexpr (L == 1) {
    static_assert(P == 1, "one pair per lane at the end");
    a = v[0];
    c = v[1];
  } else {
    constexpr int kCtrl = L == 16 ? 0x140 : L == 8 ? 0x141 : L == 4 ? 0x4E : 0xB1;
    if constexpr (P > 1) {
      const bool hi = (lig & (L / 2)) != 0;
      float w[P];
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const float keep = hi ? v[P + i] : v[i];
        const float send = hi ? v[i] : v[P + i];
        w[i] = keep + dpp_f<kCtrl>(send);
      }
      pair_sums_scatter<L / 2, P / 2>(w, lig, a, c);
    } else {
      const float w[2] = {v[0] + dpp_f<kCtrl>(v[0]), v[1] + dpp_f<kCtrl>(v[1])};
      pair_sums_scatter<L / 2, 1>(w, lig, a, c);
    }
  }
}

// Scores of a chunk's candidates from its statistics rows, stored as order
// keys: score = sigma q . mu + log(1 + sum_c (sigma q_c)^2 / 2 var_c).
template <int D, int G>
__device__ __forceinline__ void score_finish(const DecodeParams& P, int b, int g, int c_begin, int nc,
                                             const StatRows<D>& r, const float (&qs)[G][8]) {
  constexpr int LPT = StatRows<D>::LPT;
  constexpr int CPP = StatRows<D>::CPP;
  static_assert(G <= LPT && (G & (G - 1)) == 0, "whole lane groups per head");
  constexpr int LPH = LPT / G;                 // lanes holding one head's sums
  const int lig = threadIdx.x % LPT;
  const int slot = threadIdx.x / LPT;
  const int hsel = lig / LPH;                  // the head whose score this lane holds
  uint32_t* keys = P.keys + (static_cast<size_t>(b) * P.Hq + g * G) * P.sstride;   // the group's key rows
#pragma unroll
  for (int it = 0; it < StatRows<D>::NIT; ++it) {
    const float mu[8] = {r.m0[it].x, r.m0[it].y, r.m0[it].z, r.m0[it].w, r.m1[it].x, r.m1[it].y, r.m1[it].z, r.m1[it].w};
    const float va[8] = {r.v0[it].x, r.v0[it].y, r.v0[it].z, r.v0[it].w, r.v1[it].x, r.v1[it].y, r.v1[it].z, r.v1[it].w};
    float v[2 * G];   // (q . mu, sum q^2 var / 2) of each head, this lane's 8 channels
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.f, c = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        a = fmaf(qs[h][i], mu[i], a);
        c = fmaf(qs[h][i] * qs[h][i], va[i], c);
      }
      v[2 * h] = a;
      v[2 * h + 1] = 0.5f * c;
    }
    float d1, d2;
    pair_sums_scatter<LPT, G>(v, lig, d1, d2);
    const int cidx = c_begin + slot + it * CPP;
    if (lig % LPH == 0 && cidx < nc) {
      // log(1 + x) via the hardware logarithm: x >= 0, absolute error ~1e-7.
      keys[hsel * P.sstride + cidx] = f32_order_key(d1 + __logf(1.f + d2));
    }
  }
}

// One scoring workgroup of k_score_readout: the chunk's candidates for the
// G query heads of the group.  Every load of the chunk is issued before any
// arithmetic: page ids (bounded by the longest sequence, so that they need
// not wait for this one's length), then the statistics rows, then the
// queries.
template <typename KV, int D, int G>
__device__ __forceinline__ void score_part(const DecodeParams& P, int b, int g, int chunk) {
  using R = StatRows<D>;
  const int c_begin = chunk * kScoreChunk;   // < nc_max
  const int slot = threadIdx.x / R::LPT;
  const int32_t* bt = P.block_table + static_cast<size_t>(seq_of(P, b)) * P.max_blocks;
  const int lo = P.ns / P.B;   // first candidate block, whatever the length
  R r;
#pragma unroll
  for (int it = 0; it < R::NIT; ++it) r.page[it] = bt[lo + min(c_begin + slot + it * R::CPP, P.nc_max - 1)];
  const int T = first_kernel_len(P, b);
  const int nc = min(candidate_range(T, P.B, P.ns, P.W).count, P.nc_max);
  if (c_begin >= nc) return;
#pragma unroll
  for (int it = 0; it < R::NIT; ++it)
    if (c_begin + slot + it * R::CPP >= nc) r.page[it] = -1;
  stat_load<D>(P, g, r);
  float qs[G][8];
  score_query<KV, D, G>(P, b, g, qs);
  score_finish<D, G>(P, b, g, c_begin, nc, r, qs);
}

// Token-level variant ("SALS: Sparse Attention in Latent Space for KV Cache
// Compression", Approach, here on the plain keys): the scores sigma q.k_t of
// 256 candidate tokens of one (sequence, kv head) for its G query heads, as
// order keys.  D/8 lanes share a token (8 channels each); a pass covers 256 /
// (D/8) tokens, and every pass's page lookups and key rows are issued before
// the first dot product.
template <typename KV, int D, int G>
__device__ __forceinline__ void score_tokens_part(const DecodeParams& P, int b, int g, int chunk) {
  constexpr int LPT = D / 8;
  constexpr int TPP = kThreads / LPT;
  constexpr int NIT = kTokenChunk / TPP;
  static_assert(kTokenChunk % TPP == 0 && G <= LPT, "whole passes; one finishing lane per head");
  const int c_begin = chunk * kTokenChunk;
  const int tid = threadIdx.x;
  const int lig = tid % LPT;
  const int slot = tid / LPT;
  const int T = first_kernel_len(P, b);
  const CandRange cr = candidate_range(T, 1, P.ns, P.W);
  const int nc = min(cr.count, P.nc_max);
  if (c_begin >= nc) return;
  const int32_t* bt = P.block_table + static_cast<size_t>(seq_of(P, b)) * P.max_blocks;
  const char* kp = reinterpret_cast<const char*>(P.k_pages);
  Row8<KV> kr[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int t = cr.lo + min(c_begin + slot + it * TPP, nc - 1);
    const size_t page = static_cast<size_t>(bt[t / P.B]);
    kr[it].load(kp + (((page * P.Hkv + g) * P.B + t % P.B) * D + lig * 8) * KV::kBytes);
  }
  QReg<KV> qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h].load(reinterpret_cast<const char*>(P.q) + ((static_cast<size_t>(b) * P.Hq + g * G + h) * D + lig * 8) * KV::kBytes);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    float mine = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = reduce_sum_lanes<LPT>(qr[h].dot(kr[it]));
      mine = (h == lig) ? a : mine;
    }
    const int c = c_begin + slot + it * TPP;
    if (lig < G && c < nc)
      P.keys[(static_cast<size_t>(b) * P.Hq + g * G + lig) * P.sstride + c] = f32_order_key(P.sigma * mine);
  }
}

// The readout's LDS: one instance per kernel.
template <int D, int G>
struct ReadoutLds {
  // the fold's stage is done with before the readout's sums are written
  union {
    float red[kThreads / kWave][D / 4][G][4];
    uint4 fold[kFoldStageBytes / 16];   // block stage, or the statistics' sums
  };
  float zs[kRoRows];
};
template <int D, int G>
__device__ __forceinline__ ReadoutLds<D, G>& readout_lds() {
  __shared__ ReadoutLds<D, G> lds;
  return lds;
}

// The registers of one row chunk's readout, loaded by readout_load and used
// by readout_finish: thread (rg, col4) holds columns 4 col4 .. 4 col4 + 3
// of rows r0 + rg + RG i (i < NR) of S and the G heads' query entries of
// those rows; threads tid < kRoRows hold z[r0 + tid]; thread h kRoRows + r
// (h < G) holds head h's query entry of row r0 + r (for q . z).
template <int D, int G>
struct ReadoutRegs {
  static constexpr int C4 = D / 4;            // float4 columns per row
  static constexpr int RG = kThreads / C4;    // row groups
  static constexpr int NR = kRoRows / RG;     // rows per thread
  static_assert(kRoRows % RG == 0 && G * kRoRows <= kThreads, "rows per readout workgroup");
  float4 srow[NR];
  float qv[NR][G];
  float zr;
  float qz;
  uint32_t kn, vn;   // with the append, row chunk 0: element tid < D of the new key and value (storage bits)
};

// Rows [rc*32, rc*32 + 32) of the state readout: partial S^T q and q . z
// of the pair's G heads (SPLA, section "Residual Linear Attention (RLA)":
// the linear part reads the global state).  readout_load issues the loads
// (only with the linear tail; the append's fold loads the rows itself when
// it needs them without the tail).
template <typename KV, int D, int G>
__device__ __forceinline__ void readout_load(const DecodeParams& P, int b, int g, int rc, ReadoutRegs<D, G>& R) {
  using RR = ReadoutRegs<D, G>;
  const int tid = threadIdx.x;
  const int col4 = tid % RR::C4;
  const int rg = tid / RR::C4;
  const int r0 = rc * kRoRows;
  const bool app = P.app.k_new != nullptr;
  R.zr = 0.f;
  R.qz = 0.f;
  R.kn = R.vn = 0u;
  if (app && rc == 0 && tid < D) {   // the new token's row, for its page slot
    const size_t e = (static_cast<size_t>(b) * P.Hkv + g) * D + tid;
    if constexpr (KV::kBytes == 2) {
      R.kn = reinterpret_cast<const uint16_t*>(P.app.k_new)[e];
      R.vn = reinterpret_cast<const uint16_t*>(P.app.v_new)[e];
    } else {
      R.kn = reinterpret_cast<const uint32_t*>(P.app.k_new)[e];
      R.vn = reinterpret_cast<const uint32_t*>(P.app.v_new)[e];
    }
  }
  if (!P.linear_tail || rc >= D / kRoRows) return;
  const int spair = state_pair(P, b * P.Hkv + g);   // the sequence's state (the pair itself unless multi-query)
  const float* Sp = (app ? P.app.S : P.S) + static_cast<size_t>(spair) * D * D;
  const float* zp = (app ? P.app.z : P.z) + static_cast<size_t>(spair) * D + r0;
  const size_t qbase = (static_cast<size_t>(b) * P.Hq + g * G) * D;
#pragma unroll
  for (int i = 0; i < RR::NR; ++i)
    R.srow[i] = *reinterpret_cast<const float4*>(Sp + static_cast<size_t>(r0 + rg + i * RR::RG) * D + col4 * 4);
  if (tid < kRoRows) R.zr = zp[tid];
#pragma unroll
  for (int i = 0; i < RR::NR; ++i)
#pragma unroll
    for (int h = 0; h < G; ++h) R.qv[i][h] = q_elem<KV>(P.q, qbase + static_cast<size_t>(h) * D + r0 + rg + i * RR::RG);
  if (tid < G * kRoRows) R.qz = q_elem<KV>(P.q, qbase + static_cast<size_t>(tid / kRoRows) * D + r0 + tid % kRoRows);
}

// The rest of row chunk rc, once its loads are issued.  With the append
// taken in, row chunk 0 writes the new token's page slot and length, and
// when the token completes its block every chunk first adds the block to
// its rows of S and z (chunk 0 also to sv) and writes them back, so that the
// readout sees the state the stand-alone append would leave; one more chunk
// per pair (rc = d/32) computes the block's statistics.  Without the linear
// tail only the append's part runs.  t_app >= 0: the append's position and
// page_app the page of its block, as the caller already holds them; t_app <
// 0: both are read here.
template <typename KV, int D, int G>
__device__ __forceinline__ void readout_finish(const DecodeParams& P, int b, int g, int rc, ReadoutRegs<D, G>& R,
                                               int t_app, int page_app) {
  using RR = ReadoutRegs<D, G>;
  constexpr int NR = RR::NR;
  constexpr int RG = RR::RG;
  constexpr int C4 = RR::C4;
  ReadoutLds<D, G>& lds = readout_lds<D, G>();
  auto& red = lds.red;
  auto& zs = lds.zs;
  auto& fold_lds = lds.fold;
  const int tid = threadIdx.x;
  const int col4 = tid % C4;
  const int rg = tid / C4;
  const int pair = b * P.Hkv + g;
  const int r0 = rc * kRoRows;
  const bool app = P.app.k_new != nullptr;
  const bool lin = P.linear_tail != 0;
  const size_t nbase = static_cast<size_t>(pair) * D;   // k_new / v_new row of the pair
  int T = 0;
  size_t row0 = 0, page = 0;
  bool completes = false;
  if (app) {
    if (t_app >= 0) {
      T = t_app;
      page = static_cast<size_t>(page_app);
    } else {
      T = append_pos(P, b);
      page = static_cast<size_t>(P.block_table[static_cast<size_t>(b) * P.max_blocks + T / P.B]);
    }
    row0 = (page * P.Hkv + g) * P.B;   // first row of the page-head tile
    completes = (T + 1) % P.B == 0;    // uniform
  }
  if (app && rc == D / kRoRows) {   // the statistics of the block the token completes
    if (!completes) return;
    const size_t so = (page * P.Hkv + g) * D;
    filled_block_stats<KV, D, kThreads>(P.app.k_pages, P.app.k_new, row0, T % P.B, nbase, P.B, P.app.blk_mean + so,
                                        P.app.blk_var + so, *reinterpret_cast<BlockStatsLds<kThreads, D>*>(fold_lds));
    return;
  }
  if (app && rc == 0) {
    if (tid < D) {   // the values were loaded with the chunk's rows
      const size_t e = (row0 + T % P.B) * D + tid;
      if constexpr (KV::kBytes == 2) {
        reinterpret_cast<uint16_t*>(P.app.k_pages)[e] = static_cast<uint16_t>(R.kn);
        reinterpret_cast<uint16_t*>(P.app.v_pages)[e] = static_cast<uint16_t>(R.vn);
      } else {
        reinterpret_cast<uint32_t*>(P.app.k_pages)[e] = R.kn;
        reinterpret_cast<uint32_t*>(P.app.v_pages)[e] = R.vn;
      }
    }
    if (g == 0 && tid == 0 && P.app.lens_after) P.app.lens_after[b] = T + 1;
  }
  // a per-token state takes the new token now (never with the chunk form)
  const bool tok = app && P.state_all;
  if (!lin) {
    if (!completes && !tok) return;
    const float* Sp = P.app.S + static_cast<size_t>(pair) * D * D;
#pragma unroll
    for (int i = 0; i < NR; ++i)
      R.srow[i] = *reinterpret_cast<const float4*>(Sp + static_cast<size_t>(r0 + rg + i * RG) * D + col4 * 4);
    if (tid < kRoRows) R.zr = P.app.z[nbase + r0 + tid];
  }
  if (tok) {
    // S += k v^T on the chunk's rows, z += k, and chunk 0 sv += v: the same
    // arithmetic as the stand-alone append, before the readout reads them
    const float4 vv = kv_load4<KV>(P.app.v_new, nbase + col4 * 4);
    float* Sw = P.app.S + static_cast<size_t>(pair) * D * D;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const float kr = kv_elem<KV>(P.app.k_new, nbase + r0 + rg + i * RG);
      R.srow[i].x = fmaf(kr, vv.x, R.srow[i].x);
      R.srow[i].y = fmaf(kr, vv.y, R.srow[i].y);
      R.srow[i].z = fmaf(kr, vv.z, R.srow[i].z);
      R.srow[i].w = fmaf(kr, vv.w, R.srow[i].w);
      *reinterpret_cast<float4*>(Sw + static_cast<size_t>(r0 + rg + i * RG) * D + col4 * 4) = R.srow[i];
    }
    if (tid < kRoRows) {
      R.zr += kv_elem<KV>(P.app.k_new, nbase + r0 + tid);
      P.app.z[nbase + r0 + tid] = R.zr;
    }
    if (rc == 0 && tid < D) P.app.sv[nbase + tid] += kv_elem<KV>(P.app.v_new, nbase + tid);
  } else if (completes) {
    const CompletedBlock cb{P.app.k_pages, P.app.v_pages, P.app.k_new, P.app.v_new, row0, nbase, T % P.B, P.B};
    const int zrow = tid < kRoRows ? r0 + tid : -1;
    const int svcol = rc == 0 && tid < D ? tid : -1;
    float sv = svcol >= 0 ? P.app.sv[nbase + svcol] : 0.f;
    fold_completed_block<KV, D, kThreads, NR, RG>(cb, fold_lds, R.srow, r0 + rg, col4, zrow, R.zr, svcol, sv);
    __syncthreads();   // the stage is read before the readout's sums overwrite it
    float* Sw = P.app.S + static_cast<size_t>(pair) * D * D;
#pragma unroll
    for (int i = 0; i < NR; ++i)
      *reinterpret_cast<float4*>(Sw + static_cast<size_t>(r0 + rg + i * RG) * D + col4 * 4) = R.srow[i];
    if (zrow >= 0) P.app.z[nbase + zrow] = R.zr;
    if (svcol >= 0) {
      P.app.sv[nbase + svcol] = sv;
    }
  }
  if (!lin) return;
  if (tid < kRoRows) zs[tid] = R.zr;
  float acc[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.f;
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      acc[h][0] = fmaf(R.qv[i][h], R.srow[i].x, acc[h][0]);
      acc[h][1] = fmaf(R.qv[i][h], R.srow[i].y, acc[h][1]);
      acc[h][2] = fmaf(R.qv[i][h], R.srow[i].z, acc[h][2]);
      acc[h][3] = fmaf(R.qv[i][h], R.srow[i].w, acc[h][3]);
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
  // q . z over the chunk's rows: thread h kRoRows + r takes row r of head
  // h, then a sum over the 32 lanes of the head (rows of 16 lanes, then
  // the lanes 16 apart)
  float qzv = tid < G * kRoRows ? R.qz * zs[tid % kRoRows] : 0.f;
  qzv = reduce_sum_lanes<16>(qzv);
  qzv = pair_sum<16>(qzv);
  if (tid < G * kRoRows && tid % kRoRows == 0) {
    P.roz[(static_cast<size_t>(pair) * P.ro_wgs + rc) * G + tid / kRoRows] = qzv;
  }
}

// A whole row chunk: its loads, `mid` while they are in flight, the rest.
template <typename KV, int D, int G, typename Mid>
__device__ __forceinline__ void readout_part(const DecodeParams& P, int b, int g, int rc, Mid&& mid) {
  ReadoutRegs<D, G> R;
  readout_load<KV, D, G>(P, b, g, rc, R);
  mid();
  readout_finish<KV, D, G>(P, b, g, rc, R, -1, 0);
}

template <typename KV, int D, int G>
__global__ __launch_bounds__(kThreads) void k_score_readout(DecodeParams P) {
#ifdef HSLA_PHASE_TIMESTAMPS
  const PhaseSpan span(g_phase_score, kPhaseScoreWgs, static_cast<size_t>(blockIdx.y) * gridDim.x + blockIdx.x);
#endif
  const int pair = blockIdx.y;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int x = blockIdx.x;
  if (x == 0 && threadIdx.x == 0) {   // the pair's counters for the attention kernel
    if (P.dyn && P.fused_sel)
      __hip_atomic_store(P.ctr + static_cast<size_t>(pair) * kCtrStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (P.fused_merge)
      __hip_atomic_store(P.ctr + static_cast<size_t>(pair) * kCtrStride + kDoneSlot, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  if (x < P.score_wgs) {
    if (P.tokens) {
      if constexpr (G <= D / 8) score_tokens_part<KV, D, G>(P, b, g, x);
    } else {
      score_part<KV, D, G>(P, b, g, x);
    }
  } else {
    readout_part<KV, D, G>(P, b, g, x - P.score_wgs, [] {});
  }
}

// ---------------------------------------------------------------------------
// 2. Top-k selection and the union of the group's exact blocks
// ---------------------------------------------------------------------------
// Selection runs per query head: one wavefront takes the head's block-score
// order keys, finds the k-th largest by a radix search and writes the head's
// selection bitmap and its selected indices.  The union of a group's exact
// blocks (SPLA Figure 1(a)) is not materialised here: each attention
// workgroup forms its own share of it from the G bitmaps (section 3).
// Wavefront-wide min / max of uint32 without LDS: DPP permutations inside
// each row of 16 lanes, then the permlane swaps across rows.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  auto dpp = [](uint32_t x, auto ctrl) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), decltype(ctrl)::value, 0xf, 0xf, true));
  };
  v = op(v, dpp(v, std::integral_constant<int, 0xB1>{}));    // quad_perm [1,0,3,2]
  v = op(v, dpp(v, std::integral_constant<int, 0x4E>{}));    // quad_perm [2,3,0,1]
  v = op(v, dpp(v, std::integral_constant<int, 0x141>{}));   // row_half_mirror
  v = op(v, dpp(v, std::integral_constant<int, 0x140>{}));   // row_mirror
  auto r16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r16[0], r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r32[0], r32[1]);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return wave_minmax_u32<false>(v); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return wave_minmax_u32<true>(v); }
__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
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

// One radix pass step shared by the two threshold searches below: given the
// wavefront's histogram row (4 bins per lane, digit 4 lane + j), find the
// digit holding the rem-th largest key and how many of that digit's keys are
// still to take.
__device__ __forceinline__ void radix_pick(const uint4 c4, int lane, int& digit, int& rem) {
  const uint32_t mine = c4.x + c4.y + c4.z + c4.w;
  const uint32_t incl = wave_scan_incl(mine);
  const uint32_t total = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1));
  const uint32_t suffix = total - incl + mine;   // keys whose digit >= 4 * lane
  const uint32_t above = suffix - mine;          // keys whose digit > 4 * lane + 3
  const bool here = above < static_cast<uint32_t>(rem) && static_cast<uint32_t>(rem) <= suffix;
  int d = 0, rem_here = rem;
  if (here) {   // the crossing bin is one of this lane's four, scanned from the top
    uint32_t acc = above;
    bool found = false;
    const uint32_t cs[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
    for (int j = 3; j >= 0; --j) {
      if (!found && acc + cs[j] >= static_cast<uint32_t>(rem)) {
        d = 4 * lane + j;
        rem_here = rem - static_cast<int>(acc);
        found = true;
      }
      acc += cs[j];
    }
  }
  const uint64_t hm = __ballot(here);
  const int src = __ffsll(static_cast<unsigned long long>(hm)) - 1;
  digit = __builtin_amdgcn_readlane(d, src);
  rem = __builtin_amdgcn_readlane(rem_here, src);
}

// Value of lane ^ S, for S = 1 .. 32, without LDS: DPP quad permutes for 1
// and 2, two bank-masked DPP row shifts for 4 and 8 (each half of the row
// reads from the other), the gfx950 row swaps for 16 and 32.  A swap
// returns the lane's own value in one result and its partner's in the
// other; taking the one that differs from the own value is right whichever
// is which (when they are equal either is the partner's).
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  const int x = static_cast<int>(v);
  if constexpr (S == 1) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xf, 0xf, false));   // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xf, 0xf, false));   // quad_perm [2,3,0,1]
  } else if constexpr (S == 4) {
    const int t = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xf, 0x5, false);   // row_shl:4 into banks 0, 2
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(t, x, 0x114, 0xf, 0xA, false));   // row_shr:4 into 1, 3
  } else if constexpr (S == 8) {
    const int t = __builtin_amdgcn_update_dpp(x, x, 0x108, 0xf, 0x3, false);   // row_shl:8 into banks 0, 1
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(t, x, 0x118, 0xf, 0xC, false));   // row_shr:8 into 2, 3
  } else if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return r[0] == v ? r[1] : r[0];
  } else {
    static_assert(S == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r[0] == v ? r[1] : r[0];
  }
}

// One compare-exchange step of the sort below: pairs (lane, lane ^ S) of a
// run of SIZE lanes; in a run that ends descending the lower lane keeps the
// larger value.
template <int SIZE, int S>
__device__ __forceinline__ uint32_t sort_step(uint32_t v, int lane) {
  const uint32_t o = lane_xor<S>(v);
  const bool desc = (lane & SIZE) == 0;
  const bool lower = (lane & S) == 0;
  return (lower == desc) ? max(v, o) : min(v, o);
}
template <int SIZE, int S>
__device__ __forceinline__ uint32_t sort_merge(uint32_t v, int lane) {
  v = sort_step<SIZE, S>(v, lane);
  if constexpr (S > 1) v = sort_merge<SIZE, S / 2>(v, lane);
  return v;
}

// Descending bitonic sort of one value per lane across the wavefront: lane
// i ends with the (i+1)-th largest.  21 compare-exchange steps, all in
// registers.
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t v, int lane) {
  v = sort_merge<2, 1>(v, lane);
  v = sort_merge<4, 2>(v, lane);
  v = sort_merge<8, 4>(v, lane);
  v = sort_merge<16, 8>(v, lane);
  v = sort_merge<32, 16>(v, lane);
  return sort_merge<64, 32>(v, lane);
}

// k-th largest of n > k order keys held in registers (lane l: keys l,
// l + 64, ...; 0 where there is none, which orders below every key), for
// k <= 64.  The k-th largest of the lane maxima is a lower bound of the
// answer (those maxima are k of the keys); when at most `cap` keys reach
// it -- the usual case: the k largest keys rarely crowd into a few lanes --
// they are gathered into one value per lane and sorted, and the k-th of
// them is the answer.  Two wavefront sorts, no histogram.  Returns false
// (and leaves thr alone) when more keys reach the bound.
template <int KPL>
__device__ __forceinline__ bool wave_topk_sorted(const uint32_t* key, int k, int lane, uint32_t* hist,
                                                 uint32_t& thr) {
  uint32_t lmax = 0u;
#pragma unroll
  for (int j = 0; j < KPL; ++j) lmax = max(lmax, key[j]);
  const uint32_t bound =
      static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_sort_desc(lmax, lane)), k - 1));
  int c = 0;   // keys >= bound, gathered into hist[0 .. 63]
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const bool in = key[j] >= bound;
    const uint64_t m = __ballot(in);
    const int pos = c + __popcll(m & lanes_below(lane));
    if (in && pos < kWave) hist[pos] = key[j];
    c += __popcll(m);
  }
  if (c > kWave) return false;
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  uint32_t x = lane < c ? hist[lane] : 0u;
  if (c <= kWave / 2) {   // lanes 32 .. 63 hold zeros: sorting each half leaves lanes 0 .. 31 descending
    x = sort_merge<2, 1>(x, lane);
    x = sort_merge<4, 2>(x, lane);
    x = sort_merge<8, 4>(x, lane);
    x = sort_merge<16, 8>(x, lane);
    x = sort_merge<32, 16>(x, lane);
  } else {
    x = wave_sort_desc(x, lane);
  }
  thr = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), k - 1));
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // hist is read before any later use
  return true;
}

// k-th largest of n order keys for one wavefront: `thr` is that key and
// `rem` how many keys equal to it are taken (the lowest indices first).
// Radix select over 8-bit digits, skipping the high bits every key shares,
// with a 256-bin histogram private to the wavefront (no workgroup barrier).
// KPL > 0: lane l holds keys l, l + 64, ... in registers; KPL == 0: keys
// are read through key_at on every pass.
// With keys in registers and k <= 64, the smallest of the 64 lane maxima is
// a lower bound of the k-th largest key (each lane holds one key at least
// that large), so only keys at or above it take part.
template <int KPL, typename KeyAt>
__device__ __forceinline__ void wave_topk_threshold(const uint32_t* key, KeyAt key_at, int n, int k, int lane,
                                                    uint32_t* hist, uint32_t& thr, int& rem) {
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  uint32_t floor_key = 0u;   // keys below it cannot be among the k largest
  if constexpr (KPL > 0) {
    if (k <= kWave && n >= kWave) {
      uint32_t lmax = 0u;
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if (lane + kWave * j < n) lmax = max(lmax, key[j]);
      floor_key = wave_min_u32(lmax);   // every lane holds a key (n >= 64)
    }
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (lane + kWave * j < n && key[j] >= floor_key) {
        kmin = min(kmin, key[j]);
        kmax = max(kmax, key[j]);
      }
  } else {
    for (int i = lane; i < n; i += kWave) {
      const uint32_t x = key_at(i);
      kmin = min(kmin, x);
      kmax = max(kmax, x);
    }
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  const uint32_t diff = kmin ^ kmax;
  int shift = diff ? 32 - __clz(static_cast<int>(diff)) : 0;   // low bits that still vary
  uint32_t mask = (shift == 32) ? 0u : ~((1u << shift) - 1u);
  uint32_t prefix = kmax & mask;
  rem = k;
  uint4* hrow = reinterpret_cast<uint4*>(hist + 4 * lane);
  while (shift > 0) {
    const int nb = min(8, shift);
    shift -= nb;
    const uint32_t dmask = (1u << nb) - 1u;
    *hrow = make_uint4(0, 0, 0, 0);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if constexpr (KPL > 0) {
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if (lane + kWave * j < n && key[j] >= floor_key && (key[j] & mask) == prefix)
          atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
    } else {
      for (int i = lane; i < n; i += kWave) {
        const uint32_t x = key_at(i);
        if ((x & mask) == prefix) atomicAdd(&hist[(x >> shift) & dmask], 1u);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    int digit;
    radix_pick(*hrow, lane, digit, rem);
    prefix |= static_cast<uint32_t>(digit) << shift;
    mask |= dmask << shift;
  }
  thr = prefix;
}

// One head's selection: threshold, then the bitmap of selected candidates
// (word w, bit i: candidate 64 w + i) and, when `out` is set, the selected
// block indices in ascending order padded with -1.  Both are written to
// `ncopy` consecutive heads' rows (bitmap rows nwords apart, index rows k
// apart).
template <int KPL, typename KeyAt>
__device__ __forceinline__ void head_select(KeyAt key_at, const uint32_t* key, int nc, int k, int nwords, int lane,
                                            uint32_t* hist, uint64_t* bits_row, int32_t* out, int lo,
                                            int ncopy = 1) {
  const bool take_all = k >= nc;
  const bool take_none = (k <= 0) || (nc == 0);
  int nsel = 0;
  if constexpr (KPL > 0) {
    // Keys in registers, 0 where a lane holds no candidate (0 orders below
    // every key).  The selection is built as whole 64-bit masks, one per
    // register slot (word w, bit i: candidate 64 w + i), in scalar
    // registers: keys >= the threshold, and when fewer keys equal to it are
    // taken than there are, those above it plus the lowest-index equal ones.
    uint32_t kz[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) kz[j] = lane + kWave * j < nc ? key[j] : 0u;
    uint64_t sm[KPL];
    if (take_none) {
#pragma unroll
      for (int w = 0; w < KPL; ++w) sm[w] = 0ull;
    } else if (take_all) {
#pragma unroll
      for (int w = 0; w < KPL; ++w) sm[w] = __ballot(w * kWave + lane < nc);
    } else {
      uint32_t thr = 0;
      if (k > kWave || !wave_topk_sorted<KPL>(kz, k, lane, hist, thr)) {
        int rem_unused;
        wave_topk_threshold<KPL>(key, key_at, nc, k, lane, hist, thr, rem_unused);
      }
      int ge_total = 0;
#pragma unroll
      for (int w = 0; w < KPL; ++w) {
        sm[w] = __ballot(kz[w] >= thr);
        ge_total += __popcll(sm[w]);
      }
      if (ge_total > k) {   // keep only the lowest-index keys equal to thr that fit
        uint64_t em[KPL];
        int eq_total = 0;
#pragma unroll
        for (int w = 0; w < KPL; ++w) {
          em[w] = __ballot(kz[w] == thr);
          eq_total += __popcll(em[w]);
        }
        int eq_left = k - (ge_total - eq_total);
#pragma unroll
        for (int w = 0; w < KPL; ++w) {
          uint64_t e = em[w];
          const int c = __popcll(e);
          if (c > eq_left) {
            uint64_t keep = 0ull;
            for (int r = 0; r < eq_left; ++r) {
              const uint64_t low = e & (~e + 1ull);
              keep |= low;
              e ^= low;
            }
            e = keep;
          }
          eq_left -= __popcll(e);
          sm[w] = (sm[w] & ~em[w]) | e;
        }
      }
    }
    // the bitmap: word w from lane w
    uint64_t mine = 0ull;
#pragma unroll
    for (int w = 0; w < KPL; ++w)
      if (lane == w) mine = sm[w];
    if (lane < nwords)
      for (int x = 0; x < ncopy; ++x) bits_row[lane + x * nwords] = mine;
    if (out) {
#pragma unroll
      for (int w = 0; w < KPL; ++w) {
        const int pos = nsel + __popcll(sm[w] & lanes_below(lane));
        const bool sel = (sm[w] >> lane) & 1ull;
        for (int x = 0; x < ncopy; ++x)
          if (sel && pos < k) out[pos + x * k] = lo + w * kWave + lane;
        nsel += __popcll(sm[w]);
      }
    }
  } else {
    uint32_t thr = 0;
    int rem = k;
    if (!take_all && !take_none) wave_topk_threshold<KPL>(key, key_at, nc, k, lane, hist, thr, rem);
    int neq = 0;
    // When every key equal to the threshold is taken, the selection is just
    // key >= thr and no rank among equal keys is needed.
    bool simple = take_all || take_none;
    if (!simple) {
      int eq_total = 0;
      for (int w = 0; w < nwords; ++w) {
        const int i = w * kWave + lane;
        eq_total += __popcll(__ballot(i < nc && key_at(i) == thr));
      }
      simple = eq_total == rem;
    }
    for (int w = 0; w < nwords; ++w) {
      const int i = w * kWave + lane;
      const bool valid = i < nc;
      const uint32_t x = valid ? key_at(i) : 0u;
      bool sel;
      if (take_none) {
        sel = false;
      } else if (take_all) {
        sel = valid;
      } else if (simple) {
        sel = valid && x >= thr;
      } else {
        const bool eq = valid && x == thr;
        const uint64_t eqm = __ballot(eq);
        const int eqrank = neq + __popcll(eqm & lanes_below(lane));
        sel = valid && (x > thr || (eq && eqrank < rem));
        neq += __popcll(eqm);
      }
      const uint64_t sm = __ballot(sel);
      const int pos = nsel + __popcll(sm & lanes_below(lane));
      for (int c = 0; c < ncopy; ++c) {
        if (sel && out && pos < k) out[pos + c * k] = lo + i;
        if (lane == 0) bits_row[w + c * nwords] = sm;
      }
      nsel += __popcll(sm);
    }
  }
  if (out)
    for (int x = 0; x < ncopy; ++x)
      for (int j = nsel + lane; j < k; j += kWave) out[j + x * k] = -1;
}

// Selection of one (sequence, query head), one wavefront: the head's order
// keys straight into registers (KPL per lane; KPL = 0 reads them through
// memory on every pass), the threshold, then the head's selection bitmap
// (word w, bit i: candidate 64 w + i) and its selected block indices.
template <int KPL>
__global__ __launch_bounds__(kWave) void k_select(DecodeParams P) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];
  const int bh = blockIdx.x;
  const int b = bh / P.Hq;
  const int lane = threadIdx.x;
  const uint32_t* kh = P.keys + static_cast<size_t>(bh) * P.sstride;
  // The keys go into registers before the sequence length is known (the
  // row holds sstride >= nc_max keys; those past nc are never used).
  uint32_t key[KPL > 0 ? KPL : 1];
  if constexpr (KPL > 0) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) key[j] = kh[min(lane + kWave * j, P.sstride - 1)];
  }
  const int T = __builtin_amdgcn_readfirstlane(clamp_len(P.seq_lens[b], P.max_seq_len));
  const CandRange cr = candidate_range(T, P.bsel, P.ns, P.W);
  const int nc = min(cr.count, P.nc_max);
  auto key_at = [&](int i) -> uint32_t { return kh[i]; };
  int32_t* out = P.sel_idx ? P.sel_idx + static_cast<size_t>(bh) * P.top_k : nullptr;
  const int G = P.Hq / P.Hkv;
  if (P.dyn && lane == 0 && (bh % P.Hq) % G == 0)   // the pair's work counter for the attention kernel
    __hip_atomic_store(P.ctr + static_cast<size_t>(bh / G) * kCtrStride, 0, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  head_select<KPL>(key_at, key, nc, P.top_k, P.nwords, lane, hist, P.bits + static_cast<size_t>(bh) * P.nwords, out,
                   cr.lo);
}

// Grouped selection of one (sequence, kv head), one wavefront: the G heads'
// order keys are decoded back to scores; each head's scores become a softmax
// over the candidates (the head's maximum, then its sum of exponentials,
// both wavefront reductions) and the G shares are summed per block.  The
// top-k of these sums is the selection of every head of the group: its
// bitmap and indices are written to all G heads' rows, so that the union
// and attention stages run unchanged.  KPL > 0 keeps G x KPL keys per lane
// in registers; KPL == 0 streams them and writes the sums as order keys over
// the first head's key row, which the threshold search then reads.
template <int KPL, int G>
__global__ __launch_bounds__(kWave) void k_select_grouped(DecodeParams P) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[256];
  const int pair = blockIdx.x;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int lane = threadIdx.x;
  const size_t row0 = static_cast<size_t>(b) * P.Hq + g * G;
  uint32_t* k0 = P.keys + row0 * P.sstride;
  const int ss = P.sstride;
  uint32_t kr[G][KPL > 0 ? KPL : 1];
  if constexpr (KPL > 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < KPL; ++j) kr[h][j] = k0[h * ss + min(lane + kWave * j, ss - 1)];
  }
  const int T = __builtin_amdgcn_readfirstlane(clamp_len(P.seq_lens[b], P.max_seq_len));
  const CandRange cr = candidate_range(T, P.B, P.ns, P.W);
  const int nc = min(cr.count, P.nc_max);
  uint32_t agg[KPL > 0 ? KPL : 1];
  if constexpr (KPL > 0) {
    float w[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) w[j] = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      uint32_t kmax = 0u;
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if (lane + kWave * j < nc) kmax = max(kmax, kr[h][j]);
      const float m = f32_from_order_key(wave_max_u32(kmax));
      float e[KPL], sum = 0.f;
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        e[j] = lane + kWave * j < nc ? fast_exp(f32_from_order_key(kr[h][j]) - m) : 0.f;
        sum += e[j];
      }
      const float inv = 1.f / wave_sum(sum);
#pragma unroll
      for (int j = 0; j < KPL; ++j) w[j] = fmaf(e[j], inv, w[j]);
    }
#pragma unroll
    for (int j = 0; j < KPL; ++j) agg[j] = f32_order_key(w[j]);
  } else if (nc > 0) {
    float m[G], inv[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      uint32_t kmax = 0u;
      for (int i = lane; i < nc; i += kWave) kmax = max(kmax, k0[h * ss + i]);
      m[h] = f32_from_order_key(wave_max_u32(kmax));
      float sum = 0.f;
      for (int i = lane; i < nc; i += kWave) sum += fast_exp(f32_from_order_key(k0[h * ss + i]) - m[h]);
      inv[h] = 1.f / wave_sum(sum);
    }
    for (int i = lane; i < nc; i += kWave) {   // every key of index i is read before it is overwritten
      float w = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) w = fmaf(fast_exp(f32_from_order_key(k0[h * ss + i]) - m[h]), inv[h], w);
      k0[i] = f32_order_key(w);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  auto key_at = [&](int i) -> uint32_t { return k0[i]; };
  int32_t* out = P.sel_idx ? P.sel_idx + row0 * P.top_k : nullptr;
  if (P.dyn && lane == 0)   // the pair's work counter for the attention kernel
    __hip_atomic_store(P.ctr + static_cast<size_t>(pair) * kCtrStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  head_select<KPL>(key_at, agg, nc, P.top_k, P.nwords, lane, hist, P.bits + row0 * P.nwords, out, cr.lo, G);
}

// The split's share of the union, built by the attention workgroup itself
// from the G heads' selection bitmaps: the union of the group's exact blocks
// in ascending block order -- blocks below the candidates (sinks),
// candidates selected by some head or holding sink or window tokens, blocks
// past the candidates (window) -- of which split s takes positions s, s + S,
// s + 2S, ... (S = max_split), so window and sink blocks, which every head
// needs, spread over the splits.  One round trip brings the bitmaps and the
// sequence's block-table row into LDS (`smem`, laid out by SelLayout); one
// barrier later every wavefront forms the 64-block chunk masks in registers
// (lane c: chunk c), scans their counts and, by a binary search over the
// chunk prefixes and a rank search in the chunk's mask, gives lane e < ne its
// entry (block | mask of the heads that selected it << 20) and page.  Has a
// workgroup barrier: every thread calls it.  Split 0 also records the union
// size for the merge.
// FULL (the dynamic split): instead of one share, the whole list -- entries
// and pages, in union order -- is written to LDS (SelLayout::ulist), each
// wavefront writing the entries of every NW-th chunk, and a second barrier
// publishes it.
struct SplitShare {
  int T;       // sequence length (uniform)
  int ent;
  int page;    // -1 on lanes past ne
  int count;   // union size (uniform)
  int ne;      // entries of this split (uniform)
};
template <int G, bool FULL, int FK, bool GS, typename Stage, typename Early>
__device__ __forceinline__ SplitShare union_share(const DecodeParams& P, char* smem, int pair, int b, int g, int split,
                                                  Stage&& stage, Early&& early) {
  constexpr int NW = kThreads / kWave;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  uint64_t* bits = reinterpret_cast<uint64_t*>(smem + P.sl.bits);
  uint64_t* umask = reinterpret_cast<uint64_t*>(smem + P.sl.umask) + wave * kWave;
  int32_t* upre = reinterpret_cast<int32_t*>(smem + P.sl.upre) + wave * kWave;
  int32_t* btrow = reinterpret_cast<int32_t*>(smem + P.sl.btrow);
  const int nwords = P.nwords;
  const int S = P.max_split;
  const int32_t* bt = P.block_table + static_cast<size_t>(seq_of(P, b)) * P.max_blocks;
  const uint64_t* src = P.bits + (static_cast<size_t>(b) * P.Hq + g * G) * nwords;
  const int nbits = P.fused_sel ? 0 : G * nwords;   // bitmaps loaded from the selection kernel
  constexpr int HPW = (G + NW - 1) / NW;            // heads per wavefront of the fused selection

  // ---- bitmaps (or, with the selection fused here, the order keys of the
  // wavefront's heads) and block-table row.  The first round of each is
  // loaded before the sequence length is read and together with the
  // caller's own loads, which `stage` then stores, so that the usual sizes
  // take a single round trip; larger rows loop on.
  uint64_t v[2];
  int w[4];
  uint32_t kr[HPW][FK];
  auto load_keys = [&](auto ld) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      const int h = min(wave + NW * i, G - 1);
      const uint32_t* kh = P.keys + (static_cast<size_t>(b) * P.Hq + g * G + h) * P.sstride;
#pragma unroll
      for (int j = 0; j < FK; ++j) kr[i][j] = ld(kh + min(lane + kWave * j, P.sstride - 1));
    }
  };
  if (P.fused_sel) {
    load_keys([](const uint32_t* p) { return *p; });
  } else {
#pragma unroll
    for (int u = 0; u < 2; ++u) v[u] = src[min(tid + u * kThreads, max(nbits, 1) - 1)];
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) w[u] = bt[min(tid + u * kThreads, P.nblk_max - 1)];
  const int T = __builtin_amdgcn_readfirstlane(clamp_len(P.seq_lens[b], P.max_seq_len));
  // page of block j: from the staged row in LDS, else from global memory
  // (explicit address spaces: a pointer to either would be a flat access)
  auto page_of = [&](int j) __attribute__((always_inline)) -> int {
    return P.bt_staged ? ld_lds<int32_t>(btrow + j) : ld_global<int32_t>(bt + j);
  };
  const CandRange cr = candidate_range(T, P.B, P.ns, P.W);
  const int nc = min(cr.count, P.nc_max);
  const int nb = min(ceil_div(T, P.B), P.nblk_max);
  {
    const int nbt = P.bt_staged ? nb : 0;
    stage();
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (tid + u * kThreads < nbits) bits[tid + u * kThreads] = v[u];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (tid + u * kThreads < nbt) btrow[tid + u * kThreads] = w[u];
    for (int base = 2 * kThreads; base < nbits; base += 2 * kThreads) {
#pragma unroll
      for (int u = 0; u < 2; ++u) v[u] = src[min(base + tid + u * kThreads, nbits - 1)];
#pragma unroll
      for (int u = 0; u < 2; ++u)
        if (base + tid + u * kThreads < nbits) bits[base + tid + u * kThreads] = v[u];
    }
    for (int base = 4 * kThreads; base < nbt; base += 4 * kThreads) {
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = bt[min(base + tid + u * kThreads, nb - 1)];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (base + tid + u * kThreads < nbt) btrow[base + tid + u * kThreads] = w[u];
    }
  }
  HSLA_STAMP(1);
  if constexpr (FULL) {
    // The blocks past the candidates (window blocks) are in the union
    // whatever the selection: the caller may start loading them now, so that
    // they arrive while the selection runs.
    __syncthreads();   // the block-table row
    early(nc > 0 ? cr.lo + nc : 0, nb, page_of);
  }
  if constexpr (!GS) {
    if (P.fused_sel) {
      // each wavefront selects for its heads; the bitmaps go to LDS and, from
      // the pair's first workgroup, the indices to sel_idx
      uint32_t* hist = reinterpret_cast<uint32_t*>(smem + P.sl.hist) + wave * 256;
      auto no_key = [](int) -> uint32_t { return 0u; };   // the keys are all in registers
#pragma unroll
      for (int i = 0; i < HPW; ++i) {
        const int h = wave + NW * i;
        if (h < G) {
          int32_t* out = (P.sel_idx && split == 0)
                             ? P.sel_idx + (static_cast<size_t>(b) * P.Hq + g * G + h) * P.top_k
                             : nullptr;
          head_select<FK>(no_key, kr[i], nc, P.top_k, nwords, lane, hist, bits + h * nwords, out, cr.lo);
        }
      }
    }
    HSLA_STAMP_WAVE(2);
  } else if (nc > 0) {
    // grouped selection, as k_select_grouped computes it: each wavefront
    // turns its heads' scores into shares of the head's candidate mass (a
    // softmax over the candidates); wavefront 0 sums the G shares per block
    // and selects once for every head of the group
    const int ncr = ceil_div(P.nc_max, kWave) * kWave;
    float* gw = reinterpret_cast<float*>(smem + P.sl.gw);
#pragma unroll
    for (int i = 0; i < HPW; ++i) {
      const int h = wave + NW * i;
      if (h < G) {
        uint32_t kmax = 0u;
#pragma unroll
        for (int j = 0; j < FK; ++j)
          if (lane + kWave * j < nc) kmax = max(kmax, kr[i][j]);
        const float m = f32_from_order_key(wave_max_u32(kmax));
        float e[FK], sum = 0.f;
#pragma unroll
        for (int j = 0; j < FK; ++j) {
          e[j] = lane + kWave * j < nc ? fast_exp(f32_from_order_key(kr[i][j]) - m) : 0.f;
          sum += e[j];
        }
        const float inv = 1.f / wave_sum(sum);
#pragma unroll
        for (int j = 0; j < FK; ++j)
          if (lane + kWave * j < nc) gw[h * ncr + lane + kWave * j] = e[j] * inv;   // nc <= ncr
      }
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t agg[FK];
#pragma unroll
      for (int j = 0; j < FK; ++j) {
        float w = 0.f;
        if (lane + kWave * j < nc) {
#pragma unroll
          for (int h = 0; h < G; ++h) w += gw[h * ncr + lane + kWave * j];
        }
        agg[j] = f32_order_key(w);
      }
      uint32_t* hist = reinterpret_cast<uint32_t*>(smem + P.sl.hist);
      int32_t* out = (P.sel_idx && split == 0) ? P.sel_idx + (static_cast<size_t>(b) * P.Hq + g * G) * P.top_k
                                               : nullptr;
      auto no_key = [](int) -> uint32_t { return 0u; };
      head_select<FK>(no_key, agg, nc, P.top_k, nwords, lane, hist, bits, out, cr.lo, G);
    }
  } else {   // grouped, no candidates: every head's bitmap is empty
    for (int x = tid; x < G * nwords; x += kThreads) bits[x] = 0ull;
    if (P.sel_idx && split == 0)
      for (int x = tid; x < G * P.top_k; x += kThreads) P.sel_idx[(static_cast<size_t>(b) * P.Hq + g * G) * P.top_k + x] = -1;
  }
  __syncthreads();

  // Union membership of block j: every block when there are no candidates;
  // otherwise blocks below a1 (sink tokens) or from a2 on (window tokens)
  // and candidates some head selected.
  const int a1 = nc > 0 ? ceil_div(P.ns, P.B) : nb;
  const int a2 = nc > 0 ? (T - P.W) / P.B : nb;   // T - W > ns >= 0 here
  auto head_mask = [&](int j) -> int {   // heads that selected candidate j
    const int c = j - cr.lo;
    int hm = 0;
    if (nc > 0 && c >= 0 && c < nc) {
#pragma unroll
      for (int x = 0; x < G; ++x)
        hm |= static_cast<int>((bits[x * nwords + (c >> 6)] >> (c & 63)) & 1ull) << x;
    }
    return hm;
  };
  // Lanes of blocks [j0, j0 + 64) inside [x, y), as a bit mask.
  auto range_bits = [](int j0, int x, int y) -> uint64_t {
    const int lo = min(max(x - j0, 0), kWave);
    const int hi = min(max(y - j0, 0), kWave);
    if (hi <= lo) return 0ull;
    const uint64_t upto = hi == kWave ? ~0ull : ((1ull << hi) - 1ull);
    return upto & ~((1ull << lo) - 1ull);
  };
  // Selected candidates among blocks [j0, j0 + 64): the bitmaps are indexed
  // by candidate (block - lo), so each head's two overlapping words are
  // shifted into place.
  auto cand_bits = [&](int j0) -> uint64_t {
    if (nc == 0) return 0ull;
    const int a = j0 - cr.lo;
    const int kw = a >> 6;   // floor
    const int sh = a & 63;
    uint64_t m = 0ull;
#pragma unroll
    for (int x = 0; x < G; ++x) {
      const uint64_t* row = bits + x * nwords;
      const uint64_t w0 = (kw >= 0 && kw < nwords) ? row[kw] : 0ull;
      const uint64_t w1 = (sh != 0 && kw + 1 >= 0 && kw + 1 < nwords) ? row[kw + 1] : 0ull;
      m |= (w0 >> sh) | (sh != 0 ? w1 << (64 - sh) : 0ull);
    }
    return m;
  };
  SplitShare r;
  r.T = T;
  r.ent = 0;
  r.page = -1;
  const int pos = split + lane * S;   // this lane's target position
  const bool want = lane < P.bps;
  const int nch = ceil_div(nb, kWave);
  int done = 0;   // union entries in the chunks before this round
  // Rounds of 64 chunks of 64 blocks; lane c holds chunk c's mask.  Every
  // wavefront computes the whole share itself, so no barrier is needed.
  for (int c0 = 0; c0 < nch; c0 += kWave) {
    const int ncr = min(kWave, nch - c0);
    const int j0 = (c0 + lane) * kWave;
    uint64_t mymask = 0ull;
    if (lane < ncr)
      mymask = (cand_bits(j0) | range_bits(j0, 0, a1) | range_bits(j0, a2, nb)) & range_bits(j0, 0, nb);
    const uint32_t cnt_c = static_cast<uint32_t>(__popcll(mymask));
    const uint32_t incl = wave_scan_incl(cnt_c);
    const int total = __builtin_amdgcn_readlane(static_cast<int>(incl), kWave - 1);
    if constexpr (FULL) {
      // the whole list: wavefront w writes the entries of chunks w, w + NW, ...
      int32_t* uent = reinterpret_cast<int32_t*>(smem + P.sl.ulist);
      int32_t* upg = uent + P.umax;
      const int excl = done + static_cast<int>(incl - cnt_c);
      for (int c = wave; c < ncr; c += NW) {
        const uint64_t m = (static_cast<uint64_t>(static_cast<uint32_t>(
                                __builtin_amdgcn_readlane(static_cast<int>(mymask >> 32), c))) << 32) |
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(mymask), c));
        const int base = __builtin_amdgcn_readlane(excl, c);
        const int at = base + __popcll(m & lanes_below(lane));
        if (((m >> lane) & 1ull) && at < P.umax) {
          const int j = (c0 + c) * kWave + lane;
          uent[at] = j | (head_mask(j) << 20);
          upg[at] = page_of(j);
        }
      }
      done += total;
      continue;
    }
    upre[lane] = done + static_cast<int>(incl - cnt_c);   // wavefront-private copies
    umask[lane] = mymask;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if (want && pos >= done && pos < done + total && pos < P.umax) {
      int c = 0;   // last chunk of the round whose prefix is <= pos
#pragma unroll
      for (int step = 32; step >= 1; step >>= 1)
        if (c + step < ncr && upre[c + step] <= pos) c += step;
      int rnk = pos - upre[c];
      uint64_t m = umask[c];
      int bit = 0;
#pragma unroll
      for (int w = 32; w >= 1; w >>= 1) {   // rank search: the (rnk+1)-th set bit
        const int low = __popcll(m & ((1ull << w) - 1ull));
        if (rnk >= low) {
          rnk -= low;
          m >>= w;
          bit += w;
        }
      }
      const int j = (c0 + c) * kWave + bit;
      r.ent = j | (head_mask(j) << 20);
      r.page = page_of(j);
    }
    done += total;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // reads above before the next round's writes
  }
  r.count = __builtin_amdgcn_readfirstlane(min(done, P.umax));
  if constexpr (FULL) {
    __syncthreads();   // the list is complete
    r.ne = 0;
    return r;
  }
  r.ne = split < r.count ? min(P.bps, ceil_div(r.count - split, S)) : 0;
  if (lane >= r.ne) {
    r.ent = 0;
    r.page = -1;
  }
  if (split == 0 && tid == 0) P.ucount[pair] = r.count;
  return r;
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
__global__ __launch_bounds__(kThreads, 1) void k_attend(DecodeParams P) {
  constexpr int LPT = D / 8;             // lanes per token row
  constexpr int NGRP = kThreads / LPT;   // token groups per workgroup
  constexpr int U = kUnit / NGRP;        // rows per group per unit
  constexpr int NW = kThreads / kWave;
  constexpr int kAll = (1 << G) - 1;
  static_assert(kUnit == kWave, "softmax pass maps one row to one lane");
  __shared__ float s_lds[G][kUnit];
  __shared__ float2 pw_lds[G][kUnit];
  __shared__ bool lin_lds[kUnit];
  __shared__ float scale_lds[G];
  __shared__ float red[NW][G][2 * D];
  __shared__ float mll[G][4];

  const int pair = blockIdx.x / P.max_split;
  const int split = blockIdx.x % P.max_split;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int lig = tid % LPT;
  QReg<KV> qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h].load(reinterpret_cast<const char*>(P.q) +
               ((static_cast<size_t>(b) * P.Hq + g * G + h) * D + lig * 8) * KV::kBytes);
  extern __shared__ uint64_t dyn_lds[];
  const SplitShare share = union_share<G, false, kFusedKplMax, false>(
      P, reinterpret_cast<char*>(dyn_lds), pair, b, g, split, [] {}, [](int, int, auto&&) {});
  const int T = share.T;
  const int Ts = state_tokens(P, T, b);   // tokens the linear state holds
  if (split >= share.count) return;
  const int ne = share.ne;
  const int my_ent = share.ent;
  const int my_page = share.page;
  const int B = P.B;
  const int ns = P.ns;
  const int win0 = T - P.W;
  const int grp = tid / LPT;
  const int upb = BIG ? B / kUnit : 1;   // units per block
  const int epu = BIG ? 1 : kUnit / B;   // blocks per unit
  const int nu = BIG ? ne * upb : ceil_div(ne, epu);

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
        x.k[i].load_nt(kp + base + lane_off[i]);
        x.v[i].load_nt(vp + base + lane_off[i]);
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
        x.k[i].load_nt(kp + off);
        x.v[i].load_nt(vp + off);
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
    // subtraction terms only for tokens the state holds (complete blocks)
    if (lig == 0) {
#pragma unroll
      for (int i = 0; i < U; ++i) lin_lds[grp + NGRP * i] = valid[i] && x.tok[i] < Ts;
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
      const float wv = (inc && lin_lds[lane]) ? 1.f + sv : 0.f;
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
// 3b. Split-K exact attention for bf16 keys/values on the matrix cores
// ---------------------------------------------------------------------------
// Per union token the exact part costs G dot products of length D and 2G
// multiply-adds per channel (p v for the softmax, (1 + s) v for the linear
// sums that are subtracted from the global state): about 3 fp32 MACs per
// byte of K/V at G = 4, more than the vector ALUs sustain at HBM rate.  The
// two contractions run on MFMA instead:
//   scores  S[h][t]  = sum_c Q[h][c] K[t][c]       v_mfma_f32_16x16x32_bf16,
//           rows = query heads (G of 16 used), columns = 16 tokens;
//   values  O[r][c] += sum_t A[r][t] V[t][c]       v_mfma_f32_16x16x16_bf16,
//           rows r = (p_hi, p_lo, w_hi, w_lo) x G heads, columns = channels.
// p = exp(s - m) and w = 1 + s are fp32; each is split into a bf16 pair
// hi + lo (hi = bf16(x), lo = bf16(x - hi)) that carries ~16 mantissa bits,
// so the products match the fp32 vector path to ~2^-17 relative while keys,
// values and queries enter exactly (they are bf16 already).
//
// Work: the union blocks are cut into slices of 16 rows of one page.  With
// the fixed split (DYN false) wavefront w of the workgroup takes slices w,
// w + 4, ... of its split; with the dynamic split the wavefronts of all the
// pair's workgroups claim units of four slices from the pair's counter.
// Each wavefront keeps its own running maximum per head, so the slice loop
// has no workgroup barrier; the four wavefronts are combined once at the
// end.
// Lane l = 16 q + n: in the score MFMA it carries token n (channels
// q D/4 .. q D/4 + D/4 of its K row); in the value MFMA it carries tokens
// 4q .. 4q + 3 of the slice at channels (D/16) n .. (D/16) n + D/16, and its
// value tile t column n is channel (D/16) n + t.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  return fmaxf(v, dpp_f<0x140>(v));
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(f)));
}

template <int NT>
struct VSlice;
template <>
struct VSlice<8> {   // D = 128: 8 channels of a row per lane
  u32x4 r;
  __device__ __forceinline__ void load(const char* p) { r = ld_global_nt<u32x4>(p); }
  __device__ __forceinline__ void load_cached(const char* p) { r = ld_global<u32x4>(p); }
  __device__ __forceinline__ void clear() { r = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ uint32_t word(int i) const { return r[i]; }
};
template <>
struct VSlice<4> {   // D = 64: 4 channels of a row per lane
  u32x2 r;
  __device__ __forceinline__ void load(const char* p) { r = ld_global_nt<u32x2>(p); }
  __device__ __forceinline__ void load_cached(const char* p) { r = ld_global<u32x2>(p); }
  __device__ __forceinline__ void clear() { r = u32x2{0u, 0u}; }
  __device__ __forceinline__ uint32_t word(int i) const { return r[i]; }
};


// The merge of one pair's nsplit split partials and its residual linear part
// (SPLA Abstract: global state minus the exact tokens' share), done by the
// pair's last attention workgroup: thread entries (head, channel) walk the
// splits with a running maximum, kMergeBatch splits' loads issued together.
// Everything another workgroup of the launch wrote -- split partials,
// readout partials, and in the one-launch step the folded sv -- is read
// with agent-scope loads.
constexpr int kMergeBatch = 4;
template <int D, int G>
__device__ __forceinline__ void merge_pair(const DecodeParams& P, int pair, int b, int g, int nsplit, int T) {
  constexpr int RO = D / kRoRows;
  const float* pb = P.part + static_cast<size_t>(pair) * P.max_split * G * P.pstride;
  const CandRange cr = candidate_range(T, P.B, P.ns, P.W);
  const bool tail = P.linear_tail && P.top_k < min(cr.count, P.nc_max);
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int hh = idx / D;
    const int c = idx % D;
    float ro = 0.f, rz = 0.f, svc = 0.f;
    if (tail) {
#pragma unroll
      for (int rc = 0; rc < RO; ++rc) {
        ro += load_agent(P.ro + ((static_cast<size_t>(pair) * RO + rc) * G + hh) * D + c);
        rz += load_agent(P.roz + (static_cast<size_t>(pair) * RO + rc) * G + hh);
      }
      svc = load_agent(P.sv + static_cast<size_t>(state_pair(P, pair)) * D + c);
    }
    float M = 0.f;   // the linear part is in unshifted units (log-scale 0)
    float num = 0.f, den = 0.f, lnum = 0.f, lden = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += kMergeBatch) {
      float ms[kMergeBatch], ls[kMergeBatch], lw[kMergeBatch], a[kMergeBatch], la[kMergeBatch];
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        const float* ps = pb + (static_cast<size_t>(min(s0 + i, nsplit - 1)) * G + hh) * P.pstride;
        ms[i] = load_agent(ps);
        ls[i] = load_agent(ps + 1);
        lw[i] = load_agent(ps + 2);
        a[i] = load_agent(ps + 4 + c);
        la[i] = load_agent(ps + 4 + D + c);
      }
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        if (s0 + i >= nsplit) break;
        lnum += la[i];
        lden += lw[i];
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
    if (tail) {
      const float num_u = svc + P.sigma * ro - lnum;
      const float den_u = static_cast<float>(state_tokens(P, T, b)) + P.sigma * rz - lden;   // n: tokens the state holds
      const float em = __expf(-M);
      num = fmaf(em, num_u, num);
      den = fmaf(em, den_u, den);
    }
    P.out[(static_cast<size_t>(b) * P.Hq + g * G + hh) * D + c] = num / den;
  }
}

// NTL: the K/V loads are non-temporal (decode: each page is read once per
// step); the multi-query form, whose query rows of one sequence re-read the
// same pages from L2, loads them normally.
template <int D, int G, bool DYN, int FK, bool GS, bool NTL = true>
__global__ __launch_bounds__(kThreads, 2) void k_attend_mfma(DecodeParams P) {
  constexpr int NW = kThreads / kWave;
  constexpr int KS = D / 32;            // score MFMAs per slice (32 channels each)
  constexpr int NT = D / 16;            // value tiles (16 channels each)
  constexpr int MT = G <= 4 ? 1 : 2;    // value M-tiles of 16 rows
  constexpr int R = 4 * G;              // value rows used: p_hi, p_lo, w_hi, w_lo per head
  constexpr int kAll = (1 << G) - 1;
  constexpr int SL = 16;                // rows per slice
  __shared__ float red[NW][2][G][D];    // per-wavefront sums of p v and w v
  __shared__ float wst[NW][G][3];       // per-wavefront m, sum p, sum w
  __shared__ uint4 q_lds[16][D / 8 + 1];

  HSLA_STAMP(0);
#ifdef HSLA_PHASE_TIMESTAMPS
  struct ExitStamp { __device__ ~ExitStamp() { HSLA_STAMP(12); } } exit_stamp;
#endif
  const int pair = blockIdx.x / P.max_split;
  const int split = blockIdx.x % P.max_split;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);   // uniform: keeps the loop scalar
  const int lane = tid % kWave;
  const int q4 = lane / 16;
  const int n16 = lane % 16;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int B = P.B;
  const int ns = P.ns;
  const int spb = B / SL;               // slices per block

  // Query operand rows (heads; rows G..15 zero) staged in LDS, 16 bytes of
  // padding per row so that the 16 rows fall on distinct banks.  Loaded
  // first, in the same round trip as the split's union data; union_share
  // stores them and its barrier publishes q_lds.
  static_assert(16 * (D / 8) <= kThreads, "one query chunk per thread");
  const int q_row = tid / (D / 8);
  const int q_col = tid % (D / 8);
  uint4 qv = make_uint4(0, 0, 0, 0);
  if (q_row < G)
    qv = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(P.q) +
                                         (static_cast<size_t>(b) * P.Hq + g * G + q_row) * D + q_col * 8);
  auto stage_q = [&] {
    if (q_row < 16) q_lds[q_row][q_col] = qv;
  };
  const char* kp = reinterpret_cast<const char*>(P.k_pages);
  const char* vp = reinterpret_cast<const char*>(P.v_pages);
  const size_t k_lane = (static_cast<size_t>(n16) * D + 8 * q4) * 2;
  const size_t v_lane = (static_cast<size_t>(4 * q4) * D + NT * n16) * 2;

  struct Slice {
    u32x4 k[KS];
    VSlice<NT> v[4];
    int t0;   // first token (uniform); kDeadT0 for a slice without a page (no row valid)
    int fm;   // heads that selected the block (uniform)
  };
  // Slice `sub` of union entry (ent, page pg); a dead slice re-reads a live
  // one (an L2 hit) and marks every row invalid.
  auto load_slice = [&](int ent, int pg, int sub, bool live, Slice& x) __attribute__((always_inline)) {
    const size_t base = ((static_cast<size_t>(max(pg, 0)) * P.Hkv + g) * B + sub * SL) * D * 2;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      x.k[s] = NTL ? ld_global_nt<u32x4>(kp + base + k_lane + 64 * s) : ld_global<u32x4>(kp + base + k_lane + 64 * s);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (NTL) x.v[j].load(vp + base + v_lane + static_cast<size_t>(j) * D * 2);
      else x.v[j].load_cached(vp + base + v_lane + static_cast<size_t>(j) * D * 2);
    }
    x.t0 = (live && pg >= 0) ? (ent & 0xFFFFF) * B + sub * SL : kDeadT0;
    x.fm = (ent >> 20) & kAll;
    // keep the loads ahead of the previous slice's arithmetic
    __builtin_amdgcn_sched_barrier(0);
  };
  // Dynamic split: this wavefront's slices of the window blocks, loaded
  // before the selection: slices r = split * NW + wave + m S NW (m < kPre)
  // of the window region, so that its first npre slices are taken this way.
  // One per wavefront measured faster than two or three: more window
  // traffic in flight delays the selection's own loads.
  constexpr int kPre = 1;
  Slice pre[kPre];
  int npre = 0, nwin_sl = 0;
  auto early = [&](int jw0, int nbk, auto&& page_of) __attribute__((always_inline)) {
    nwin_sl = (nbk - jw0) * spb;
    const int span = P.max_split * NW;
    npre = min(kPre * span, nwin_sl);
#pragma unroll
    for (int m = 0; m < kPre; ++m) {
      const int r = split * NW + wave + m * span;
      const bool live = DYN && r < npre;
      const int j = jw0 + (live ? r : 0) / spb;
      const int sub = (live ? r : 0) % spb;
      load_slice(j, live ? page_of(j) : 0, sub, live, pre[m]);
    }
  };
  extern __shared__ uint64_t dyn_lds[];
  const SplitShare share =
      union_share<G, DYN, FK, GS>(P, reinterpret_cast<char*>(dyn_lds), pair, b, g, split, stage_q, early);
  HSLA_STAMP(6);
  const int T = share.T;
  const int Ts = state_tokens(P, T, b);           // tokens the linear state holds
  const int win0 = T - P.W;
  if (!DYN && split >= share.count) return;
  const int ne = share.ne;
  const int my_ent = share.ent;
  const int my_page = share.page;
  const int nsl = ne * spb;             // slices of the split
  const int nk = nsl > wave ? ceil_div(nsl - wave, NW) : 0;   // slices of this wavefront

  f32x4_t acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[mt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // Lane (q4, n16) scores column n16, i.e. head hl, and builds value-operand
  // rows 16 mt + n16, which belong to the same head: its scores never leave
  // the lane.  m_ref is the head's reference maximum: exponentials are taken
  // against it, and it moves (with a rescale of the sums) only when a score
  // exceeds it by more than kLazyMax, so p = e^(s - m_ref) <= e^kLazyMax.
  const int hl = n16 % G;
  constexpr float kLazyMax = 8.f;
  float m_ref = kNegInf;
  float l_acc[MT];                       // sum of this lane's value-operand row (fp32)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) l_acc[mt] = 0.f;

  // Static split: slice kk of this wavefront is slice wave + NW kk of the
  // split, whose entries lane e holds.
  auto fetch = [&](int kk, Slice& x) __attribute__((always_inline)) {
    const bool live = kk < nk;
    const int sl = wave + NW * (live ? kk : max(nk - 1, 0));
    const int e = sl / spb;
    const int sub = sl - e * spb;
    load_slice(__builtin_amdgcn_readlane(my_ent, e), __builtin_amdgcn_readlane(my_page, e), sub, live, x);
  };

  // Every fetched slice of the loop is processed, without a branch around
  // it, so that no load stays in flight across the loop back edge.
  auto process = [&](Slice& x) __attribute__((always_inline)) {
    // ---- scores, transposed: row 4 q4 + i is token t0 + 4 q4 + i, column
    // n16 is head hl (the K operand rows are tokens; channels 32 s + 8 q4
    // .. + 8 of both operands)
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x.k[s]),
                                                   __builtin_bit_cast(bf16x8_t, q_lds[hl][4 * s + q4]), sc, 0, 0, 0);
    const int tb = x.t0 + 4 * q4;       // the lane's first token
    const bool sel = (x.fm >> hl) & 1;
    float sv[4];
    bool over = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = tb + j;
      const bool inc = t < T && (sel || t < ns || t >= win0);
      sv[j] = inc ? P.sigma * sc[j] : kNegInf;
      over |= sv[j] > m_ref + kLazyMax;
    }
    // ---- a reference moves (uniform branch, rare after the first slices):
    // the head's new maximum over the slice's 16 tokens (lanes n16 + 16 q4),
    // then the p rows of the sums are rescaled
    if (__builtin_amdgcn_ballot_w64(over) != 0) {
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      float a, c;
      lane_pair<16>(mx, a, c);
      mx = fmaxf(a, c);
      lane_pair<32>(mx, a, c);
      mx = fmaxf(a, c);
      const float mnew = fmaxf(m_ref, mx);
      const float cf = mnew == m_ref ? 1.f : fast_exp(m_ref - mnew);   // m_ref = -inf: 0
      m_ref = mnew;
      float cfh[G];   // head h's factor sits in lane h
#pragma unroll
      for (int h = 0; h < G; ++h) cfh[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cf), h));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mt + 4 * q4 + i;   // acc row: type r / G, head r % G
          float f = 1.f;
#pragma unroll
          for (int h = 0; h < G; ++h) f = (r < 2 * G && r % G == h) ? cfh[h] : f;
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) acc[mt][tt][i] *= f;
        }
        if ((16 * mt + n16) < 2 * G) l_acc[mt] *= cf;   // the lane's own p row
      }
    }
    // ---- value operand rows: lane (q4, n16) builds row r = 16 mt + n16
    // (type r / G: 0 p_hi, 1 p_lo, 2 w_hi, 3 w_lo, >= 4 unused) for tokens
    // tb .. tb + 3
    float pv[4], wv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool inc = sv[j] != kNegInf;
      pv[j] = inc ? fast_exp(sv[j] - m_ref) : 0.f;
      // subtraction terms only for tokens the state holds (complete blocks)
      wv[j] = (inc && tb + j < Ts) ? 1.f + sv[j] : 0.f;
    }
    s16x4_t av[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int typ = (16 * mt + n16) / G;
      uint32_t bits[4];
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float val = typ < 2 ? pv[j] : wv[j];
        val = typ < 4 ? val : 0.f;
        rs += val;
        const uint32_t hi = bf16_bits_rne(val);
        const uint32_t lo = bf16_bits_rne(val - __uint_as_float(hi << 16));
        bits[j] = (typ & 1) ? lo : hi;
      }
      l_acc[mt] += rs;
      av[mt] = __builtin_bit_cast(s16x4_t, make_uint2(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16)));
    }
    // ---- values: tile t takes channel t of each lane's V rows; rows past
    // the end of the sequence may hold anything and enter as zero (uniform
    // branch: only a sequence's last slice, or a dead one, has such rows)
    if (x.t0 + SL > T) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (tb + j >= T) x.v[j].clear();
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const uint32_t selw = (tt & 1) ? 0x07060302u : 0x05040100u;
      uint32_t vw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) vw[j] = x.v[j].word(tt / 2);
      const uint32_t lo = __builtin_amdgcn_perm(vw[1], vw[0], selw);
      const uint32_t hi = __builtin_amdgcn_perm(vw[3], vw[2], selw);
      const s16x4_t bv = __builtin_bit_cast(s16x4_t, make_uint2(lo, hi));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt][tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[mt], bv, acc[mt][tt], 0, 0, 0);
    }
  };

  // The next slice is in flight while one is processed.  Two (16 KB per
  // wavefront) measured faster than three or four: deeper queues only
  // lengthen the memory latency that the prologue loads and the last slices
  // wait through.
  Slice sa, sb;
  if constexpr (DYN) {
    // The pair's slices, in units of kUnitSlices, go to whichever wavefront
    // of the pair's workgroups claims them next (a device-scope counter per
    // pair, zeroed by the selection kernel), so that workgroups on a slower
    // XCD take fewer.  A wavefront claims its next unit when it starts one
    // and reads the claim when it prefetches that unit's first slice, three
    // slices later: the atomic's latency stays hidden, and no wavefront holds
    // more than the unit it is working on.
    const int32_t* uent = reinterpret_cast<const int32_t*>(reinterpret_cast<const char*>(dyn_lds) + P.sl.ulist);
    const int32_t* upg = uent + P.umax;
    const int total = share.count * spb;
    // the window region is the list's tail; its first npre slices were
    // prefetched, the rest of the list is claimed
    const int w0 = total - nwin_sl;
    const int nclaim = total - npre;
    const int nunits = ceil_div(nclaim, kUnitSlices);
    int32_t* ctr = P.ctr + static_cast<size_t>(pair) * kCtrStride;
    auto claim = [&]() -> int {   // the claimed unit, in lane 0
      int v = 0;
      if (lane == 0) v = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return v;
    };
    auto fetch_u = [&](int u, int i, Slice& x) __attribute__((always_inline)) {
      const int qc = u * kUnitSlices + i;
      const bool live = u >= 0 && u < nunits && qc < nclaim;
      const int q = qc < w0 ? qc : qc + npre;
      const int e = (live ? q : 0) / spb;
      const int sub = (live ? q : 0) - e * spb;
      load_slice(__builtin_amdgcn_readfirstlane(uent[e]), __builtin_amdgcn_readfirstlane(upg[e]), sub, live, x);
    };
    static_assert(kUnitSlices == 4, "the loop body processes four slices");
    int ua = __builtin_amdgcn_readfirstlane(claim());
    fetch_u(ua, 0, sb);
#pragma unroll
    for (int m = 0; m < kPre; ++m)   // the prefetched window slices (masked if none)
      if (m == 0 || pre[m].t0 != kDeadT0) process(pre[m]);
    while (ua < nunits) {
      const int cn = claim();
      fetch_u(ua, 1, sa);
      process(sb);
      fetch_u(ua, 2, sb);
      process(sa);
      fetch_u(ua, 3, sa);
      process(sb);
      ua = __builtin_amdgcn_readfirstlane(cn);
      fetch_u(ua, 0, sb);
      process(sa);
    }
  } else {
    // Static split.  The loop has a single exit: an odd count ends with a
    // fully masked slice.
    fetch(0, sa);
    for (int kk = 0; kk < nk; kk += 2) {
      fetch(kk + 1, sb);
      process(sa);
      fetch(kk + 2, sa);
      process(sb);
    }
  }

  HSLA_STAMP_WAVE(7);
  // ---- per-wavefront sums: hi + lo rows, then p v / w v per head to LDS
  // Row r of value tile (mt, t) sits in lane group q4 = (r % 16) / 4, entry
  // r % 4, column n16 = channel NT n16 + t.
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int c = NT * n16 + tt;
    if constexpr (G == 1) {
      if (q4 == 0) {
        red[wave][0][0][c] = acc[0][tt][0] + acc[0][tt][1];
        red[wave][1][0][c] = acc[0][tt][2] + acc[0][tt][3];
      }
    } else if constexpr (G == 2) {
      if (q4 < 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) red[wave][q4][h][c] = acc[0][tt][h] + acc[0][tt][h + 2];
      }
    } else if constexpr (G == 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = pair_sum<16>(acc[0][tt][i]);   // hi row + lo row
        if (q4 == 0 || q4 == 2) red[wave][q4 / 2][i][c] = v;
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = pair_sum<32>(acc[mt][tt][i]);
          if (q4 < 2) red[wave][mt][4 * q4 + i][c] = v;
        }
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const float v = pair_sum<32>(pair_sum<16>(l_acc[mt]));   // over the four token groups
    const int r = 16 * mt + n16;
    if (q4 == 0 && r < R) {
      const int typ = r / G;
      if (typ == 0) wst[wave][r % G][1] = v;
      if (typ == 2) wst[wave][r % G][2] = v;
    }
  }
  if (lane < G) wst[wave][lane][0] = m_ref;   // lane h < G scores head h
  __syncthreads();

  float* outp = P.part + (static_cast<size_t>(pair) * P.max_split + split) * G * P.pstride;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int c = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wst[w][h][0]);
    float a = 0.f, la = 0.f, l = 0.f, ld = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = wst[w][h][0];
      const float e = mw == kNegInf ? 0.f : fast_exp(mw - M);
      a = fmaf(e, red[w][0][h][c], a);
      l = fmaf(e, wst[w][h][1], l);
      la += red[w][1][h][c];
      ld += wst[w][h][2];
    }
    float* o = outp + static_cast<size_t>(h) * P.pstride;
    if (P.fused_merge) {
      store_agent(o + 4 + c, a);
      store_agent(o + 4 + D + c, la);
      if (c == 0) {
        store_agent(o, M);
        store_agent(o + 1, l);
        store_agent(o + 2, ld);
      }
    } else {
      o[4 + c] = a;
      o[4 + D + c] = la;
      if (c == 0) {
        o[0] = M;
        o[1] = l;
        o[2] = ld;
        o[3] = 0.f;
      }
    }
  }
  HSLA_STAMP(11);
  if (P.fused_merge) {
    // The pair's last workgroup to finish merges: every thread's partial
    // stores complete first, then one thread counts the workgroup done.
    __shared__ int is_last;
    stores_complete();
    __syncthreads();
    const int writers = DYN ? P.max_split : min(share.count, P.max_split);
    int32_t* done = P.ctr + static_cast<size_t>(pair) * kCtrStride + kDoneSlot;
    if (tid == 0)
      is_last = __hip_atomic_fetch_add(done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == writers - 1;
    __syncthreads();
    if (is_last) {
      // the reader's side of the hand-off: drop any non-coherent cached
      // copy before the partial loads (an invalidate, no L2 writeback)
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      merge_pair<D, G>(P, pair, b, g, writers, T);
    }
  }
}

// ---------------------------------------------------------------------------
// 4. Merge of the splits and the residual linear part
// ---------------------------------------------------------------------------
// One workgroup per (sequence, query head); NP = 256 / D lanes share a
// channel and walk the splits with a running maximum, then combine.  Every
// load of the usual case -- the first NP * NPC splits' partials, the readout
// partials, sv, the union size and the sequence length -- goes out in one
// round trip: partials of splits past the union size are loaded and ignored.
// NPC (splits per lane loaded together) is the launch's splits per lane,
// rounded up to 2, 4, 8 or 16, so that up to 16 NP splits take one round
// trip and few splits issue no surplus loads.
template <int D, int G, int NPC>
__global__ __launch_bounds__(kThreads) void k_merge(DecodeParams P) {
  constexpr int NP = kThreads / D;
  constexpr int RO = D / kRoRows;   // readout partials per head
  __shared__ float part_m[NP][D], part_num[NP][D], part_den[NP][D], part_lnum[NP][D], part_lden[NP][D];
#ifdef HSLA_PHASE_TIMESTAMPS
  const PhaseSpan span(g_phase_merge, kPhaseMergeWgs, blockIdx.x);
#endif
  const int bh = blockIdx.x;
  const int b = bh / P.Hq;
  const int h = bh % P.Hq;
  const int g = h / G;
  const int hh = h % G;
  const int pair = b * P.Hkv + g;
  const int tid = threadIdx.x;
  const int c = tid % D;
  const int pp = tid / D;
  const size_t sstride = static_cast<size_t>(G) * P.pstride;
  const float* pb = P.part + (static_cast<size_t>(pair) * P.max_split * G + hh) * P.pstride;

  float ms[NPC], ls[NPC], lds[NPC], a[NPC], la[NPC];
  auto load_chunk = [&](int s0, int bound) {
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const float* ps = pb + min(s0 + i * NP, bound - 1) * sstride;
      ms[i] = ps[0];
      ls[i] = ps[1];
      lds[i] = ps[2];
      a[i] = ps[4 + c];
      la[i] = ps[4 + D + c];
    }
  };
  load_chunk(pp, P.max_split);
  float ro_p[RO], rz_p[RO], svc = 0.f;
  if (P.linear_tail) {
#pragma unroll
    for (int rc = 0; rc < RO; ++rc) {
      ro_p[rc] = P.ro[((static_cast<size_t>(pair) * RO + rc) * G + hh) * D + c];
      rz_p[rc] = P.roz[(static_cast<size_t>(pair) * RO + rc) * G + hh];
    }
    svc = P.sv[static_cast<size_t>(state_pair(P, pair)) * D + c];
  }
  const int count = min(P.ucount[pair], P.umax);
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  // static: split s holds entries s, s + max_split, ...; dynamic: every
  // workgroup of the pair wrote a partial (possibly empty)
  const int nsplit = P.dyn ? P.max_split : min(count, P.max_split);

  float M = 0.f;   // the linear part is in unshifted units (log-scale 0)
  float num = 0.f, den = 0.f, lnum = 0.f, lden = 0.f;
  for (int s0 = pp; s0 < nsplit; s0 += NP * NPC) {
    if (s0 != pp) load_chunk(s0, nsplit);
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
  const CandRange cr = candidate_range(T, P.bsel, P.ns, P.W);
  if (P.linear_tail && P.top_k < min(cr.count, P.nc_max)) {
    float ro = 0.f, rz = 0.f;
#pragma unroll
    for (int rc = 0; rc < RO; ++rc) {
      ro += ro_p[rc];
      rz += rz_p[rc];
    }
    const float num_u = svc + P.sigma * ro - lnum;
    const float den_u = static_cast<float>(state_tokens(P, T, b)) + P.sigma * rz - lden;   // n: tokens the state holds
    const float em = __expf(-M);
    num = fmaf(em, num_u, num);
    den = fmaf(em, den_u, den);
  }
  P.out[(static_cast<size_t>(b) * P.Hq + h) * D + c] = num / den;
}

// ---------------------------------------------------------------------------
// Token-level variant: per-head top-k over the candidate tokens
// ---------------------------------------------------------------------------
// One workgroup of 1024 threads per (sequence, query head).  Rows hold tens
// of thousands of keys, so the whole workgroup runs the radix select: three passes over
// 11-, 11- and 10-bit digits, each streaming the row (16 keys per thread in
// flight) into a 2048-bin LDS histogram of the keys that match the digits
// found so far, and a suffix scan picks the digit that holds the k-th
// largest key.  Then each
// wavefront takes a sixteenth of the row's 64-key words: it counts its keys
// above and equal to the threshold, the counts are exchanged, and a second
// walk writes the bitmap words and the ascending indices (keys equal to the
// threshold are taken lowest index first).
template <int NT>
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t v, uint32_t* wtot) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const uint32_t incl = wave_scan_incl(v);
  if (lane == kWave - 1) wtot[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) before += w < wave ? wtot[w] : 0u;
  __syncthreads();
  return incl + before;
}

constexpr int kSelThreads = 1024;   // token-level selection: threads per head
constexpr size_t kSelCacheBytes = 128 * 1024;   // token rows up to this size stay in LDS
constexpr int kUnionThreads = 1024; // token-level exact lists: threads per (sequence, kv head)

template <bool CACHE>
__global__ __launch_bounds__(kSelThreads) void k_select_tokens(DecodeParams P) {
  extern __shared__ uint32_t krow[];   // CACHE: the row's keys, filled by the first pass
  constexpr int NT = kSelThreads;
  constexpr int NW = NT / kWave;
  constexpr int UK = 16;            // keys in flight per thread
  constexpr int NB = 2048;          // histogram bins (11-bit digits)
  constexpr int BPT = NB / NT;      // bins per thread
  __shared__ uint32_t hist[NB];
  __shared__ uint32_t wtot[NW];
  __shared__ int pick[2];
  __shared__ int wcnt[NW][2];
  const int bh = blockIdx.x;
  const int b = bh / P.Hq;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const uint32_t* kh = P.keys + static_cast<size_t>(bh) * P.sstride;
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const CandRange cr = candidate_range(T, 1, P.ns, P.W);
  const int nc = min(cr.count, P.nc_max);
  const int k = P.top_k;
  const int nw = ceil_div(nc, kWave);
  uint64_t* bits_row = P.bits + static_cast<size_t>(bh) * P.nwords;
  int32_t* out = P.sel_idx ? P.sel_idx + static_cast<size_t>(bh) * k : nullptr;
  const bool take_all = k >= nc;
  const bool take_none = k <= 0 || nc == 0;
  const bool cached = CACHE && !take_all && !take_none;   // the radix passes fill krow

  uint32_t thr = 0u;
  int rem = k;   // keys equal to thr still to take, lowest indices first
  if (!take_all && !take_none) {
    uint32_t prefix = 0u, pmask = 0u;
    // digits: bits 21..31, 10..20, 0..9
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
      const uint32_t dmask = pass == 2 ? 1023u : 2047u;
#pragma unroll
      for (int j = 0; j < BPT; ++j) hist[tid * BPT + j] = 0u;
      __syncthreads();
      for (int i0 = 0; i0 < nc; i0 += NT * UK) {
        uint32_t x[UK];
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          const int i = min(i0 + u * NT + tid, nc - 1);
          x[u] = (CACHE && pass > 0) ? krow[i] : kh[i];
        }
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          if (i0 + u * NT + tid < nc) {
            if (CACHE && pass == 0) krow[i0 + u * NT + tid] = x[u];
            if ((x[u] & pmask) == prefix) atomicAdd(&hist[(x[u] >> shift) & dmask], 1u);
          }
        }
      }
      __syncthreads();
      // thread tid holds the BPT bins counted from the top: digits
      // NB-1 - (tid*BPT + j)
      uint32_t cb[BPT];
      uint32_t mine = 0u;
#pragma unroll
      for (int j = 0; j < BPT; ++j) {
        cb[j] = hist[NB - 1 - (tid * BPT + j)];
        mine += cb[j];
      }
      const uint32_t incl = block_scan_incl<NT>(mine, wtot);   // keys whose digit >= the thread's lowest
      uint32_t above = incl - mine;
      if (above < static_cast<uint32_t>(rem) && static_cast<uint32_t>(rem) <= incl) {
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
          if (above < static_cast<uint32_t>(rem) && static_cast<uint32_t>(rem) <= above + cb[j]) {
            pick[0] = NB - 1 - (tid * BPT + j);
            pick[1] = rem - static_cast<int>(above);
          }
          above += cb[j];
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(pick[0]) << shift;
      pmask |= dmask << shift;
      rem = pick[1];
      __syncthreads();
    }
    thr = prefix;
  }

  // an equal share of the words per wavefront, UK words in flight
  const int wpw = ceil_div(nw, NW);
  const int wb = min(wave * wpw, nw);
  const int we = min(wb + wpw, nw);
  auto masks = [&](int w, uint32_t x, uint64_t& gt, uint64_t& eq, uint64_t& valid) __attribute__((always_inline)) {
    const bool v = w * kWave + lane < nc;
    valid = __ballot(v);
    gt = __ballot(v && x > thr);
    eq = __ballot(v && x == thr);
  };
  int n_eq = 0, n_gt = 0;
  for (int w0 = wb; w0 < we; w0 += UK) {
    uint32_t x[UK];
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int i = min((w0 + u) * kWave + lane, max(nc - 1, 0));
      x[u] = cached ? krow[i] : kh[i];
    }
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      if (w0 + u >= we) break;
      uint64_t gt, eq, valid;
      masks(w0 + u, x[u], gt, eq, valid);
      n_eq += __popcll(eq);
      n_gt += __popcll(gt);
    }
  }
  if (lane == 0) {
    wcnt[wave][0] = n_eq;
    wcnt[wave][1] = n_gt;
  }
  __syncthreads();
  int eq_before = 0, pos = 0, total = 0, eq_acc = 0;
  for (int w = 0; w < NW; ++w) {   // keys each wavefront selects, in index order
    const int e = wcnt[w][0];
    const int taken = take_all ? e + wcnt[w][1] : take_none ? 0 : wcnt[w][1] + min(max(rem - eq_acc, 0), e);
    if (w < wave) {
      pos += taken;
      eq_before += e;
    }
    total += taken;
    eq_acc += e;
  }
  for (int w0 = wb; w0 < we; w0 += UK) {
    uint32_t x[UK];
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int i = min((w0 + u) * kWave + lane, max(nc - 1, 0));
      x[u] = cached ? krow[i] : kh[i];
    }
#pragma unroll
    for (int u = 0; u < UK; ++u) {
      const int w = w0 + u;
      if (w >= we) break;
      uint64_t gt, eq, valid;
      masks(w, x[u], gt, eq, valid);
      uint64_t sm;
      if (take_none) {
        sm = 0ull;
      } else if (take_all) {
        sm = valid;
      } else {
        // equal keys of this word whose rank among all equal keys is < rem
        uint64_t keep = 0ull, e = eq;
        int r = eq_before;
        while (e && r < rem) {
          const uint64_t low = e & (~e + 1ull);
          keep |= low;
          e ^= low;
          ++r;
        }
        eq_before += __popcll(eq);
        sm = gt | keep;
      }
      if (lane == 0) bits_row[w] = sm;
      const bool sel = (sm >> lane) & 1ull;
      const int at = pos + __popcll(sm & lanes_below(lane));
      if (sel && out && at < k) out[at] = cr.lo + w * kWave + lane;
      pos += __popcll(sm);
    }
  }
  if (out)   // padding after the selection
    for (int j = total + tid; j < k; j += NT) out[j] = -1;
}

// ---------------------------------------------------------------------------
// Token-level variant: exact token list and attention over it
// ---------------------------------------------------------------------------
// One workgroup per (sequence, kv head) lists the pair's exact tokens in
// ascending order: the sinks and the window for every head, and between them
// every candidate token some head selected, with the mask of the heads that
// selected it and the token's page (token | heads << 20, page), so that the
// attention kernel reaches the rows in one round trip.  Each thread takes a contiguous run of
// bitmap words; a workgroup scan of their counts places the runs.
template <int G>
__global__ __launch_bounds__(kUnionThreads) void k_token_union(DecodeParams P) {
  constexpr int NT = kUnionThreads;
  __shared__ int wave_total[NT / kWave];
  const int pair = blockIdx.x;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const CandRange cr = candidate_range(T, 1, P.ns, P.W);
  const int nc = min(cr.count, P.nc_max);
  const int nw = ceil_div(nc, kWave);
  const int nsink = min(P.ns, T);
  const int w0 = max(T - P.W, nsink);   // first window token that is not a sink
  constexpr int kAll = (1 << G) - 1;
  int2* list = reinterpret_cast<int2*>(P.tlist) + static_cast<size_t>(pair) * P.umax;
  const int32_t* bt = P.block_table + static_cast<size_t>(seq_of(P, b)) * P.max_blocks;
  const uint64_t* bits = P.bits + (static_cast<size_t>(b) * P.Hq + g * G) * P.nwords;

  const int wpt = ceil_div(nw, NT);   // bitmap words per thread
  const int wb = min(tid * wpt, nw);
  const int we = min(wb + wpt, nw);
  int mine = 0;
  for (int w = wb; w < we; ++w) {
    uint64_t any = 0ull;
#pragma unroll
    for (int h = 0; h < G; ++h) any |= bits[static_cast<size_t>(h) * P.nwords + w];
    mine += __popcll(any);
  }
  const uint32_t incl = wave_scan_incl(static_cast<uint32_t>(mine));
  if (lane == kWave - 1) wave_total[wave] = static_cast<int>(incl);
  __syncthreads();
  int before = static_cast<int>(incl) - mine;
  int total = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    before += w < wave ? wave_total[w] : 0;
    total += wave_total[w];
  }
  int at = nsink + before;
  for (int w = wb; w < we; ++w) {
    uint64_t hb[G];
    uint64_t any = 0ull;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      hb[h] = bits[static_cast<size_t>(h) * P.nwords + w];
      any |= hb[h];
    }
    // the word's 64 tokens span at most 64 / B + 1 <= 5 blocks: their pages
    // are read together, before the entries are written
    const int blk0 = (cr.lo + w * kWave) / P.B;
    const int blk1 = (cr.lo + min(w * kWave + kWave, nc) - 1) / P.B;   // the word's last candidate
    int pg[5];
#pragma unroll
    for (int q = 0; q < 5; ++q) pg[q] = bt[min(blk0 + q, blk1)];
    while (any) {
      const int j = __ffsll(static_cast<unsigned long long>(any)) - 1;
      any &= any - 1ull;
      int heads = 0;
#pragma unroll
      for (int h = 0; h < G; ++h) heads |= static_cast<int>((hb[h] >> j) & 1ull) << h;
      const int t = cr.lo + w * kWave + j;
      const int q = t / P.B - blk0;
      const int page = q == 0 ? pg[0] : q == 1 ? pg[1] : q == 2 ? pg[2] : q == 3 ? pg[3] : pg[4];
      list[at++] = make_int2(t | (heads << 20), page);
    }
  }
  for (int i = tid; i < nsink; i += NT) list[i] = make_int2(i | (kAll << 20), bt[i / P.B]);
  const int nwin = T - w0;
  for (int i = tid; i < nwin; i += NT)
    list[nsink + total + i] = make_int2((w0 + i) | (kAll << 20), bt[(w0 + i) / P.B]);
  if (tid == 0) P.ucount[pair] = nsink + total + nwin;
}

// Split-K exact attention over a pair's token list (token-level variant):
// split s takes a contiguous run of the list.  D/8 lanes share a token (8
// channels of its key and value row each, gathered through the block
// table); a wavefront takes 64 / (D/8) tokens at a time, U deep, and every
// token group keeps its own running maximum, sums and first-order sums per
// head.  The groups are combined inside the wavefront (lane swaps), the
// wavefronts through LDS, and the split's partial is written in the layout
// the merge reads.  Subtraction sums take only the tokens the state holds
// (complete blocks).
template <typename KV, int D, int G>
__global__ __launch_bounds__(kThreads) void k_token_attend(DecodeParams P) {
  constexpr int LPT = D / 8;            // lanes per token
  constexpr int TPW = kWave / LPT;      // tokens per wavefront at a time
  constexpr int NW = kThreads / kWave;
  constexpr int U = 4;                  // tokens in flight per token group (8 measured slower)
  __shared__ float red[NW][G][2][D];
  __shared__ float wst[NW][G][3];
  const int pair = blockIdx.x / P.max_split;
  const int split = blockIdx.x % P.max_split;
  const int b = pair / P.Hkv;
  const int g = pair % P.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int tg = lane / LPT;
  const int lig = lane % LPT;
  const int T = clamp_len(P.seq_lens[b], P.max_seq_len);
  const int Ts = state_tokens(P, T, b);           // tokens the linear state holds
  const int count = min(P.ucount[pair], P.umax);
  const int per = ceil_div(count, P.max_split);
  const int e0 = min(split * per, count);
  const int e1 = min(e0 + per, count);
  const int2* list = reinterpret_cast<const int2*>(P.tlist) + static_cast<size_t>(pair) * P.umax;
  const char* kp = reinterpret_cast<const char*>(P.k_pages);
  const char* vp = reinterpret_cast<const char*>(P.v_pages);

  QReg<KV> qr[G];
#pragma unroll
  for (int h = 0; h < G; ++h)
    qr[h].load(reinterpret_cast<const char*>(P.q) + ((static_cast<size_t>(b) * P.Hq + g * G + h) * D + lig * 8) * KV::kBytes);
  float m[G], l[G], ld[G], acc[G][8], lacc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = ld[h] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] = lacc[h][j] = 0.f;
  }

  constexpr int STEP = NW * TPW * U;    // list entries per workgroup iteration
  const int niter = ceil_div(e1 - e0, STEP);
  // list entries of iteration it (dead ones repeat the first entry)
  auto fetch_list = [&](int it, int2 (&en)[U]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = e0 + it * STEP + (u * NW + wave) * TPW + tg;
      en[u] = list[e < e1 ? e : e0];
      if (e >= e1) en[u].x &= 0xFFFFF;   // no heads
    }
  };
  int2 nxt[U];
  if (niter > 0) fetch_list(0, nxt);
  for (int it = 0; it < niter; ++it) {
    int tok[U], heads[U];
    Row8<KV> kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      tok[u] = nxt[u].x & 0xFFFFF;
      heads[u] = nxt[u].x >> 20;
      const size_t off = (((static_cast<size_t>(nxt[u].y) * P.Hkv + g) * P.B + tok[u] % P.B) * D + lig * 8) *
                         KV::kBytes;
      kr[u].load_nt(kp + off);
      vr[u].load_nt(vp + off);
    }
    if (it + 1 < niter) fetch_list(it + 1, nxt);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
      vr[u].to_f32(vf);
      const bool held = tok[u] < Ts;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float s = P.sigma * reduce_sum_lanes<LPT>(qr[h].dot(kr[u]));
        if ((heads[u] >> h) & 1) {
          const float mn = fmaxf(m[h], s);
          const float c = m[h] == kNegInf ? 0.f : __expf(m[h] - mn);
          const float pv = __expf(s - mn);
          l[h] = fmaf(l[h], c, pv);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(acc[h][j], c, pv * vf[j]);
          m[h] = mn;
          if (held) {
            const float w = 1.f + s;
            ld[h] += w;
#pragma unroll
            for (int j = 0; j < 8; ++j) lacc[h][j] = fmaf(w, vf[j], lacc[h][j]);
          }
        }
      }
    }
  }

  // token groups of the wavefront: common maximum, rescale, sum
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = m[h];
    if constexpr (LPT <= 8) M = fmaxf(M, __shfl_xor(M, 8));
    if constexpr (LPT <= 16) M = fmaxf(M, __shfl_xor(M, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float f = m[h] == kNegInf ? 0.f : __expf(m[h] - M);
    l[h] *= f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[h][j] *= f;
    auto gsum = [&](float x) {
      if constexpr (LPT <= 8) x = pair_sum<8>(x);
      if constexpr (LPT <= 16) x = pair_sum<16>(x);
      return pair_sum<32>(x);
    };
    l[h] = gsum(l[h]);
    ld[h] = gsum(ld[h]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[h][j] = gsum(acc[h][j]);
      lacc[h][j] = gsum(lacc[h][j]);
    }
    m[h] = M;
    if (tg == 0) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        red[wave][h][0][lig * 8 + j] = acc[h][j];
        red[wave][h][1][lig * 8 + j] = lacc[h][j];
      }
    }
    if (lane == 0) {
      wst[wave][h][0] = M;
      wst[wave][h][1] = l[h];
      wst[wave][h][2] = ld[h];
    }
  }
  __syncthreads();
  float* outp = P.part + (static_cast<size_t>(pair) * P.max_split + split) * G * P.pstride;
  for (int idx = tid; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int c = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wst[w][h][0]);
    float a = 0.f, la = 0.f, lsum = 0.f, lw = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = wst[w][h][0];
      const float e = mw == kNegInf ? 0.f : __expf(mw - M);
      a = fmaf(e, red[w][h][0][c], a);
      lsum = fmaf(e, wst[w][h][1], lsum);
      la += red[w][h][1][c];
      lw += wst[w][h][2];
    }
    float* o = outp + static_cast<size_t>(h) * P.pstride;
    o[4 + c] = a;
    o[4 + D + c] = la;
    if (c == 0) {
      o[0] = M;
      o[1] = lsum;
      o[2] = lw;
      o[3] = 0.f;
    }
  }
}

// The token-level variant after the scoring launch: per-head selection over
// the candidate tokens, the pairs' exact token lists, attention over them,
// merge.
// The merge kernel with NPC matched to the splits each of its lanes walks.
template <int D, int G>
hipError_t launch_merge(const Problem& p, const DecodeLayout& L, const DecodeParams& P, hipStream_t stream) {
  const int per_lane = ceil_div(L.max_split, kThreads / D);
  const dim3 grid(p.batch * p.Hq);
  if (per_lane <= 2)
    hipLaunchKernelGGL((k_merge<D, G, 2>), grid, dim3(kThreads), 0, stream, P);
  else if (per_lane <= 4)
    hipLaunchKernelGGL((k_merge<D, G, 4>), grid, dim3(kThreads), 0, stream, P);
  else if (per_lane <= 8)
    hipLaunchKernelGGL((k_merge<D, G, 8>), grid, dim3(kThreads), 0, stream, P);
  else
    hipLaunchKernelGGL((k_merge<D, G, 16>), grid, dim3(kThreads), 0, stream, P);
  return launch_status("k_merge");
}

template <typename KV, int D, int G>
hipError_t launch_tokens(const Problem& p, const DecodeLayout& L, const DecodeParams& P, hipStream_t stream,
                         RecordFn rec, void* ctx, int ev) {
  const int pairs = p.batch * p.Hkv;
  if (rec) rec(ctx, ev++, "select");
  {
    // short rows: one wavefront per head with the keys in registers; long
    // rows: the whole workgroup
    const dim3 grid(p.batch * p.Hq);
    if (p.nc_max <= 8 * kWave)
      hipLaunchKernelGGL((k_select<8>), grid, dim3(kWave), 0, stream, P);
    else if (p.nc_max <= 32 * kWave)
      hipLaunchKernelGGL((k_select<32>), grid, dim3(kWave), 0, stream, P);
    else if (static_cast<size_t>(p.nc_max) * sizeof(uint32_t) <= kSelCacheBytes) {
      // the row fits in LDS: only the first radix pass reads it from memory
      const size_t lds = static_cast<size_t>(p.nc_max) * sizeof(uint32_t);
      hipError_t a = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_select_tokens<true>),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (a != hipSuccess) return a;
      hipLaunchKernelGGL((k_select_tokens<true>), grid, dim3(kSelThreads), lds, stream, P);
    } else {
      hipLaunchKernelGGL((k_select_tokens<false>), grid, dim3(kSelThreads), 0, stream, P);
    }
    hipError_t e = launch_status("k_select");
    if (e != hipSuccess) return e;
  }
  if (rec) rec(ctx, ev++, "token_union");
  hipLaunchKernelGGL((k_token_union<G>), dim3(pairs), dim3(kUnionThreads), 0, stream, P);
  hipError_t e = launch_status("k_token_union");
  if (e != hipSuccess) return e;
  if (rec) rec(ctx, ev++, "attend");
  hipLaunchKernelGGL((k_token_attend<KV, D, G>), dim3(pairs * L.max_split), dim3(kThreads), 0, stream, P);
  e = launch_status("k_token_attend");
  if (e != hipSuccess) return e;
  if (rec) rec(ctx, ev++, "merge");
  e = launch_merge<D, G>(p, L, P, stream);
  if (e != hipSuccess) return e;
  if (rec) rec(ctx, ev, nullptr);
  return hipSuccess;
}

template <typename KV, int D, int G>
hipError_t launch_typed(const Problem& p, const DecodeLayout& L, const DecodeParams& P,
                        hipStream_t stream, RecordFn rec, void* ctx) {
  const int pairs = p.batch * p.Hkv;
  int ev = 0;   // profiling events: one before each launched kernel, one after the last
  // with the append taken in, the row-chunk workgroups run whatever the
  // linear tail (they apply the state update)
  const int ro_launch = P.app.k_new ? D / kRoRows + 1 : L.ro_wgs;   // + the statistics workgroup
  if (rec) rec(ctx, ev++, P.app.k_new ? "append_score_readout" : "score_readout");
  // neither candidates nor a linear tail: nothing to score or read out, and
  // the launch only runs when a counter of the attention kernel needs zeroing
  if (L.score_wgs + ro_launch > 0 || P.fused_merge) {
    dim3 grid(std::max(1, L.score_wgs + ro_launch), pairs);
    hipLaunchKernelGGL((k_score_readout<KV, D, G>), grid, dim3(kThreads), 0, stream, P);
    hipError_t e = launch_status("k_score_readout");
    if (e != hipSuccess) return e;
  }
  if (p.tokens) return launch_tokens<KV, D, G>(p, L, P, stream, rec, ctx, ev);
  if (L.fused_sel) {
    // selection runs in the attention prologue
  } else if (p.grouped) {
    if (rec) rec(ctx, ev++, "select");
    // keys in registers up to G x KPL <= 64 per lane
    const dim3 grid(pairs);
    const int kpl = p.nc_max <= 4 * kWave ? 4 : p.nc_max <= 8 * kWave ? 8 : p.nc_max <= 16 * kWave ? 16 : 0;
    if (kpl == 4) {
      hipLaunchKernelGGL((k_select_grouped<4, G>), grid, dim3(kWave), 0, stream, P);
    } else if (kpl == 8) {
      hipLaunchKernelGGL((k_select_grouped<8, G>), grid, dim3(kWave), 0, stream, P);
    } else if (kpl == 16 && G <= 4) {
      if constexpr (G <= 4) hipLaunchKernelGGL((k_select_grouped<16, G>), grid, dim3(kWave), 0, stream, P);
    } else {
      hipLaunchKernelGGL((k_select_grouped<0, G>), grid, dim3(kWave), 0, stream, P);
    }
    hipError_t e = launch_status("k_select_grouped");
    if (e != hipSuccess) return e;
  } else {
    if (rec) rec(ctx, ev++, "select");
    const dim3 grid(p.batch * p.Hq);
    if (p.nc_max <= 4 * kWave)
      hipLaunchKernelGGL((k_select<4>), grid, dim3(kWave), 0, stream, P);
    else if (p.nc_max <= 8 * kWave)
      hipLaunchKernelGGL((k_select<8>), grid, dim3(kWave), 0, stream, P);
    else if (p.nc_max <= 16 * kWave)
      hipLaunchKernelGGL((k_select<16>), grid, dim3(kWave), 0, stream, P);
    else if (p.nc_max <= 32 * kWave)
      hipLaunchKernelGGL((k_select<32>), grid, dim3(kWave), 0, stream, P);
    else
      hipLaunchKernelGGL((k_select<0>), grid, dim3(kWave), 0, stream, P);
    hipError_t e = launch_status("k_select");
    if (e != hipSuccess) return e;
  }
  if (rec) rec(ctx, ev++, "attend");
  {
    const size_t lds = L.sl.total;   // union data; within the default dynamic LDS limit
    const dim3 grid(pairs * L.max_split);
    if constexpr (KV::kBytes == 2) {
      // keys per lane of the fused selection: 8 up to 512 candidates
      const bool fk8 = p.nc_max <= 8 * kWave;
      const bool rows = p.qrows > 1;   // multi-query form: cached K/V loads
      if (rows && !P.dyn && L.fused_sel && p.grouped)
        hipLaunchKernelGGL((k_attend_mfma<D, G, false, 8, true, false>), grid, dim3(kThreads), lds, stream, P);
      else if (rows && !P.dyn && !(L.fused_sel && p.grouped) && fk8)
        hipLaunchKernelGGL((k_attend_mfma<D, G, false, 8, false, false>), grid, dim3(kThreads), lds, stream, P);
      else if (rows && !P.dyn && !(L.fused_sel && p.grouped))
        hipLaunchKernelGGL((k_attend_mfma<D, G, false, 16, false, false>), grid, dim3(kThreads), lds, stream, P);
      else if (L.fused_sel && p.grouped && P.dyn)   // fused grouped selection: up to 512 candidates
        hipLaunchKernelGGL((k_attend_mfma<D, G, true, 8, true>), grid, dim3(kThreads), lds, stream, P);
      else if (L.fused_sel && p.grouped)
        hipLaunchKernelGGL((k_attend_mfma<D, G, false, 8, true>), grid, dim3(kThreads), lds, stream, P);
      else if (P.dyn && fk8)
        hipLaunchKernelGGL((k_attend_mfma<D, G, true, 8, false>), grid, dim3(kThreads), lds, stream, P);
      else if (P.dyn)
        hipLaunchKernelGGL((k_attend_mfma<D, G, true, 16, false>), grid, dim3(kThreads), lds, stream, P);
      else if (fk8)
        hipLaunchKernelGGL((k_attend_mfma<D, G, false, 8, false>), grid, dim3(kThreads), lds, stream, P);
      else
        hipLaunchKernelGGL((k_attend_mfma<D, G, false, 16, false>), grid, dim3(kThreads), lds, stream, P);
    }
    else if (p.B >= kUnit)
      hipLaunchKernelGGL((k_attend<KV, D, G, true>), grid, dim3(kThreads), lds, stream, P);
    else
      hipLaunchKernelGGL((k_attend<KV, D, G, false>), grid, dim3(kThreads), lds, stream, P);
    hipError_t e = launch_status("k_attend");
    if (e != hipSuccess) return e;
  }
  if (!P.fused_merge) {   // else the last attention workgroup of each pair merged it
    if (rec) rec(ctx, ev++, "merge");
    hipError_t e = launch_merge<D, G>(p, L, P, stream);
    if (e != hipSuccess) return e;
  }
  if (rec) rec(ctx, ev, nullptr);
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
  if (p.tokens) L.score_chunk = kTokenChunk;
  L.score_wgs = p.nc_max > 0 ? ceil_div(p.nc_max, L.score_chunk) : 0;
  L.ro_rows = kRoRows;
  L.ro_wgs = p.linear_tail ? p.D / L.ro_rows : 0;
  const int sink_blocks = p.ns / p.B;
  const long sel_blocks = std::min<long>(static_cast<long>(p.grouped ? 1 : p.G) * p.top_k, p.nc_max);
  const long bound = static_cast<long>(sink_blocks) + sel_blocks + 2 + p.W / p.B + 1;
  L.umax = static_cast<int>(std::max<long>(1, std::min<long>(bound, p.nblk_max)));
  if (p.tokens)   // the exact token list: sinks, the heads' selected tokens, the window
    L.umax = static_cast<int>(std::min<long>(static_cast<long>(p.ns) + std::min<long>(static_cast<long>(p.G) * p.top_k,
                                                                                     p.nc_max) + p.W + 1,
                                             static_cast<long>(p.max_seq_len) + 1));
  // Dynamic attention (bf16 path): the pair's workgroups share its union
  // list, which the prologue keeps whole in LDS.
  // The grouped selection is fused on the bf16 path up to 512 candidates
  // (eight keys per lane); past that its registers spill.
  L.fused_sel = (!p.tokens && (p.grouped ? (p.bf16 && p.nc_max <= kFusedKplGrouped * kWave)
                                         : p.nc_max <= kFusedKplMax * kWave)) ? 1 : 0;
  // with the selection fused, the scoring kernel zeroes the work counters,
  // so the dynamic split needs that launch
  const bool scores_launched = (p.nc_max > 0) || p.linear_tail;
  L.dyn = (p.bf16 && !p.tokens && p.deterministic == HSLA_SPLIT_DYNAMIC && L.umax <= kMaxDynList &&
           (!L.fused_sel || scores_launched))
              ? 1 : 0;
  {
    const int want = std::max(1, (kAttendWgsTarget + pairs / 2) / pairs);
    if (L.dyn) {
      L.max_split = std::min(L.umax, want);
      L.bps = ceil_div(L.umax, L.max_split);
    } else {
      const int splits = std::min(L.umax, std::max(want, ceil_div(L.umax, kWave)));
      L.bps = ceil_div(L.umax, splits);   // <= 64: one union entry per lane
      L.max_split = ceil_div(L.umax, L.bps);
    }
  }
  if (p.tokens) {   // about kTokensPerSplit list entries per attention workgroup, at least want
    const int want = std::max(1, (kAttendWgsTarget + pairs / 2) / pairs);
    L.max_split = std::max(want, ceil_div(L.umax, kTokensPerSplit));
    L.bps = ceil_div(L.umax, L.max_split);
  }
  // bf16 attention with few splits per pair: its last workgroup merges
  L.fused_merge = (p.bf16 && !p.tokens && L.max_split <= kFusedMergeSplits) ? 1 : 0;
  L.pstride = 2 * p.D + 4;
  L.sstride = std::max(4, (p.nc_max + 3) / 4 * 4);
  L.nwords = std::max(1, (p.nc_max + 63) / 64);
  L.bt_staged = static_cast<size_t>(p.nblk_max) * sizeof(int32_t) <= kBtStageBytes ? 1 : 0;
  {
    uint32_t o = 0;
    auto take = [&](uint32_t bytes) {
      const uint32_t at = o;
      o += (bytes + 15u) & ~15u;
      return at;
    };
    L.sl.bits = take(static_cast<uint32_t>(p.G * L.nwords * sizeof(uint64_t)));
    L.sl.umask = take((kThreads / kWave) * kWave * sizeof(uint64_t));
    L.sl.upre = take((kThreads / kWave) * kWave * sizeof(int32_t));
    L.sl.btrow = take(L.bt_staged ? static_cast<uint32_t>(p.nblk_max * sizeof(int32_t)) : 0u);
    L.sl.ulist = take(L.dyn ? static_cast<uint32_t>(2 * L.umax * sizeof(int32_t)) : 0u);
    L.sl.hist = take(L.fused_sel ? static_cast<uint32_t>((kThreads / kWave) * 256 * sizeof(uint32_t)) : 0u);
    L.sl.gw = take(L.fused_sel && p.grouped
                       ? static_cast<uint32_t>(p.G * ((p.nc_max + kWave - 1) / kWave) * kWave * sizeof(float))
                       : 0u);
    L.sl.total = o;
  }
  size_t off = 0;
  L.off_scores = off;
  off = align_up(off + sizeof(uint32_t) * static_cast<size_t>(p.batch) * p.Hq * L.sstride);
  L.off_ro = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(pairs) * std::max(1, L.ro_wgs) * p.G * p.D);
  L.off_roz = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(pairs) * std::max(1, L.ro_wgs) * p.G);
  L.off_bits = off;
  off = align_up(off + sizeof(uint64_t) * static_cast<size_t>(p.batch) * p.Hq * L.nwords);
  L.off_ucount = off;
  off = align_up(off + sizeof(int32_t) * static_cast<size_t>(pairs));
  L.off_ctr = off;
  off = align_up(off + sizeof(int32_t) * static_cast<size_t>(pairs) * kCtrStride);
  L.off_part = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(pairs) * L.max_split * p.G * L.pstride);
  L.off_tlist = off;
  off = align_up(off + (p.tokens ? 2 * sizeof(int32_t) * static_cast<size_t>(pairs) * L.umax : 0));
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
  P.keys = reinterpret_cast<uint32_t*>(a.ws + L.off_scores);
  P.bits = reinterpret_cast<uint64_t*>(a.ws + L.off_bits);
  P.ro = reinterpret_cast<float*>(a.ws + L.off_ro);
  P.roz = reinterpret_cast<float*>(a.ws + L.off_roz);
  P.ucount = reinterpret_cast<int32_t*>(a.ws + L.off_ucount);
  P.ctr = reinterpret_cast<int32_t*>(a.ws + L.off_ctr);
  P.dyn = L.dyn;
  P.fused_sel = L.fused_sel;
  P.fused_merge = L.fused_merge;
  P.tokens = p.tokens;
  P.qrows = p.qrows;
  P.chunk = p.chunk;
  P.state_all = p.state_all;
  P.bsel = p.tokens ? 1 : p.B;
  P.tlist = reinterpret_cast<int32_t*>(a.ws + L.off_tlist);
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
  P.sstride = L.sstride;
  P.nwords = L.nwords;
  P.bt_staged = L.bt_staged;
  P.sl = L.sl;
  P.app = DecodeAppend{a.app.k_pages, a.app.v_pages, a.app.blk_mean, a.app.blk_var, a.app.S, a.app.z, a.app.sv,
                       a.app.k_new, a.app.v_new, a.app.seq_lens_before, a.app.seq_lens_after};
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

size_t phase_bytes() {
#ifdef HSLA_PHASE_TIMESTAMPS
  return sizeof(g_phase_attend) + sizeof(g_phase_score) + sizeof(g_phase_merge);
#else
  return 0;
#endif
}

hipError_t phase_copy(void* host, bool clear) {
#ifdef HSLA_PHASE_TIMESTAMPS
  char* h = static_cast<char*>(host);
  hipError_t e = hipMemcpyFromSymbol(h, HIP_SYMBOL(g_phase_attend), sizeof(g_phase_attend));
  if (e == hipSuccess) e = hipMemcpyFromSymbol(h + sizeof(g_phase_attend), HIP_SYMBOL(g_phase_score), sizeof(g_phase_score));
  if (e == hipSuccess)
    e = hipMemcpyFromSymbol(h + sizeof(g_phase_attend) + sizeof(g_phase_score), HIP_SYMBOL(g_phase_merge),
                            sizeof(g_phase_merge));
  if (e == hipSuccess && clear) {
    void* a = nullptr;
    for (const void* sym : {reinterpret_cast<const void*>(&g_phase_attend), reinterpret_cast<const void*>(&g_phase_score),
                            reinterpret_cast<const void*>(&g_phase_merge)}) {
      size_t n = 0;
      if (e == hipSuccess) e = hipGetSymbolAddress(&a, sym);
      if (e == hipSuccess) e = hipGetSymbolSize(&n, sym);
      if (e == hipSuccess) e = hipMemset(a, 0, n);
    }
  }
  return e;
#else
  (void)host;
  (void)clear;
  return hipErrorNotSupported;
#endif
}

}  // namespace hsla
