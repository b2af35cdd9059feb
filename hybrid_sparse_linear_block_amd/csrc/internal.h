// Host-side plumbing between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>

#include "hsla.h"

namespace hsla {

// Status of the launch just made; failures are reported on stderr with the
// kernel's name and HIP's error string.
inline hipError_t launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) fprintf(stderr, "libhsla: launch of %s failed: %s\n", what, hipGetErrorString(e));
  return e;
}

// Resolved, validated problem description handed to the launchers.
struct Problem {
  int Hq, Hkv, G, D, B, top_k, ns, W, linear_tail, bf16;
  int grouped;     // one selection per kv head (HSLA_SEL_GROUPED)
  int deterministic;  // HSLA_SPLIT_*: only HSLA_SPLIT_DYNAMIC selects the dynamic split-K attention
  int tokens;      // token-level variant (HSLA_SEL_TOKEN): candidates are single tokens
  int qrows;       // query rows per sequence: 1, or the chunk length of the multi-query form
                   // (then batch counts query rows: sequences x qrows)
  int chunk;       // multi-query form: the state holds the whole blocks before the chunk
  int state_all;   // HSLA_STATE_TOKENS: the state holds all T tokens (n = T)
  float sigma;
  int batch, max_seq_len;
  int max_blocks;  // block table row stride
  int nc_max;      // candidate blocks at max_seq_len
  int nblk_max;    // blocks of a max_seq_len sequence
};

// ---------------------------------------------------------------- decode
// Byte offsets into the dynamic LDS of an attention workgroup, where it
// builds its share of the union: the G heads' selection bitmaps [G][nwords]
// (uint64), wavefront-private union chunk masks [4][64] (uint64) and chunk
// prefixes [4][64] (int32), when staged the sequence's block-table row
// [nblk_max] (int32), for dynamic attention the whole union list: entries
// [umax] and pages [umax] (int32), for the fused selection the
// wavefronts' radix histograms [4][256] (uint32), and for the fused grouped
// selection the heads' candidate shares [G][round64(nc_max)] (float).
struct SelLayout {
  uint32_t bits, umask, upre, btrow, ulist, hist, gw, total;
};

struct DecodeLayout {
  int score_chunk;     // candidates per scoring workgroup
  int score_wgs;       // scoring workgroups per (sequence, kv head)
  int ro_wgs;          // readout workgroups per (sequence, kv head)
  int ro_rows;         // rows of S per readout workgroup
  int umax;            // union-list capacity per (sequence, kv head)
  int bps;             // union blocks per attention split (fixed split)
  int max_split;       // attention workgroups per (sequence, kv head)
  int pstride;         // floats per (split, head) partial
  int sstride;         // order keys per (sequence, head) row, multiple of 4
  int nwords;          // 64-bit words of a per-head selection bitmap
  int bt_staged;       // block-table row staged in LDS
  int dyn;             // attention workgroups of a pair claim its slices dynamically
  int fused_sel;       // per-head selection in the attention prologue
  int fused_merge;     // the last attention workgroup of a pair merges (no merge kernel)
  SelLayout sl;
  size_t off_scores, off_ro, off_roz, off_bits, off_ucount, off_ctr, off_part, off_tlist, total;
};
DecodeLayout decode_layout(const Problem& p);

// Diagnostic build (HSLA_PHASE_TIMESTAMPS): the per-workgroup phase stamps
// of the last decode launches, attention [kPhaseAttendWgs][kPhaseSlots]
// then scoring [kPhaseScoreWgs][2] then merge [kPhaseMergeWgs][2] (uint64);
// phase_bytes() is 0 in the release build.
constexpr int kPhaseAttendWgs = 4096;
constexpr int kPhaseSlots = 16;
constexpr int kPhaseScoreWgs = 16384;
constexpr int kPhaseMergeWgs = 8192;
size_t phase_bytes();
hipError_t phase_copy(void* host, bool clear);

// ---------------------------------------------------------------- append
struct AppendArgs {
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
};

// A decode; app.k_new != nullptr: the token append is taken in by the first
// kernel (hsla_append_decode), seq_lens is then app.seq_lens_after.
struct DecodeArgs {
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
  char* ws;
  AppendArgs app;
};

// Launches score+readout, select, attend, merge.  `record` is called with the
// kernel index before each launch and with the kernel count after the last.
typedef void (*RecordFn)(void* ctx, int idx, const char* name);
hipError_t launch_decode(const Problem& p, const DecodeLayout& L, const DecodeArgs& a,
                         hipStream_t stream, RecordFn rec, void* rec_ctx);

// ---------------------------------------------------------------- build
struct BuildLayout {
  int tile;      // tokens staged in LDS at a time (multiple of 64 and of B)
  int chunk;     // tokens per workgroup
  int nchunk;    // workgroups per (sequence, kv head)
  size_t part_stride;  // floats per chunk partial (D*D + 2*D)
  size_t total;
};
BuildLayout build_layout(const Problem& p);

struct BuildArgs {
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
};
hipError_t launch_build(const Problem& p, const BuildLayout& L, const BuildArgs& a,
                        hipStream_t stream);

// ---------------------------------------------------------------- append
// Append of `count` tokens per sequence (k_new / v_new [batch, count, Hkv, D]):
// kAppendWriteRows writes their page slots (and, with row_lens, each query
// row's length T0 + 1 + i), kAppendFold folds the block they complete (at
// most one: count <= B) into the state and statistics and sets
// seq_lens_after.  A token append is count 1 with both.
constexpr int kAppendWriteRows = 1;
constexpr int kAppendFold = 2;
hipError_t launch_append(const Problem& p, const AppendArgs& a, hipStream_t stream, int count = 1,
                         int mode = kAppendWriteRows | kAppendFold, int32_t* row_lens = nullptr);

// ---------------------------------------------------------------- checks
// Lengths and block-table entries as the kernels use them: a row's length T
// must satisfy min_len <= T and T + extra <= max_seq_len (extra = tokens
// the call appends), and its entries j < ceil((T + extra) / B) must be pages
// in [0, num_pages).  result[0] receives the number of violations, result[1]
// the key of the first (row b's length: b (max_blocks + 1); its entry j:
// b (max_blocks + 1) + j + 1), INT_MAX when there is none.
struct CheckTablesArgs {
  const int32_t* block_table;
  const int32_t* seq_lens;
  int32_t* result;
  int batch, max_blocks, num_pages, B, max_seq_len, extra, min_len;
};
hipError_t launch_check_tables(const CheckTablesArgs& a, hipStream_t stream);   // device arrays
void check_tables_host(const CheckTablesArgs& a);                               // host arrays

}  // namespace hsla
