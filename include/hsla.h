/*
 * hsla.h -- C ABI of libhsla, hybrid sparse-plus-linear decode attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages (title, then the part of the page):
 *   [SPLA]  "SPLA: Block Sparse Plus Linear Attention for Long Context
 *           Modeling" -- TL;DR, Abstract, sections "Page Attention and
 *           Selection", "Principled Block Selection via Taylor Expansion",
 *           "Residual Linear Attention (RLA)", "Recurrence",
 *           "IO-Efficient Implementation", Figure 1.
 *   [SALSA] "SALSA: Training-Consistent Sparse Caching with Sink
 *           Preservation for Linearized LLMs" -- abstract (sliding window,
 *           sparse global cache, linear hidden state, sink tokens).
 *   [SLAKE] "SLAKE: Softmax-Approximated Training-Free Linear Attention with
 *           KV-Cache Eviction for Long-Sequence LLMs" -- abstract (first-order
 *           Taylor linearisation of softmax for low-importance tokens).
 *
 * Definitions used throughout (T = tokens of a sequence including the
 * current one, B = block_size, d = head_dim, sigma = scale or 1/sqrt(d)):
 *   - query head h reads kv head h / (num_q_heads / num_kv_heads);
 *   - block j of a sequence holds tokens [jB, (j+1)B); it is "full" when
 *     (j+1)B <= T.  Block statistics: mean_j = (1/B) sum k_t and the
 *     population variance var_j,c = (1/B) sum (k_t,c - mean_j,c)^2;
 *   - sinks are tokens [0, num_sink), the window is [T - window, T) (it holds
 *     the current token); candidate blocks intersect [num_sink, T - window);
 *   - block score = sigma q.mean_j + log1p(sigma^2/2 sum_c q_c^2 var_j,c)
 *     (second-order Taylor expansion of exp(sigma q.k) around the block mean,
 *     averaged over the block) [SPLA, "Principled Block Selection ..."];
 *   - each query head keeps its top_k candidates by (score desc, index asc);
 *     exact set E = sinks U window U selected blocks, residual U = rest;
 *   - global linear state with phi(q).phi(k) = 1 + sigma q.k [SLAKE]:
 *     S = sum_t k_t v_t^T (d x d, S[i][j] = sum k_t,i v_t,j), z = sum k_t,
 *     sv = sum v_t, n = number of tokens summed, taken over the tokens of
 *     complete blocks, t < Ts = T - T % B.  The incomplete last block lies
 *     inside the window (window >= B), so its tokens are always exact and
 *     never part of U; the state takes a block when it completes;
 *   - out = (sum_E e^{s_t} v_t + num_U) / (sum_E e^{s_t} + den_U), s_t =
 *     sigma q.k_t, with num_U = sv + sigma S^T q - sum_{E, t<Ts} (1+s_t) v_t
 *     and den_U = n + sigma q.z - sum_{E, t<Ts} (1+s_t) (global minus
 *     selected, so U is never read) [SPLA Abstract]; num_U = den_U = 0 when
 *     U is empty or the linear tail is off.  This equals the sum over U of
 *     the state built over all T tokens.
 *
 * Conventions for every entry point:
 *   - Memory: every pointer is a device pointer unless stated otherwise and
 *     is owned by the caller.  The library never allocates or frees memory,
 *     keeps no pointer after returning and has no global mutable state.
 *     Tensor pointers must be 16-byte aligned.
 *   - Asynchrony: all work is enqueued on `stream`; results are valid once
 *     the stream has synchronised.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued; on a negative status nothing has been enqueued, except
 *     HSLA_ERR_HIP, which reports a failed launch.  Device-side contents
 *     (block tables, lengths) are trusted: a length above max_seq_len or a
 *     page index outside [0, num_pages) is undefined behaviour, which
 *     hsla_check_tables / hsla_check_tables_host detect on request and the
 *     debug build (libhsla_debug.so) on every call.
 */
#ifndef HSLA_H
#define HSLA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hsla_status {
  HSLA_OK = 0,
  HSLA_ERR_INVALID_ARG = -1, /* null pointer, bad size, misaligned pointer */
  HSLA_ERR_UNSUPPORTED = -2, /* valid but not built: head_dim, group, block size, dtype,
                                or more candidate blocks than one workgroup's selection
                                bitmaps hold (G * ceil(n_candidates / 64) * 8 > 16384) */
  HSLA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  HSLA_ERR_HIP = -4          /* a kernel launch failed */
} hsla_status;

typedef enum hsla_dtype { HSLA_F32 = 0, HSLA_BF16 = 1 } hsla_dtype;

/* Block selection.
 * HSLA_SEL_PER_HEAD: every query head keeps its own top_k blocks (the method
 *   as defined above).
 * HSLA_SEL_GROUPED: the G query heads of a kv head share one selection
 *   [SPLA table of contents, "Grouped Sparsity"; the section's text is not on
 *   the page, so this is a reading]: each head's block scores become a
 *   softmax over its candidates, the G softmaxes are summed per block, and
 *   the top_k blocks by that sum (lower index first on ties) are the
 *   selection of every head of the group.  With G = 1 it equals
 *   HSLA_SEL_PER_HEAD.
 * HSLA_SEL_TOKEN: token-level variant ["SALS: Sparse Attention in Latent
 *   Space for KV Cache Compression", Approach; here on the plain keys, with
 *   no latent projection]: the candidates are the tokens of
 *   [num_sink, T - window), a token's score is sigma q.k_t, each query head
 *   keeps its top_k tokens (score descending, lower index first), and
 *   sel_idx receives token indices.  Sinks, window, the linear tail and the
 *   merge are unchanged.  Supported for max_seq_len < 2^20. */
typedef enum hsla_selection {
  HSLA_SEL_PER_HEAD = 0,
  HSLA_SEL_GROUPED = 1,
  HSLA_SEL_TOKEN = 2
} hsla_selection;

/* The problem statement's parameters.
 * num_q_heads, num_kv_heads: GQA heads; num_q_heads / num_kv_heads must be
 *   1, 2, 4 or 8.
 * head_dim: 64 or 128.
 * block_size: tokens per block and per KV page: 16, 32, 64, 128 or 256
 *   [SPLA, "Page Attention and Selection": selection at page granularity].
 * top_k: selected blocks per query head (tokens with HSLA_SEL_TOKEN), >= 0
 *   [SPLA Abstract].
 * num_sink: initial sink tokens, >= 0; window: sliding-window length
 *   including the current token, >= block_size [SALSA abstract].
 * linear_tail: 1 = residual linear attention over U [SPLA, "Residual Linear
 *   Attention (RLA)"]; 0 = drop U (plain block-sparse attention, the
 *   "discard" behaviour of SPLA Figure 1(c)).
 * kv_dtype: hsla_dtype of keys, values, queries and appended tokens.
 * scale: sigma; 0 selects 1/sqrt(head_dim).
 * selection: hsla_selection (0 = per head).
 * deterministic: how the attention workgroups of a (sequence, kv head)
 *   share its exact blocks.  HSLA_SPLIT_FIXED (1): each takes a fixed share;
 *   results are bitwise reproducible.  HSLA_SPLIT_DYNAMIC (2): they claim
 *   the blocks from a shared counter as they go, so that workgroups on
 *   faster XCDs take more; the summation order, and so the last bits of
 *   the output, then vary from run to run (selections do not).
 *   HSLA_SPLIT_DEFAULT (0): the library's choice, the fixed split (it
 *   measured as fast or faster at every workload here).  fp32 keys/values
 *   always run the fixed split.  Other values: HSLA_ERR_INVALID_ARG. */
#define HSLA_SPLIT_DEFAULT 0
#define HSLA_SPLIT_FIXED 1
#define HSLA_SPLIT_DYNAMIC 2
/* state_span: which tokens the global linear state (hsla_state) holds
 *   [SPLA, "Residual Linear Attention (RLA)", "Recurrence"].
 *   HSLA_STATE_BLOCKS (0): the tokens of complete blocks, n = T - T % B.
 *     The library keeps it so: hsla_build_state builds it, and the appends
 *     fold a block in when it completes.
 *   HSLA_STATE_TOKENS (1): every token, n = T, as a state updated at every
 *     token holds it.  hsla_build_state builds it over all T tokens,
 *     hsla_append_token and hsla_append_decode (and its no-alloc variant)
 *     add each appended token to it (S += k v^T, z += k, sv += v; a
 *     completed block still gets its statistics), and the decode subtracts
 *     every exact token from it.  hsla_prefill_chunk, whose queries read
 *     the state as it was before the chunk, folds whole blocks only and
 *     returns HSLA_ERR_UNSUPPORTED.  Both spans give the same residual, up
 *     to rounding, since the tokens of the incomplete block are in the
 *     window.
 *   Other values: HSLA_ERR_INVALID_ARG. */
#define HSLA_STATE_BLOCKS 0
#define HSLA_STATE_TOKENS 1
typedef struct hsla_config {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t top_k;
  int32_t num_sink;
  int32_t window;
  int32_t linear_tail;
  int32_t kv_dtype;
  float scale;
  int32_t selection;
  int32_t deterministic;
  int32_t state_span;
} hsla_config;

/* Paged KV cache [SPLA, "Page Attention and Selection"].
 * k_pages, v_pages: [num_pages, num_kv_heads, block_size, head_dim] kv_dtype;
 *   page p, kv head g holds one block of one sequence for that head.
 * blk_mean, blk_var: [num_pages, num_kv_heads, head_dim] float32 statistics
 *   of the block stored in that page (defined only for full blocks).
 * block_table: [batch, max_blocks_per_seq] int32, row-major; entry (b, j) is
 *   the page of block j of sequence b.  The kernels may load any entry
 *   j < ceil(max_seq_len / B) of a row (they prefetch the row before the
 *   sequence's length is known), but only entries j < ceil(T_b / B) (and
 *   entry T_b / B by an append) are used as page indices, so the rest may
 *   hold anything. */
typedef struct hsla_kv_pool {
  void* k_pages;
  void* v_pages;
  float* blk_mean;
  float* blk_var;
  const int32_t* block_table;
  int32_t max_blocks_per_seq;
  int32_t num_pages;
} hsla_kv_pool;

/* Global linear state per (sequence, kv head) [SPLA, "Residual Linear
 * Attention (RLA)", "Recurrence"]: S [batch, Hkv, d, d], z and sv
 * [batch, Hkv, d], all float32, over the tokens of the sequence's complete
 * blocks (n = T - T % B follows from the length), or over all T tokens
 * (n = T) with state_span = HSLA_STATE_TOKENS. */
typedef struct hsla_state {
  float* S;
  float* z;
  float* sv;
} hsla_state;

/* Optional timing hook.  The caller creates `capacity` HIP events; the
 * library records events[i] on `stream` just before its i-th kernel launch and
 * one more after the last, sets `recorded`, and names the kernels in
 * `names[i]` (static strings).  Pass NULL to record nothing. */
#define HSLA_MAX_PROFILE_EVENTS 8
typedef struct hsla_profile {
  hipEvent_t events[HSLA_MAX_PROFILE_EVENTS];
  int32_t capacity;
  int32_t recorded;
  const char* names[HSLA_MAX_PROFILE_EVENTS];
} hsla_profile;

/* Static description of a status code (never NULL). */
const char* hsla_status_string(hsla_status status);

/* Library version string (static). */
const char* hsla_version(void);

/* Bytes of workspace hsla_build_state needs for this shape (0 on invalid
 * arguments).  Pure host function. */
size_t hsla_build_workspace_size(const hsla_config* cfg, int32_t batch, int32_t max_seq_len);

/* Build the block statistics of every full block and the global linear state
 * of every (sequence, kv head) from a prefilled paged cache [SPLA TL;DR,
 * Abstract; "Recurrence"].
 * seq_lens: device [batch] int32, T_b <= max_seq_len (host value, sizes the
 *   launch; >= 1).
 * Writes pool->blk_mean / blk_var for the pages of full blocks, and
 * state->S, z, sv for every (b, g) over the tokens of full blocks.  The sums are reduced in a fixed order,
 * so repeated builds are bitwise identical.
 * workspace: device scratch of at least hsla_build_workspace_size() bytes;
 *   contents on entry are ignored. */
hsla_status hsla_build_state(const hsla_config* cfg, const hsla_kv_pool* pool,
                             const hsla_state* state, const int32_t* seq_lens,
                             int32_t batch, int32_t max_seq_len, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* Append one token per (sequence, kv head) [SPLA, "Recurrence"].
 * k_new, v_new: device [batch, Hkv, head_dim] kv_dtype.
 * seq_lens_before: device [batch]; the token goes to position T_b =
 *   seq_lens_before[b], i.e. slot T_b % B of page block_table[b][T_b / B],
 *   which the caller must have mapped.  T_b + 1 <= max_seq_len.
 * seq_lens_after: device [batch] or NULL; receives T_b + 1.  Must not alias
 *   seq_lens_before.
 * Writes the token's page slot.  When position T_b completes its block, the
 * state takes the block (S += K_b^T V_b, z += sum k, sv += sum v over its B
 * tokens) and the block's statistics are computed. */
hsla_status hsla_append_token(const hsla_config* cfg, const hsla_kv_pool* pool,
                              const hsla_state* state, const void* k_new, const void* v_new,
                              const int32_t* seq_lens_before, int32_t* seq_lens_after,
                              int32_t batch, int32_t max_seq_len, hipStream_t stream);

/* Checks of what the kernels trust [SPLA, "Page Attention and Selection":
 * the paged cache they read through the block table].  Every row b must
 * satisfy min_len <= T_b and T_b + extra <= max_seq_len, where T_b =
 * seq_lens[b], extra = tokens the call appends (0 for hsla_decode and
 * hsla_build_state, whose lengths include the current token; 1 for the
 * seq_lens_before of hsla_append_token and hsla_append_decode; q_len for
 * hsla_prefill_chunk) and min_len = 1 when extra is 0, else 0; and every
 * entry j < ceil((T_b + extra) / B) of the row must be a page in
 * [0, num_pages).  Entries past that are not checked (the kernels never use
 * them as page indices).
 * result: int32[2]: result[0] = number of violations; result[1] = the first
 *   one as a key: b (max_blocks_per_seq + 1) for row b's length,
 *   b (max_blocks_per_seq + 1) + j + 1 for its entry j; INT32_MAX if none.
 * hsla_check_tables: block_table (pool), seq_lens and result are device
 *   pointers; the check is enqueued on `stream` (two small kernels, no
 *   memset, capturable) and result is valid once the stream has
 *   synchronised.  Returns HSLA_OK once enqueued.
 * hsla_check_tables_host: the same check on host arrays (block_table
 *   [batch, max_blocks_per_seq], seq_lens [batch], result [2]); runs on the
 *   calling thread, needs no GPU, and returns HSLA_OK when there is no
 *   violation, else HSLA_ERR_INVALID_ARG with result filled.
 * A library built with HSLA_DEBUG_CHECKS (libhsla_debug.so) runs the device
 * check inside every entry point that enqueues work, waits for it, and on a
 * violation returns HSLA_ERR_INVALID_ARG with the first violation on stderr,
 * enqueueing nothing else. */
hsla_status hsla_check_tables(const hsla_config* cfg, const hsla_kv_pool* pool, const int32_t* seq_lens,
                              int32_t batch, int32_t max_seq_len, int32_t extra, int32_t* result,
                              hipStream_t stream);
hsla_status hsla_check_tables_host(const hsla_config* cfg, int32_t max_blocks_per_seq, int32_t num_pages,
                                   const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                                   int32_t max_seq_len, int32_t extra, int32_t* result);

/* Bytes of workspace hsla_decode needs for this shape (0 on invalid
 * arguments).  Pure host function. */
size_t hsla_decode_workspace_size(const hsla_config* cfg, int32_t batch, int32_t max_seq_len);

/* One decode step for every (sequence, query head): block scores from the
 * statistics, top-k selection, exact softmax attention over E, residual
 * linear readout over U by subtraction from the global state, merge
 * [SPLA Abstract, Figure 1; SALSA abstract; SLAKE abstract].
 * q: device [batch, Hq, head_dim] kv_dtype (the current token's queries).
 * seq_lens: device [batch], T_b including the current token, 1 <= T_b <=
 *   max_seq_len.  The current token must already be in the cache and the
 *   statistics of every full block and the state must be up to date.
 * out: device [batch, Hq, head_dim] float32.
 * sel_idx: device [batch, Hq, top_k] int32 or NULL; receives each head's
 *   selected block indices (token indices with HSLA_SEL_TOKEN) in ascending
 *   order, padded with -1.
 * workspace: device scratch of at least hsla_decode_workspace_size() bytes;
 *   contents on entry are ignored.  Calls that share a workspace must not
 *   run concurrently.
 * prof: optional timing hook (NULL for none). */
hsla_status hsla_decode(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state,
                        const void* q, const int32_t* seq_lens, int32_t batch,
                        int32_t max_seq_len, float* out, int32_t* sel_idx, void* workspace,
                        size_t workspace_bytes, hipStream_t stream, hsla_profile* prof);

/* The token append and the decode of the grown sequences in one call
 * [SPLA, "Recurrence", Abstract, Figure 1]: the same results as
 * hsla_append_token(k_new, v_new, seq_lens_before, seq_lens_after) followed by
 * hsla_decode(seq_lens_after), with one launch fewer.  The first decode
 * kernel applies the append (page slot, seq_lens_after and, when the token
 * completes its block, the block into the state and its statistics) while
 * it reads the state, so the state's rows are read once.  Arguments as in the two
 * calls: the token goes to position T_b = seq_lens_before[b] (page mapped by
 * the caller), the decode runs at T_b + 1 <= max_seq_len.  seq_lens_after is
 * required and must not alias seq_lens_before; state is required whatever
 * linear_tail says (the append maintains it).  Workspace as for hsla_decode
 * (hsla_decode_workspace_size). */
hsla_status hsla_append_decode(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state,
                               const void* k_new, const void* v_new, const int32_t* seq_lens_before,
                               int32_t* seq_lens_after, const void* q, int32_t batch, int32_t max_seq_len,
                               float* out, int32_t* sel_idx, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, hsla_profile* prof);

/* Scratch of hsla_append_decode_noalloc: 16 MiB per GPU. */
#define HSLA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* Bytes of that scratch (HSLA_NOALLOC_SCRATCH_BYTES).  Pure host function. */
size_t hsla_noalloc_scratch_bytes(void);

/* hsla_append_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Arguments and results as hsla_append_decode, without the
 * workspace and the timing hook.  The workspace is instead a fixed array of
 * HSLA_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends (its first call on a device looks up the array's address
 * there).  The call allocates nothing.
 * Limits and errors: when hsla_decode_workspace_size(cfg, batch,
 * max_seq_len) exceeds HSLA_NOALLOC_SCRATCH_BYTES it returns
 * HSLA_ERR_WORKSPACE (and says so on stderr) and enqueues nothing; other
 * errors as hsla_append_decode.  Every call on one GPU shares that GPU's
 * array: calls whose work overlaps on one GPU (other host threads, other
 * streams) race and give wrong results; calls ordered on one stream, or
 * synchronised, are safe. */
hsla_status hsla_append_decode_noalloc(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state,
                                       const void* k_new, const void* v_new, const int32_t* seq_lens_before,
                                       int32_t* seq_lens_after, const void* q, int32_t batch, int32_t max_seq_len,
                                       float* out, int32_t* sel_idx, hipStream_t stream);

/* Diagnostics: per-workgroup phase timestamps of the decode kernels (not
 * part of the method; for measuring where a step's time goes).  Only a
 * library built with HSLA_PHASE_TIMESTAMPS (libhsla_phases.so) records
 * them; there every workgroup of the last launch of each decode kernel
 * stamps its phases with the device's 100 MHz real-time counter (uint64):
 * attention workgroups [4096][16] (slots: 0 entry, 1 prologue loads staged,
 * 2..5 selection done per wavefront, 6 prologue done, 7..10 loop done per
 * wavefront, 11 partials written, 12 exit; row = workgroup index), then
 * scoring workgroups [16384][2] (entry, exit; row = pair x scoring grid +
 * workgroup), then merge workgroups [8192][2]; unused rows are 0.
 * hsla_phase_timestamp_bytes: the size of that host buffer; 0 in other
 * builds.  Pure host function.
 * hsla_phase_timestamps: copies the stamps into `host` (a host pointer of
 * at least that many bytes) and, when clear != 0, zeroes them on the device.
 * Synchronous on the null stream.  HSLA_ERR_UNSUPPORTED in other builds,
 * HSLA_ERR_INVALID_ARG for a missing or short buffer. */
size_t hsla_phase_timestamp_bytes(void);
hsla_status hsla_phase_timestamps(void* host, size_t bytes, int32_t clear);

/* Bytes of workspace hsla_prefill_chunk needs (0 on invalid arguments or
 * an unsupported chunk).  Pure host function. */
size_t hsla_prefill_chunk_workspace_size(const hsla_config* cfg, int32_t batch, int32_t q_len,
                                         int32_t max_seq_len);

/* Multi-query form: a chunk of q_len consecutive tokens per sequence is
 * appended and each of its queries is decoded causally at its own position
 * [SALSA abstract: the same sparse + window + linear partition at training
 * and inference; SPLA Figure 1(a), "Recurrence"].  Query i of sequence b sits
 * at position T0 = seq_lens_before[b] plus i, sees tokens 0 .. T0 + i, and
 * gets exactly the output hsla_decode gives at length T0 + i + 1 (its own
 * candidates, top-k, sinks, window and linear tail): what q_len rounds of
 * hsla_append_decode compute, up to rounding (every query's linear part is
 * taken from the state as it stood before the chunk), in three launches: the
 * chunk's page slots, the q_len x batch decodes, then the fold of the block
 * the chunk completed (at most one) into the state and statistics.  The
 * cache afterwards (pages, statistics, state, lengths) is bitwise what
 * q_len hsla_append_token calls leave.
 * k_chunk, v_chunk: device [batch, q_len, Hkv, head_dim] kv_dtype; the pages
 *   of positions T0 .. T0 + q_len - 1 must be mapped by the caller.
 * q: device [batch, q_len, Hq, head_dim] kv_dtype.
 * seq_lens_before: device [batch], T0 >= 0 with T0 + q_len <= max_seq_len;
 * seq_lens_after: device [batch], receives T0 + q_len; must not alias
 *   seq_lens_before.
 * out: device [batch, q_len, Hq, head_dim] float32; sel_idx: device
 *   [batch, q_len, Hq, top_k] int32 or NULL (as for hsla_decode).
 * Limits: 1 <= q_len <= min(block_size, window - block_size + 1), so that
 *   every query's window covers the tokens between the state (whole blocks
 *   before the chunk) and the query; block selection only
 *   (HSLA_SEL_TOKEN -> HSLA_ERR_UNSUPPORTED).  state is required.
 * workspace: at least hsla_prefill_chunk_workspace_size() bytes. */
hsla_status hsla_prefill_chunk(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state,
                               const void* k_chunk, const void* v_chunk, const int32_t* seq_lens_before,
                               int32_t* seq_lens_after, const void* q, int32_t batch, int32_t q_len,
                               int32_t max_seq_len, float* out, int32_t* sel_idx, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HSLA_H */
