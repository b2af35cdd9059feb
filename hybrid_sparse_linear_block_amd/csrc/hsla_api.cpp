// C ABI of libhsla: argument validation, workspace sizing and launch order.
// The operations and their definitions are documented in include/hsla.h.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "common.h"
#include "hsla.h"
#include "internal.h"

namespace {

using hsla::Problem;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validates the configuration and resolves the problem description.
hsla_status resolve(const hsla_config* cfg, int32_t batch, int32_t max_seq_len,
                    int32_t max_blocks, Problem* out) {
  if (!cfg) return HSLA_ERR_INVALID_ARG;
  if (cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0 || cfg->num_q_heads % cfg->num_kv_heads != 0)
    return HSLA_ERR_INVALID_ARG;
  if (cfg->top_k < 0 || cfg->num_sink < 0 || cfg->window < 1) return HSLA_ERR_INVALID_ARG;
  if (cfg->linear_tail != 0 && cfg->linear_tail != 1) return HSLA_ERR_INVALID_ARG;
  if (cfg->selection != HSLA_SEL_PER_HEAD && cfg->selection != HSLA_SEL_GROUPED && cfg->selection != HSLA_SEL_TOKEN)
    return HSLA_ERR_INVALID_ARG;
  if (cfg->deterministic < HSLA_SPLIT_DEFAULT || cfg->deterministic > HSLA_SPLIT_DYNAMIC) return HSLA_ERR_INVALID_ARG;
  if (!(cfg->scale >= 0.0f) || !isfinite(cfg->scale)) return HSLA_ERR_INVALID_ARG;
  if (cfg->state_span != HSLA_STATE_BLOCKS && cfg->state_span != HSLA_STATE_TOKENS) return HSLA_ERR_INVALID_ARG;
  if (batch < 1 || max_seq_len < 1) return HSLA_ERR_INVALID_ARG;
  const int G = cfg->num_q_heads / cfg->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return HSLA_ERR_UNSUPPORTED;
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return HSLA_ERR_UNSUPPORTED;
  const int B = cfg->block_size;
  if (B != 16 && B != 32 && B != 64 && B != 128 && B != 256) return HSLA_ERR_UNSUPPORTED;
  if (cfg->kv_dtype != HSLA_F32 && cfg->kv_dtype != HSLA_BF16) return HSLA_ERR_UNSUPPORTED;
  if (cfg->window < B) return HSLA_ERR_INVALID_ARG;  // candidates must be full blocks
  const long nblk = (static_cast<long>(max_seq_len) + B - 1) / B;
  if (nblk >= (1L << 20)) return HSLA_ERR_UNSUPPORTED;  // block index field of the union list
  if (max_blocks >= 0 && max_blocks < nblk) return HSLA_ERR_INVALID_ARG;
  Problem p{};
  p.Hq = cfg->num_q_heads;
  p.Hkv = cfg->num_kv_heads;
  p.G = G;
  p.D = cfg->head_dim;
  p.B = B;
  p.top_k = cfg->top_k;
  p.ns = cfg->num_sink;
  p.W = cfg->window;
  p.linear_tail = cfg->linear_tail;
  p.grouped = cfg->selection == HSLA_SEL_GROUPED ? 1 : 0;
  p.tokens = cfg->selection == HSLA_SEL_TOKEN ? 1 : 0;
  p.qrows = 1;
  p.deterministic = cfg->deterministic;
  p.state_all = cfg->state_span == HSLA_STATE_TOKENS ? 1 : 0;
  p.bf16 = cfg->kv_dtype == HSLA_BF16;
  p.sigma = cfg->scale > 0.0f ? cfg->scale : 1.0f / sqrtf(static_cast<float>(cfg->head_dim));
  p.batch = batch;
  p.max_seq_len = max_seq_len;
  p.max_blocks = max_blocks;
  p.nblk_max = static_cast<int>(nblk);
  if (p.tokens) {
    // token indices share a 32-bit list entry with the heads' mask
    if (max_seq_len >= (1 << 20)) return HSLA_ERR_UNSUPPORTED;
    p.nc_max = hsla::candidate_range(max_seq_len, 1, p.ns, p.W).count;
  } else {
    p.nc_max = hsla::candidate_range(max_seq_len, B, p.ns, p.W).count;
    // Per-head selection bitmaps of an attention workgroup live in LDS.
    const size_t bitmap = static_cast<size_t>(G) * ((p.nc_max + 63) / 64) * 8;
    if (bitmap > 16 * 1024) return HSLA_ERR_UNSUPPORTED;
  }
  *out = p;
  return HSLA_OK;
}

hsla_status check_pool(const hsla_kv_pool* pool, bool need_stats) {
  if (!pool || !pool->k_pages || !pool->v_pages || !pool->block_table) return HSLA_ERR_INVALID_ARG;
  if (need_stats && (!pool->blk_mean || !pool->blk_var)) return HSLA_ERR_INVALID_ARG;
  if (pool->num_pages < 1 || pool->max_blocks_per_seq < 1) return HSLA_ERR_INVALID_ARG;
  if (!aligned(pool->k_pages, 16) || !aligned(pool->v_pages, 16) || !aligned(pool->block_table, 4))
    return HSLA_ERR_INVALID_ARG;
  if (need_stats && (!aligned(pool->blk_mean, 16) || !aligned(pool->blk_var, 16))) return HSLA_ERR_INVALID_ARG;
  return HSLA_OK;
}

hsla_status check_state(const hsla_state* st) {
  if (!st || !st->S || !st->z || !st->sv) return HSLA_ERR_INVALID_ARG;
  if (!aligned(st->S, 16) || !aligned(st->z, 16) || !aligned(st->sv, 16)) return HSLA_ERR_INVALID_ARG;
  return HSLA_OK;
}

struct ProfileCtx {
  hsla_profile* prof;
  hipStream_t stream;
  bool failed;
};

void record_event(void* ctx, int idx, const char* name) {
  ProfileCtx* c = static_cast<ProfileCtx*>(ctx);
  if (!c->prof || idx >= c->prof->capacity || idx >= HSLA_MAX_PROFILE_EVENTS) return;
  if (hipEventRecord(c->prof->events[idx], c->stream) != hipSuccess) c->failed = true;
  c->prof->names[idx] = name;
  c->prof->recorded = idx + 1;
}

hsla::CheckTablesArgs check_args(const Problem& p, const hsla_kv_pool* pool, const int32_t* lens, int extra,
                                 int32_t* result) {
  hsla::CheckTablesArgs a{};
  a.block_table = pool->block_table;
  a.seq_lens = lens;
  a.result = result;
  a.batch = p.batch;
  a.max_blocks = pool->max_blocks_per_seq;
  a.num_pages = pool->num_pages;
  a.B = p.B;
  a.max_seq_len = p.max_seq_len;
  a.extra = extra;
  a.min_len = extra > 0 ? 0 : 1;
  return a;
}

#ifdef HSLA_DEBUG_CHECKS
// Debug build: before anything is enqueued, every entry point checks the
// lengths and block-table entries its kernels will use (on the GPU, into a
// file-scope device array; the call waits for the result), and returns
// HSLA_ERR_INVALID_ARG with the first violation on stderr instead of
// launching on a bad table.  Calls are serialised; the wait makes them
// unsuitable for graph capture.
static __device__ int32_t debug_result[2];
std::mutex g_debug_mutex;
void* g_debug_ptr[64] = {};

hsla_status debug_check_tables(const Problem& p, const hsla_kv_pool* pool, const int32_t* lens, int extra,
                               hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_debug_mutex);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return HSLA_ERR_HIP;
  if (!g_debug_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(debug_result)) != hipSuccess || !ptr) return HSLA_ERR_HIP;
    g_debug_ptr[dev] = ptr;
  }
  int32_t* res = static_cast<int32_t*>(g_debug_ptr[dev]);
  const hsla::CheckTablesArgs a = check_args(p, pool, lens, extra, res);
  (void)hipGetLastError();
  if (hsla::launch_check_tables(a, stream) != hipSuccess || hipStreamSynchronize(stream) != hipSuccess)
    return HSLA_ERR_HIP;
  int32_t r[2] = {0, 0};
  if (hipMemcpy(r, res, sizeof(r), hipMemcpyDeviceToHost) != hipSuccess) return HSLA_ERR_HIP;
  if (r[0] == 0) return HSLA_OK;
  const long m = static_cast<long>(a.max_blocks) + 1;
  const int b = static_cast<int>(r[1] / m);
  const long j = r[1] % m - 1;
  int32_t v = 0;
  if (j < 0) {
    (void)hipMemcpy(&v, lens + b, sizeof(v), hipMemcpyDeviceToHost);
    fprintf(stderr, "libhsla (debug checks): %d violation(s); first: sequence %d has length %d (allowed %d .. %d)\n",
            r[0], b, v, a.min_len, a.max_seq_len - a.extra);
  } else {
    (void)hipMemcpy(&v, a.block_table + static_cast<size_t>(b) * a.max_blocks + j, sizeof(v), hipMemcpyDeviceToHost);
    fprintf(stderr, "libhsla (debug checks): %d violation(s); first: block %ld of sequence %d maps to page %d, "
            "outside [0, %d)\n", r[0], j, b, v, a.num_pages);
  }
  return HSLA_ERR_INVALID_ARG;
}
#define HSLA_DEBUG_CHECK(p, pool, lens, extra, stream)                                   \
  do {                                                                                   \
    const hsla_status dbg_ = debug_check_tables((p), (pool), (lens), (extra), (stream)); \
    if (dbg_ != HSLA_OK) return dbg_;                                                    \
  } while (0)
#else
#define HSLA_DEBUG_CHECK(p, pool, lens, extra, stream) \
  do {                                                 \
  } while (0)
#endif

}  // namespace

extern "C" {

const char* hsla_status_string(hsla_status s) {
  switch (s) {
    case HSLA_OK: return "HSLA_OK: success";
    case HSLA_ERR_INVALID_ARG: return "HSLA_ERR_INVALID_ARG: null, misaligned or out-of-range argument";
    case HSLA_ERR_UNSUPPORTED: return "HSLA_ERR_UNSUPPORTED: head_dim, GQA group, block size, dtype or size not built";
    case HSLA_ERR_WORKSPACE: return "HSLA_ERR_WORKSPACE: workspace missing or too small";
    case HSLA_ERR_HIP: return "HSLA_ERR_HIP: a HIP launch failed";
  }
  return "unknown hsla_status";
}

const char* hsla_version(void) { return "hsla 0.1.0 gfx950"; }

size_t hsla_build_workspace_size(const hsla_config* cfg, int32_t batch, int32_t max_seq_len) {
  Problem p;
  if (resolve(cfg, batch, max_seq_len, -1, &p) != HSLA_OK) return 0;
  return hsla::build_layout(p).total;
}

hsla_status hsla_build_state(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state,
                             const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  Problem p;
  hsla_status st = resolve(cfg, batch, max_seq_len, pool ? pool->max_blocks_per_seq : 0, &p);
  if (st != HSLA_OK) return st;
  if ((st = check_pool(pool, true)) != HSLA_OK) return st;
  if ((st = check_state(state)) != HSLA_OK) return st;
  if (!seq_lens || !aligned(seq_lens, 4)) return HSLA_ERR_INVALID_ARG;
  const hsla::BuildLayout L = hsla::build_layout(p);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, 16)) return HSLA_ERR_WORKSPACE;
  hsla::BuildArgs a{};
  a.k_pages = pool->k_pages;
  a.v_pages = pool->v_pages;
  a.blk_mean = pool->blk_mean;
  a.blk_var = pool->blk_var;
  a.block_table = pool->block_table;
  a.S = state->S;
  a.z = state->z;
  a.sv = state->sv;
  a.seq_lens = seq_lens;
  a.ws = static_cast<float*>(workspace);
  HSLA_DEBUG_CHECK(p, pool, seq_lens, 0, stream);
  (void)hipGetLastError();  // a stale error from another runtime user is not ours
  return hsla::launch_build(p, L, a, stream) == hipSuccess ? HSLA_OK : HSLA_ERR_HIP;
}

hsla_status hsla_append_token(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state,
                              const void* k_new, const void* v_new, const int32_t* seq_lens_before,
                              int32_t* seq_lens_after, int32_t batch, int32_t max_seq_len,
                              hipStream_t stream) {
  Problem p;
  hsla_status st = resolve(cfg, batch, max_seq_len, pool ? pool->max_blocks_per_seq : 0, &p);
  if (st != HSLA_OK) return st;
  if ((st = check_pool(pool, true)) != HSLA_OK) return st;
  if ((st = check_state(state)) != HSLA_OK) return st;
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return HSLA_ERR_INVALID_ARG;
  if (!seq_lens_before || !aligned(seq_lens_before, 4)) return HSLA_ERR_INVALID_ARG;
  if (seq_lens_after && (!aligned(seq_lens_after, 4) || seq_lens_after == seq_lens_before))
    return HSLA_ERR_INVALID_ARG;
  hsla::AppendArgs a{};
  a.k_pages = pool->k_pages;
  a.v_pages = pool->v_pages;
  a.blk_mean = pool->blk_mean;
  a.blk_var = pool->blk_var;
  a.block_table = pool->block_table;
  a.S = state->S;
  a.z = state->z;
  a.sv = state->sv;
  a.k_new = k_new;
  a.v_new = v_new;
  a.seq_lens_before = seq_lens_before;
  a.seq_lens_after = seq_lens_after;
  HSLA_DEBUG_CHECK(p, pool, seq_lens_before, 1, stream);
  (void)hipGetLastError();
  return hsla::launch_append(p, a, stream) == hipSuccess ? HSLA_OK : HSLA_ERR_HIP;
}

size_t hsla_decode_workspace_size(const hsla_config* cfg, int32_t batch, int32_t max_seq_len) {
  Problem p;
  if (resolve(cfg, batch, max_seq_len, -1, &p) != HSLA_OK) return 0;
  return hsla::decode_layout(p).total;
}

hsla_status hsla_check_tables(const hsla_config* cfg, const hsla_kv_pool* pool, const int32_t* seq_lens,
                              int32_t batch, int32_t max_seq_len, int32_t extra, int32_t* result,
                              hipStream_t stream) {
  Problem p;
  hsla_status st = resolve(cfg, batch, max_seq_len, pool ? pool->max_blocks_per_seq : 0, &p);
  if (st != HSLA_OK) return st;
  if (!pool || !pool->block_table || !aligned(pool->block_table, 4) || pool->num_pages < 1 ||
      pool->max_blocks_per_seq < 1)
    return HSLA_ERR_INVALID_ARG;
  if (!seq_lens || !aligned(seq_lens, 4) || !result || !aligned(result, 4) || extra < 0) return HSLA_ERR_INVALID_ARG;
  (void)hipGetLastError();
  return hsla::launch_check_tables(check_args(p, pool, seq_lens, extra, result), stream) == hipSuccess
             ? HSLA_OK
             : HSLA_ERR_HIP;
}

hsla_status hsla_check_tables_host(const hsla_config* cfg, int32_t max_blocks_per_seq, int32_t num_pages,
                                   const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                                   int32_t max_seq_len, int32_t extra, int32_t* result) {
  Problem p;
  hsla_status st = resolve(cfg, batch, max_seq_len, max_blocks_per_seq, &p);
  if (st != HSLA_OK) return st;
  if (!block_table || !seq_lens || !result || num_pages < 1 || max_blocks_per_seq < 1 || extra < 0)
    return HSLA_ERR_INVALID_ARG;
  hsla_kv_pool pool{};
  pool.block_table = block_table;
  pool.max_blocks_per_seq = max_blocks_per_seq;
  pool.num_pages = num_pages;
  hsla::check_tables_host(check_args(p, &pool, seq_lens, extra, result));
  return result[0] == 0 ? HSLA_OK : HSLA_ERR_INVALID_ARG;
}

}  // extern "C"

namespace {

// hsla_decode, with the token append taken in when `app` is given.
hsla_status decode_impl(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state, const void* q,
                        const int32_t* seq_lens, int32_t batch, int32_t max_seq_len, float* out, int32_t* sel_idx,
                        void* workspace, size_t workspace_bytes, hipStream_t stream, hsla_profile* prof,
                        const hsla::AppendArgs* app) {
  Problem p;
  hsla_status st = resolve(cfg, batch, max_seq_len, pool ? pool->max_blocks_per_seq : 0, &p);
  if (st != HSLA_OK) return st;
  if ((st = check_pool(pool, true)) != HSLA_OK) return st;
  if ((p.linear_tail || app) && (st = check_state(state)) != HSLA_OK) return st;
  if (!q || !aligned(q, 16) || !out || !aligned(out, 16)) return HSLA_ERR_INVALID_ARG;
  if (!seq_lens || !aligned(seq_lens, 4)) return HSLA_ERR_INVALID_ARG;
  if (sel_idx && !aligned(sel_idx, 4)) return HSLA_ERR_INVALID_ARG;
  if (prof && (prof->capacity < 0 || prof->capacity > HSLA_MAX_PROFILE_EVENTS)) return HSLA_ERR_INVALID_ARG;
  const hsla::DecodeLayout L = hsla::decode_layout(p);
  if (!workspace || workspace_bytes < L.total || !aligned(workspace, 16)) return HSLA_ERR_WORKSPACE;
  hsla::DecodeArgs a{};
  a.k_pages = pool->k_pages;
  a.v_pages = pool->v_pages;
  a.blk_mean = pool->blk_mean;
  a.blk_var = pool->blk_var;
  a.block_table = pool->block_table;
  a.S = p.linear_tail ? state->S : nullptr;
  a.z = p.linear_tail ? state->z : nullptr;
  a.sv = p.linear_tail ? state->sv : nullptr;
  a.q = q;
  a.seq_lens = seq_lens;
  a.out = out;
  a.sel_idx = sel_idx;
  a.ws = static_cast<char*>(workspace);
  if (app) a.app = *app;
  if (app) {
    HSLA_DEBUG_CHECK(p, pool, app->seq_lens_before, 1, stream);
  } else {
    HSLA_DEBUG_CHECK(p, pool, seq_lens, 0, stream);
  }
  ProfileCtx ctx{prof, stream, false};
  if (prof) prof->recorded = 0;
  (void)hipGetLastError();
  const hipError_t e = hsla::launch_decode(p, L, a, stream, prof ? record_event : nullptr, &ctx);
  if (e != hipSuccess || ctx.failed) return HSLA_ERR_HIP;
  return HSLA_OK;
}

}  // namespace

extern "C" {

hsla_status hsla_decode(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state,
                        const void* q, const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                        float* out, int32_t* sel_idx, void* workspace, size_t workspace_bytes,
                        hipStream_t stream, hsla_profile* prof) {
  return decode_impl(cfg, pool, state, q, seq_lens, batch, max_seq_len, out, sel_idx, workspace, workspace_bytes,
                     stream, prof, nullptr);
}

hsla_status hsla_append_decode(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state,
                               const void* k_new, const void* v_new, const int32_t* seq_lens_before,
                               int32_t* seq_lens_after, const void* q, int32_t batch, int32_t max_seq_len,
                               float* out, int32_t* sel_idx, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, hsla_profile* prof) {
  if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16)) return HSLA_ERR_INVALID_ARG;
  if (!seq_lens_before || !aligned(seq_lens_before, 4)) return HSLA_ERR_INVALID_ARG;
  if (!seq_lens_after || !aligned(seq_lens_after, 4) || seq_lens_after == seq_lens_before)
    return HSLA_ERR_INVALID_ARG;
  if (!state) return HSLA_ERR_INVALID_ARG;
  if (!pool) return HSLA_ERR_INVALID_ARG;
  hsla::AppendArgs a{};
  a.k_pages = pool->k_pages;
  a.v_pages = pool->v_pages;
  a.blk_mean = pool->blk_mean;
  a.blk_var = pool->blk_var;
  a.block_table = pool->block_table;
  a.S = state->S;
  a.z = state->z;
  a.sv = state->sv;
  a.k_new = k_new;
  a.v_new = v_new;
  a.seq_lens_before = seq_lens_before;
  a.seq_lens_after = seq_lens_after;
  return decode_impl(cfg, pool, state, q, seq_lens_after, batch, max_seq_len, out, sel_idx, workspace,
                     workspace_bytes, stream, prof, &a);
}

}  // extern "C"

namespace {

// The no-allocation variant of hsla_append_decode: the decode workspace is a
// file-scope device array of fixed size.  Every GPU the library runs on
// holds its own copy (until the process ends); its address on a device is
// looked up once, with that device current, and kept.  Like the workspace
// it stands in for, its contents on entry do not matter.
constexpr size_t kNoAllocScratchBytes = HSLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device (nullptr on a
// HIP error).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

// The multi-query form's shapes: `seq` over the sequences (append), `rows`
// over the batch x q_len query rows (decode).  Workspace: the decode's, then
// the rows' lengths.
hsla_status resolve_chunk(const hsla_config* cfg, int32_t batch, int32_t q_len, int32_t max_seq_len,
                          int32_t max_blocks, Problem* seq, Problem* rows, size_t* ws_rows, size_t* ws_total) {
  hsla_status st = resolve(cfg, batch, max_seq_len, max_blocks, seq);
  if (st != HSLA_OK) return st;
  if (seq->tokens || seq->state_all) return HSLA_ERR_UNSUPPORTED;
  if (q_len < 1 || q_len > seq->B || q_len > seq->W - seq->B + 1 || q_len > max_seq_len) return HSLA_ERR_INVALID_ARG;
  if (static_cast<long>(batch) * q_len > (1L << 24)) return HSLA_ERR_INVALID_ARG;
  if ((st = resolve(cfg, batch * q_len, max_seq_len, max_blocks, rows)) != HSLA_OK) return st;
  rows->qrows = q_len;
  rows->chunk = 1;
  const size_t dec = hsla::decode_layout(*rows).total;
  *ws_rows = (dec + 255) / 256 * 256;
  *ws_total = *ws_rows + sizeof(int32_t) * static_cast<size_t>(batch) * q_len;
  return HSLA_OK;
}

}  // namespace

extern "C" {

size_t hsla_prefill_chunk_workspace_size(const hsla_config* cfg, int32_t batch, int32_t q_len,
                                         int32_t max_seq_len) {
  Problem seq, rows;
  size_t off = 0, total = 0;
  if (resolve_chunk(cfg, batch, q_len, max_seq_len, -1, &seq, &rows, &off, &total) != HSLA_OK) return 0;
  return total;
}

hsla_status hsla_prefill_chunk(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state,
                               const void* k_chunk, const void* v_chunk, const int32_t* seq_lens_before,
                               int32_t* seq_lens_after, const void* q, int32_t batch, int32_t q_len,
                               int32_t max_seq_len, float* out, int32_t* sel_idx, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  Problem seq, rows;
  size_t off = 0, total = 0;
  hsla_status st = resolve_chunk(cfg, batch, q_len, max_seq_len, pool ? pool->max_blocks_per_seq : 0, &seq, &rows,
                                 &off, &total);
  if (st != HSLA_OK) return st;
  if ((st = check_pool(pool, true)) != HSLA_OK) return st;
  if ((st = check_state(state)) != HSLA_OK) return st;
  if (!k_chunk || !v_chunk || !aligned(k_chunk, 16) || !aligned(v_chunk, 16)) return HSLA_ERR_INVALID_ARG;
  if (!seq_lens_before || !aligned(seq_lens_before, 4)) return HSLA_ERR_INVALID_ARG;
  if (!seq_lens_after || !aligned(seq_lens_after, 4) || seq_lens_after == seq_lens_before)
    return HSLA_ERR_INVALID_ARG;
  if (!q || !aligned(q, 16) || !out || !aligned(out, 16)) return HSLA_ERR_INVALID_ARG;
  if (sel_idx && !aligned(sel_idx, 4)) return HSLA_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < total || !aligned(workspace, 16)) return HSLA_ERR_WORKSPACE;
  int32_t* row_lens = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + off);

  hsla::AppendArgs a{};
  a.k_pages = pool->k_pages;
  a.v_pages = pool->v_pages;
  a.blk_mean = pool->blk_mean;
  a.blk_var = pool->blk_var;
  a.block_table = pool->block_table;
  a.S = state->S;
  a.z = state->z;
  a.sv = state->sv;
  a.k_new = k_chunk;
  a.v_new = v_chunk;
  a.seq_lens_before = seq_lens_before;
  a.seq_lens_after = seq_lens_after;

  hsla::DecodeArgs d{};
  d.k_pages = pool->k_pages;
  d.v_pages = pool->v_pages;
  d.blk_mean = pool->blk_mean;
  d.blk_var = pool->blk_var;
  d.block_table = pool->block_table;
  d.S = rows.linear_tail ? state->S : nullptr;
  d.z = rows.linear_tail ? state->z : nullptr;
  d.sv = rows.linear_tail ? state->sv : nullptr;
  d.q = q;
  d.seq_lens = row_lens;
  d.out = out;
  d.sel_idx = sel_idx;
  d.ws = static_cast<char*>(workspace);

  HSLA_DEBUG_CHECK(seq, pool, seq_lens_before, q_len, stream);
  (void)hipGetLastError();
  // 1. the chunk's page slots and the query rows' lengths; 2. every query
  // against the cache as it stood before the chunk's blocks were folded; 3.
  // the fold of the completed block and the new lengths
  if (hsla::launch_append(seq, a, stream, q_len, hsla::kAppendWriteRows, row_lens) != hipSuccess) return HSLA_ERR_HIP;
  if (hsla::launch_decode(rows, hsla::decode_layout(rows), d, stream, nullptr, nullptr) != hipSuccess)
    return HSLA_ERR_HIP;
  if (hsla::launch_append(seq, a, stream, q_len, hsla::kAppendFold, nullptr) != hipSuccess) return HSLA_ERR_HIP;
  return HSLA_OK;
}

}  // extern "C"

extern "C" {

size_t hsla_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

hsla_status hsla_append_decode_noalloc(const hsla_config* cfg, const hsla_kv_pool* pool, const hsla_state* state,
                                       const void* k_new, const void* v_new, const int32_t* seq_lens_before,
                                       int32_t* seq_lens_after, const void* q, int32_t batch, int32_t max_seq_len,
                                       float* out, int32_t* sel_idx, hipStream_t stream) {
  const size_t need = hsla_decode_workspace_size(cfg, batch, max_seq_len);
  if (need == 0) {   // the configuration itself is rejected: the same status as the workspace form
    Problem p;
    const hsla_status st = resolve(cfg, batch, max_seq_len, -1, &p);
    return st != HSLA_OK ? st : HSLA_ERR_INVALID_ARG;
  }
  if (need > kNoAllocScratchBytes) {
    fprintf(stderr, "libhsla: hsla_append_decode_noalloc needs %zu bytes of scratch, more than its %zu\n", need,
            kNoAllocScratchBytes);
    return HSLA_ERR_WORKSPACE;
  }
  void* ws = scratch_on_current_device();
  if (!ws) return HSLA_ERR_HIP;
  return hsla_append_decode(cfg, pool, state, k_new, v_new, seq_lens_before, seq_lens_after, q, batch, max_seq_len,
                            out, sel_idx, ws, kNoAllocScratchBytes, stream, nullptr);
}

size_t hsla_phase_timestamp_bytes(void) { return hsla::phase_bytes(); }

hsla_status hsla_phase_timestamps(void* host, size_t bytes, int32_t clear) {
  const size_t need = hsla::phase_bytes();
  if (need == 0) return HSLA_ERR_UNSUPPORTED;
  if (!host || bytes < need) return HSLA_ERR_INVALID_ARG;
  return hsla::phase_copy(host, clear != 0) == hipSuccess ? HSLA_OK : HSLA_ERR_HIP;
}

}  // extern "C"
