// extern "C" entry points of libamdoscar.so (see include/oscar.h): argument
// validation on the host, then kernel launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

#include "../../include/oscar.h"
#include "calibrate.h"
#include "launchers.h"

using namespace oscar;

namespace {

oscar_status check_desc(const oscar_layer_desc* d) {
  if (!d) return OSCAR_ERR_INVALID;
  if (d->head_dim != 128 || d->page_size != 16 || d->n_sink != 64 || d->n_recent != 256 || d->group_size != 32)
    return OSCAR_ERR_UNSUPPORTED;
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0) return OSCAR_ERR_INVALID;
  if (d->num_q_heads % d->num_kv_heads != 0) return OSCAR_ERR_INVALID;
  const int g = d->num_q_heads / d->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return OSCAR_ERR_UNSUPPORTED;
  return OSCAR_OK;
}

oscar_status check_pool(const oscar_pool* p, bool need_hist_tiers) {
  if (!p) return OSCAR_ERR_INVALID;
  if (!p->sink_k || !p->sink_v || !p->recent_k || !p->recent_v) return OSCAR_ERR_INVALID;
  if (need_hist_tiers && (!p->hist || !p->page_table)) return OSCAR_ERR_INVALID;
  if (!p->rot_k || !p->rot_v || !p->clip_k || !p->clip_v) return OSCAR_ERR_INVALID;
  if (p->rot_per_kv_head != 0 && p->rot_per_kv_head != 1) return OSCAR_ERR_INVALID;
  if (p->code_bits != 2 && p->code_bits != 4) return OSCAR_ERR_UNSUPPORTED;
  if (p->n_slots <= 0 || p->max_pages_per_seq < 0 || p->num_pages < 0) return OSCAR_ERR_INVALID;
  return OSCAR_OK;
}

thread_local char g_hip_error[160] = "";

// elements between consecutive KV heads' rotations / clip thresholds (0:
// one pair shared by the layer)
int rot_stride(const oscar_pool* p) { return p->rot_per_kv_head ? 128 * 128 : 0; }
int clip_stride(const oscar_pool* p) { return p->rot_per_kv_head ? 128 : 0; }

oscar_status hip_status(hipError_t e) {
  if (e == hipSuccess) return OSCAR_OK;
  snprintf(g_hip_error, sizeof(g_hip_error), "HIP runtime error: %s (%s)", hipGetErrorName(e), hipGetErrorString(e));
  return OSCAR_ERR_HIP;
}

}  // namespace

namespace {
// Several query tokens per sequence: the query heads' virtual heads (t, h)
// of one KV head are split into work-item column groups of `group` columns,
// the largest power of two (at most max_group) that divides n_query * G.
// The INT2 kernel takes 16 columns (one head per column) only when that still
// leaves two or more groups: at 16 virtual heads, two 8-column groups keep
// twice the workgroups busy and are faster on one long sequence.
constexpr int kMaxQueryTokens = 256;
struct QueryColumns {
  int group;
  int n_colgroups;
};
QueryColumns query_columns(const oscar_layer_desc* d, int n_query, int max_group) {
  const int v = n_query * (d->num_q_heads / d->num_kv_heads);
  int group = max_group;
  while (v % group != 0) group >>= 1;
  return QueryColumns{group, v / group};
}
QueryColumns int2_query_columns(const oscar_layer_desc* d, int n_query) {
  const int v = n_query * (d->num_q_heads / d->num_kv_heads);
  return query_columns(d, n_query, v >= 32 ? 16 : 8);
}
constexpr int kMaxBf16Columns = 8;
}  // namespace

// which launches of a tiered decode call run
enum DecodePhases { kPhaseSplits = 1, kPhaseMerge = 2, kPhaseBoth = 3 };
static oscar_status decode_tiered(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                                  const int32_t* seq_len, const void* q, int32_t n_query, float* out,
                                  void* workspace, size_t ws_bytes, int32_t batch, int32_t max_seq_len, void* stream,
                                  int phases = kPhaseBoth, const void* k_new = nullptr, const void* v_new = nullptr,
                                  int len_offset = 0);

namespace {
oscar_status check_append(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                          const int32_t* position, const void* k_new, const void* v_new, int32_t batch) {
  oscar_status st = check_desc(desc);
  if (st != OSCAR_OK) return st;
  if ((st = check_pool(pool, true)) != OSCAR_OK) return st;
  if (!position || !k_new || !v_new || batch <= 0) return OSCAR_ERR_INVALID;
  if (!seq_slot && batch > pool->n_slots) return OSCAR_ERR_INVALID;
  return OSCAR_OK;
}

AppendArgs append_args(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                       const int32_t* position, const void* k_new, const void* v_new) {
  AppendArgs a{};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.seq_slot = seq_slot;
  a.position = position;
  a.sink_k = static_cast<uint16_t*>(pool->sink_k);
  a.sink_v = static_cast<uint16_t*>(pool->sink_v);
  a.recent_k = static_cast<uint16_t*>(pool->recent_k);
  a.recent_v = static_cast<uint16_t*>(pool->recent_v);
  a.hist = pool->hist;
  a.page_table = pool->page_table;
  a.rot_k = pool->rot_k; a.rot_v = pool->rot_v;
  a.clip_k = pool->clip_k; a.clip_v = pool->clip_v;
  a.rot_kv_stride = rot_stride(pool); a.clip_kv_stride = clip_stride(pool);
  a.code_bits = pool->code_bits;
  a.hkv = desc->num_kv_heads;
  a.max_pages = pool->max_pages_per_seq;
  return a;
}
}  // namespace

extern "C" {

int32_t oscar_abi_version(void) { return OSCAR_ABI_VERSION; }

const char* oscar_status_string(oscar_status s) {
  switch (s) {
    case OSCAR_OK: return "ok";
    case OSCAR_ERR_INVALID: return "invalid argument";
    case OSCAR_ERR_UNSUPPORTED: return "unsupported shape";
    case OSCAR_ERR_CAPACITY: return "workspace or page table too small";
    case OSCAR_ERR_HIP: return g_hip_error[0] ? g_hip_error : "HIP runtime error";
    case OSCAR_ERR_NUMERIC: return "non-finite or out-of-range calibration value";
  }
  return "unknown status";
}

oscar_status oscar_calibrate_layers(const oscar_layer_desc* desc, const oscar_calib_opts* opts, int32_t n_layers,
                                    const float* q, const float* k, const float* v, int64_t n_tokens, float* rot_k,
                                    float* rot_v, float* clip_k, float* clip_v) {
  oscar_status st = check_desc(desc);
  if (st != OSCAR_OK) return st;
  if (!opts || !q || !k || !v || !rot_k || !rot_v || !clip_k || !clip_v || n_tokens < 2 || n_layers < 1)
    return OSCAR_ERR_INVALID;
  if (opts->hadamard_block != 32 && opts->hadamard_block != 128) return OSCAR_ERR_UNSUPPORTED;
  if (!(opts->clip_percentile > 0.0f && opts->clip_percentile <= 100.0f)) return OSCAR_ERR_INVALID;
  if (opts->rotation < OSCAR_ROT_SPECTRAL || opts->rotation > OSCAR_ROT_IDENTITY) return OSCAR_ERR_INVALID;
  if (opts->per_kv_head != 0 && opts->per_kv_head != 1) return OSCAR_ERR_INVALID;
  const int rc = calibrate_layers(desc->num_q_heads, desc->num_kv_heads, n_layers, opts->hadamard_block,
                                  opts->clip_percentile, opts->rotation, opts->per_kv_head == 1, q, k, v, n_tokens,
                                  rot_k, rot_v, clip_k, clip_v);
  return rc == 0 ? OSCAR_OK : (rc == -2 ? OSCAR_ERR_INVALID : OSCAR_ERR_NUMERIC);
}

oscar_status oscar_calibrate(const oscar_layer_desc* desc, const oscar_calib_opts* opts, const float* q,
                             const float* k, const float* v, int64_t n_tokens, float* rot_k, float* rot_v,
                             float* clip_k, float* clip_v) {
  return oscar_calibrate_layers(desc, opts, 1, q, k, v, n_tokens, rot_k, rot_v, clip_k, clip_v);
}

oscar_status oscar_append(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                          const int32_t* position, const void* k_new, const void* v_new, int32_t batch,
                          void* stream) {
  const oscar_status st = check_append(desc, pool, seq_slot, position, k_new, v_new, batch);
  if (st != OSCAR_OK) return st;
  const AppendArgs a = append_args(desc, pool, seq_slot, position, k_new, v_new);
  return hip_status(launch_append(a, batch, static_cast<hipStream_t>(stream)));
}

static oscar_status demote_common(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                                  const int32_t* hist_start, const int32_t* length, const void* k, const void* v,
                                  int32_t src_kind, int32_t batch, int32_t src_tokens, int32_t src_tok0,
                                  int32_t n_tokens, int32_t max_count, void* stream) {
  DemoteArgs a{};
  if (src_kind == OSCAR_SRC_BF16) {
    a.src_k = static_cast<const uint16_t*>(k);
    a.src_v = static_cast<const uint16_t*>(v);
  } else if (src_kind == OSCAR_SRC_F32_ROTATED) {
    a.src_k_f32 = static_cast<const float*>(k);
    a.src_v_f32 = static_cast<const float*>(v);
  } else {
    return OSCAR_ERR_INVALID;
  }
  a.src_tokens = src_tokens;
  a.src_tok0 = src_tok0;
  a.n_tokens = n_tokens;
  a.length = length;
  a.hist_start = hist_start;
  a.seq_slot = seq_slot;
  a.rot_k = pool->rot_k; a.rot_v = pool->rot_v;
  a.clip_k = pool->clip_k; a.clip_v = pool->clip_v;
  a.rot_kv_stride = rot_stride(pool); a.clip_kv_stride = clip_stride(pool);
  a.code_bits = pool->code_bits;
  a.hist = pool->hist;
  a.page_table = pool->page_table;
  a.max_pages = pool->max_pages_per_seq;
  a.hkv = desc->num_kv_heads;
  return hip_status(launch_demote(a, batch, max_count, src_kind == OSCAR_SRC_F32_ROTATED,
                                  static_cast<hipStream_t>(stream)));
}

oscar_status oscar_demote(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                          const int32_t* hist_start, const void* k, const void* v, int32_t src_kind, int32_t batch,
                          int32_t n_tokens, void* stream) {
  oscar_status st = check_desc(desc);
  if (st != OSCAR_OK) return st;
  if ((st = check_pool(pool, true)) != OSCAR_OK) return st;
  if (!hist_start || !k || !v || batch <= 0 || n_tokens < 0) return OSCAR_ERR_INVALID;
  if (!seq_slot && batch > pool->n_slots) return OSCAR_ERR_INVALID;
  if (n_tokens == 0) return OSCAR_OK;
  return demote_common(desc, pool, seq_slot, hist_start, nullptr, k, v, src_kind, batch, n_tokens, 0, n_tokens,
                       n_tokens, stream);
}

oscar_status oscar_prefill(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                           const int32_t* length, const void* k, const void* v, int32_t batch, int32_t max_len,
                           void* stream) {
  oscar_status st = check_desc(desc);
  if (st != OSCAR_OK) return st;
  if ((st = check_pool(pool, max_len > 320)) != OSCAR_OK) return st;
  if (!length || !k || !v || batch <= 0 || max_len <= 0) return OSCAR_ERR_INVALID;
  if (!seq_slot && batch > pool->n_slots) return OSCAR_ERR_INVALID;
  const int max_hist = max_len - 320;
  if (max_hist > 0 && (max_hist + 15) / 16 > pool->max_pages_per_seq) return OSCAR_ERR_CAPACITY;
  PrefillArgs pa{};
  pa.src_k = static_cast<const uint16_t*>(k);
  pa.src_v = static_cast<const uint16_t*>(v);
  pa.length = length;
  pa.seq_slot = seq_slot;
  pa.sink_k = static_cast<uint16_t*>(pool->sink_k);
  pa.sink_v = static_cast<uint16_t*>(pool->sink_v);
  pa.recent_k = static_cast<uint16_t*>(pool->recent_k);
  pa.recent_v = static_cast<uint16_t*>(pool->recent_v);
  pa.max_len = max_len;
  pa.hkv = desc->num_kv_heads;
  const oscar_status rs = hip_status(launch_prefill_route(pa, batch, static_cast<hipStream_t>(stream)));
  if (rs != OSCAR_OK) return rs;
  if (max_hist <= 0) return OSCAR_OK;
  return demote_common(desc, pool, seq_slot, nullptr, length, k, v, OSCAR_SRC_BF16, batch, max_len, 64, 0,
                       max_hist, stream);
}

size_t oscar_decode_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t max_seq_len) {
  return oscar_decode_multi_workspace_bytes(desc, batch, 1, max_seq_len);
}

size_t oscar_decode_multi_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t n_query,
                                          int32_t max_seq_len) {
  if (check_desc(desc) != OSCAR_OK || batch <= 0 || max_seq_len <= 0 || n_query < 1 || n_query > kMaxQueryTokens)
    return 0;
  const QueryColumns c = int2_query_columns(desc, n_query);
  return plan_decode(batch, desc->num_kv_heads, c.group, c.n_colgroups, max_seq_len).workspace_bytes;
}

oscar_status oscar_decode(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                          const int32_t* seq_len, const void* q, float* out, void* workspace, size_t ws_bytes,
                          int32_t batch, int32_t max_seq_len, void* stream) {
  return oscar_decode_multi(desc, pool, seq_slot, seq_len, q, 1, out, workspace, ws_bytes, batch, max_seq_len, stream);
}

oscar_status oscar_decode_multi(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                                const int32_t* seq_len, const void* q, int32_t n_query, float* out, void* workspace,
                                size_t ws_bytes, int32_t batch, int32_t max_seq_len, void* stream) {
  return decode_tiered(desc, pool, seq_slot, seq_len, q, n_query, out, workspace, ws_bytes, batch, max_seq_len,
                       stream);
}

oscar_status oscar_decode_partials(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                                   const int32_t* seq_len, const void* q, void* workspace, size_t ws_bytes,
                                   int32_t batch, int32_t max_seq_len, void* stream) {
  return decode_tiered(desc, pool, seq_slot, seq_len, q, 1, nullptr, workspace, ws_bytes, batch, max_seq_len,
                       stream, kPhaseSplits);
}

oscar_status oscar_decode_merge(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_len,
                                float* out, void* workspace, size_t ws_bytes, int32_t batch, int32_t max_seq_len,
                                void* stream) {
  return decode_tiered(desc, pool, nullptr, seq_len, nullptr, 1, out, workspace, ws_bytes, batch, max_seq_len,
                       stream, kPhaseMerge);
}
}  // extern "C"

// Tiered decode (split kernel + merge, or one of them).  The fused step
// passes the new token (k_new, v_new) and its positions as seq_len with
// len_offset 1.
static oscar_status decode_tiered(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                                  const int32_t* seq_len, const void* q, int32_t n_query, float* out,
                                  void* workspace, size_t ws_bytes, int32_t batch, int32_t max_seq_len, void* stream,
                                  int phases, const void* k_new, const void* v_new, int len_offset) {
  oscar_status st = check_desc(desc);
  if (st != OSCAR_OK) return st;
  if ((st = check_pool(pool, max_seq_len > 320)) != OSCAR_OK) return st;
  if (!seq_len || !workspace || batch <= 0 || max_seq_len <= 0) return OSCAR_ERR_INVALID;
  if (((phases & kPhaseSplits) && !q) || ((phases & kPhaseMerge) && !out)) return OSCAR_ERR_INVALID;
  if (n_query < 1 || max_seq_len < n_query) return OSCAR_ERR_INVALID;
  if (n_query > kMaxQueryTokens) return OSCAR_ERR_UNSUPPORTED;
  if ((phases & kPhaseSplits) && !seq_slot && batch > pool->n_slots) return OSCAR_ERR_INVALID;
  const int hkv = desc->num_kv_heads, g = desc->num_q_heads / hkv;
  const int max_hist = max_seq_len - 320;
  if (max_hist > 0 && (max_hist + 15) / 16 > pool->max_pages_per_seq) return OSCAR_ERR_CAPACITY;
  const QueryColumns c = int2_query_columns(desc, n_query);
  const DecodePlan plan = plan_decode(batch, hkv, c.group, c.n_colgroups, max_seq_len);
  if (!plan.ok) return OSCAR_ERR_UNSUPPORTED;
  if (ws_bytes < plan.workspace_bytes) return OSCAR_ERR_CAPACITY;
  DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.out = out;
  a.seq_slot = seq_slot;
  a.seq_len = seq_len;
  a.len_offset = len_offset;
  a.sink_k = static_cast<const uint16_t*>(pool->sink_k);
  a.sink_v = static_cast<const uint16_t*>(pool->sink_v);
  a.recent_k = static_cast<const uint16_t*>(pool->recent_k);
  a.recent_v = static_cast<const uint16_t*>(pool->recent_v);
  a.hist = pool->hist;
  a.page_table = pool->page_table;
  a.rot_k = pool->rot_k;
  a.rot_v = pool->rot_v;
  a.rot_kv_stride = rot_stride(pool);
  a.clip_k = pool->clip_k;
  a.clip_v = pool->clip_v;
  a.clip_kv_stride = clip_stride(pool);
  a.code_bits = pool->code_bits;
  // the fused step: this step's token reaches its sink or ring slot, and the
  // token leaving the ring its history slot, in the decode launch
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.partials = static_cast<float*>(workspace);
  a.hkv = hkv;
  a.max_pages = pool->max_pages_per_seq;
  a.n_hist_splits = plan.n_hist_splits;
  a.pages_per_split = plan.pages_per_split;
  a.n_tile_splits = plan.n_tile_splits;
  a.tile_tokens = plan.tile_tokens;
  a.tiles_last = plan.tiles_last ? 1 : 0;
  a.n_groups_total = batch * hkv * c.n_colgroups;
  a.grid_per_xcd = plan.grid / 8;
  a.q_tokens = n_query;
  a.g_model = g;
  a.n_colgroups = c.n_colgroups;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((phases & kPhaseSplits) && (st = hip_status(launch_decode(a, c.group, plan.grid, hs))) != OSCAR_OK) return st;
  if (!(phases & kPhaseMerge)) return OSCAR_OK;
  MergeArgs m{};
  m.partials = a.partials;
  m.seq_len = seq_len;
  m.len_offset = len_offset;
  m.rot = pool->rot_v;
  m.rot_kv_stride = rot_stride(pool);
  m.out = out;
  m.hkv = hkv;
  m.group = c.group;
  m.q_tokens = n_query;
  m.g_model = g;
  m.n_colgroups = c.n_colgroups;
  m.n_splits_total = plan.n_splits_total;
  m.n_plain_slots = plan.n_tile_splits;
  m.pages_per_split = plan.pages_per_split;
  m.tiered = 1;
  m.tile_tokens = plan.tile_tokens;
  return hip_status(launch_merge(m, batch * n_query * desc->num_q_heads, hs));
}

extern "C" {

size_t oscar_decode_bf16_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t max_seq_len) {
  return oscar_decode_bf16_multi_workspace_bytes(desc, batch, 1, max_seq_len);
}

size_t oscar_decode_bf16_multi_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t n_query,
                                               int32_t max_seq_len) {
  if (check_desc(desc) != OSCAR_OK || batch <= 0 || max_seq_len <= 0 || n_query < 1 || n_query > kMaxQueryTokens)
    return 0;
  const QueryColumns c = query_columns(desc, n_query, kMaxBf16Columns);
  return plan_decode_bf16(batch, desc->num_kv_heads, c.group, c.n_colgroups, max_seq_len).workspace_bytes;
}

oscar_status oscar_decode_bf16(const oscar_layer_desc* desc, const oscar_bf16_pool* pool, const int32_t* seq_slot,
                               const int32_t* seq_len, const void* q, float* out, void* workspace, size_t ws_bytes,
                               int32_t batch, int32_t max_seq_len, void* stream) {
  return oscar_decode_bf16_multi(desc, pool, seq_slot, seq_len, q, 1, out, workspace, ws_bytes, batch, max_seq_len,
                                 stream);
}

oscar_status oscar_decode_bf16_multi(const oscar_layer_desc* desc, const oscar_bf16_pool* pool,
                                     const int32_t* seq_slot, const int32_t* seq_len, const void* q, int32_t n_query,
                                     float* out, void* workspace, size_t ws_bytes, int32_t batch,
                                     int32_t max_seq_len, void* stream) {
  oscar_status st = check_desc(desc);
  if (st != OSCAR_OK) return st;
  if (!pool || !pool->kv || !pool->page_table || pool->n_slots <= 0) return OSCAR_ERR_INVALID;
  if (!seq_len || !q || !out || !workspace || batch <= 0 || max_seq_len <= 0) return OSCAR_ERR_INVALID;
  if (n_query < 1 || max_seq_len < n_query) return OSCAR_ERR_INVALID;
  if (n_query > kMaxQueryTokens) return OSCAR_ERR_UNSUPPORTED;
  if (!seq_slot && batch > pool->n_slots) return OSCAR_ERR_INVALID;
  if ((max_seq_len + 15) / 16 > pool->max_pages_per_seq) return OSCAR_ERR_CAPACITY;
  const int hkv = desc->num_kv_heads, g = desc->num_q_heads / hkv;
  const QueryColumns c = query_columns(desc, n_query, kMaxBf16Columns);
  const DecodePlan plan = plan_decode_bf16(batch, hkv, c.group, c.n_colgroups, max_seq_len);
  if (!plan.ok) return OSCAR_ERR_UNSUPPORTED;
  if (ws_bytes < plan.workspace_bytes) return OSCAR_ERR_CAPACITY;
  DecodeBf16Args a{};
  a.q = static_cast<const uint16_t*>(q);
  a.out = out;
  a.seq_slot = seq_slot;
  a.seq_len = seq_len;
  a.kv = static_cast<const uint16_t*>(pool->kv);
  a.page_table = pool->page_table;
  a.partials = static_cast<float*>(workspace);
  a.hkv = hkv;
  a.max_pages = pool->max_pages_per_seq;
  a.n_splits = plan.n_splits_total;
  a.pages_per_split = plan.pages_per_split;
  a.n_groups_total = batch * hkv * c.n_colgroups;
  a.grid_per_xcd = plan.grid / 8;
  a.q_tokens = n_query;
  a.g_model = g;
  a.n_colgroups = c.n_colgroups;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((st = hip_status(launch_decode_bf16(a, c.group, plan.grid, hs))) != OSCAR_OK) return st;
  MergeArgs m{};
  m.partials = a.partials;
  m.seq_len = seq_len;
  m.rot = nullptr;
  m.out = out;
  m.hkv = hkv;
  m.group = c.group;
  m.q_tokens = n_query;
  m.g_model = g;
  m.n_colgroups = c.n_colgroups;
  m.n_splits_total = plan.n_splits_total;
  m.n_plain_slots = plan.n_splits_total;
  m.pages_per_split = plan.pages_per_split;
  m.tiered = 0;
  return hip_status(launch_merge(m, batch * n_query * desc->num_q_heads, hs));
}

size_t oscar_step_workspace_bytes(const oscar_layer_desc* desc, int32_t batch, int32_t max_seq_len) {
  return oscar_decode_workspace_bytes(desc, batch, max_seq_len);
}

oscar_status oscar_step(const oscar_layer_desc* desc, const oscar_pool* pool, const int32_t* seq_slot,
                        const int32_t* position, const void* k_new, const void* v_new, const void* q, float* out,
                        void* workspace, size_t ws_bytes, int32_t batch, int32_t max_seq_len, void* stream) {
  oscar_status st = check_append(desc, pool, seq_slot, position, k_new, v_new, batch);
  if (st != OSCAR_OK) return st;
  if (!q || !out || !workspace || max_seq_len < 1) return OSCAR_ERR_INVALID;
  const size_t need = oscar_step_workspace_bytes(desc, batch, max_seq_len);
  if (need == 0) return OSCAR_ERR_UNSUPPORTED;
  if (ws_bytes < need) return OSCAR_ERR_CAPACITY;
  // one decode launch appends (the new token into its tier; from position
  // 320 on, the token leaving the ring into history) and attends; the
  // cached length is position + 1
  return decode_tiered(desc, pool, seq_slot, position, q, 1, out, workspace, ws_bytes, batch, max_seq_len, stream,
                       kPhaseBoth, k_new, v_new, 1);
}

}  // extern "C"
