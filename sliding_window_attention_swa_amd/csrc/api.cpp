// C ABI of libswa: argument checks on the host, then kernel launches on the
// caller's stream.  Every check runs before any HIP call, so argument errors
// never touch the device.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

#include "common.hpp"

namespace {

constexpr int32_t kHeadDim = 128;
// gfx950 (MI355X) has 256 compute units.  A full-layer split is streamed by
// one wavefront per (request, kv head, split); planning targets about four such
// streams per CU: more streams only add outstanding requests to a path whose
// limit is address translation and DRAM, not issue slots.
constexpr int64_t kTargetStreams = 1024;
constexpr int64_t kMinKeysPerSplit = 512;
constexpr int32_t kMaxSplits = 1024;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_group(int32_t q_heads, int32_t kv_heads) {
  if (kv_heads <= 0 || q_heads <= 0 || q_heads % kv_heads) return false;
  const int32_t g = q_heads / kv_heads;
  return g == 1 || g == 2 || g == 4 || g == 8 || g == 16;
}

swa_status_t from_hip(hipError_t e) { return e == hipSuccess ? SWA_OK : SWA_E_HIP; }

swa_status_t check_layer(const swa_kv_layer_t *layer) {
  if (!layer || !layer->k || !layer->v) return SWA_E_ARG;
  if (layer->rows < 1 || layer->kv_heads < 1 || layer->head_dim < 1) return SWA_E_ARG;
  if (layer->dtype != SWA_F32 && layer->dtype != SWA_BF16 && layer->dtype != SWA_FP8_E4M3) return SWA_E_DTYPE;
  if (!aligned16(layer->k) || !aligned16(layer->v)) return SWA_E_ARG;
  if (layer->dtype == SWA_FP8_E4M3) {
    if (!(layer->k_scale > 0.f) || !(layer->v_scale > 0.f) || !std::isfinite(layer->k_scale) ||
        !std::isfinite(layer->v_scale))
      return SWA_E_ARG;
  }
  return SWA_OK;
}

swa_status_t check_index(const swa_index_t *idx, bool need_r2t) {
  if (!idx || idx->batch < 0) return SWA_E_ARG;
  if (idx->batch == 0) return SWA_OK;
  if (!idx->seq_lens) return SWA_E_ARG;
  if (need_r2t) {
    if (!idx->req_to_token || !idx->req_pool_idx || idx->r2t_rows < 1 || idx->r2t_stride < 1) return SWA_E_ARG;
  }
  if (idx->full_to_swa && idx->map_len < 2) return SWA_E_ARG;
  return SWA_OK;
}

// Slots pass through int32 window tables, so a pool addressed through them
// must have fewer than 2^31 rows.
constexpr int64_t kMaxRows = INT32_MAX;

}  // namespace

extern "C" {

swa_status_t swa_pool_config(int64_t avail_bytes, double ratio, int32_t page_size, int32_t window,
                             int32_t n_full_layers, int64_t full_bytes_per_token, int32_t n_swa_layers,
                             int64_t swa_bytes_per_token, int64_t *n_full_tokens, int64_t *n_swa_tokens) {
  if (!n_full_tokens || !n_swa_tokens) return SWA_E_ARG;
  if (page_size <= 0 || avail_bytes < 0 || !(ratio >= 0.0) || !std::isfinite(ratio) || window < -1 ||
      n_full_layers < 0 || n_swa_layers < 0 || full_bytes_per_token < 0 || swa_bytes_per_token < 0)
    return SWA_E_ARG;
  const double cell = static_cast<double>(full_bytes_per_token) * n_full_layers +
                      ratio * static_cast<double>(swa_bytes_per_token) * n_swa_layers;
  if (!(cell > 0.0)) return SWA_E_ARG;
  int64_t n_full = static_cast<int64_t>(std::floor(static_cast<double>(avail_bytes) / cell));
  n_full = n_full / page_size * page_size;
  int64_t n_swa = static_cast<int64_t>(std::floor(ratio * static_cast<double>(n_full)));
  n_swa = n_swa / page_size * page_size;
  *n_full_tokens = n_full;
  *n_swa_tokens = n_swa;
  if (n_swa <= static_cast<int64_t>(window) + page_size) return SWA_E_NOSPACE;
  return SWA_OK;
}

swa_status_t swa_translate_loc(const int64_t *full_loc, int64_t n, const int64_t *full_to_swa, int64_t map_len,
                               int64_t *swa_loc, hipStream_t stream) {
  if (n < 0) return SWA_E_ARG;
  if (n == 0) return SWA_OK;
  if (!full_loc || !full_to_swa || !swa_loc || map_len < 2) return SWA_E_ARG;
  if (full_loc == swa_loc) return SWA_E_ARG;
  return from_hip(swa::launch_translate_loc(full_loc, n, full_to_swa, map_len, swa_loc, stream));
}

swa_status_t swa_translate_window(const swa_index_t *idx, int32_t window, const int32_t *prefix_lens,
                                  int32_t *slot_table, int32_t *table_indptr, int64_t table_capacity,
                                  hipStream_t stream) {
  swa_status_t st = check_index(idx, true);
  if (st != SWA_OK) return st;
  if (window < -1 || table_capacity < 0 || !table_indptr) return SWA_E_ARG;
  if (table_capacity > 0 && !slot_table) return SWA_E_ARG;
  return from_hip(swa::launch_translate_window(*idx, window, 0, prefix_lens, slot_table, table_indptr,
                                               table_capacity, stream));
}

swa_status_t swa_translate_window_chunked(const swa_index_t *idx, int32_t window, int32_t chunk,
                                          const int32_t *prefix_lens, int32_t *slot_table, int32_t *table_indptr,
                                          int64_t table_capacity, hipStream_t stream) {
  swa_status_t st = check_index(idx, true);
  if (st != SWA_OK) return st;
  if (window < -1 || chunk < 0 || table_capacity < 0 || !table_indptr) return SWA_E_ARG;
  if (table_capacity > 0 && !slot_table) return SWA_E_ARG;
  return from_hip(swa::launch_translate_window(*idx, window, chunk, prefix_lens, slot_table, table_indptr,
                                               table_capacity, stream));
}

swa_status_t swa_translate_window_ring(const swa_index_t *idx, int64_t ring_rows, int32_t window, int32_t chunk,
                                       const int32_t *prefix_lens, int32_t *slot_table, int32_t *table_indptr,
                                       int64_t table_capacity, hipStream_t stream) {
  swa_status_t st = check_index(idx, false);
  if (st != SWA_OK) return st;
  if (ring_rows < 1 || window < -1 || chunk < 0 || table_capacity < 0 || !table_indptr) return SWA_E_ARG;
  if (idx->r2t_rows < 1 || idx->r2t_stride < 1 || (idx->batch > 0 && !idx->req_pool_idx)) return SWA_E_ARG;
  if (table_capacity > 0 && !slot_table) return SWA_E_ARG;
  if (ring_rows > kMaxRows / idx->r2t_rows) return SWA_E_SHAPE;  // ring rows travel through int32 tables
  return from_hip(swa::launch_translate_window_ring(*idx, ring_rows, window, chunk, prefix_lens, slot_table,
                                                    table_indptr, table_capacity, stream));
}

swa_status_t swa_ring_locs(const swa_index_t *idx, int64_t ring_rows, const int32_t *prefix_lens, int64_t *out,
                           int64_t n_out, hipStream_t stream) {
  swa_status_t st = check_index(idx, false);
  if (st != SWA_OK) return st;
  if (ring_rows < 1 || n_out < 0 || (n_out > 0 && !out)) return SWA_E_ARG;
  if (idx->r2t_rows < 1 || (idx->batch > 0 && !idx->req_pool_idx)) return SWA_E_ARG;
  if (ring_rows > INT64_MAX / idx->r2t_rows) return SWA_E_SHAPE;
  return from_hip(swa::launch_ring_locs(*idx, ring_rows, prefix_lens, out, n_out, stream));
}

}  // extern "C"

namespace {

// The checks of swa_kv_store (every check runs before a launch).
swa_status_t store_check(const swa_kv_layer_t *layer, const int64_t *loc, int64_t n, const void *k_new,
                         const void *v_new, int32_t in_dtype) {
  swa_status_t st = check_layer(layer);
  if (st != SWA_OK) return st;
  if (n < 0) return SWA_E_ARG;
  const int32_t out = layer->dtype;
  const bool pair_ok = (in_dtype == out && in_dtype != SWA_FP8_E4M3) || (in_dtype == SWA_F32 && out == SWA_BF16) ||
                       (in_dtype == SWA_BF16 && out == SWA_FP8_E4M3) || (in_dtype == SWA_F32 && out == SWA_FP8_E4M3);
  if (!pair_ok) return SWA_E_DTYPE;
  if ((static_cast<int64_t>(layer->kv_heads) * layer->head_dim) % 8) return SWA_E_SHAPE;
  if (n == 0) return SWA_OK;
  if (!loc || !k_new || !v_new || !aligned16(k_new) || !aligned16(v_new)) return SWA_E_ARG;
  return SWA_OK;
}

}  // namespace

extern "C" {

swa_status_t swa_kv_store(const swa_kv_layer_t *layer, const int64_t *loc, int64_t n, const void *k_new,
                          const void *v_new, int32_t in_dtype, hipStream_t stream) {
  const swa_status_t st = store_check(layer, loc, n, k_new, v_new, in_dtype);
  if (st != SWA_OK || n == 0) return st;
  return from_hip(swa::launch_kv_store(*layer, loc, n, k_new, v_new, in_dtype, stream));
}

swa_status_t swa_decode_plan(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim, int32_t window,
                             int64_t max_seq_len, int32_t *num_splits, size_t *workspace_bytes) {
  if (!num_splits || !workspace_bytes) return SWA_E_ARG;
  if (batch < 0 || window < -1 || max_seq_len < 0) return SWA_E_ARG;
  if (head_dim != kHeadDim) return SWA_E_SHAPE;
  if (!valid_group(q_heads, kv_heads)) return SWA_E_SHAPE;
  int64_t splits = 1;
  // Full layers, and windows past the one-split window kernel (W + 1 > 256
  // keys), stream their keys and are split by length: a request holds at most
  // W + 1 keys of a window.
  const bool streamed = window < 0 || window > swa::kMaxFusedWindow;
  if (streamed && batch > 0) {
    const int64_t keys = (window >= 0 && window + 1 < max_seq_len) ? window + 1 : max_seq_len;
    const int64_t by_fill = (kTargetStreams + static_cast<int64_t>(batch) * kv_heads - 1) /
                            (static_cast<int64_t>(batch) * kv_heads);
    const int64_t by_len = (keys + kMinKeysPerSplit - 1) / kMinKeysPerSplit;
    splits = by_fill < by_len ? by_fill : by_len;
    if (splits < 1) splits = 1;
    if (splits > kMaxSplits) splits = kMaxSplits;
  }
  *num_splits = static_cast<int32_t>(splits);
  *workspace_bytes = splits > 1 ? static_cast<size_t>(batch) * q_heads * splits * (2 + kHeadDim) * sizeof(float) : 0;
  return SWA_OK;
}

size_t swa_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t head_dim, int32_t max_keys) {
  if (batch <= 0 || q_heads <= 0 || head_dim != kHeadDim || max_keys <= 0) return 0;
  int64_t splits = (static_cast<int64_t>(max_keys) + kMinKeysPerSplit - 1) / kMinKeysPerSplit;  // the planner's cap
  if (splits > kMaxSplits) splits = kMaxSplits;
  if (splits <= 1) return 0;
  return static_cast<size_t>(batch) * q_heads * splits * (2 + kHeadDim) * sizeof(float);
}

}  // extern "C"

namespace {

// Checks shared by swa_decode and swa_decode_store (fused: with the store);
// on SWA_OK `a` holds the launch.  An empty batch passes the same checks, may
// leave q, out, loc and the new rows NULL, and launches nothing.
swa_status_t decode_prepare(const void *q, int32_t q_dtype, int32_t q_heads, const swa_kv_layer_t *layer,
                            const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                            int64_t table_capacity, int32_t window, const float *sinks, float sm_scale, void *out,
                            int32_t out_dtype, int32_t num_splits, void *workspace, size_t workspace_bytes,
                            bool fused, const int64_t *loc, const void *k_new, const void *v_new,
                            swa::DecodeArgs &a) {
  swa_status_t st = check_layer(layer);
  if (st != SWA_OK) return st;
  st = check_index(idx, table_indptr == nullptr);
  if (st != SWA_OK) return st;
  const bool empty = idx->batch == 0;
  if ((!empty && (!q || !out)) || window < -1 || num_splits < 1 || num_splits > kMaxSplits) return SWA_E_ARG;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return SWA_E_ARG;
  if (table_indptr && (!slot_table || table_capacity < 0)) return SWA_E_ARG;
  // the kernels translate through the window table only: a mapping without
  // one would read full-pool slots from this pool
  if (idx->full_to_swa && !table_indptr) return SWA_E_ARG;
  if (layer->head_dim != kHeadDim) return SWA_E_SHAPE;
  if (!valid_group(q_heads, layer->kv_heads)) return SWA_E_SHAPE;
  if (layer->rows > kMaxRows) return SWA_E_SHAPE;
  const bool f32_path = q_dtype == SWA_F32 && layer->dtype == SWA_F32;
  const bool mfma_path = q_dtype == SWA_BF16 && (layer->dtype == SWA_BF16 || layer->dtype == SWA_FP8_E4M3);
  if (!f32_path && !mfma_path) return SWA_E_DTYPE;
  if (out_dtype != SWA_F32 && out_dtype != SWA_BF16) return SWA_E_DTYPE;
  if (!aligned16(q) || !aligned16(out)) return SWA_E_ARG;
  if (num_splits > 1 && !empty) {
    const size_t need = static_cast<size_t>(idx->batch) * q_heads * num_splits * (2 + kHeadDim) * sizeof(float);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return SWA_E_WORKSPACE;
  }
  if (fused) {
    if (!empty && (!loc || !k_new || !v_new)) return SWA_E_ARG;
    if (!aligned16(k_new) || !aligned16(v_new)) return SWA_E_ARG;
    if (!mfma_path) return SWA_E_DTYPE;
    if (window < 0 || window > swa::kMaxFusedWindow || num_splits != 1) return SWA_E_SHAPE;
  }
  a = swa::DecodeArgs{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.q_heads = q_heads;
  a.layer = *layer;
  a.idx = *idx;
  a.table = slot_table;
  a.indptr = table_indptr;
  a.capacity = table_capacity;
  a.window = window;
  a.sinks = sinks;
  a.sm_scale = sm_scale;
  a.out = out;
  a.out_dtype = out_dtype;
  a.num_splits = num_splits;
  a.ws = static_cast<float *>(workspace);
  a.new_loc = loc;
  a.k_new = k_new;
  a.v_new = v_new;
  return SWA_OK;
}

swa_status_t decode_impl(const void *q, int32_t q_dtype, int32_t q_heads, const swa_kv_layer_t *layer,
                         const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                         int64_t table_capacity, int32_t window, const float *sinks, float sm_scale, void *out,
                         int32_t out_dtype, int32_t num_splits, void *workspace, size_t workspace_bytes, bool fused,
                         const int64_t *loc, const void *k_new, const void *v_new, hipStream_t stream) {
  swa::DecodeArgs a;
  const swa_status_t st = decode_prepare(q, q_dtype, q_heads, layer, idx, slot_table, table_indptr, table_capacity,
                                         window, sinks, sm_scale, out, out_dtype, num_splits, workspace,
                                         workspace_bytes, fused, loc, k_new, v_new, a);
  if (st != SWA_OK) return st;
  return from_hip(swa::launch_decode(a, stream));
}

}  // namespace

extern "C" {

swa_status_t swa_decode(const void *q, int32_t q_dtype, int32_t q_heads, const swa_kv_layer_t *layer,
                        const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                        int64_t table_capacity, int32_t window, const float *sinks, float sm_scale, void *out,
                        int32_t out_dtype, int32_t num_splits, void *workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return decode_impl(q, q_dtype, q_heads, layer, idx, slot_table, table_indptr, table_capacity, window, sinks,
                     sm_scale, out, out_dtype, num_splits, workspace, workspace_bytes, false, nullptr, nullptr,
                     nullptr, stream);
}

swa_status_t swa_decode_noalloc(const void *q, int32_t q_dtype, int32_t q_heads, const swa_kv_layer_t *layer,
                                const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                                int64_t table_capacity, int32_t window, const float *sinks, float sm_scale, void *out,
                                int32_t out_dtype, int32_t num_splits, hipStream_t stream) {
  // every argument check first, with no workspace: SWA_E_WORKSPACE then means
  // that the plan has split partials, which go to the static scratch if they fit
  swa::DecodeArgs a;
  swa_status_t st = decode_prepare(q, q_dtype, q_heads, layer, idx, slot_table, table_indptr, table_capacity, window,
                                   sinks, sm_scale, out, out_dtype, num_splits, nullptr, 0, false, nullptr, nullptr,
                                   nullptr, a);
  if (st == SWA_E_WORKSPACE) {
    const size_t need = static_cast<size_t>(idx->batch) * q_heads * num_splits * (2 + kHeadDim) * sizeof(float);
    if (need > swa::kStaticScratchBytes) return SWA_E_WORKSPACE;
    void *ws = nullptr;
    if (swa::static_scratch(&ws) != hipSuccess) return SWA_E_HIP;
    st = decode_prepare(q, q_dtype, q_heads, layer, idx, slot_table, table_indptr, table_capacity, window, sinks,
                        sm_scale, out, out_dtype, num_splits, ws, swa::kStaticScratchBytes, false, nullptr, nullptr,
                        nullptr, a);
  }
  if (st != SWA_OK) return st;
  return from_hip(swa::launch_decode(a, stream));
}

swa_status_t swa_decode_store(const void *q, int32_t q_dtype, int32_t q_heads, const swa_kv_layer_t *layer,
                              const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                              int64_t table_capacity, int32_t window, const float *sinks, float sm_scale,
                              const int64_t *loc, const void *k_new, const void *v_new, int32_t new_dtype,
                              void *out, int32_t out_dtype, hipStream_t stream) {
  if (new_dtype != SWA_BF16) return SWA_E_DTYPE;
  return decode_impl(q, q_dtype, q_heads, layer, idx, slot_table, table_indptr, table_capacity, window, sinks,
                     sm_scale, out, out_dtype, 1, nullptr, 0, true, loc, k_new, v_new, stream);
}

namespace {

// One layer's work in a decode step, checked before anything is launched.
struct StepLaunch {
  bool store;                 // swa_kv_store first
  swa_kv_layer_t store_layer;
  const int64_t *store_loc;
  const void *k_new, *v_new;
  swa::DecodeArgs decode;
};

swa_status_t step_plan(const swa_decode_step_t *st, const swa_index_t *idx, int64_t max_seq_len,
                       int32_t *full_splits, size_t *workspace_bytes) {
  *full_splits = 1;
  *workspace_bytes = 0;
  if (!st || !idx || idx->batch < 0 || max_seq_len < 0 || st->n_layers < 0) return SWA_E_ARG;
  if (st->n_layers > 0 && !st->layers_mapping) return SWA_E_ARG;
  if (st->n_full_layers < 0 || st->n_swa_layers < 0) return SWA_E_ARG;
  if ((st->n_full_layers > 0 && !st->full_layers) || (st->n_swa_layers > 0 && !st->swa_layers)) return SWA_E_ARG;
  int32_t full_kv = 0;
  for (int32_t l = 0; l < st->n_layers; ++l) {
    const swa_layer_map_t &m = st->layers_mapping[l];
    const int32_t n = m.is_swa ? st->n_swa_layers : st->n_full_layers;
    if ((m.is_swa != 0 && m.is_swa != 1) || m.pool_layer < 0 || m.pool_layer >= n) return SWA_E_ARG;
    if (!m.is_swa) {
      const int32_t kv = st->full_layers[m.pool_layer].kv_heads;
      full_kv = kv > full_kv ? kv : full_kv;
    }
  }
  if (full_kv == 0) return SWA_OK;
  // the split count of the widest full layer's plan serves every full layer
  // (the workspace holds batch * q_heads * splits partials whatever kv_heads is)
  size_t ws = 0;
  const swa_status_t s = swa_decode_plan(idx->batch, st->q_heads, full_kv, kHeadDim, -1, max_seq_len, full_splits, &ws);
  if (s != SWA_OK) return s;
  *workspace_bytes = ws;
  return SWA_OK;
}

}  // namespace

extern "C" {

size_t swa_decode_step_workspace_bytes(const swa_decode_step_t *step, const swa_index_t *idx, int64_t max_seq_len) {
  int32_t splits;
  size_t ws;
  return step_plan(step, idx, max_seq_len, &splits, &ws) == SWA_OK ? ws : 0;
}

swa_status_t swa_decode_step(const swa_decode_step_t *st, const swa_index_t *idx, int64_t max_seq_len,
                             int32_t *slot_table, int32_t *table_indptr, int64_t table_capacity, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  int32_t full_splits;
  size_t ws_need;
  swa_status_t status = step_plan(st, idx, max_seq_len, &full_splits, &ws_need);
  if (status != SWA_OK) return status;
  if (!st->q || !st->out) return SWA_E_ARG;
  if (st->window < 0) return SWA_E_ARG;
  const bool store = st->k_new || st->v_new || st->full_loc;
  if (store && (!st->k_new || !st->v_new || !st->full_loc)) return SWA_E_ARG;
  const int32_t B = idx->batch;
  bool any_swa = false;
  for (int32_t l = 0; l < st->n_layers; ++l) any_swa = any_swa || st->layers_mapping[l].is_swa;
  const bool translate = store && any_swa && idx->full_to_swa;  // the store's SWA slots: full_loc translated
  if (translate && !st->swa_loc) return SWA_E_ARG;
  const int64_t *swa_loc = idx->full_to_swa ? st->swa_loc : st->full_loc;
  if (any_swa) {
    status = check_index(idx, true);
    if (status != SWA_OK) return status;
    if (!table_indptr || table_capacity < 0 || (table_capacity > 0 && !slot_table)) return SWA_E_ARG;
  }
  if (translate && B > 0 && idx->map_len < 2) return SWA_E_ARG;
  // full layers read req_to_token directly: the same batch without the mapping
  swa_index_t full_idx = *idx;
  full_idx.full_to_swa = nullptr;
  full_idx.map_len = 0;

  std::vector<StepLaunch> plan(static_cast<size_t>(st->n_layers));
  for (int32_t l = 0; l < st->n_layers; ++l) {
    const swa_layer_map_t &m = st->layers_mapping[l];
    const swa_kv_layer_t *layer = m.is_swa ? &st->swa_layers[m.pool_layer] : &st->full_layers[m.pool_layer];
    const float *sinks = st->sinks ? st->sinks[l] : nullptr;
    StepLaunch &x = plan[static_cast<size_t>(l)];
    x.store = false;
    const void *kn = store ? st->k_new[l] : nullptr;
    const void *vn = store ? st->v_new[l] : nullptr;
    // the new token is fused into the window kernel for bf16 pools; e4m3 pools
    // store with their own launch (the fused e4m3 kernel holds more registers,
    // which costs a workgroup per CU)
    const bool fuse = store && m.is_swa && layer->dtype == SWA_BF16 && st->window <= swa::kMaxFusedWindow &&
                      st->q_dtype == SWA_BF16;
    if (store && !fuse) {
      x.store = true;
      x.store_layer = *layer;
      x.store_loc = m.is_swa ? swa_loc : st->full_loc;
      x.k_new = kn;
      x.v_new = vn;
      status = store_check(layer, x.store_loc, B, kn, vn, SWA_BF16);
      if (status != SWA_OK) return status;
    }
    if (m.is_swa) {
      status = decode_prepare(st->q[l], st->q_dtype, st->q_heads, layer, idx, slot_table, table_indptr,
                              table_capacity, st->window, sinks, st->sm_scale, st->out[l], st->out_dtype, 1, nullptr, 0,
                              fuse, fuse ? swa_loc : nullptr, fuse ? kn : nullptr, fuse ? vn : nullptr, x.decode);
    } else {
      status = decode_prepare(st->q[l], st->q_dtype, st->q_heads, layer, &full_idx, nullptr, nullptr, 0, -1, sinks,
                              st->sm_scale, st->out[l], st->out_dtype, full_splits, workspace, workspace_bytes, false,
                              nullptr, nullptr, nullptr, x.decode);
    }
    if (status != SWA_OK) return status;
  }
  if (B == 0) return SWA_OK;

  // a3 once for every SWA layer, a2 once for the store, then the layers in order
  if (any_swa) {
    status = from_hip(swa::launch_translate_window(*idx, st->window, 0, nullptr, slot_table, table_indptr,
                                                   table_capacity, stream));
    if (status != SWA_OK) return status;
  }
  if (translate) {
    status = from_hip(swa::launch_translate_loc(st->full_loc, B, idx->full_to_swa, idx->map_len, st->swa_loc, stream));
    if (status != SWA_OK) return status;
  }
  for (const StepLaunch &x : plan) {
    if (x.store) {
      status = from_hip(swa::launch_kv_store(x.store_layer, x.store_loc, B, x.k_new, x.v_new, SWA_BF16, stream));
      if (status != SWA_OK) return status;
    }
    status = from_hip(swa::launch_decode(x.decode, stream));
    if (status != SWA_OK) return status;
  }
  return SWA_OK;
}

}  // extern "C"

namespace {

swa_status_t extend_impl(const void *q, int32_t q_dtype, int32_t q_heads, const int32_t *qo_indptr,
                         const int32_t *prefix_lens, int64_t total_q, const swa_kv_layer_t *layer,
                         const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                         int64_t table_capacity, int32_t window, int32_t chunk, const float *sinks, float sm_scale,
                         void *out, int32_t out_dtype, hipStream_t stream) {
  swa_status_t st = check_layer(layer);
  if (st != SWA_OK) return st;
  st = check_index(idx, true);
  if (st != SWA_OK) return st;
  if (total_q < 0 || window < -1 || chunk < 0 || !(sm_scale > 0.f) || !std::isfinite(sm_scale)) return SWA_E_ARG;
  if (idx->batch > 0 && (!qo_indptr || !prefix_lens)) return SWA_E_ARG;
  if (total_q > 0 && (!q || !out)) return SWA_E_ARG;
  if (table_indptr && (!slot_table || table_capacity < 0)) return SWA_E_ARG;
  if (idx->full_to_swa && !table_indptr) return SWA_E_ARG;  // as in decode: no translation without the table
  if (layer->head_dim != kHeadDim) return SWA_E_SHAPE;
  if (!valid_group(q_heads, layer->kv_heads)) return SWA_E_SHAPE;
  if (layer->rows > kMaxRows || total_q > INT32_MAX) return SWA_E_SHAPE;
  if (q_dtype != SWA_BF16 || layer->dtype != SWA_BF16) return SWA_E_DTYPE;
  if (out_dtype != SWA_F32 && out_dtype != SWA_BF16) return SWA_E_DTYPE;
  if (total_q > 0 && (!aligned16(q) || !aligned16(out))) return SWA_E_ARG;
  swa::ExtendArgs a{};
  a.q = q;
  a.q_heads = q_heads;
  a.qo_indptr = qo_indptr;
  a.prefix_lens = prefix_lens;
  a.total_q = total_q;
  a.layer = *layer;
  a.idx = *idx;
  a.table = slot_table;
  a.indptr = table_indptr;
  a.capacity = table_capacity;
  a.window = window;
  a.chunk = chunk;
  a.sinks = sinks;
  a.sm_scale = sm_scale;
  a.out = out;
  a.out_dtype = out_dtype;
  return from_hip(swa::launch_extend(a, stream));
}

}  // namespace

swa_status_t swa_extend(const void *q, int32_t q_dtype, int32_t q_heads, const int32_t *qo_indptr,
                        const int32_t *prefix_lens, int64_t total_q, const swa_kv_layer_t *layer,
                        const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                        int64_t table_capacity, int32_t window, const float *sinks, float sm_scale, void *out,
                        int32_t out_dtype, hipStream_t stream) {
  return extend_impl(q, q_dtype, q_heads, qo_indptr, prefix_lens, total_q, layer, idx, slot_table, table_indptr,
                     table_capacity, window, 0, sinks, sm_scale, out, out_dtype, stream);
}

swa_status_t swa_extend_chunked(const void *q, int32_t q_dtype, int32_t q_heads, const int32_t *qo_indptr,
                                const int32_t *prefix_lens, int64_t total_q, const swa_kv_layer_t *layer,
                                const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                                int64_t table_capacity, int32_t window, int32_t chunk, const float *sinks,
                                float sm_scale, void *out, int32_t out_dtype, hipStream_t stream) {
  return extend_impl(q, q_dtype, q_heads, qo_indptr, prefix_lens, total_q, layer, idx, slot_table, table_indptr,
                     table_capacity, window, chunk, sinks, sm_scale, out, out_dtype, stream);
}

namespace {

int64_t dtype_bytes(int32_t dtype) {
  return dtype == SWA_F32 ? 4 : dtype == SWA_BF16 ? 2 : dtype == SWA_FP8_E4M3 ? 1 : 0;
}

// Geometry of one unified sub-pool, or false on bad or oversized arguments:
// bytes of one row, of one page envelope (2L row blocks), and kernel-facing rows.
bool unified_geometry(int32_t layer_num, int32_t kv_heads, int32_t head_dim, int32_t dtype, int32_t page_size,
                      int64_t num_pages, int64_t &row_bytes, int64_t &page_bytes, int64_t &n_rows) {
  const int64_t item = dtype_bytes(dtype);
  if (!item || layer_num < 1 || kv_heads < 1 || head_dim < 1 || page_size < 1 || num_pages < 1) return false;
  if (layer_num > 4096 || kv_heads > 4096 || head_dim > 4096 || page_size > (1 << 20) || num_pages > (1ll << 40))
    return false;
  row_bytes = static_cast<int64_t>(kv_heads) * head_dim * item;
  const int64_t blocks = 2ll * layer_num;
  page_bytes = page_size * blocks * row_bytes;
  if (num_pages > INT64_MAX / 2 / page_bytes) return false;
  n_rows = num_pages * blocks * page_size;
  return true;
}

}  // namespace

int64_t swa_unified_pool_bytes(int32_t layer_num, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                               int32_t page_size, int64_t num_pages) {
  int64_t row_bytes, page_bytes, n_rows;
  if (!unified_geometry(layer_num, kv_heads, head_dim, dtype, page_size, num_pages, row_bytes, page_bytes, n_rows))
    return -1;
  return num_pages * page_bytes + page_bytes;  // the envelopes, then one envelope of tail pad
}

swa_status_t swa_unified_layer_views(void *raw, int64_t raw_bytes, int64_t anchor_bytes, int32_t layer_num,
                                     int32_t kv_heads, int32_t head_dim, int32_t dtype, int32_t page_size,
                                     int64_t num_pages, float k_scale, float v_scale, swa_kv_layer_t *views) {
  if (!raw || !views || raw_bytes < 0 || anchor_bytes < 0 || (anchor_bytes & 15)) return SWA_E_ARG;
  if (!aligned16(raw)) return SWA_E_ARG;
  if (dtype_bytes(dtype) == 0) return SWA_E_DTYPE;
  int64_t row_bytes, page_bytes, n_rows;
  if (!unified_geometry(layer_num, kv_heads, head_dim, dtype, page_size, num_pages, row_bytes, page_bytes, n_rows))
    return SWA_E_ARG;
  if (row_bytes & 15) return SWA_E_SHAPE;     // rows must keep 16-byte alignment
  if (n_rows > kMaxRows) return SWA_E_SHAPE;  // kernel-facing ids travel through int32 tables
  // the last view (layer L-1's V) ends (2L - 1) * P rows past the last envelope
  if (anchor_bytes > raw_bytes || raw_bytes - anchor_bytes < num_pages * page_bytes + page_bytes) return SWA_E_SHAPE;
  char *base = static_cast<char *>(raw) + anchor_bytes;
  for (int32_t l = 0; l < layer_num; ++l) {
    swa_kv_layer_t &v = views[l];
    v.k = base + (2ll * l) * page_size * row_bytes;
    v.v = base + (2ll * l + 1) * page_size * row_bytes;
    v.rows = n_rows;
    v.kv_heads = kv_heads;
    v.head_dim = head_dim;
    v.dtype = dtype;
    v.k_scale = k_scale;
    v.v_scale = v_scale;
  }
  return SWA_OK;
}

swa_status_t swa_translate_kernel_ids(const int64_t *virt, int64_t n, const int64_t *v2p, int64_t n_pages,
                                      int32_t page_size, int32_t multiplier, int64_t *out, hipStream_t stream) {
  if (n < 0 || n_pages < 1 || !v2p || page_size < 1 || multiplier < 1) return SWA_E_ARG;
  if (n > 0 && (!virt || !out)) return SWA_E_ARG;
  return from_hip(swa::launch_translate_ids(virt, n, v2p, n_pages, page_size, multiplier, out, stream));
}

swa_status_t swa_translate_window_unified(const swa_index_t *idx, const int64_t *v2p, int64_t n_pages,
                                          int32_t multiplier, int32_t window, const int32_t *prefix_lens,
                                          int32_t *slot_table, int32_t *table_indptr, int64_t table_capacity,
                                          hipStream_t stream) {
  swa_status_t st = check_index(idx, true);
  if (st != SWA_OK) return st;
  if (!v2p || n_pages < 1 || multiplier < 1 || idx->page_size < 1) return SWA_E_ARG;
  if (window < -1 || table_capacity < 0 || !table_indptr) return SWA_E_ARG;
  if (table_capacity > 0 && !slot_table) return SWA_E_ARG;
  // every kernel-facing id must fit the int32 table
  if (n_pages > kMaxRows / idx->page_size / multiplier) return SWA_E_SHAPE;
  return from_hip(swa::launch_translate_window_unified(*idx, v2p, n_pages, multiplier, window, prefix_lens,
                                                       slot_table, table_indptr, table_capacity, stream));
}

int64_t swa_alloc_pages_needed(const int32_t *pre_lens, const int32_t *seq_lens, int32_t batch, int32_t page_size) {
  if (batch < 0 || page_size < 1 || (batch > 0 && !seq_lens)) return -1;
  int64_t n = 0;
  for (int32_t b = 0; b < batch; ++b) {
    int64_t seq = seq_lens[b];
    int64_t pre = pre_lens ? pre_lens[b] : seq - 1;
    if (pre < 0) pre = 0;
    if (seq < pre) seq = pre;
    n += (seq + page_size - 1) / page_size - (pre + page_size - 1) / page_size;
  }
  return n;
}

namespace {

// The sufficiency check that must pass before an allocation kernel reads a
// free list: the optimistic bound first, then (with host copies of the
// lengths) the exact count.
swa_status_t alloc_fits(int32_t batch, int32_t page, int64_t bound, const int32_t *pre_host,
                        const int32_t *seq_host, int64_t avail) {
  if (bound <= avail) return SWA_OK;
  if (!seq_host) return SWA_E_NOSPACE;
  const int64_t exact = swa_alloc_pages_needed(pre_host, seq_host, batch, page);
  return exact <= avail ? SWA_OK : SWA_E_NOSPACE;
}

swa_status_t alloc_impl(bool decode, int32_t batch, int32_t page_size, const int32_t *pre_lens,
                        const int32_t *seq_lens, const int64_t *last_loc, const swa_free_list_t *full,
                        const swa_free_list_t *swa_list, int64_t *full_to_swa, int64_t map_len, int64_t n_tokens,
                        const int32_t *pre_host, const int32_t *seq_host, int64_t *out_full, int64_t *out_swa,
                        int64_t *new_pages, hipStream_t stream) {
  if (batch < 0 || page_size < 1 || n_tokens < 0 || !full || full->count < 0) return SWA_E_ARG;
  if (batch > 0 && (!seq_lens || !last_loc || (!decode && !pre_lens))) return SWA_E_ARG;
  if (full->count > 0 && !full->pages) return SWA_E_ARG;
  if (n_tokens > 0 && !out_full) return SWA_E_ARG;
  if (swa_list) {
    if (swa_list->count < 0 || (swa_list->count > 0 && !swa_list->pages)) return SWA_E_ARG;
    if (!full_to_swa || map_len < 2) return SWA_E_ARG;
  }
  int64_t avail = full->count;
  if (swa_list && swa_list->count < avail) avail = swa_list->count;
  const int64_t bound = decode ? batch : n_tokens / page_size + batch + 1;
  const swa_status_t fits = alloc_fits(batch, page_size, bound, decode ? nullptr : pre_host, seq_host, avail);
  if (fits != SWA_OK) return fits;
  swa::AllocArgs a{};
  a.batch = batch;
  a.page_size = page_size;
  a.decode = decode;
  a.pre_lens = decode ? nullptr : pre_lens;
  a.seq_lens = seq_lens;
  a.last_loc = last_loc;
  a.free_full = full->pages;
  a.n_free_full = full->count;
  a.free_swa = swa_list ? swa_list->pages : nullptr;
  a.n_free_swa = swa_list ? swa_list->count : 0;
  a.full_to_swa = swa_list ? full_to_swa : nullptr;
  a.map_len = swa_list ? map_len : 0;
  a.out_full = out_full;
  a.out_swa = swa_list ? out_swa : nullptr;
  a.capacity = n_tokens;
  a.new_pages = new_pages;
  return from_hip(swa::launch_alloc(a, stream));
}

}  // namespace

swa_status_t swa_alloc_extend(int32_t batch, int32_t page_size, const int32_t *pre_lens, const int32_t *seq_lens,
                              const int64_t *last_loc, const swa_free_list_t *full, const swa_free_list_t *swa_list,
                              int64_t *full_to_swa, int64_t map_len, int64_t extend_num_tokens,
                              const int32_t *pre_lens_host, const int32_t *seq_lens_host, int64_t *out_full,
                              int64_t *out_swa, int64_t *new_pages, hipStream_t stream) {
  return alloc_impl(false, batch, page_size, pre_lens, seq_lens, last_loc, full, swa_list, full_to_swa, map_len,
                    extend_num_tokens, pre_lens_host, seq_lens_host, out_full, out_swa, new_pages, stream);
}

swa_status_t swa_alloc_decode(int32_t batch, int32_t page_size, const int32_t *seq_lens, const int64_t *last_loc,
                              const swa_free_list_t *full, const swa_free_list_t *swa_list, int64_t *full_to_swa,
                              int64_t map_len, const int32_t *seq_lens_host, int64_t *out_full, int64_t *out_swa,
                              int64_t *new_pages, hipStream_t stream) {
  return alloc_impl(true, batch, page_size, nullptr, seq_lens, last_loc, full, swa_list, full_to_swa, map_len, batch,
                    nullptr, seq_lens_host, out_full, out_swa, new_pages, stream);
}

size_t swa_evict_workspace_bytes(int32_t batch, int64_t r2t_stride, int32_t page_size) {
  if (batch <= 0 || r2t_stride < 1 || page_size < 1) return 0;
  return static_cast<size_t>(swa::evict_cand_offset(batch, r2t_stride, page_size)) +
         static_cast<size_t>(batch) * static_cast<size_t>(swa::evict_cands(r2t_stride, page_size)) * sizeof(int64_t);
}

swa_status_t swa_evict(const swa_index_t *idx, int64_t *full_to_swa, const int32_t *pre_lens,
                       const int32_t *protected_lens, int32_t *evicted_lens, int32_t window, int32_t mode,
                       int32_t interval, int64_t *freed_pages, int64_t freed_capacity, int64_t *freed_count,
                       void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!idx || idx->batch < 0 || !full_to_swa || !freed_count) return SWA_E_ARG;
  swa_status_t st = check_index(idx, true);
  if (st != SWA_OK) return st;
  if (idx->map_len < 2 || idx->page_size < 1 || window < 0 || (mode != 0 && mode != 1) || interval < 0 ||
      freed_capacity < 0)
    return SWA_E_ARG;
  if (idx->batch > 0 && (!pre_lens || !evicted_lens)) return SWA_E_ARG;
  if (freed_capacity > 0 && !freed_pages) return SWA_E_ARG;
  if (idx->batch > 0 && swa::evict_chunks(idx->r2t_stride, idx->page_size) > 65535) return SWA_E_SHAPE;
  if (idx->batch > 0 &&
      (!workspace || workspace_bytes < swa_evict_workspace_bytes(idx->batch, idx->r2t_stride, idx->page_size) ||
       (reinterpret_cast<uintptr_t>(workspace) & 7u)))
    return SWA_E_WORKSPACE;
  return from_hip(swa::launch_evict(*idx, full_to_swa, pre_lens, protected_lens, evicted_lens, window, mode,
                                    interval, freed_pages, freed_capacity, freed_count,
                                    static_cast<int32_t *>(workspace), stream));
}

// Workspace of swa_validate: 16 int64 counters, then one bit per pool row.
constexpr int64_t kValidateCounterBytes = 16 * sizeof(int64_t);

size_t swa_validate_workspace_bytes(int64_t pool_rows) {
  if (pool_rows < 0) return 0;
  return static_cast<size_t>(kValidateCounterBytes + (pool_rows + 31) / 32 * 4);
}

swa_status_t swa_validate(const swa_index_t *idx, int32_t window, const int32_t *prefix_lens,
                          const int32_t *qo_indptr, int64_t total_q, int64_t pool_rows, const int64_t *store_loc,
                          int64_t n_store, void *workspace, size_t workspace_bytes, swa_validate_report_t *report,
                          hipStream_t stream) {
  if (!report || !idx || idx->batch < 0 || window < -1 || pool_rows < 0 || n_store < 0 || total_q < 0)
    return SWA_E_ARG;
  if (idx->page_size < 1) return SWA_E_ARG;
  swa_status_t st = check_index(idx, true);
  if (st != SWA_OK) return st;
  if (n_store > 0 && !store_loc) return SWA_E_ARG;
  if (!workspace || !aligned16(workspace)) return SWA_E_WORKSPACE;
  const size_t need = n_store > 0 ? swa_validate_workspace_bytes(pool_rows) : kValidateCounterBytes;
  if (workspace_bytes < need) return SWA_E_WORKSPACE;
  hipError_t e = swa::launch_validate(*idx, window, prefix_lens, qo_indptr, total_q, pool_rows, store_loc, n_store,
                                      workspace, kValidateCounterBytes, stream);
  if (e != hipSuccess) return SWA_E_HIP;
  int64_t c[16];
  e = hipMemcpyAsync(c, workspace, sizeof(c), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return SWA_E_HIP;
  report->bad_requests = c[0];
  report->positions = c[1];
  report->full_out_of_range = c[2];
  report->tombstones = c[3];
  report->sentinels = c[4];
  report->slot_out_of_range = c[5];
  report->store_locs = c[6];
  report->store_out_of_range = c[7];
  report->store_duplicates = c[8];
  report->qo_bad = c[9];
  return SWA_OK;
}

const char *swa_status_string(swa_status_t status) {
  switch (status) {
    case SWA_OK: return "ok";
    case SWA_E_ARG: return "invalid argument";
    case SWA_E_DTYPE: return "unsupported dtype";
    case SWA_E_SHAPE: return "unsupported shape";
    case SWA_E_NOSPACE: return "SWA pool cannot hold window + page";
    case SWA_E_WORKSPACE: return "workspace missing or too small";
    case SWA_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"
