/*
 * swa.h — C ABI of libswa: sliding-window attention (SWA) over a two-pool paged
 * KV cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources.  The operations are the ones three web pages describe:
 *   [SWA]   zdszero.github.io/swa.html — SWA design note
 *   [POOLS] pinghaoyang.com.cn, "SGLang 源码完全拆解(十五): 内存池与显存管理"
 *   [PR]    prhub.com.cn digest of sglang pull request 34602
 * Each declaration below names the section it follows.
 *
 * Conventions shared by every call.
 *   - Pointers are DEVICE pointers owned by the caller unless marked [host].
 *     No call allocates or frees device memory, and none synchronises the
 *     device except swa_validate, which is a debugging aid.
 *   - Device work is enqueued on `stream` (a hipStream_t; NULL is the null
 *     stream).  Argument errors are detected on the host, before anything is
 *     enqueued, and returned synchronously; a failed launch returns SWA_E_HIP.
 *   - Kernels never fault on bad index data.  A slot, loc or position outside
 *     its table or pool is replaced by 0, the padding row / page 0 sink of every
 *     pool and table ([POOLS] 一重映射 and 二重映射: row 0 of req_to_token and
 *     slot 0 of each KV buffer absorb padded reads and writes); a store to a loc
 *     outside the pool is dropped.  swa_validate reports such data.
 *   - The library is stateless and thread-safe; calls that share output
 *     buffers on different streams race, as any two kernels would.
 *   - Every index is an element index, never a byte offset; slot offsets are
 *     computed in 64-bit arithmetic, so pools may exceed 2^31 rows x bytes
 *     ([PR] 实现拆解: the kernel-facing row bound of int32 index buffers).
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Negative values are errors. */
typedef enum swa_status {
  SWA_OK = 0,
  SWA_E_ARG = -1,       /* null pointer, negative size, inconsistent arguments */
  SWA_E_DTYPE = -2,     /* unsupported dtype or dtype combination */
  SWA_E_SHAPE = -3,     /* unsupported head_dim / head counts / group size */
  SWA_E_NOSPACE = -4,   /* pool sizing: the SWA pool cannot hold one request;
                           allocation: a free list is (or cannot be shown to be)
                           too short */
  SWA_E_WORKSPACE = -5, /* workspace missing or smaller than required */
  SWA_E_HIP = -6        /* the HIP runtime reported an error (launch / query) */
} swa_status_t;

/* Element types.  fp8 pools hold raw bytes ([POOLS] 二重映射: fp8 KV caches
 * are stored as uint8 and re-interpreted on read); the format is OCP e4m3fn. */
typedef enum swa_dtype {
  SWA_F32 = 0,
  SWA_BF16 = 1,
  SWA_FP8_E4M3 = 2
} swa_dtype_t;

/* One layer's dense K and V views of a pool ([POOLS] 二重映射: per-layer
 * k_buffer / v_buffer of shape (size + page_size, head_num, head_dim);
 * [SWA] 双池与映射表: the full pool and the SWA pool are two ordinary pools).
 * k and v are row-major (rows, kv_heads, head_dim) arrays of `dtype`;
 * row 0 is the padding sink.  k_scale / v_scale dequantise fp8 (value = code
 * * scale); they are ignored for f32 / bf16 and must be 1 there. */
typedef struct swa_kv_layer {
  void *k;
  void *v;
  int64_t rows;      /* = N + page_size */
  int32_t kv_heads;
  int32_t head_dim;
  int32_t dtype;     /* swa_dtype_t */
  float k_scale;
  float v_scale;
} swa_kv_layer_t;

/* The batch's index structures.
 *   req_to_token  int32 (r2t_rows, r2t_stride): full-pool slot of each position
 *                 of each request row; row 0 is padding ([POOLS] 一重映射).
 *   req_pool_idx  int32 (batch): the req_to_token row of each request.
 *   seq_lens      int32 (batch): tokens of each request INCLUDING the ones
 *                 being computed (decode: the current token is stored first).
 *   full_to_swa   int64 (map_len): SWA slot of each full slot, 0 = no SWA slot
 *                 (tombstone), last entry -1 so that -1 translates to -1
 *                 ([SWA] 双池与映射表; [POOLS] 双池 + 映射表).  map_len is
 *                 full pool size + page_size + 1.  NULL for full layers.
 *   page_size     pages of both pools; kernels translate per token, so it is
 *                 used only for validation. */
typedef struct swa_index {
  const int32_t *req_to_token;
  int64_t r2t_rows;
  int64_t r2t_stride;
  const int32_t *req_pool_idx;
  const int32_t *seq_lens;
  const int64_t *full_to_swa;
  int64_t map_len;
  int32_t batch;
  int32_t page_size;
} swa_index_t;

/* ---------------------------------------------------------------------------
 * Pool sizing — [SWA] 显存怎么分 (--swa-full-tokens-ratio).  All [host].
 *   cell   = full_bytes_per_token * n_full_layers
 *          + ratio * swa_bytes_per_token * n_swa_layers
 *   N_full = floor(avail_bytes / cell), N_swa = floor(ratio * N_full), both
 *   rounded down to page_size.  *_bytes_per_token is num_kv_heads *
 *   (head_dim + v_head_dim) * dtype_size of one layer.
 * Returns SWA_E_NOSPACE when N_swa <= window + page_size (the startup error on
 * the page), SWA_E_ARG for non-positive page_size, negative sizes or ratio, or
 * null outputs.  Outputs are written on SWA_OK and on SWA_E_NOSPACE. */
swa_status_t swa_pool_config(int64_t avail_bytes, double ratio, int32_t page_size, int32_t window,
                             int32_t n_full_layers, int64_t full_bytes_per_token,
                             int32_t n_swa_layers, int64_t swa_bytes_per_token,
                             int64_t *n_full_tokens, int64_t *n_swa_tokens);

/* ---------------------------------------------------------------------------
 * translate_loc — [SWA] Attention backend (translate_loc_from_full_to_swa is
 * full_to_swa[idx]) and 双池与映射表 (the -1 sentinel).
 *   swa_loc[i] = full_to_swa[full_loc[i]]  for 0 <= full_loc[i] < map_len - 1
 *              = full_to_swa[map_len - 1] (= -1) for full_loc[i] == -1
 *              = 0 for any other value.
 * full_loc, swa_loc: int64 (n); may not alias.  n == 0 is a no-op. */
swa_status_t swa_translate_loc(const int64_t *full_loc, int64_t n, const int64_t *full_to_swa,
                               int64_t map_len, int64_t *swa_loc, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * translate_window — the fused index translation + window gather, done once
 * per batch and shared by every SWA layer ([SWA] Attention backend: backends
 * build the window's translated indices once per batch; FlashInfer keeps W+1
 * positions, which is why W excludes the current token, [SWA] 实现).
 * For request b with row r = req_pool_idx[b], L = seq_lens[b],
 * p = prefix_lens ? prefix_lens[b] : L - 1 (decode):
 *   positions lo .. L-1, lo = (window < 0) ? 0 : max(0, p - window)
 *   slot_table[table_indptr[b] + k] = T(req_to_token[r][lo + k])
 * with T = full_to_swa (0 for an index outside the table, -1 -> -1) when
 * idx->full_to_swa is set, identity otherwise.
 * table_indptr: int32 (batch + 1), written by the kernel (exclusive prefix sum
 * of the counts L - lo, clamped at 0).  Entries past table_capacity are not
 * written; the caller sizes the table (decode: batch * (window + 1)). */
swa_status_t swa_translate_window(const swa_index_t *idx, int32_t window, const int32_t *prefix_lens,
                                  int32_t *slot_table, int32_t *table_indptr,
                                  int64_t table_capacity, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * kv_store — scatter new K/V rows into a pool ([SWA] Attention backend: SWA
 * layers receive an already translated swa_loc and the pool never translates;
 * [POOLS] 谁在往页里写 (KVWriteLoc) and 二重映射).
 *   layer->k[loc[i]] = cvt(k_new[i]), layer->v[loc[i]] = cvt(v_new[i])
 * k_new, v_new: (n, kv_heads, head_dim) of in_dtype.  loc: int64 (n), physical
 * rows of THIS pool; rows outside [0, rows) are skipped.  Conversions:
 * same dtype -> byte copy; f32 -> bf16 and f32/bf16 -> e4m3 round to nearest
 * even, e4m3 saturates to +-448 and maps NaN to 0x7F.  Duplicate locs (other
 * than the padding row 0) race; swa_validate reports them. */
swa_status_t swa_kv_store(const swa_kv_layer_t *layer, const int64_t *loc, int64_t n,
                          const void *k_new, const void *v_new, int32_t in_dtype,
                          hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Decode planning [host]: number of key splits per (request, kv head) and the
 * workspace swa_decode needs.  max_seq_len is a host-side upper bound of
 * seq_lens (a performance hint: any split count gives correct results).
 * Windows of up to 256 keys (0 <= window <= 255) use one split and no
 * workspace.  Full layers (window = -1) and longer windows (a per-layer
 * sliding_window_size, [SWA] 实现) are split by their key count,
 * min(max_seq_len, window + 1) for a window, into pieces of at least 512 keys,
 * up to about four (request, kv head, split) streams per compute unit. */
swa_status_t swa_decode_plan(int32_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                             int32_t window, int64_t max_seq_len, int32_t *num_splits,
                             size_t *workspace_bytes);

/* [host] Workspace bytes that suffice for every split count swa_decode_plan
 * can return for this batch, q_heads and head_dim when no request has more than
 * max_keys keys (its split count is capped at ceil(max_keys / 512)): an upper
 * bound for callers that size the workspace once.  0 when no split is needed
 * or the arguments are out of range. */
size_t swa_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t head_dim, int32_t max_keys);

/* ---------------------------------------------------------------------------
 * decode — one query per request at position i = seq_lens[b] - 1 ([SWA]
 * opening paragraph: each query sees the most recent window; 实现: W excludes
 * the current token, -1 = full; 设计: learnable per-head sink):
 *   keys j in [max(0, i - W), i] (all of [0, i] for window = -1)
 *   s_j = sm_scale * q_h . k_j, with kv head g = h / (q_heads / kv_heads)
 *   m   = max(max_j s_j, sink_h)
 *   o_h = sum_j e^{s_j - m} v_j / (sum_j e^{s_j - m} + e^{sink_h - m})
 * sinks NULL means no sink (sink_h = -inf).
 * Keys come from the window table when table_indptr is given (SWA layers: the
 * output of swa_translate_window with the same window), otherwise from
 * req_to_token directly (full layers, or single-pool windowed attention).
 * q: (batch, q_heads, head_dim) of q_dtype; out: same shape of out_dtype
 * (SWA_F32, or SWA_BF16 = the f32 result rounded to nearest even).
 * Supported: head_dim 128; q_dtype f32 with f32 K/V; q_dtype bf16 with bf16 or
 * e4m3 K/V; q_heads / kv_heads in {1, 2, 4, 8, 16}.
 * Precision: with bf16 or e4m3 K/V, P.V runs in f16 (weights rounded to f16,
 * V converted to f16, fp32 accumulation), so bf16 V values must satisfy
 * |v| <= 65504 (larger ones overflow to inf; e4m3 codes always fit); values
 * below 2^-14 in magnitude become f16 subnormals, accurate to 2^-25.  V is
 * not checked: an out-of-range V gives inf/NaN outputs, no error.
 * num_splits and workspace come from swa_decode_plan for the same shape.
 * An empty batch (idx->batch == 0) launches nothing and returns SWA_OK after
 * the same argument checks; q, out and the workspace may then be NULL. */
swa_status_t swa_decode(const void *q, int32_t q_dtype, int32_t q_heads, const swa_kv_layer_t *layer,
                        const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                        int64_t table_capacity, int32_t window, const float *sinks, float sm_scale,
                        void *out, int32_t out_dtype, int32_t num_splits, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * decode that allocates nothing — for callers that cannot allocate device
 * memory or hand over a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  swa_decode with the same
 * arguments minus the workspace: the split-K partials of a plan with
 * num_splits > 1 go to a static device array of 32 MiB that the library holds
 * on every GPU it runs on until the process ends; its address is looked up once
 * per device.  No hipMalloc / hipFree.  A plan whose partials
 * (batch * q_heads * num_splits * 520 bytes) exceed 32 MiB returns
 * SWA_E_WORKSPACE before any device call.  Every call on one GPU shares that
 * array: calls that overlap on one GPU (other streams, concurrent threads)
 * race.  Each call writes every partial it reads, so nothing carries over from
 * an earlier call. */
swa_status_t swa_decode_noalloc(const void *q, int32_t q_dtype, int32_t q_heads, const swa_kv_layer_t *layer,
                                const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                                int64_t table_capacity, int32_t window, const float *sinks, float sm_scale, void *out,
                                int32_t out_dtype, int32_t num_splits, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * decode with the current token's store fused in — the same result as
 *   swa_kv_store(layer, loc, batch, k_new, v_new, new_dtype);
 *   swa_decode(..., num_splits = 1, ...);
 * in one launch ([SWA] Attention backend: the new token's K/V are written to
 * the layer's pool right before its attention; [POOLS] 谁在往页里写).
 * loc (batch): the pool slot of each request's current token, i.e. of
 * position seq_lens[b] - 1, which its window's last entry resolves to (SWA
 * layers: the translated swa_loc); a loc outside [0, rows) is not stored.
 * k_new, v_new: bf16 (batch, kv_heads, head_dim), 16-byte aligned.  The
 * current token is attended from these rows converted to the pool format
 * exactly as stored.  Supported: windowed layers with 0 <= window <= 255,
 * bf16 q, bf16 or e4m3 pools, new_dtype SWA_BF16; other cases return
 * SWA_E_DTYPE / SWA_E_SHAPE (use the two calls).  An empty batch launches
 * nothing; q, out, loc, k_new and v_new may then be NULL. */
swa_status_t swa_decode_store(const void *q, int32_t q_dtype, int32_t q_heads, const swa_kv_layer_t *layer,
                              const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                              int64_t table_capacity, int32_t window, const float *sinks, float sm_scale,
                              const int64_t *loc, const void *k_new, const void *v_new, int32_t new_dtype,
                              void *out, int32_t out_dtype, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * One decode step of a hybrid model ([SWA] 双池与映射表: SWAKVPool holds a
 * full pool and an SWA pool, and layers_mapping sends each global layer id to
 * (its layer number inside its pool, whether it is an SWA layer); 设计:
 * MiMo-V2-Flash mixes 39 SWA layers with 9 full-attention layers; Attention
 * backend: the window's translated indices are built once per batch and
 * shared by every SWA layer; 实现: -1 is full attention).
 *
 * The step enqueues, in this order:
 *   1. swa_translate_window(idx, window) once, when any layer is an SWA layer;
 *   2. with a store and a mapping: swa_translate_loc(full_loc -> swa_loc) once;
 *   3. for each global layer l in order, through layers_mapping[l]:
 *      SWA layer  (swa_layers[pool_layer], window W):  the current token's
 *                 K/V stored at swa_loc (fused into the decode launch for bf16
 *                 pools, a separate swa_kv_store otherwise), then swa_decode
 *                 over the shared window table;
 *      full layer (full_layers[pool_layer], W = -1): the current token's K/V
 *                 stored at full_loc, then swa_decode over req_to_token with
 *                 the split count swa_decode_plan gives for max_seq_len and the
 *                 widest full layer's kv heads; the split partials use the
 *                 workspace, one layer at a time.
 * Every argument of every layer is checked before anything is enqueued; an
 * error launches nothing.  Without a mapping (idx->full_to_swa NULL, the
 * single-pool windowed mode) the SWA layers' window table and store use full
 * slots directly.
 *   layers_mapping, full_layers, swa_layers, q, out, sinks, k_new, v_new:
 *                [host] arrays (q, out, sinks, k_new, v_new: n_layers device
 *                pointers each, indexed by the global layer id; sinks may be
 *                NULL, or hold NULL entries for layers without sinks).
 *   q, out       (batch, q_heads, 128) of q_dtype / out_dtype, as swa_decode.
 *   full_loc     device int64 (batch): full slot of each request's current
 *                token (position seq_lens[b] - 1); NULL together with k_new and
 *                v_new: no store.
 *   swa_loc      device int64 (batch), written by the step (the translated
 *                full_loc); needed with a store, SWA layers and a mapping.
 *   k_new, v_new bf16 (batch, the layer's kv_heads, 128) per layer.
 *   slot_table, table_indptr, table_capacity: the window table
 *                (capacity >= batch * (window + 1)).
 *   workspace    swa_decode_step_workspace_bytes(step, idx, max_seq_len) bytes.
 * Errors: those of the calls above, plus SWA_E_ARG for a mapping entry outside
 * its pool's layer list, window < 0, or a store with a missing buffer. */
typedef struct swa_layer_map {
  int32_t pool_layer; /* index into full_layers or swa_layers */
  int32_t is_swa;     /* 1: SWA layer, 0: full-attention layer */
} swa_layer_map_t;

typedef struct swa_decode_step {
  int32_t n_layers;
  const swa_layer_map_t *layers_mapping;
  const swa_kv_layer_t *full_layers;
  int32_t n_full_layers;
  const swa_kv_layer_t *swa_layers;
  int32_t n_swa_layers;
  int32_t window;     /* the SWA layers' window, >= 0 */
  int32_t q_heads;
  int32_t q_dtype;
  int32_t out_dtype;
  const void *const *q;
  void *const *out;
  const float *const *sinks;
  float sm_scale;
  const int64_t *full_loc;
  int64_t *swa_loc;
  const void *const *k_new;
  const void *const *v_new;
} swa_decode_step_t;

/* [host] Workspace bytes swa_decode_step needs (0 without full layers or on
 * bad arguments). */
size_t swa_decode_step_workspace_bytes(const swa_decode_step_t *step, const swa_index_t *idx, int64_t max_seq_len);

swa_status_t swa_decode_step(const swa_decode_step_t *step, const swa_index_t *idx, int64_t max_seq_len,
                             int32_t *slot_table, int32_t *table_indptr, int64_t table_capacity, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * extend — windowed-causal prefill of a chunk over a cached prefix ([SWA]
 * 运行时: chunked prefill; same formula as decode).  Request b owns query rows
 * qo_indptr[b] .. qo_indptr[b+1]-1 holding positions prefix_lens[b] ..
 * seq_lens[b]-1; query i sees keys [max(0, i - W), i].  The chunk's own K/V
 * must already be in the pool (swa_kv_store first).
 * q, out: (total_q, q_heads, head_dim).  total_q (host) is the row count of q
 * and out, i.e. qo_indptr[batch].  Keys come from the window table built by
 * swa_translate_window(prefix_lens) when table_indptr is given, else from
 * req_to_token directly.  Supported: head_dim 128, bf16 q with bf16 K/V,
 * q_heads / kv_heads in {1, 2, 4, 8, 16}.  P.V runs in f16 as in swa_decode,
 * so V values must satisfy |v| <= 65504 (not checked).  Requests with no new tokens
 * (qo_indptr[b] == qo_indptr[b+1]) contribute nothing; an empty batch or
 * total_q == 0 launches nothing, and q and out may then be NULL. */
swa_status_t swa_extend(const void *q, int32_t q_dtype, int32_t q_heads, const int32_t *qo_indptr,
                        const int32_t *prefix_lens, int64_t total_q, const swa_kv_layer_t *layer,
                        const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                        int64_t table_capacity, int32_t window, const float *sinks, float sm_scale,
                        void *out, int32_t out_dtype, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Attention variants.
 *
 * Chunked local attention ([SWA] 设计: Llama4's chunked local layers).  With a
 * chunk size C > 0, positions form chunks of C from position 0 and query i
 * sees only the earlier positions of its own chunk and itself: keys
 * [max(first, C * floor(i / C)), i], where first is i - W for a window W >= 0
 * and 0 for W = -1.  swa_translate_window_chunked builds the slot table of
 * those keys (for extend: from the first new query's first key on);
 * swa_extend_chunked is swa_extend with the chunk bound in its masks and
 * reads the table built with the same W and C.  Decode needs no variant: a
 * decode reads exactly the keys its table lists, so swa_decode with the
 * chunked table (window = C - 1 when C <= 256, else -1 with a split plan for
 * C keys) is chunked local decode.  C = 0 is the plain window.
 */
swa_status_t swa_translate_window_chunked(const swa_index_t *idx, int32_t window, int32_t chunk,
                                          const int32_t *prefix_lens, int32_t *slot_table, int32_t *table_indptr,
                                          int64_t table_capacity, hipStream_t stream);

swa_status_t swa_extend_chunked(const void *q, int32_t q_dtype, int32_t q_heads, const int32_t *qo_indptr,
                                const int32_t *prefix_lens, int64_t total_q, const swa_kv_layer_t *layer,
                                const swa_index_t *idx, const int32_t *slot_table, const int32_t *table_indptr,
                                int64_t table_capacity, int32_t window, int32_t chunk, const float *sinks,
                                float sm_scale, void *out, int32_t out_dtype, hipStream_t stream);

/* Per-request SWA ring ([POOLS] SWATokenToKVPoolAllocator, per-request SWA
 * ring: each request slot owns the ring size rounded up to a page, the SWA
 * capacity is request slots x that, the paged SWA indices go unused).  Request
 * slot r (req_pool_idx) owns pool rows [r * R, (r + 1) * R) and position j lives
 * at row r * R + j mod R, with R = ring_rows (the rounded ring size): no
 * mapping, no eviction.  Valid while the positions one call reads or writes
 * span at most R (decode: W + 1; extend: W + the chunk).
 * swa_translate_window_ring writes the window's ring rows as the slot table
 * (req_to_token is not read; idx->r2t_rows bounds the request slots,
 * idx->r2t_stride the positions); swa_ring_locs writes the ring rows of the
 * new positions [prefix_lens[b], seq_lens[b]) of every request packed in
 * request order (prefix_lens NULL: decode, one position seq_lens[b] - 1 per
 * request) for swa_kv_store / swa_decode_store; at most n_out are written.
 * The layer views the ring pool, rows = request slots x R.  Errors: SWA_E_ARG,
 * SWA_E_SHAPE (ring rows of all slots reach 2^31). */
swa_status_t swa_translate_window_ring(const swa_index_t *idx, int64_t ring_rows, int32_t window, int32_t chunk,
                                       const int32_t *prefix_lens, int32_t *slot_table, int32_t *table_indptr,
                                       int64_t table_capacity, hipStream_t stream);

swa_status_t swa_ring_locs(const swa_index_t *idx, int64_t ring_rows, const int32_t *prefix_lens, int64_t *out,
                           int64_t n_out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * SWA eviction — release the SWA KV of positions that left each request's
 * window ([SWA] 运行时: free_swa_out_of_window_slots; 双池与映射表: free_swa).
 * For request b (row req_pool_idx[b] of req_to_token) the released positions
 * are [lo, hi) with
 *   lo = max(evicted_lens[b], protected_lens[b])        (protected_lens NULL: 0)
 *   hi = floor_page(pre_lens[b] - W)            mode 0, chunk cache
 *   hi = floor_page(pre_lens[b] - max(W, P))    mode 1, radix cache
 * (floor_page rounds down to a multiple of idx->page_size; a negative bound is
 * 0), and nothing when interval > 0 and hi - evicted_lens[b] < interval (the
 * decode eviction interval, 128 on the page).  For each released position whose
 * full slot f has full_to_swa[f] > 0, that SWA slot is released and
 * full_to_swa[f] is set to 0; entries that are already 0 release nothing, so a
 * repeated call frees nothing twice.  A request that releases a range gets
 * evicted_lens[b] = hi.
 *   full_to_swa  the mapping (map_len = idx->map_len entries), modified in
 *                place; idx->full_to_swa is not used.
 *   freed_pages  int64 (freed_capacity): the released SWA pages (slot / P), in
 *                request order, then position order; a page is reported at the
 *                first released position of a range and at every released
 *                position that starts a page.  Entries past the capacity are
 *                not written; *freed_count (device int64) receives the full
 *                number, so the caller can detect a short buffer.
 *   pre_lens, evicted_lens, protected_lens  device int32 [batch]
 *                (evicted_lens read and updated in place).
 *   workspace    device, swa_evict_workspace_bytes(batch, r2t_stride, page)
 *                bytes, 8-aligned; overwritten.
 * Ranges of different requests must not share full slots (a shared prefix is
 * protected).  Positions or slots outside their tables release nothing.
 * Errors: SWA_E_ARG (null or inconsistent arguments, window < 0, mode not 0/1,
 * interval < 0), SWA_E_WORKSPACE (workspace missing, short or misaligned),
 * SWA_E_SHAPE (req_to_token rows longer than 65,535 x 2,048 positions). */
size_t swa_evict_workspace_bytes(int32_t batch, int64_t r2t_stride, int32_t page_size);

swa_status_t swa_evict(const swa_index_t *idx, int64_t *full_to_swa, const int32_t *pre_lens,
                       const int32_t *protected_lens, int32_t *evicted_lens, int32_t window, int32_t mode,
                       int32_t interval, int64_t *freed_pages, int64_t freed_capacity, int64_t *freed_count,
                       void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Unified pool ([PR] 功能与动机 and 实现拆解, steps 1-3: build_mha_views,
 * view_tail_pad_bytes, _assert_kernel_id_bound, translate_kv_loc_for_kernel).
 * One raw byte buffer holds a sub-pool of L layers as page-major envelopes
 * [L0_K*P | L0_V*P | L1_K*P | L1_V*P | ...]: page p is 2L row blocks of P rows,
 * a row being kv_heads * head_dim elements.  Layer l's K view starts at block
 * 2l of page 0 and its V view at block 2l + 1; both are ordinary dense
 * (n_rows, kv_heads, head_dim) layers with n_rows = num_pages * 2L * P, so
 * row kernel_id(t) = v2p[t / P] * (P * 2L) + t % P of the view is the row of
 * virtual token t, and every kernel of this library runs on them unchanged.
 * The last view reaches (2L - 1) * P rows past the last envelope: the buffer
 * must hold one envelope of tail pad after the envelopes. */

/* [host] Bytes a sub-pool needs from its anchor on: num_pages envelopes plus
 * the tail pad.  -1 on bad arguments. */
int64_t swa_unified_pool_bytes(int32_t layer_num, int32_t kv_heads, int32_t head_dim, int32_t dtype,
                               int32_t page_size, int64_t num_pages);

/* [host] Fill views[0 .. layer_num) (host array) with the per-layer K/V views
 * of the sub-pool at raw + anchor_bytes (device buffer of raw_bytes bytes).
 * No device work.  Errors: SWA_E_ARG (null / misaligned: raw and anchor must
 * be 16-byte aligned), SWA_E_DTYPE, SWA_E_SHAPE (rows not a multiple of 16
 * bytes, the views would run past the buffer (tail pad missing), or
 * n_rows >= 2^31, the bound of int32 index buffers). */
swa_status_t swa_unified_layer_views(void *raw, int64_t raw_bytes, int64_t anchor_bytes, int32_t layer_num,
                                     int32_t kv_heads, int32_t head_dim, int32_t dtype, int32_t page_size,
                                     int64_t num_pages, float k_scale, float v_scale, swa_kv_layer_t *views);

/* Virtual token ids -> kernel-facing ids: out[i] = v2p[t / P] * (P *
 * multiplier) + t % P for t = virt[i], with multiplier = 2L, the row blocks
 * per page; a tombstoned page (v2p = -1) and an id outside the page table
 * (t < 0 or t / P >= n_pages) give 0, the sink row.  virt / out: device
 * int64 [n] (may be the same buffer); v2p: device int64 [n_pages]. */
swa_status_t swa_translate_kernel_ids(const int64_t *virt, int64_t n, const int64_t *v2p, int64_t n_pages,
                                      int32_t page_size, int32_t multiplier, int64_t *out, hipStream_t stream);

/* swa_translate_window on a unified pool: req_to_token holds virtual ids and
 * each window position's slot is its kernel-facing id (as above), written to
 * the int32 slot table; idx->full_to_swa is not used.  Errors as
 * swa_translate_window, plus SWA_E_SHAPE when a kernel-facing id could reach
 * 2^31. */
swa_status_t swa_translate_window_unified(const swa_index_t *idx, const int64_t *v2p, int64_t n_pages,
                                          int32_t multiplier, int32_t window, const int32_t *prefix_lens,
                                          int32_t *slot_table, int32_t *table_indptr, int64_t table_capacity,
                                          hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Paired allocation ([POOLS] 三重映射, alloc_extend, alloc_decode, 扩容与不足
 * and SWATokenToKVPoolAllocator; [SWA] 双池与映射表: alloc, alloc_extend and
 * alloc_decode take the same number of slots from both allocators, then write
 * the mapping).
 *
 * A paged allocator's free list is an array of page numbers handed out from
 * its head; page 0 is never on it.  The caller passes each list from its
 * current head and advances the head by the number of pages taken (*new_pages,
 * or swa_alloc_pages_needed on host copies of the lengths); freeing is the
 * caller's (pages released by swa_evict go back on the SWA list).
 *
 * For request b (page size P, pre = pre_lens[b], seq = seq_lens[b]) the new
 * positions [pre, seq) get, in order and packed after the earlier requests'
 * new positions in out_full / out_swa:
 *   - positions before ceil_P(pre) (the rest of the page the prefix ends in):
 *     last + 1, last + 2, ..., where last is last_loc[b] on the full side and
 *     full_to_swa[last_loc[b]] on the SWA side (-1, no prefix, stays -1);
 *   - position p >= ceil_P(pre): page * P + p mod P, with page the request's
 *     ((p - ceil_P(pre)) / P)-th new page; the request's new pages are
 *     ceil(seq/P) - ceil(pre/P) consecutive entries of each free list, after
 *     the earlier requests' new pages.
 * Then full_to_swa[full slot] = SWA slot for every new position.  With
 * swa_list NULL only the full pool is allocated (one-pool cache) and
 * full_to_swa is not used.
 *
 * Before anything is launched the host proves that the free lists are long
 * enough, as the pages do: first with the bound extend_num_tokens / P + batch
 * + 1 (decode: batch); if that does not fit, with the exact count from the host
 * copies of the lengths; if those are NULL or the count does not fit, the call
 * returns SWA_E_NOSPACE and changes nothing.  The kernels never read past a
 * free list (a page beyond it would read as page 0) and never write more than
 * extend_num_tokens (decode: batch) outputs.
 *   pre_lens, seq_lens  device int32 [batch]; last_loc device int64 [batch]:
 *                the full slot of position pre - 1 (decode: seq - 2), or -1.
 *   full, swa_list  [host] structs naming device int64 free lists.
 *   full_to_swa  the mapping (map_len entries, trailing -1), written in place.
 *   extend_num_tokens  [host] sum of seq - pre, the length of the outputs.
 *   pre_lens_host, seq_lens_host  [host] optional copies for the exact count.
 *   out_full, out_swa  device int64 (out_swa may be NULL).
 *   new_pages  optional device int64: the pages taken from each list.
 * Errors: SWA_E_ARG, SWA_E_NOSPACE. */
typedef struct swa_free_list {
  const int64_t *pages; /* device int64 page numbers, taken from index 0 on */
  int64_t count;        /* entries available */
} swa_free_list_t;

/* [host] The exact number of new pages: sum of ceil(seq/P) - ceil(pre/P) over
 * host arrays (pre_lens NULL: decode, pre = seq - 1).  -1 on bad arguments. */
int64_t swa_alloc_pages_needed(const int32_t *pre_lens, const int32_t *seq_lens, int32_t batch, int32_t page_size);

swa_status_t swa_alloc_extend(int32_t batch, int32_t page_size, const int32_t *pre_lens, const int32_t *seq_lens,
                              const int64_t *last_loc, const swa_free_list_t *full, const swa_free_list_t *swa_list,
                              int64_t *full_to_swa, int64_t map_len, int64_t extend_num_tokens,
                              const int32_t *pre_lens_host, const int32_t *seq_lens_host, int64_t *out_full,
                              int64_t *out_swa, int64_t *new_pages, hipStream_t stream);

/* One new token per request (pre = seq - 1): last + 1 while it stays in its
 * page, else the start of the next free page ([POOLS] alloc_decode). */
swa_status_t swa_alloc_decode(int32_t batch, int32_t page_size, const int32_t *seq_lens, const int64_t *last_loc,
                              const swa_free_list_t *full, const swa_free_list_t *swa_list, int64_t *full_to_swa,
                              int64_t map_len, const int32_t *seq_lens_host, int64_t *out_full, int64_t *out_swa,
                              int64_t *new_pages, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Validation (debugging aid; SYNCHRONOUS: waits for `stream`).  Counts the
 * index data that the kernels above silently absorb, per the contracts of
 * [SWA] 双池与映射表 and 运行时 (a live window never holds a tombstone: eviction
 * frees only positions that left the window) and [POOLS] 一重映射, 二重映射
 * and 释放 (indices stay inside their tables; a slot is handed out once, page
 * 0 being the shared sink of padded writes).
 *
 * Window part (idx->batch requests): request b is bad when req_pool_idx[b]
 * is outside [0, r2t_rows), seq_lens[b] outside [0, r2t_stride] or, with
 * prefix_lens, prefix_lens[b] outside [0, seq_lens[b]]; its positions are then
 * skipped.  Otherwise every position of its window (the ones swa_translate_
 * window would emit for the same window and prefix_lens) is classified:
 *   full_out_of_range  with a map: req_to_token entry outside [-1, map_len-1)
 *   tombstones         SWA slot 0 (with a map) / full slot 0 (without)
 *   sentinels          SWA slot -1 (with a map)
 *   slot_out_of_range  any other slot outside [0, pool_rows)
 * Store part (n_store locs, may be 0 / NULL): locs outside [0, pool_rows), and
 * repeats of a loc outside page 0 (each occurrence after the first counts).
 * Extend part (qo_indptr may be NULL): qo_bad counts requests b whose query
 * rows qo_indptr[b] .. qo_indptr[b+1]-1 are not in order inside [0, total_q],
 * or (for a request that is not bad, with prefix_lens) are not exactly its
 * seq_lens[b] - prefix_lens[b] new positions.  swa_extend clamps such rows
 * into [0, total_q] and never reads or writes outside q and out.
 * pool_rows: rows of the pool the window and the locs address (the SWA pool
 * with a map, the full pool without).
 * workspace: device, at least swa_validate_workspace_bytes(pool_rows) bytes,
 * 16-byte aligned; its contents are overwritten.  report: [host].
 * Returns SWA_E_ARG for null / negative arguments or page_size < 1. */
typedef struct swa_validate_report {
  int64_t bad_requests;
  int64_t positions;
  int64_t full_out_of_range;
  int64_t tombstones;
  int64_t sentinels;
  int64_t slot_out_of_range;
  int64_t store_locs;
  int64_t store_out_of_range;
  int64_t store_duplicates;
  int64_t qo_bad;
} swa_validate_report_t;

size_t swa_validate_workspace_bytes(int64_t pool_rows);

swa_status_t swa_validate(const swa_index_t *idx, int32_t window, const int32_t *prefix_lens,
                          const int32_t *qo_indptr, int64_t total_q, int64_t pool_rows, const int64_t *store_loc,
                          int64_t n_store, void *workspace, size_t workspace_bytes, swa_validate_report_t *report,
                          hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *swa_status_string(swa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
