// Internal helpers shared by the HIP kernels of libswa (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "swa.h"

namespace swa {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;   // MFMA bf16 operand
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;    // 16x16 MFMA accumulator
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;  // packed conversion result

constexpr float kLog2e = 1.4426950408889634f;
// Finite stand-in for -inf as a running maximum: exp2(x - kNegBig) stays 0 for
// x = -inf and exp2(kNegBig - kNegBig) = 1, so empty ranges never produce NaN.
constexpr float kNegBig = -1.0e30f;

// bf16 <-> f32.  bf16 is the upper half of an IEEE binary32 word.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even; NaN -> quiet NaN 0x7FC0.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_rne(lo)) | (static_cast<uint32_t>(f32_to_bf16_rne(hi)) << 16);
}

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
// For finite inputs it equals pack_bf16x2; NaN payloads are the hardware's.
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2_hw(float lo, float hi) {
  f32x2v_t x = {lo, hi};
  bf16x2v_t r = __builtin_convertvector(x, bf16x2v_t);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

// The P.V product of the MFMA attention kernels runs in IEEE binary16 (f16):
// the softmax weights are rounded to f16 (11 significant bits, against 8 for
// bf16) and the V rows are staged as f16, which holds every bf16 value in
// [2^-14, 65504] exactly (smaller values to within 2^-25; larger ones
// overflow to inf, so V must stay inside f16's range).  A query whose output
// is dominated by a few keys is as large as a V row while the output's RMS is
// that of an average over the window; with bf16 weights the rounding of the
// few large weights alone could then reach 2% of the RMS, with f16 it stays
// below 0.5%.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));   // MFMA f16 operand
typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4v_t __attribute__((ext_vector_type(4)));

// Two floats -> two f16 (round to nearest even) in one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack_f16x2_hw(float lo, float hi) {
  f32x2v_t x = {lo, hi};
  f16x2v_t r = __builtin_convertvector(x, f16x2v_t);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

// acc + both f16 values of a packed pair, in f32 (v_dot2c_f32_f16 against
// (1, 1); the products are exact): the normaliser sums the same rounded
// weights that enter P.V, so the output is an exact convex combination of the
// staged V rows (plus the sink).
__device__ __forceinline__ float f16x2_acc(uint32_t u, float acc) {
  f16x2v_t a, ones;
  const uint32_t one2 = 0x3C003C00u;
  __builtin_memcpy(&a, &u, 4);
  __builtin_memcpy(&ones, &one2, 4);
  return __builtin_amdgcn_fdot2(a, ones, acc, false);
}

// Eight bf16 (a 16-byte piece of a row) -> eight f16 in the same order.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(const uint4 &x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = pack_f16x2_hw(__uint_as_float(w[i] << 16), __uint_as_float(w[i] & 0xFFFF0000u));
  return make_uint4(r[0], r[1], r[2], r[3]);
}

// c + A B on the f16 matrix cores (16x16x32), operands carried as 8 x 16 bits.
__device__ __forceinline__ f32x4_t mfma_f16(const bf16x8_t &a, const bf16x8_t &b, const f32x4_t &c) {
  f16x8_t x, y;
  __builtin_memcpy(&x, &a, 16);
  __builtin_memcpy(&y, &b, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(x, y, c, 0, 0, 0);
}

// Reductions over the four 16-lane rows of a wavefront (lanes l, l^16, l^32,
// l^48).  gfx950's row swaps do it in the VALU: v_permlane16_swap pairs rows
// (0, 1) and (2, 3), v_permlane32_swap the two halves, so no LDS round trip
// (and no wait on LDS loads issued before it) sits in the softmax.
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane r supplies the LDS
// address of 4 consecutive 16-bit elements (row r of a 16 x 4 block M);
// lane i receives M[i/4 + 4e][i%4] for e = 0..3.
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
__device__ __forceinline__ i16x4_t lds_read_tr16(const uint16_t *lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t *)(const_cast<uint16_t *>(lds_ptr)));
}

// OCP e4m3fn encoder: round to nearest even, saturate finite overflow (and inf)
// to +-448, NaN -> 0x7F.  Normal range: the binary32 word is rounded at the
// 20-bit boundary (3 mantissa bits kept) and re-biased (127 - 7 = 120);
// below 2^-6 the value is a multiple of 2^-9 and rintf gives the RNE count.
__device__ __forceinline__ uint8_t f32_to_e4m3_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7F;
  uint32_t code;
  if (a < 0x3C800000u) {  // |f| < 2^-6: subnormal codes 0..8
    code = static_cast<uint32_t>(rintf(__uint_as_float(a) * 512.0f));
  } else {
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return static_cast<uint8_t>(sign | code);
}

// 64-bit row offset of (slot, head) in a (rows, heads, dim) array, in elements.
__device__ __forceinline__ int64_t row_elem(int64_t slot, int32_t heads, int32_t head, int32_t dim) {
  return (slot * heads + head) * static_cast<int64_t>(dim);
}

}  // namespace swa

// Launchers implemented in the .hip translation units (host side, internal).
namespace swa {
hipError_t launch_translate_loc(const int64_t *full_loc, int64_t n, const int64_t *map, int64_t map_len,
                                int64_t *out, hipStream_t stream);
hipError_t launch_translate_window(const swa_index_t &idx, int32_t window, int32_t chunk, const int32_t *prefix_lens,
                                   int32_t *table, int32_t *indptr, int64_t capacity, hipStream_t stream);
hipError_t launch_translate_window_ring(const swa_index_t &idx, int64_t ring_rows, int32_t window, int32_t chunk,
                                        const int32_t *prefix_lens, int32_t *table, int32_t *indptr,
                                        int64_t capacity, hipStream_t stream);
hipError_t launch_ring_locs(const swa_index_t &idx, int64_t ring_rows, const int32_t *prefix_lens, int64_t *out,
                            int64_t capacity, hipStream_t stream);
hipError_t launch_kv_store(const swa_kv_layer_t &layer, const int64_t *loc, int64_t n, const void *k_new,
                           const void *v_new, int32_t in_dtype, hipStream_t stream);

struct DecodeArgs {
  const void *q;
  int32_t q_dtype;
  int32_t q_heads;
  swa_kv_layer_t layer;
  swa_index_t idx;
  const int32_t *table;
  const int32_t *indptr;
  int64_t capacity;
  int32_t window;
  const float *sinks;
  float sm_scale;
  void *out;
  int32_t out_dtype;
  int32_t num_splits;
  float *ws;  // partials: m, l (batch*q_heads*num_splits each), acc (... * head_dim)
  // fused store of the current token (null: none): bf16 (batch, kv_heads,
  // head_dim) rows written to pool slot new_loc[b]
  const void *k_new;
  const void *v_new;
  const int64_t *new_loc;
};
// Largest window the one-split window kernel (and so the fused store) handles.
constexpr int32_t kMaxFusedWindow = 255;
hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
// Static scratch of the no-allocation decode (split-K partials): its size, and
// its device address on the current device.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
hipError_t static_scratch(void **ptr);

hipError_t launch_validate(const swa_index_t &idx, int32_t window, const int32_t *prefix_lens,
                           const int32_t *qo_indptr, int64_t total_q, int64_t pool_rows, const int64_t *store_loc,
                           int64_t n_store, void *workspace, int64_t counters_bytes, hipStream_t stream);

// Eviction works on chunks of positions that start at page boundaries: the
// smallest multiple of the page size that is at least one apply pass (256
// threads x kEvictApplyPerThread positions).
#ifndef SWA_EVICT_APPLY_PER_THREAD
#define SWA_EVICT_APPLY_PER_THREAD 8
#endif
constexpr int kEvictApplyPerThread = SWA_EVICT_APPLY_PER_THREAD;
__host__ __device__ inline int64_t evict_chunk(int32_t page) {
  const int64_t pass = 256 * kEvictApplyPerThread;
  return (pass + static_cast<int64_t>(page) - 1) / page * page;
}
__host__ __device__ inline int64_t evict_chunks(int64_t r2t_stride, int32_t page) {
  const int64_t c = evict_chunk(page);
  return (r2t_stride + c - 1) / c;
}

// Candidates of one request's range (its first position and each page start in
// it): at most this many for a req_to_token row of r2t_stride positions.
__host__ __device__ inline int64_t evict_cands(int64_t r2t_stride, int32_t page) { return r2t_stride / page + 2; }
// Byte offset of the candidates' mapping values in the workspace (8-aligned).
__host__ __device__ inline int64_t evict_cand_offset(int32_t batch, int64_t r2t_stride, int32_t page) {
  return (static_cast<int64_t>(batch) * (3 + evict_chunks(r2t_stride, page)) * 4 + 7) / 8 * 8;
}

// workspace: int32 [batch] counts, [batch][2] ranges, [batch][evict_chunks] bases,
// then (8-aligned) int64 [batch][evict_cands] the candidates' mapping values
hipError_t launch_evict(const swa_index_t &idx, int64_t *full_to_swa, const int32_t *pre_lens,
                        const int32_t *protected_lens, int32_t *evicted_lens, int32_t window, int32_t radix,
                        int32_t interval, int64_t *freed_pages, int64_t capacity, int64_t *freed_count,
                        int32_t *workspace, hipStream_t stream);

hipError_t launch_translate_window_unified(const swa_index_t &idx, const int64_t *v2p, int64_t n_pages,
                                           int32_t multiplier, int32_t window, const int32_t *prefix_lens,
                                           int32_t *table, int32_t *indptr, int64_t capacity, hipStream_t stream);
hipError_t launch_translate_ids(const int64_t *virt, int64_t n, const int64_t *v2p, int64_t n_pages,
                                int32_t page_size, int32_t multiplier, int64_t *out, hipStream_t stream);

struct AllocArgs {
  int32_t batch;
  int32_t page_size;
  bool decode;              // one new token per request (pre = seq - 1; pre_lens unused)
  const int32_t *pre_lens;  // device
  const int32_t *seq_lens;  // device
  const int64_t *last_loc;  // device: full slot of position pre - 1, or -1
  const int64_t *free_full;
  int64_t n_free_full;
  const int64_t *free_swa;  // null: one pool
  int64_t n_free_swa;
  int64_t *full_to_swa;
  int64_t map_len;
  int64_t *out_full;
  int64_t *out_swa;
  int64_t capacity;
  int64_t *new_pages;
};

hipError_t launch_alloc(const AllocArgs &a, hipStream_t stream);

struct ExtendArgs {
  int32_t chunk;  // chunked local attention: chunk size, 0 = none
  const void *q;
  int32_t q_heads;
  const int32_t *qo_indptr;
  const int32_t *prefix_lens;
  int64_t total_q;
  swa_kv_layer_t layer;
  swa_index_t idx;
  const int32_t *table;
  const int32_t *indptr;
  int64_t capacity;
  int32_t window;
  const float *sinks;
  float sm_scale;
  void *out;
  int32_t out_dtype;
};
hipError_t launch_extend(const ExtendArgs &a, hipStream_t stream);
}  // namespace swa
