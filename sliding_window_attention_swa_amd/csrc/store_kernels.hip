// kv_store: scatter new K/V rows into one layer's pool rows.
//
// SWA note (zdszero.github.io/swa.html), section Attention backend: SWA layers
// receive an already translated swa_loc and the pool never translates.
// SGLang memory-pool article (pinghaoyang.com.cn), sections 二重映射 (per-layer
// (size + page, heads, dim) buffers; fp8 held as bytes) and 谁在往页里写
// (KVWriteLoc).
//
// A pool row (all kv heads of one slot) is contiguous, so each token moves one
// contiguous run of kv_heads * head_dim elements.  Each thread converts one
// 16-byte source vector; consecutive threads cover consecutive bytes of a row,
// so both the reads and the row writes are coalesced.
#include "common.hpp"

namespace swa {
namespace {

template <typename In, typename Out>
struct Cvt;

// Vector width: 8 source elements per thread for 2-byte inputs, 4 for 4-byte.
template <>
struct Cvt<uint16_t, uint16_t> {  // bf16 -> bf16 copy
  static constexpr int kVec = 8;
  __device__ static void run(const uint16_t *src, uint16_t *dst) {
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
  }
};
template <>
struct Cvt<float, float> {  // f32 -> f32 copy
  static constexpr int kVec = 4;
  __device__ static void run(const float *src, float *dst) {
    *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
  }
};
template <>
struct Cvt<float, uint16_t> {  // f32 -> bf16, nearest even
  static constexpr int kVec = 4;
  __device__ static void run(const float *src, uint16_t *dst) {
    float4 x = *reinterpret_cast<const float4 *>(src);
    uint2 o;
    o.x = pack_bf16x2(x.x, x.y);
    o.y = pack_bf16x2(x.z, x.w);
    *reinterpret_cast<uint2 *>(dst) = o;
  }
};
template <>
struct Cvt<uint16_t, uint8_t> {  // bf16 -> e4m3fn, nearest even, saturating
  static constexpr int kVec = 8;
  __device__ static void run(const uint16_t *src, uint8_t *dst) {
    uint4 x = *reinterpret_cast<const uint4 *>(src);
    uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t o[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint16_t h = static_cast<uint16_t>(w[e >> 1] >> ((e & 1) * 16));
      o[e >> 2] |= static_cast<uint32_t>(f32_to_e4m3_rne(bf16_to_f32(h))) << ((e & 3) * 8);
    }
    *reinterpret_cast<uint2 *>(dst) = make_uint2(o[0], o[1]);
  }
};
template <>
struct Cvt<float, uint8_t> {  // f32 -> e4m3fn
  static constexpr int kVec = 4;
  __device__ static void run(const float *src, uint8_t *dst) {
    float4 x = *reinterpret_cast<const float4 *>(src);
    uint32_t o = static_cast<uint32_t>(f32_to_e4m3_rne(x.x)) | (static_cast<uint32_t>(f32_to_e4m3_rne(x.y)) << 8) |
                 (static_cast<uint32_t>(f32_to_e4m3_rne(x.z)) << 16) |
                 (static_cast<uint32_t>(f32_to_e4m3_rne(x.w)) << 24);
    *reinterpret_cast<uint32_t *>(dst) = o;
  }
};

// grid.y = 2 (0: K, 1: V); grid.x * block covers n * vecs_per_row vectors.
template <typename In, typename Out>
__global__ void __launch_bounds__(256) kv_store_kernel(Out *__restrict__ pool_k, Out *__restrict__ pool_v,
                                                       int64_t rows, const int64_t *__restrict__ loc, int64_t n,
                                                       const In *__restrict__ k_new, const In *__restrict__ v_new,
                                                       int32_t row_elems) {
  constexpr int kVec = Cvt<In, Out>::kVec;
  const int32_t vecs_per_row = row_elems / kVec;
  const int64_t total = n * vecs_per_row;
  Out *__restrict__ pool = blockIdx.y ? pool_v : pool_k;
  const In *__restrict__ src = blockIdx.y ? v_new : k_new;
  const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; t < total; t += step) {
    const int64_t tok = t / vecs_per_row;
    const int32_t vec = static_cast<int32_t>(t - tok * vecs_per_row);
    const int64_t slot = loc[tok];
    if (slot < 0 || slot >= rows) continue;  // outside the pool: dropped
    Cvt<In, Out>::run(src + tok * row_elems + vec * kVec, pool + slot * row_elems + vec * kVec);
  }
}

template <typename In, typename Out>
hipError_t launch_typed(const swa_kv_layer_t &layer, const int64_t *loc, int64_t n, const void *k_new,
                        const void *v_new, hipStream_t stream) {
  const int32_t row_elems = layer.kv_heads * layer.head_dim;
  const int64_t total = n * (row_elems / Cvt<In, Out>::kVec);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((kv_store_kernel<In, Out>), dim3(static_cast<uint32_t>(blocks), 2), dim3(256), 0, stream,
                     static_cast<Out *>(layer.k), static_cast<Out *>(layer.v), layer.rows, loc, n,
                     static_cast<const In *>(k_new), static_cast<const In *>(v_new), row_elems);
  return hipGetLastError();
}

}  // namespace

// The API layer has checked the dtype pair and that a row is a whole number
// of vectors (kv_heads * head_dim divisible by 8).
hipError_t launch_kv_store(const swa_kv_layer_t &layer, const int64_t *loc, int64_t n, const void *k_new,
                           const void *v_new, int32_t in_dtype, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int32_t out = layer.dtype;
  if (in_dtype == SWA_BF16 && out == SWA_BF16) return launch_typed<uint16_t, uint16_t>(layer, loc, n, k_new, v_new, stream);
  if (in_dtype == SWA_F32 && out == SWA_F32) return launch_typed<float, float>(layer, loc, n, k_new, v_new, stream);
  if (in_dtype == SWA_F32 && out == SWA_BF16) return launch_typed<float, uint16_t>(layer, loc, n, k_new, v_new, stream);
  if (in_dtype == SWA_BF16 && out == SWA_FP8_E4M3) return launch_typed<uint16_t, uint8_t>(layer, loc, n, k_new, v_new, stream);
  if (in_dtype == SWA_F32 && out == SWA_FP8_E4M3) return launch_typed<float, uint8_t>(layer, loc, n, k_new, v_new, stream);
  return hipErrorInvalidValue;
}

}  // namespace swa
