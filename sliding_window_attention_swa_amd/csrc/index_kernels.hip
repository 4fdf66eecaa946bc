// Index translation kernels: flat full -> SWA loc translation and the fused
// window gather (req_to_token -> full slot -> full_to_swa -> SWA slot), and
// their unified-pool forms (virtual id -> kernel-facing row through a page
// table).
//
// SWA note (zdszero.github.io/swa.html), sections 双池与映射表 and Attention
// backend: the full index is the primary address; the SWA slot of a token is
// full_to_swa[full], 0 meaning "no SWA slot" and a trailing -1 making -1
// translate to -1; backends translate the window once per batch.  SGLang
// memory-pool article (pinghaoyang.com.cn), section 一重映射: req_to_token
// rows hold each position's full slot, row 0 is padding.
#include "common.hpp"

namespace swa {
namespace {

__device__ __forceinline__ int64_t map_full(const int64_t *__restrict__ map, int64_t map_len, int64_t full) {
  if (full == -1) return map[map_len - 1];
  if (full < 0 || full >= map_len - 1) return 0;
  return map[full];
}

__global__ void __launch_bounds__(256) translate_loc_kernel(const int64_t *__restrict__ full_loc, int64_t n,
                                                            const int64_t *__restrict__ map, int64_t map_len,
                                                            int64_t *__restrict__ out) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (; i < n; i += step) out[i] = map_full(map, map_len, full_loc[i]);
}

// Unified pool (prhub.com.cn digest of sglang pull request 34602, 实现拆解:
// translate_kv_loc_for_kernel): a virtual id t addresses row
// v2p[t / P] * (P * multiplier) + t % P of a dense per-layer view, multiplier
// being the row blocks per page (2 x layers); a tombstoned page (-1) lands on
// row 0, the sink.  Ids outside the page table read row 0 as well.
struct PageTable {
  const int64_t *__restrict__ v2p;
  int64_t n_pages;
  int32_t page;
  int64_t stride;  // page * multiplier
  __device__ __forceinline__ int64_t operator()(int64_t, int64_t, int64_t virt) const {
    if (virt < 0) return 0;
    const int64_t pg = virt / page;
    if (pg >= n_pages) return 0;
    const int64_t id = v2p[pg] * stride + virt % page;
    return id > 0 ? id : 0;
  }
};

// The two-pool translation (or none: a full layer reads req_to_token directly).
struct MapTable {
  const int64_t *__restrict__ map;
  int64_t map_len;
  __device__ __forceinline__ int64_t operator()(int64_t, int64_t, int64_t full) const {
    return map ? map_full(map, map_len, full) : full;
  }
};

// Per-request SWA ring ("SGLang 源码完全拆解(十五)", SWATokenToKVPoolAllocator:
// each request slot owns a ring of the ring size rounded up to a page, the
// paged SWA indices go unused): position `pos` of request slot `row` lives at
// row * R + pos mod R; req_to_token is not read.
struct RingTable {
  int64_t ring_rows;
  __device__ __forceinline__ int64_t operator()(int64_t row, int64_t pos, int64_t) const {
    return row * ring_rows + pos % ring_rows;
  }
};

__global__ void __launch_bounds__(256) translate_ids_kernel(const int64_t *__restrict__ virt, int64_t n,
                                                            PageTable tr, int64_t *__restrict__ out) {
  int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (; i < n; i += step) out[i] = tr(0, 0, virt[i]);
}

// Pool rows of the new positions [prefix, seq) of every request in a ring
// (decode: prefix = seq - 1), packed in request order.  One workgroup per
// request; the output offset is the earlier requests' new positions.
__global__ void __launch_bounds__(256) ring_locs_kernel(const int32_t *__restrict__ req_idx, int64_t n_slots,
                                                        const int32_t *__restrict__ seq_lens,
                                                        const int32_t *__restrict__ prefix_lens, int64_t ring_rows,
                                                        int64_t *__restrict__ out, int64_t capacity) {
  __shared__ int64_t partial[4];
  const int32_t b = blockIdx.x;
  auto span = [&](int32_t r, int64_t &pre, int64_t &seq) {
    seq = seq_lens[r];
    pre = prefix_lens ? prefix_lens[r] : seq - 1;
    if (pre < 0) pre = 0;
    if (seq < pre) seq = pre;
  };
  int64_t before = 0;
  for (int32_t r = threadIdx.x; r < b; r += blockDim.x) {
    int64_t pre, seq;
    span(r, pre, seq);
    before += seq - pre;
  }
  for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o);
  if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = before;
  __syncthreads();
  before = partial[0] + partial[1] + partial[2] + partial[3];
  int64_t pre, seq;
  span(b, pre, seq);
  int64_t row = req_idx[b];
  if (row < 0 || row >= n_slots) row = 0;
  for (int64_t k = threadIdx.x; k < seq - pre; k += blockDim.x) {
    const int64_t at = before + k;
    if (at < capacity) out[at] = row * ring_rows + (pre + k) % ring_rows;
  }
}

// Number of window entries of request b: positions lo .. L-1.
// The first key of query position i: i - W (W >= 0), the start of i's chunk of
// C positions (chunked local attention, C > 0), the later of the two, >= 0.
__device__ __forceinline__ int32_t first_key(int32_t i, int32_t window, int32_t chunk) {
  int32_t lo = 0;
  if (window >= 0 && i - window > lo) lo = i - window;
  if (chunk > 0 && i > 0 && i - i % chunk > lo) lo = i - i % chunk;
  return lo;
}

__device__ __forceinline__ int32_t window_count(const int32_t *__restrict__ seq_lens,
                                                const int32_t *__restrict__ prefix_lens, int32_t window,
                                                int32_t chunk, int64_t stride, int32_t b, int32_t *lo_out) {
  int32_t L = seq_lens[b];
  if (L < 0) L = 0;
  if (L > stride) L = static_cast<int32_t>(stride);
  int32_t p = prefix_lens ? prefix_lens[b] : L - 1;
  if (p > L) p = L;
  const int32_t lo = first_key(p, window, chunk);
  if (lo_out) *lo_out = lo;
  int32_t c = L - lo;
  return c > 0 ? c : 0;
}

// One workgroup per request.  The workgroup first sums the counts of the
// requests before it (an exclusive prefix sum done redundantly per request,
// which avoids a separate scan launch and any host read of device lengths),
// then gathers and translates its window with coalesced int32 reads.
template <typename Translate>
__global__ void __launch_bounds__(256) translate_window_kernel(
    const int32_t *__restrict__ r2t, int64_t r2t_rows, int64_t r2t_stride, const int32_t *__restrict__ req_idx,
    const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ prefix_lens, Translate tr, int32_t batch,
    int32_t window, int32_t chunk, int32_t *__restrict__ table, int32_t *__restrict__ indptr, int64_t capacity) {
  __shared__ int64_t partial[256];
  const int32_t b = blockIdx.x;
  if (batch == 0) {  // empty batch: the prefix sum is the single 0
    if (threadIdx.x == 0) indptr[0] = 0;
    return;
  }
  int64_t acc = 0;
  for (int32_t t = threadIdx.x; t < b; t += blockDim.x)
    acc += window_count(seq_lens, prefix_lens, window, chunk, r2t_stride, t, nullptr);
  partial[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (threadIdx.x < s) partial[threadIdx.x] += partial[threadIdx.x + s];
    __syncthreads();
  }
  const int64_t base = partial[0];
  int32_t lo = 0;
  const int32_t count = window_count(seq_lens, prefix_lens, window, chunk, r2t_stride, b, &lo);
  if (threadIdx.x == 0) {
    indptr[b] = static_cast<int32_t>(base);
    if (b == batch - 1) indptr[batch] = static_cast<int32_t>(base + count);
  }
  int64_t row = req_idx[b];
  if (row < 0 || row >= r2t_rows) row = 0;
  const int32_t *__restrict__ src = r2t ? r2t + row * r2t_stride + lo : nullptr;  // none: ring mode
  for (int32_t k = threadIdx.x; k < count; k += blockDim.x) {
    const int64_t dst = base + k;
    if (dst >= capacity) break;
    table[dst] = static_cast<int32_t>(tr(row, lo + k, src ? src[k] : 0));
  }
}

}  // namespace

hipError_t launch_translate_loc(const int64_t *full_loc, int64_t n, const int64_t *map, int64_t map_len,
                                int64_t *out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(translate_loc_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, full_loc, n,
                     map, map_len, out);
  return hipGetLastError();
}

hipError_t launch_translate_window(const swa_index_t &idx, int32_t window, int32_t chunk, const int32_t *prefix_lens,
                                   int32_t *table, int32_t *indptr, int64_t capacity, hipStream_t stream) {
  const uint32_t grid = idx.batch > 0 ? static_cast<uint32_t>(idx.batch) : 1u;
  hipLaunchKernelGGL(translate_window_kernel<MapTable>, dim3(grid), dim3(256), 0, stream, idx.req_to_token,
                     idx.r2t_rows, idx.r2t_stride, idx.req_pool_idx, idx.seq_lens, prefix_lens,
                     MapTable{idx.full_to_swa, idx.map_len}, idx.batch, window, chunk, table, indptr, capacity);
  return hipGetLastError();
}

hipError_t launch_translate_window_ring(const swa_index_t &idx, int64_t ring_rows, int32_t window, int32_t chunk,
                                        const int32_t *prefix_lens, int32_t *table, int32_t *indptr,
                                        int64_t capacity, hipStream_t stream) {
  const uint32_t grid = idx.batch > 0 ? static_cast<uint32_t>(idx.batch) : 1u;
  // positions are bounded by the row length r2t_stride; rows by r2t_rows (the request slots)
  hipLaunchKernelGGL(translate_window_kernel<RingTable>, dim3(grid), dim3(256), 0, stream, nullptr,
                     idx.r2t_rows, idx.r2t_stride, idx.req_pool_idx, idx.seq_lens, prefix_lens, RingTable{ring_rows},
                     idx.batch, window, chunk, table, indptr, capacity);
  return hipGetLastError();
}

hipError_t launch_ring_locs(const swa_index_t &idx, int64_t ring_rows, const int32_t *prefix_lens, int64_t *out,
                            int64_t capacity, hipStream_t stream) {
  if (idx.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(ring_locs_kernel, dim3(static_cast<uint32_t>(idx.batch)), dim3(256), 0, stream,
                     idx.req_pool_idx, idx.r2t_rows, idx.seq_lens, prefix_lens, ring_rows, out, capacity);
  return hipGetLastError();
}

hipError_t launch_translate_window_unified(const swa_index_t &idx, const int64_t *v2p, int64_t n_pages,
                                           int32_t multiplier, int32_t window, const int32_t *prefix_lens,
                                           int32_t *table, int32_t *indptr, int64_t capacity, hipStream_t stream) {
  const uint32_t grid = idx.batch > 0 ? static_cast<uint32_t>(idx.batch) : 1u;
  const PageTable tr{v2p, n_pages, idx.page_size, static_cast<int64_t>(idx.page_size) * multiplier};
  hipLaunchKernelGGL(translate_window_kernel<PageTable>, dim3(grid), dim3(256), 0, stream, idx.req_to_token,
                     idx.r2t_rows, idx.r2t_stride, idx.req_pool_idx, idx.seq_lens, prefix_lens, tr, idx.batch,
                     window, 0, table, indptr, capacity);
  return hipGetLastError();
}

hipError_t launch_translate_ids(const int64_t *virt, int64_t n, const int64_t *v2p, int64_t n_pages,
                                int32_t page_size, int32_t multiplier, int64_t *out, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const PageTable tr{v2p, n_pages, page_size, static_cast<int64_t>(page_size) * multiplier};
  hipLaunchKernelGGL(translate_ids_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream, virt, n, tr,
                     out);
  return hipGetLastError();
}

}  // namespace swa
