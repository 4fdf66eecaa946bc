// Index-data validation (debug aid): counts the contract violations that the
// hot-path kernels silently absorb.
//
// The contracts (SWA note, zdszero.github.io/swa.html, sections 双池与映射表
// and 运行时; "SGLang 源码完全拆解(十五): 内存池与显存管理", sections 一重映射,
// 二重映射, 释放 and SWATokenToKVPoolAllocator):
//   * every position inside a live window has a slot: an SWA mapping of 0
//     (tombstone) or -1 (the trailing sentinel) there is a bug, because
//     eviction only releases positions that left the window;
//   * req_to_token rows, full slots and SWA slots index inside their tables;
//   * a store location is used once per batch, except in page 0, the padding
//     sink that padded (dummy) writes share;
//   * (extend) request b's query rows qo_indptr[b] .. qo_indptr[b+1]-1 lie in
//     order inside the query array and are its new positions, seq - prefix.
//
// Workspace layout (device, caller-owned): 16 int64 counters, then a bitmap of
// ceil(pool_rows / 32) 32-bit words used to find repeated store locations.
#include "common.hpp"

namespace swa {
namespace {

enum Counter {
  kBadRequests = 0,
  kPositions,
  kFullOutOfRange,
  kTombstones,
  kSentinels,
  kSlotOutOfRange,
  kStoreLocs,
  kStoreOutOfRange,
  kStoreDuplicates,
  kQoBad,
  kNumCounters
};

__global__ void validate_clear_kernel(uint32_t *ws, int64_t words) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < words;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    ws[i] = 0u;
}

// Sum of one int64 per thread over the workgroup, added to counters[c] by one lane.
__device__ void block_add(unsigned long long *counters, int c, int64_t v, int64_t *red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t t = 0;
    for (int i = 0; i < static_cast<int>(blockDim.x >> 6); ++i) t += red[i];
    if (t) atomicAdd(counters + c, static_cast<unsigned long long>(t));
  }
}

// One workgroup per request: walk its window and classify every position.
__global__ void __launch_bounds__(256) validate_window_kernel(swa_index_t idx, int32_t window,
                                                              const int32_t *prefix_lens, const int32_t *qo_indptr,
                                                              int64_t total_q, int64_t pool_rows,
                                                              unsigned long long *counters) {
  __shared__ int64_t red[4];
  const int32_t b = blockIdx.x;
  const int64_t row = idx.req_pool_idx[b];
  const int64_t len = idx.seq_lens[b];
  const int64_t pre = prefix_lens ? prefix_lens[b] : len - 1;
  const bool bad = row < 0 || row >= idx.r2t_rows || len < 0 || len > idx.r2t_stride ||
                   (prefix_lens && (pre < 0 || pre > len));
  int64_t n_pos = 0, n_full = 0, n_tomb = 0, n_sent = 0, n_slot = 0;
  if (!bad && len > 0) {
    const int64_t lo = window < 0 ? 0 : (pre - window > 0 ? pre - window : 0);
    const int32_t *r2t = idx.req_to_token + row * idx.r2t_stride;
    for (int64_t j = lo + threadIdx.x; j < len; j += blockDim.x) {
      ++n_pos;
      const int64_t full = r2t[j];
      if (idx.full_to_swa) {
        // valid full slots index the mapping; -1 reads its trailing sentinel entry
        if (full < -1 || full >= idx.map_len - 1) {
          ++n_full;
          continue;
        }
        const int64_t s = idx.full_to_swa[full < 0 ? idx.map_len - 1 : full];
        if (s == 0)
          ++n_tomb;
        else if (s == -1)
          ++n_sent;
        else if (s < 0 || s >= pool_rows)
          ++n_slot;
      } else {
        if (full == 0)
          ++n_tomb;
        else if (full < 0 || full >= pool_rows)
          ++n_slot;
      }
    }
  }
  // query rows of an extend: inside [0, total_q], in order, and (for a request
  // whose row and lengths are valid) as many as its new positions
  bool qo_bad = false;
  if (qo_indptr && threadIdx.x == 0) {
    const int64_t q0 = qo_indptr[b], q1 = qo_indptr[b + 1];
    qo_bad = q0 < 0 || q1 < q0 || q1 > total_q || (!bad && prefix_lens && q1 - q0 != len - pre);
  }
  block_add(counters, kQoBad, qo_bad ? 1 : 0, red);
  block_add(counters, kBadRequests, (bad && threadIdx.x == 0) ? 1 : 0, red);
  block_add(counters, kPositions, n_pos, red);
  block_add(counters, kFullOutOfRange, n_full, red);
  block_add(counters, kTombstones, n_tomb, red);
  block_add(counters, kSentinels, n_sent, red);
  block_add(counters, kSlotOutOfRange, n_slot, red);
}

// Grid-stride over the store locations: out of range, or seen before (outside page 0).
__global__ void __launch_bounds__(256) validate_store_kernel(const int64_t *loc, int64_t n, int64_t pool_rows,
                                                             int32_t page_size, uint32_t *bitmap,
                                                             unsigned long long *counters) {
  __shared__ int64_t red[4];
  int64_t n_out = 0, n_dup = 0, n_seen = 0;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    ++n_seen;
    const int64_t x = loc[i];
    if (x < 0 || x >= pool_rows) {
      ++n_out;
      continue;
    }
    if (x < page_size) continue;  // page 0 absorbs padded writes
    const uint32_t bit = 1u << (x & 31);
    const uint32_t old = atomicOr(bitmap + (x >> 5), bit);
    if (old & bit) ++n_dup;
  }
  block_add(counters, kStoreLocs, n_seen, red);
  block_add(counters, kStoreOutOfRange, n_out, red);
  block_add(counters, kStoreDuplicates, n_dup, red);
}

}  // namespace

hipError_t launch_validate(const swa_index_t &idx, int32_t window, const int32_t *prefix_lens,
                           const int32_t *qo_indptr, int64_t total_q, int64_t pool_rows, const int64_t *store_loc,
                           int64_t n_store, void *workspace, int64_t counters_bytes, hipStream_t stream) {
  unsigned long long *counters = static_cast<unsigned long long *>(workspace);
  uint32_t *bitmap = reinterpret_cast<uint32_t *>(static_cast<char *>(workspace) + counters_bytes);
  const int64_t words = counters_bytes / 4 + (store_loc && n_store > 0 ? (pool_rows + 31) / 32 : 0);
  int64_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(validate_clear_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     static_cast<uint32_t *>(workspace), words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (idx.batch > 0) {
    hipLaunchKernelGGL(validate_window_kernel, dim3(static_cast<uint32_t>(idx.batch)), dim3(256), 0, stream, idx,
                       window, prefix_lens, qo_indptr, total_q, pool_rows, counters);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (store_loc && n_store > 0) {
    int64_t sb = (n_store + 255) / 256;
    if (sb > 4096) sb = 4096;
    hipLaunchKernelGGL(validate_store_kernel, dim3(static_cast<uint32_t>(sb)), dim3(256), 0, stream, store_loc,
                       n_store, pool_rows, idx.page_size, bitmap, counters);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace swa
