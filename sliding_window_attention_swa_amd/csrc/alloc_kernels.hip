// Paired allocation: the slots of every request's new positions in the full
// pool and, for a two-pool cache, in the SWA pool, plus the mapping entries
// that tie them.
//
// "SGLang 源码完全拆解(十五): 内存池与显存管理", sections 三重映射 (a paged
// allocator hands out pages from the head of its free list), alloc_extend and
// alloc_decode (each request's outputs start after the earlier requests' new
// tokens, its new pages after the earlier requests' new pages; positions left
// in the page the prefix ends in continue from last_loc + 1, every later
// position p sits at offset p mod P of the request's (p - ceil_P(pre)) / P-th new
// page), and SWATokenToKVPoolAllocator (the SWA side continues from the mapping
// of last_loc -- the trailing -1 entry turns a -1 into -1 -- and
// full_to_swa[full] = swa is written afterwards).  SWA note
// (zdszero.github.io/swa.html), section 双池与映射表: both allocators take the
// same number of slots.
//
// The pages' three parts (rest of the half-full page, whole new pages, tail
// page) collapse into one formula per position here, so every thread of the
// workgroup handles any position.
#include "common.hpp"

namespace swa {
namespace {

constexpr int kThreads = 256;

struct AllocParams {
  int32_t batch;
  int32_t page;
  const int32_t *pre_lens;  // null: decode (pre = seq - 1)
  const int32_t *seq_lens;
  const int64_t *last_loc;
  const int64_t *free_full;
  int64_t n_free_full;
  const int64_t *free_swa;  // null: one pool
  int64_t n_free_swa;
  int64_t *map;
  int64_t map_len;
  int64_t *out_full;
  int64_t *out_swa;
  int64_t capacity;  // entries of out_full / out_swa
  int64_t *new_pages;
  int32_t page_shift;  // log2(page) for a power-of-two page, else -1
};

__device__ __forceinline__ int64_t ceil_page(int64_t x, int32_t page) { return (x + page - 1) / page; }

// Request b's prefix and sequence lengths (a negative prefix counts as 0, a
// sequence shorter than its prefix adds nothing).
__device__ __forceinline__ void lens_of(const AllocParams &p, int32_t b, int64_t &pre, int64_t &seq) {
  seq = p.seq_lens[b];
  pre = p.pre_lens ? p.pre_lens[b] : seq - 1;
  if (pre < 0) pre = 0;
  if (seq < pre) seq = pre;
}

__device__ __forceinline__ int64_t page_at(const int64_t *list, int64_t n, int64_t i) {
  return i < n ? list[i] : 0;  // past the list: page 0, the padding sink (the host proved it never happens)
}

// Sums over the workgroup of two values per thread.
__device__ __forceinline__ void block_sum2(int64_t &a, int64_t &c, int64_t *red) {
  for (int o = 32; o > 0; o >>= 1) {
    a += __shfl_xor(a, o);
    c += __shfl_xor(c, o);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[w] = a;
    red[4 + w] = c;
  }
  __syncthreads();
  a = red[0] + red[1] + red[2] + red[3];
  c = red[4] + red[5] + red[6] + red[7];
}

// gridDim.y workgroups per request, striding over its new positions
// (positions are below 2^31: the lengths are int32).
__global__ void __launch_bounds__(kThreads) alloc_extend_kernel(AllocParams p) {
  __shared__ int64_t red[8];
  const int32_t b = blockIdx.x;
  const int32_t c = blockIdx.y;
  {
    int64_t pre, seq;
    lens_of(p, b, pre, seq);
    if (c > 0 && static_cast<int64_t>(c) * kThreads >= seq - pre) return;  // workgroup-uniform: nothing here
  }
  // where this request's outputs and new pages start: the earlier requests' totals
  int64_t out_start = 0, page_start = 0;
  for (int32_t i = threadIdx.x; i < b; i += kThreads) {
    int64_t pre, seq;
    lens_of(p, i, pre, seq);
    out_start += seq - pre;
    page_start += ceil_page(seq, p.page) - ceil_page(pre, p.page);
  }
  block_sum2(out_start, page_start, red);

  int64_t pre, seq;
  lens_of(p, b, pre, seq);
  if (b == p.batch - 1 && c == 0 && threadIdx.x == 0 && p.new_pages)
    *p.new_pages = page_start + ceil_page(seq, p.page) - ceil_page(pre, p.page);
  const int64_t n = seq - pre;
  if (n == 0) return;
  const int64_t last = p.last_loc[b];
  const bool paired = p.free_swa != nullptr;
  // the SWA side continues from the mapped last_loc; -1 (no prefix) stays -1
  const int64_t last_swa = (paired && last >= 0 && last < p.map_len - 1) ? p.map[last] : -1;
  const int64_t first_new = ceil_page(pre, p.page) * p.page;  // first position on a new page
  const uint32_t pg = static_cast<uint32_t>(p.page);
  for (int64_t i = static_cast<int64_t>(c) * kThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.y) * kThreads) {
    const int64_t j = pre + i;
    int64_t full, swa_slot = 0;
    if (j < first_new) {
      full = last + 1 + i;
      swa_slot = last_swa + 1 + i;
    } else {
      const uint32_t d = static_cast<uint32_t>(j - first_new), ju = static_cast<uint32_t>(j);
      const int64_t q = page_start + (p.page_shift >= 0 ? d >> p.page_shift : d / pg);
      const int64_t off = p.page_shift >= 0 ? ju & (pg - 1) : ju % pg;
      full = page_at(p.free_full, p.n_free_full, q) * p.page + off;
      if (paired) swa_slot = page_at(p.free_swa, p.n_free_swa, q) * p.page + off;
    }
    const int64_t at = out_start + i;
    if (at < p.capacity) {
      p.out_full[at] = full;
      if (p.out_swa) p.out_swa[at] = swa_slot;
    }
    if (paired && full >= 0 && full < p.map_len - 1) p.map[full] = swa_slot;
  }
}

// One thread per request; a workgroup ranks its requests' new pages with
// ballots on top of the earlier workgroups' total.
__global__ void __launch_bounds__(kThreads) alloc_decode_kernel(AllocParams p) {
  __shared__ int64_t red[8];
  __shared__ int32_t wave_new[4];
  const int32_t first = blockIdx.x * kThreads;
  int64_t before = 0, dummy = 0;
  for (int32_t i = threadIdx.x; i < first; i += kThreads) {
    const int64_t s = p.seq_lens[i];
    before += (s >= 1 && (s - 1) % p.page == 0) ? 1 : 0;
  }
  block_sum2(before, dummy, red);

  const int32_t b = first + threadIdx.x;
  const bool live = b < p.batch;
  const int64_t seq = live ? p.seq_lens[b] : 0;
  const bool valid = live && seq >= 1;
  const bool opens = valid && (seq - 1) % p.page == 0;  // the new token starts a page
  const uint64_t mask = __ballot(opens);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  if (lane == 0) wave_new[w] = __popcll(mask);
  __syncthreads();
  int64_t rank = before + __popcll(mask & ((1ull << lane) - 1ull));
  int64_t total = before;
  for (int v = 0; v < 4; ++v) {
    rank += v < w ? wave_new[v] : 0;
    total += wave_new[v];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0 && p.new_pages) *p.new_pages = total;
  if (!live) return;
  int64_t full = 0, swa_slot = 0;
  const bool paired = p.free_swa != nullptr;
  if (valid) {
    const int64_t last = p.last_loc[b];
    if (opens) {
      full = page_at(p.free_full, p.n_free_full, rank) * p.page;
      if (paired) swa_slot = page_at(p.free_swa, p.n_free_swa, rank) * p.page;
    } else {
      full = last + 1;
      const int64_t last_swa = (paired && last >= 0 && last < p.map_len - 1) ? p.map[last] : -1;
      swa_slot = last_swa + 1;
    }
  }
  if (b < p.capacity) {
    p.out_full[b] = full;
    if (p.out_swa) p.out_swa[b] = swa_slot;
  }
  if (valid && paired && full >= 0 && full < p.map_len - 1) p.map[full] = swa_slot;
}

__global__ void alloc_zero_kernel(int64_t *new_pages) { *new_pages = 0; }

}  // namespace

hipError_t launch_alloc(const AllocArgs &a, hipStream_t stream) {
  if (a.batch == 0) {  // nothing to allocate; the page count is still reported
    if (a.new_pages) hipLaunchKernelGGL(alloc_zero_kernel, dim3(1), dim3(1), 0, stream, a.new_pages);
    return hipGetLastError();
  }
  AllocParams p{};
  p.batch = a.batch;
  p.page = a.page_size;
  p.pre_lens = a.pre_lens;
  p.seq_lens = a.seq_lens;
  p.last_loc = a.last_loc;
  p.free_full = a.free_full;
  p.n_free_full = a.n_free_full;
  p.free_swa = a.free_swa;
  p.n_free_swa = a.n_free_swa;
  p.map = a.full_to_swa;
  p.map_len = a.map_len;
  p.out_full = a.out_full;
  p.out_swa = a.out_swa;
  p.capacity = a.capacity;
  p.new_pages = a.new_pages;
  p.page_shift = (a.page_size & (a.page_size - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(a.page_size)) : -1;
  if (a.decode) {
    const uint32_t blocks = static_cast<uint32_t>((a.batch + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(alloc_decode_kernel, dim3(blocks), dim3(kThreads), 0, stream, p);
  } else {
    // about 2,048 workgroups in all (at least one and at most 16 per request)
    int64_t split = (2048 + a.batch - 1) / a.batch;
    split = split < 1 ? 1 : split > 16 ? 16 : split;
    hipLaunchKernelGGL(alloc_extend_kernel, dim3(static_cast<uint32_t>(a.batch), static_cast<uint32_t>(split)),
                       dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace swa
