// SWA eviction: release the SWA slots of positions that left each request's
// window and clear their mapping entries.
//
// SWA note (zdszero.github.io/swa.html), section 运行时: per request, the
// released range starts at the larger of the request's evicted length and its
// protected (radix-managed) prefix and ends at pre_len - W (chunk cache) or
// pre_len - max(W, page) (radix cache), aligned down to a page; in decode the
// release waits until `interval` tokens have left the window.  Section
// 双池与映射表: free_swa releases only mapping values > 0 and then sets them to
// 0, so releasing a range twice frees nothing twice.
//
// Only a page's first released position can report it (the range's first
// position, or a position that starts a page), so the report order is fixed by
// those candidates alone.  Two launches:
//   scan:  one workgroup per request walks its candidates (about 1/page of the
//          range), keeps each candidate's mapping value for the apply, counts
//          the reports, records for every chunk of the range the number of
//          reports before it, stores the range and advances the evicted length;
//   apply: one workgroup per (request, chunk of about 2048 positions) clears
//          the chunk's mapping entries and writes its reports at
//          (reports of earlier requests) + (reports of earlier chunks) + rank.
// The report order (request, then position) is therefore deterministic, and
// the mapping is cleared by the whole grid in parallel.
#include "common.hpp"

namespace swa {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 4;                  // scan: candidates per thread and pass
constexpr int kBatch = kThreads * kPerThread;
constexpr int kApplyPerThread = kEvictApplyPerThread;  // apply: positions per thread and pass

struct EvictParams {
  const int32_t *r2t;
  int64_t r2t_rows;
  int64_t r2t_stride;
  const int32_t *req_idx;
  int32_t batch;
  int32_t page;
  int64_t chunk;   // positions per apply workgroup, a multiple of page
  int32_t nchunk;  // chunks per request row
  int64_t *map;
  int64_t map_len;
  const int32_t *pre_lens;
  const int32_t *protected_lens;
  int32_t *evicted_lens;
  int32_t window;
  int32_t radix;
  int32_t interval;
  int64_t *freed_pages;
  int64_t capacity;
  int64_t *freed_count;
  int32_t *counts;  // [batch] reports per request
  int32_t *range;   // [batch][2] lo, hi (hi <= lo: nothing released)
  int32_t *base;    // [batch][nchunk] reports of the request before each chunk
  int64_t *cand;    // [batch][ncand] each candidate's mapping value (0: reports nothing)
  int64_t ncand;    // candidates per request row at most
  int32_t page_shift;  // log2(page) for a power-of-two page, else -1
};

// Page of position j (positions are below 2^31, as the int32 lengths and
// ranges already require).
__device__ __forceinline__ uint32_t page_of(const EvictParams &p, uint32_t j) {
  return p.page_shift >= 0 ? j >> p.page_shift : j / static_cast<uint32_t>(p.page);
}

// The range [lo, hi) request b releases; hi is the new evicted length when the
// range is not empty.  Positions at or beyond the row length are never read.
__device__ __forceinline__ void evict_range(const EvictParams &p, int32_t b, int64_t &lo, int64_t &hi) {
  const int64_t pre = p.pre_lens[b];
  const int64_t ev = p.evicted_lens[b];
  const int64_t prot = p.protected_lens ? p.protected_lens[b] : 0;
  const int64_t keep = p.radix ? (p.window > p.page ? p.window : p.page) : p.window;
  const int64_t bound = pre - keep;
  hi = bound > 0 ? bound / p.page * p.page : 0;
  lo = ev > prot ? ev : prot;
  if (lo < 0) lo = 0;  // negative lengths count as 0
  if (p.interval > 0 && hi - ev < p.interval) hi = lo;
}

// The full slot of position j of request row `row` (-1 when the row, the
// position or the slot lies outside its table) and its mapping value (0 when
// there is none).
__device__ __forceinline__ void load_position(const EvictParams &p, int64_t row, int64_t j, int64_t &full,
                                              int64_t &slot) {
  full = -1;
  slot = 0;
  if (row < 0 || row >= p.r2t_rows || j < 0 || j >= p.r2t_stride) return;
  const int64_t f = p.r2t[row * p.r2t_stride + j];
  if (f < 0 || f >= p.map_len - 1) return;
  full = f;
  slot = p.map[f];
}

// Exclusive rank of each set flag among the workgroup's kPerThread x kThreads
// flags in the order i-major, then thread; also the number set.
__device__ __forceinline__ void block_ranks(const bool (&flag)[kPerThread], int32_t (&rank)[kPerThread],
                                            int32_t &total, int32_t *cnt /* LDS [kPerThread][4] */) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  uint64_t mask[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    mask[i] = __ballot(flag[i]);
    if (lane == 0) cnt[i * 4 + w] = __popcll(mask[i]);
  }
  __syncthreads();
  int32_t run = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    int32_t before = run;
    for (int v = 0; v < 4; ++v) {
      before += v < w ? cnt[i * 4 + v] : 0;
      run += cnt[i * 4 + v];
    }
    rank[i] = before + __popcll(mask[i] & ((1ull << lane) - 1ull));
  }
  total = run;
  __syncthreads();  // cnt may be reused
}

__global__ void __launch_bounds__(kThreads) evict_scan_kernel(EvictParams p) {
  __shared__ int32_t cnt[kPerThread * 4];
  const int32_t b = blockIdx.x;
  int64_t lo, hi;
  evict_range(p, b, lo, hi);
  const int64_t row = p.req_idx[b];
  const int64_t end = hi < p.r2t_stride ? hi : p.r2t_stride;  // positions read
  // candidates: lo, then every page start in (lo, end)
  const int64_t first = (lo / p.page + 1) * p.page;
  const int64_t n_cand = end > lo ? 1 + (first < end ? (end - first - 1) / p.page + 1 : 0) : 0;
  int32_t run = 0;
  for (int64_t c0 = 0; c0 < n_cand; c0 += kBatch) {  // workgroup-uniform trip count
    int64_t j[kPerThread], slot[kPerThread];
    bool flag[kPerThread];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int64_t c = c0 + i * kThreads + threadIdx.x;
      j[i] = c == 0 ? lo : first + (c - 1) * p.page;
      int64_t full;
      slot[i] = 0;
      if (c < n_cand) load_position(p, row, j[i], full, slot[i]);
      flag[i] = slot[i] > 0;
    }
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {  // the apply reads these instead of the mapping
      const int64_t c = c0 + i * kThreads + threadIdx.x;
      if (c < n_cand) p.cand[static_cast<int64_t>(b) * p.ncand + c] = slot[i];
    }
    int32_t rank[kPerThread], n;
    block_ranks(flag, rank, n, cnt);
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int64_t c = c0 + i * kThreads + threadIdx.x;
      // the chunk's first candidate records the reports before the chunk
      const uint32_t ju = static_cast<uint32_t>(j[i]), k = ju / static_cast<uint32_t>(p.chunk);
      if (c < n_cand && (c == 0 || k * static_cast<uint32_t>(p.chunk) == ju)) {
        if (k < p.nchunk) p.base[static_cast<int64_t>(b) * p.nchunk + k] = run + rank[i];
      }
    }
    run += n;
  }
  __syncthreads();  // every thread has read evicted_lens[b]
  if (threadIdx.x == 0) {
    p.counts[b] = run;
    p.range[2 * b] = static_cast<int32_t>(lo);
    p.range[2 * b + 1] = static_cast<int32_t>(hi);
    if (hi > lo) p.evicted_lens[b] = static_cast<int32_t>(hi);
  }
}

// Apply: one workgroup per (request, chunk).  Two memory phases: the
// independent per-block values (range, chunk base, request row, the earlier
// requests' counts), then the chunk's req_to_token entries together with its
// candidates' mapping values as the scan read them; one barrier ranks the
// reports and sums the counts together.  The mapping itself is only written.
__global__ void __launch_bounds__(kThreads) evict_apply_kernel(EvictParams p) {
  __shared__ int32_t cnt[kApplyPerThread * 4];
  __shared__ int64_t red[4];
  const int32_t b = blockIdx.x;
  const int32_t k = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const bool first_block = b == 0 && k == 0;  // also reports the total

  const int64_t lo = p.range[2 * b];
  const int64_t hi = p.range[2 * b + 1];
  const int64_t row = p.req_idx[b];
  const int64_t base = p.base[static_cast<int64_t>(b) * p.nchunk + k];  // read only for a live chunk
  int64_t before = 0;  // reports of requests [0, b) (block (0, 0): of all requests)
  const int32_t upto = first_block ? p.batch : b;
  for (int32_t i = threadIdx.x; i < upto; i += kThreads) before += p.counts[i];

  const int64_t c_lo = k * p.chunk > lo ? k * p.chunk : lo;
  int64_t c_hi = (k + 1) * p.chunk < hi ? (k + 1) * p.chunk : hi;
  if (c_hi > p.r2t_stride) c_hi = p.r2t_stride;
  const bool live = c_lo < c_hi;
  if (!live && !first_block) return;  // workgroup-uniform
  constexpr int64_t kPass = kThreads * kApplyPerThread;
  // block (0, 0) makes one pass even with nothing of its own, to write the total
  const int64_t n_pass = live ? (c_hi - c_lo + kPass - 1) / kPass : 1;
  const bool rows_ok = row >= 0 && row < p.r2t_rows;
  const uint32_t lo_page = page_of(p, static_cast<uint32_t>(lo));
  const int64_t *cand = p.cand + static_cast<int64_t>(b) * p.ncand;

  int64_t run = 0;
  for (int64_t ps = 0; ps < n_pass; ++ps) {  // workgroup-uniform trip count
    const int64_t j0 = c_lo + ps * kPass;
    int32_t full[kApplyPerThread];
    int64_t slot[kApplyPerThread];
    bool flag[kApplyPerThread], clear[kApplyPerThread];
#pragma unroll
    for (int i = 0; i < kApplyPerThread; ++i) {
      const int64_t j = j0 + i * kThreads + threadIdx.x;
      full[i] = (rows_ok && j < c_hi) ? p.r2t[row * p.r2t_stride + j] : -1;
    }
    // A candidate's mapping value comes from the scan: candidate 0 is lo, then
    // one per page start, so a page start's candidate is its page minus lo's.
    // Every position's entry is cleared without being read: a value that is
    // already 0 stays 0 and reports nothing either way.  Full slot 0 (padding)
    // and the trailing sentinel are never written.
#pragma unroll
    for (int i = 0; i < kApplyPerThread; ++i) {
      const int64_t j = j0 + i * kThreads + threadIdx.x;
      const uint32_t ju = static_cast<uint32_t>(j);
      const uint32_t pj = page_of(p, ju);
      const bool is_cand = j < c_hi && (j == lo || pj * static_cast<uint32_t>(p.page) == ju);
      slot[i] = is_cand ? cand[pj - lo_page] : 0;
    }
#pragma unroll
    for (int i = 0; i < kApplyPerThread; ++i) {
      clear[i] = full[i] > 0 && full[i] < p.map_len - 1;
      flag[i] = slot[i] > 0;
    }
    // ranks of the reports in position order, and (first pass) the counts' sum,
    // behind one barrier
    uint64_t mask[kApplyPerThread];
#pragma unroll
    for (int i = 0; i < kApplyPerThread; ++i) {
      mask[i] = __ballot(flag[i]);
      if (lane == 0) cnt[i * 4 + w] = __popcll(mask[i]);
    }
    if (ps == 0) {
      for (int o = 32; o > 0; o >>= 1) before += __shfl_xor(before, o);
      if (lane == 0) red[w] = before;
    }
    __syncthreads();
    if (ps == 0) {
      before = red[0] + red[1] + red[2] + red[3];
      if (first_block) {
        if (threadIdx.x == 0) *p.freed_count = before;
        before = 0;
      }
    }
    const int64_t out = before + base + run;
    int32_t acc = 0;
#pragma unroll
    for (int i = 0; i < kApplyPerThread; ++i) {
      int32_t r = acc;
      for (int v = 0; v < 4; ++v) {
        r += v < w ? cnt[i * 4 + v] : 0;
        acc += cnt[i * 4 + v];
      }
      if (flag[i]) {
        const int64_t at = out + r + __popcll(mask[i] & ((1ull << lane) - 1ull));
        if (at < p.capacity) p.freed_pages[at] = slot[i] / p.page;
      }
      if (clear[i]) p.map[full[i]] = 0;
    }
    run += acc;
    if (ps + 1 < n_pass) __syncthreads();  // cnt is reused by the next pass
  }
}

__global__ void evict_zero_kernel(int64_t *freed_count) { *freed_count = 0; }

}  // namespace

hipError_t launch_evict(const swa_index_t &idx, int64_t *full_to_swa, const int32_t *pre_lens,
                        const int32_t *protected_lens, int32_t *evicted_lens, int32_t window, int32_t radix,
                        int32_t interval, int64_t *freed_pages, int64_t capacity, int64_t *freed_count,
                        int32_t *workspace, hipStream_t stream) {
  if (idx.batch == 0) {  // nothing to release; the count is still reported
    hipLaunchKernelGGL(evict_zero_kernel, dim3(1), dim3(1), 0, stream, freed_count);
    return hipGetLastError();
  }
  EvictParams p{};
  p.r2t = idx.req_to_token;
  p.r2t_rows = idx.r2t_rows;
  p.r2t_stride = idx.r2t_stride;
  p.req_idx = idx.req_pool_idx;
  p.batch = idx.batch;
  p.page = idx.page_size;
  p.chunk = evict_chunk(idx.page_size);
  p.nchunk = static_cast<int32_t>(evict_chunks(idx.r2t_stride, idx.page_size));
  p.map = full_to_swa;
  p.map_len = idx.map_len;
  p.pre_lens = pre_lens;
  p.protected_lens = protected_lens;
  p.evicted_lens = evicted_lens;
  p.window = window;
  p.radix = radix;
  p.interval = interval;
  p.freed_pages = freed_pages;
  p.capacity = capacity;
  p.freed_count = freed_count;
  p.counts = workspace;
  p.range = workspace + idx.batch;
  p.base = workspace + 3 * static_cast<int64_t>(idx.batch);
  p.ncand = evict_cands(idx.r2t_stride, idx.page_size);
  p.page_shift = (idx.page_size & (idx.page_size - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(idx.page_size)) : -1;
  p.cand = reinterpret_cast<int64_t *>(reinterpret_cast<char *>(workspace) +
                                       evict_cand_offset(idx.batch, idx.r2t_stride, idx.page_size));
  hipLaunchKernelGGL(evict_scan_kernel, dim3(static_cast<uint32_t>(idx.batch)), dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(evict_apply_kernel, dim3(static_cast<uint32_t>(idx.batch), static_cast<uint32_t>(p.nchunk)),
                     dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace swa
