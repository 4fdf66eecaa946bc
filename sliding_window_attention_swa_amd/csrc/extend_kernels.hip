// Windowed-causal extend (chunked prefill) over a cached prefix.
//
// SWA note (zdszero.github.io/swa.html): each query i attends to keys
// [max(0, i - W), i] (opening paragraph and section 实现; W excludes the current
// token, -1 = full attention), with an optional per-head sink (section 设计);
// section 运行时 describes chunked prefill, where the chunk's K/V are written to
// the pool and the chunk's queries read the prefix's last window plus the chunk.
//
// MI355X design (not the pages' kernels):
//   * a tile = 16 consecutive queries x the G query heads of one kv head (GQA
//     packed into the M side), so each K/V row staged in LDS serves G heads;
//     G = 16 is split into two groups of 8 (eight heads fill the four
//     wavefronts at two heads each; four each would spill registers); the key
//     range of a tile is only its band [i0 - W, i0 + 15];
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 and O^T = V^T P^T on
//     v_mfma_f32_16x16x32_f16, both with fp32 accumulation; P is rounded to f16
//     (V is staged as f16, exact for bf16 values in f16's range) and never leaves
//     registers (the first product's accumulator layout is the second's B
//     operand layout); the V^T operand is read from a row-major LDS tile with
//     gfx950's transposing ds_read_b64_tr_b16; online softmax in base 2;
//   * one workgroup walks a run of consecutive tiles of one (request, kv
//     head).  At W = 128 a full tile's band is exactly 9 blocks of 16 keys and
//     the next tile's band is the same minus its first block plus one new
//     block, so the band lives in a 9-slot LDS ring: while a tile is computed,
//     the next tile's queries and its one new K/V block are already in flight
//     (and the slots of the block after that), so a tile costs its arithmetic,
//     not a memory round trip.  Other tiles (other windows, band clipped at
//     position 0, partial tiles) take a general path that stages the band in
//     chunks of 9 blocks;
//   * runs are numbered (request, kv head, run, q-head group) and dealt to the 8 XCDs in
//     contiguous ranges, so neighbouring runs, which share band blocks, hit the
//     same L2.
#include "common.hpp"

// Long-band kernel shape: row blocks per wavefront, wavefronts per workgroup,
// workgroups per CU.
#ifndef SWA_BAND_RB
#define SWA_BAND_RB 2
#endif
#ifndef SWA_BAND_NW
#define SWA_BAND_NW 8
#endif
#ifndef SWA_BAND_WGS
#define SWA_BAND_WGS 1
#endif


namespace swa {
namespace {

constexpr int kD = 128;
constexpr int kNW = 4;         // wavefronts per workgroup
constexpr int kTQ = 16;        // queries per tile
constexpr int kKB = 9;         // key blocks (of 16) per chunk / ring slots
constexpr int kBand = 16 * kKB;  // keys of a full band at W = 128
constexpr int kKRow = kD + 8;  // LDS K row: 272 bytes (16-byte aligned rows, 4-bank skew)
constexpr int kVRow = kD + 16;  // LDS V row: 288 bytes (8-bank skew: conflict-free transposed reads)

struct ExtendParams {
  const uint16_t *q;
  const uint16_t *k;
  const uint16_t *v;
  int64_t rows;
  int32_t kv_heads;
  int32_t q_heads;
  int32_t group;
  int32_t batch;
  const int32_t *qo_indptr;
  const int32_t *prefix_lens;
  int64_t total_q;
  const int32_t *r2t;
  int64_t r2t_rows;
  int64_t r2t_stride;
  const int32_t *req_idx;
  const int32_t *seq_lens;
  const int32_t *table;
  const int32_t *indptr;
  int64_t capacity;
  int32_t window;
  const float *sinks;
  float scale2;
  void *out;
  int32_t run_tiles;  // tiles per workgroup run
  int32_t chunk;      // chunked local attention: chunk size, 0 = none
  int32_t halves;     // q-head groups per kv head (G = 16: two groups of 8)
  int32_t ghead;      // q heads per group, G / halves
};

// First key position query i sees: i - W (W >= 0), the start of i's chunk of C
// positions (chunked local attention, SWA note section 设计: Llama4's chunked
// local layers; C > 0), the later of the two, never below 0.  It never
// decreases with i, so a tile's first query has the tile's first key and its
// last query the latest first key.
__device__ __forceinline__ int32_t first_key(int32_t i, int32_t window, int32_t chunk) {
  int32_t lo = 0;
  if (window >= 0 && i - window > lo) lo = i - window;
  if (chunk > 0 && i > 0 && i - i % chunk > lo) lo = i - i % chunk;
  return lo;
}

__device__ __forceinline__ float wave_max_q(float x) { return rows_max(x); }  // lanes l, l^16, l^32, l^48
__device__ __forceinline__ float wave_sum_q(float x) { return rows_sum(x); }

// Workgroup barrier for LDS data only.  __syncthreads() also fences global
// memory, i.e. waits for every outstanding global load and store of the wave;
// the ring's barriers must not wait for the next tile's prefetches or this
// tile's output stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Query rows of request b: [qo0, qo0 + n).  The entries are clamped into
// [0, total_q], so a bad qo_indptr never reads or writes outside q and out (a
// decreasing pair is an empty request).
struct QoRows {
  int32_t qo0;
  int32_t n;
};

__device__ __forceinline__ QoRows qo_rows(const ExtendParams &p, int32_t b) {
  int64_t lo = p.qo_indptr[b], hi = p.qo_indptr[b + 1];
  if (lo < 0) lo = 0;
  if (lo > p.total_q) lo = p.total_q;
  if (hi > p.total_q) hi = p.total_q;
  return QoRows{static_cast<int32_t>(lo), hi > lo ? static_cast<int32_t>(hi - lo) : 0};
}

__device__ __forceinline__ int32_t new_count(const ExtendParams &p, int32_t b) { return qo_rows(p, b).n; }

// Key position -> pool slot for one request: src[pos - pos_base], 0 <= . < hi.
struct KeySrc {
  const int32_t *src;
  int64_t hi;
  int32_t pos_base;
};

template <bool CHUNKED>
__device__ __forceinline__ KeySrc key_src(const ExtendParams &p, int32_t b, int32_t prefix) {
  KeySrc ks;
  if (p.indptr) {
    int64_t lo = p.indptr[b], hi = p.indptr[b + 1];
    if (lo < 0) lo = 0;
    if (hi > p.capacity) hi = p.capacity;
    ks.src = p.table + lo;
    ks.hi = hi > lo ? hi - lo : 0;
    if constexpr (CHUNKED) {
      ks.pos_base = first_key(prefix, p.window, p.chunk);
    } else {
      int32_t base = p.window < 0 ? 0 : prefix - p.window;
      ks.pos_base = base < 0 ? 0 : base;
    }
  } else {
    int64_t row = p.req_idx[b];
    if (row < 0 || row >= p.r2t_rows) row = 0;
    ks.src = p.r2t + row * p.r2t_stride;
    ks.hi = p.r2t_stride;
    ks.pos_base = 0;
  }
  return ks;
}

// Slot of key position `pos` (a position outside the source reads entry 0;
// callers only use such slots for rows they mask or zero).
__device__ __forceinline__ int32_t slot_at(const KeySrc &ks, int64_t pos) {
  if (ks.hi <= 0) return 0;
  const int64_t si = pos - ks.pos_base;
  return ks.src[si >= 0 && si < ks.hi ? si : 0];
}

struct Tile {
  int32_t row0;    // first q row of the tile
  int32_t i0;      // position of its first query
  int32_t i_last;  // position of its last valid query
  int32_t kj0;     // first key position of its band
  int32_t nkeys;   // keys in the band
  bool steady;     // W = 128, 16 valid queries, band inside position 0.. and the key source
};

template <bool CHUNKED>
__device__ __forceinline__ Tile tile_at(const ExtendParams &p, const KeySrc &ks, int32_t qo0, int32_t qt,
                                        int32_t prefix, int32_t n_new, int32_t seq) {
  Tile t;
  const int32_t W = p.window;
  t.row0 = qo0 + qt * kTQ;
  t.i0 = prefix + qt * kTQ;
  int32_t il = t.i0 + kTQ - 1;
  if (il > prefix + n_new - 1) il = prefix + n_new - 1;
  if (il > seq - 1) il = seq - 1;
  t.i_last = il;
  int32_t kj0 = W < 0 ? 0 : t.i0 - W;
  t.kj0 = kj0 < 0 ? 0 : kj0;
  if constexpr (CHUNKED) t.kj0 = first_key(t.i0, W, p.chunk);
  t.nkeys = il >= t.kj0 ? il - t.kj0 + 1 : 0;
  t.steady = !CHUNKED && W == kBand - 16 && t.i0 - W >= 0 && qt * kTQ + kTQ <= n_new && il == t.i0 + kTQ - 1 &&
             static_cast<int64_t>(t.row0) + kTQ <= p.total_q && static_cast<int64_t>(t.kj0) - ks.pos_base >= 0 &&
             static_cast<int64_t>(t.kj0) - ks.pos_base + kBand <= ks.hi;
  return t;
}

// Slot of a key position known to lie inside the key source (steady tiles).
__device__ __forceinline__ int32_t slot_in(const KeySrc &ks, int32_t pos) { return ks.src[pos - ks.pos_base]; }

// Q^T operands of this lane: query row `qrow`, heads w*MB + m.  Contraction
// block c takes dims 32c + 8lq .. +7 from lane group lq (K operands are read
// from LDS in the same order), so each load instruction reads 64 contiguous
// bytes of every query row.  Padding heads read a real head; their columns
// are never stored.
template <int MB>
__device__ __forceinline__ void load_q(const ExtendParams &p, int64_t qrow, int32_t hq0, int32_t w, int32_t lq,
                                       uint4 (&raw)[MB][4]) {
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int32_t hh = w * MB + m;
    const uint16_t *qp = p.q + (qrow * p.q_heads + hq0 + (hh < p.ghead ? hh : 0)) * kD + 8 * lq;
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[m][c] = *reinterpret_cast<const uint4 *>(qp + 32 * c);
  }
}

// This thread's 16-byte piece of one K row and one V row (16 threads per row).
__device__ __forceinline__ void fetch_piece(const ExtendParams &p, int32_t slot, int32_t g, uint4 &k, uint4 &v) {
  const int64_t sl = (slot < 0 || slot >= p.rows) ? 0 : static_cast<int64_t>(slot);
  const int64_t off = row_elem(sl, p.kv_heads, g, kD) + 8 * (threadIdx.x & 15);
  k = *reinterpret_cast<const uint4 *>(p.k + off);
  v = *reinterpret_cast<const uint4 *>(p.v + off);
}

// K rows are staged as bf16 (the operand of QK^T), V rows as f16 (the operand
// of the f16 P.V product).
__device__ __forceinline__ void put_piece(uint16_t *ktile, uint16_t *vtile, int32_t row, const uint4 &k,
                                          const uint4 &v) {
  const int32_t piece = threadIdx.x & 15;
  *reinterpret_cast<uint4 *>(ktile + row * kKRow + 8 * piece) = k;
  *reinterpret_cast<uint4 *>(vtile + row * kVRow + 8 * piece) = bf16x8_to_f16x8(v);
}

// Steady tiles read the band from the ring: band block j lives in ring slot
// (q0 + j) mod 9.  Block 0 is the band's lower edge (query kr sees key offsets
// k >= kr), block 8 the diagonal (k <= kr), the rest are inside the band for
// every query.
__device__ __forceinline__ int32_t ring_slot(int32_t q0, int j) { return q0 + j < kKB ? q0 + j : q0 + j - kKB; }

// A steady tile, one head at a time.  With two heads per wavefront the two
// heads' phases are staggered (head 1's QK^T next to head 0's softmax, head 0's
// P.V next to head 1's softmax, head 1's P.V next to head 0's normalisation),
// so the MFMAs of one head run while the other head's VALU work issues (C3:
// 81 -> 78 us); K and V are then read from LDS once per head instead of once
// per pair of heads (LDS was 14% busy).

// One head's S^T = K Q^T over the band (block j + 1's K rows read while block
// j's MFMAs run), band edges masked.
__device__ __forceinline__ void head_scores(const uint16_t *ktile, const int32_t (&slot)[kKB],
                                            const bf16x8_t (&qop)[4], f32x4_t (&s)[kKB]) {
  const int32_t lane = threadIdx.x & 63;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  bf16x8_t kop[2][4];
  {
    const uint16_t *kp = ktile + (slot[0] * 16 + kr) * kKRow + 8 * lq;
#pragma unroll
    for (int c = 0; c < 4; ++c) __builtin_memcpy(&kop[0][c], kp + 32 * c, 16);
  }
#pragma unroll
  for (int j = 0; j < kKB; ++j) {
    if (j + 1 < kKB) {
      const uint16_t *kp = ktile + (slot[j + 1] * 16 + kr) * kKRow + 8 * lq;
#pragma unroll
      for (int c = 0; c < 4; ++c) __builtin_memcpy(&kop[(j + 1) & 1][c], kp + 32 * c, 16);
    }
    s[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) s[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[j & 1][c], qop[c], s[j], 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int32_t k = 4 * lq + r;
    s[0][r] = (k >= kr) ? s[0][r] : -INFINITY;
    s[kKB - 1][r] = (k <= kr) ? s[kKB - 1][r] : -INFINITY;
  }
}

// One head's softmax numerators: pw holds the weights 2^(s - m), rounded to
// f16 and packed in pairs (keys 4lq + {0,1} and 4lq + {2,3} of each block), m
// the band's max and l the sum of the rounded weights (the weights that enter
// P.V), taken block by block.  The whole band at once: no rescaling.  Packing
// here halves the registers the weights hold while P.V runs.
__device__ __forceinline__ void head_weights(float scale2, const f32x4_t (&s)[kKB], uint32_t (&pw)[kKB][2],
                                             float &m_run, float &l_run) {
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kKB; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[j][r]);
  const float m_new = wave_max_q(mx) * scale2;  // finite: every query sees its own key
  m_run = m_new;
  float l = 0.f;
#pragma unroll
  for (int j = 0; j < kKB; ++j) {
    float e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) e[r] = __builtin_amdgcn_exp2f(fmaf(s[j][r], scale2, -m_new));
    pw[j][0] = pack_f16x2_hw(e[0], e[1]);
    pw[j][1] = pack_f16x2_hw(e[2], e[3]);
    l = f16x2_acc(pw[j][1], f16x2_acc(pw[j][0], l));
  }
  l_run = l;
}

// One head's O^T = V^T P^T over block pairs (2u, 2u+1) of its band.  acc is
// written, not accumulated into: the first pair starts from zero, so acc holds
// no registers while the scores are computed.  Each pair's 16 transposed reads
// go out before its MFMAs, so their LDS latency overlaps instead of stalling
// every step (C3: 90.5 -> 84.6 us).
__device__ __forceinline__ void head_pv(const uint16_t *vtile, const int32_t (&slot)[kKB], const uint32_t (&pw)[kKB][2],
                                        f32x4_t (&acc)[8]) {
  const int32_t lane = threadIdx.x & 63;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  const int32_t voff = (4 * lq + (kr >> 2)) * kVRow + 4 * (kr & 3);
#pragma unroll
  for (int u = 0; u < (kKB + 1) / 2; ++u) {
    const bool second = 2 * u + 1 < kKB;
    const int ja = 2 * u;
    const int jb = second ? 2 * u + 1 : 2 * u;
    bf16x8_t pop;
    {
      uint32_t u4[4] = {pw[ja][0], pw[ja][1], second ? pw[jb][0] : 0u, second ? pw[jb][1] : 0u};
      __builtin_memcpy(&pop, u4, 16);
    }
    const uint16_t *va = vtile + slot[ja] * 16 * kVRow + voff;
    const uint16_t *vb = vtile + slot[jb] * 16 * kVRow + voff;
    i16x4_t lo[8], hi[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      lo[n] = lds_read_tr16(va + 16 * n);
      hi[n] = second ? lds_read_tr16(vb + 16 * n) : i16x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const bf16x8_t vop = __builtin_shufflevector(lo[n], hi[n], 0, 1, 2, 3, 4, 5, 6, 7);
      acc[n] = mfma_f16(vop, pop, u == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : acc[n]);
    }
  }
}

// General tile: the band staged in chunks of up to 9 blocks, online softmax
// across chunks, per-key masks on blocks that touch the band's edges.
template <int MB, bool CHUNKED>
__device__ void tile_general(const ExtendParams &p, const KeySrc &ks, const Tile &tl, const bf16x8_t (&qop)[MB][4],
                             int32_t g, uint16_t *ktile, uint16_t *vtile, f32x4_t (&acc)[MB][8], float (&m_run)[MB],
                             float (&l_run)[MB]) {
  const int32_t lane = threadIdx.x & 63;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  const int32_t W = p.window;
  const int32_t qpos = tl.i0 + kr;  // position of the query in this lane's column
  // chunked local attention: the start of this lane's query's chunk and of the
  // tile's last query's chunk (the latest chunk start of the tile)
  const int32_t q_chunk0 = CHUNKED ? qpos - qpos % p.chunk : 0;
  const int32_t tile_chunk0 = CHUNKED ? tl.i_last - tl.i_last % p.chunk : 0;
  for (int32_t c0 = 0; c0 < tl.nkeys; c0 += kKB * 16) {
    const int32_t nbk = min(kKB, (tl.nkeys - c0 + 15) / 16);
    const int32_t chunk_pos = tl.kj0 + c0;  // position of key 0 of the chunk

    // ---- stage K and V rows of the chunk in LDS (16 threads per 256-byte
    // row).  Every thread issues all its loads before writing any; keys past
    // the band re-read the chunk's first key and are zeroed when written.
    __syncthreads();  // previous chunk (or tile) fully consumed
    {
      int32_t slot[kKB];
#pragma unroll
      for (int i = 0; i < kKB; ++i) {
        const int32_t key = (threadIdx.x >> 4) + 16 * i;
        const bool kv_ok = i < nbk && c0 + key < tl.nkeys;
        slot[i] = slot_at(ks, chunk_pos + (kv_ok ? key : 0));
      }
      uint4 kreg[kKB], vreg[kKB];
#pragma unroll
      for (int i = 0; i < kKB; ++i) fetch_piece(p, slot[i], g, kreg[i], vreg[i]);
#pragma unroll
      for (int i = 0; i < kKB; ++i) {
        const int32_t key = (threadIdx.x >> 4) + 16 * i;
        const bool kv_ok = i < nbk && c0 + key < tl.nkeys;
        put_piece(ktile, vtile, key, kv_ok ? kreg[i] : make_uint4(0, 0, 0, 0),
                  kv_ok ? vreg[i] : make_uint4(0, 0, 0, 0));
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T: block kb, lane holds keys 4lq..4lq+3 for query kr
    f32x4_t sacc[MB][kKB];
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
#pragma unroll
      for (int m = 0; m < MB; ++m) sacc[m][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (kb < nbk) {
        bf16x8_t kop[4];
        const uint16_t *kp = ktile + (kb * 16 + kr) * kKRow + 8 * lq;
#pragma unroll
        for (int c = 0; c < 4; ++c) __builtin_memcpy(&kop[c], kp + 32 * c, 16);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            sacc[m][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[c], qop[m][c], sacc[m][kb], 0, 0, 0);
      }
    }

    // ---- mask: only blocks that touch the band's edges or the chunk end need
    // a per-key test (a block is inside the band for every query of the tile
    // when its last key <= i0 and its first key >= i_last - W and, with chunks,
    // >= the start of i_last's chunk).
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const int32_t j0 = chunk_pos + kb * 16;
      const bool interior =
          kb < nbk && c0 + kb * 16 + 15 < tl.nkeys && j0 + 15 <= tl.i0 && (W < 0 || j0 >= tl.i_last - W) &&
          (!CHUNKED || j0 >= tile_chunk0);
      if (!interior) {  // workgroup-uniform
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t j = j0 + 4 * lq + r;
          const bool ok = kb < nbk && (c0 + kb * 16 + 4 * lq + r) < tl.nkeys && j <= qpos &&
                          (W < 0 || j >= qpos - W) && (!CHUNKED || j >= q_chunk0);
#pragma unroll
          for (int m = 0; m < MB; ++m) sacc[m][kb][r] = ok ? sacc[m][kb][r] : -INFINITY;
        }
      }
    }
    // ---- online softmax in base 2; the running max is kept in the scaled
    // domain, scores are scaled inside the exponent (one fma per score)
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[m][kb][r]);
      const float m_new = fmaxf(m_run[m], wave_max_q(mx) * p.scale2);
      const float alpha = __builtin_amdgcn_exp2f(m_run[m] - m_new);
      m_run[m] = m_new;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[m][kb][r] = __builtin_amdgcn_exp2f(fmaf(sacc[m][kb][r], p.scale2, -m_new));
      l_run[m] *= alpha;  // the chunk's rounded weights are added below, as they are packed
      if (c0 > 0) {
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] *= alpha;
      }
    }

    // ---- O^T += V^T P^T over block pairs (2u, 2u+1): lane (kr, lq) gets
    // V[4lq + e][16n + kr], e = 0..3, of each block of the pair.
    const uint16_t *vrow = vtile + (4 * lq + (kr >> 2)) * kVRow + 4 * (kr & 3);
#pragma unroll
    for (int u = 0; u < (kKB + 1) / 2; ++u) {
      if (2 * u < nbk) {
        const bool second = 2 * u + 1 < nbk;
        bf16x8_t pop[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const int kb1 = (2 * u + 1) < kKB ? 2 * u + 1 : 2 * u;
          uint32_t u4[4] = {pack_f16x2_hw(sacc[m][2 * u][0], sacc[m][2 * u][1]),
                            pack_f16x2_hw(sacc[m][2 * u][2], sacc[m][2 * u][3]),
                            second ? pack_f16x2_hw(sacc[m][kb1][0], sacc[m][kb1][1]) : 0u,
                            second ? pack_f16x2_hw(sacc[m][kb1][2], sacc[m][kb1][3]) : 0u};
          l_run[m] = f16x2_acc(u4[3], f16x2_acc(u4[2], f16x2_acc(u4[1], f16x2_acc(u4[0], l_run[m]))));
          __builtin_memcpy(&pop[m], u4, 16);
        }
        // the pair's transposed reads go out before its MFMAs, so their LDS
        // latency overlaps
        i16x4_t lo[8], hi[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          lo[n] = lds_read_tr16(vrow + (32 * u) * kVRow + 16 * n);
          hi[n] = second ? lds_read_tr16(vrow + (32 * u + 16) * kVRow + 16 * n) : i16x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          bf16x8_t vop = {lo[n][0], lo[n][1], lo[n][2], lo[n][3], hi[n][0], hi[n][1], hi[n][2], hi[n][3]};
#pragma unroll
          for (int m = 0; m < MB; ++m)
            acc[m][n] = mfma_f16(vop, pop[m], acc[m][n]);
        }
      }
    }
  }
}

// A finished tile's normalised output for this lane, packed for its stores.
template <bool OUT_BF16>
struct HeadOut {  // bf16: 8 consecutive dims per lane and block pair (see finish_head)
  using type = uint4[4];
};
template <>
struct HeadOut<false> {
  using type = float4[8];
};
template <int MB, bool OUT_BF16>
struct TileOut {
  typename HeadOut<OUT_BF16>::type v[MB];
};

// One head: the sink once, normalise, and (bf16) pack for the stores.
template <bool OUT_BF16>
__device__ __forceinline__ void finish_head(const ExtendParams &p, const f32x4_t (&acc)[8], float M, float l_run,
                                            float sink2, typename HeadOut<OUT_BF16>::type &ov) {
  {
    float L = wave_sum_q(l_run);
    float a = 1.f;
    if (p.sinks) {
      const float Mn = fmaxf(M, sink2);
      a = __builtin_amdgcn_exp2f(M - Mn);
      L = L * a + __builtin_amdgcn_exp2f(sink2 - Mn);
    }
    const float inv = L > 0.f ? a / L : 0.f;
    if constexpr (OUT_BF16) {
      // Lane (query kr, group lq) holds dims 16n + 4lq + 0..3 of block n.  For
      // each block pair (2t, 2t+1), rows lq and lq ^ 1 swap halves (gfx950's
      // row swap), so that the even row gets dims 32t + 8(lq/2) + 0..7 and the
      // odd row dims 32t + 16 + 8(lq/2) + 0..7: 16-byte stores that cover 64
      // contiguous bytes of a query row per instruction.
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x4_t &x0 = acc[2 * t], &x1 = acc[2 * t + 1];
        const uint32_t a0 = pack_bf16x2_hw(x0[0] * inv, x0[1] * inv), a1 = pack_bf16x2_hw(x0[2] * inv, x0[3] * inv);
        const uint32_t b0 = pack_bf16x2_hw(x1[0] * inv, x1[1] * inv), b1 = pack_bf16x2_hw(x1[2] * inv, x1[3] * inv);
        const auto s0 = __builtin_amdgcn_permlane16_swap(a0, b0, false, false);
        const auto s1 = __builtin_amdgcn_permlane16_swap(a1, b1, false, false);
        ov[t] = make_uint4(s0[0], s1[0], s0[1], s1[1]);
      }
    } else {
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const float o0 = acc[n][0] * inv, o1 = acc[n][1] * inv, o2 = acc[n][2] * inv, o3 = acc[n][3] * inv;
        ov[n] = make_float4(o0, o1, o2, o3);
      }
    }
  }
}

template <int MB, bool OUT_BF16>
__device__ __forceinline__ void finish_tile(const ExtendParams &p, const f32x4_t (&acc)[MB][8],
                                            const float (&m_run)[MB], const float (&l_run)[MB],
                                            const float (&sink2)[MB], TileOut<MB, OUT_BF16> &o) {
#pragma unroll
  for (int m = 0; m < MB; ++m) finish_head<OUT_BF16>(p, acc[m], m_run[m], l_run[m], sink2[m], o.v[m]);
}

// Stores this lane's query row `qrow` of q head `hq`.
template <bool OUT_BF16>
__device__ __forceinline__ void write_head(const ExtendParams &p, const typename HeadOut<OUT_BF16>::type &ov,
                                           int32_t hq, int32_t qrow) {
  const int32_t lq = (threadIdx.x & 63) >> 4;
  const int64_t hbase = (static_cast<int64_t>(qrow) * p.q_heads + hq) * kD;
  if constexpr (OUT_BF16) {
    const int32_t d0 = 16 * (lq & 1) + 8 * (lq >> 1);  // see finish_head
#pragma unroll
    for (int t = 0; t < 4; ++t) *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(p.out) + hbase + 32 * t + d0) = ov[t];
  } else {
#pragma unroll
    for (int n = 0; n < 8; ++n)
      *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + hbase + 4 * lq + 16 * n) = ov[n];
  }
}

// Stores this lane's query row (when qvalid) of every head of the wave.
// ALLH: the group has exactly kNW * MB heads (8 at two heads per wavefront, 4
// at one), so every head of every wavefront is valid and the steady tiles'
// stores are branch-free: the wait for the next tile's queries (loaded before
// these stores, and counted with them in issue order) then leaves the stores
// in flight.  A store under a branch makes that wait drain every store of the
// tile (C3: 84 -> 81 us without the branch).
template <int MB, bool OUT_BF16, bool ALLH>
__device__ __forceinline__ void write_tile(const ExtendParams &p, const TileOut<MB, OUT_BF16> &o, int32_t hq0,
                                           int32_t row0, bool qvalid = true) {
  const int32_t w = threadIdx.x >> 6;
  const int32_t kr = threadIdx.x & 15;
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int32_t hh = w * MB + m;
    if ((!ALLH && hh >= p.ghead) || !qvalid) continue;
    write_head<OUT_BF16>(p, o.v[m], hq0 + hh, row0 + kr);
  }
}

template <int MB>
__device__ __forceinline__ void q_operands(const uint4 (&raw)[MB][4], bf16x8_t (&qop)[MB][4]) {
#pragma unroll
  for (int m = 0; m < MB; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) __builtin_memcpy(&qop[m][c], &raw[m][c], 16);
}

// The tiles [qt_begin, qt_end) of request b, kv head g ("a run") are done in
// two passes: the steady tiles through the ring (run_steady), then the other
// tiles (band clipped at position 0, partial tiles, other windows) through the
// general path (run_general).  Tiles are independent; the kernel runs all
// first passes of its runs, then all second passes, which keeps the two
// paths' registers apart.
template <int MB, bool OUT_BF16, bool ALLH>
__device__ __forceinline__ void run_steady(const ExtendParams &p, uint16_t *ktile, uint16_t *vtile, int32_t b,
                                          int32_t g, int32_t hq0, int32_t qt_begin, int32_t qt_end) {
  const int32_t lane = threadIdx.x & 63;
  const int32_t w = threadIdx.x >> 6;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  const int32_t row = threadIdx.x >> 4;  // K/V row this thread stages within a block

  // Everything the tile loop needs from memory about the request (and the
  // sinks of this wave's heads) is read once here: a load inside the loop
  // would make the wave wait for all of its older memory operations, i.e. the
  // previous tile's output stores and the prefetches.
  const QoRows qrows = qo_rows(p, b);
  const int32_t n_new = qrows.n;
  const int32_t qo0 = qrows.qo0;
  int32_t seq = p.seq_lens[b];
  if (seq > p.r2t_stride) seq = static_cast<int32_t>(p.r2t_stride);
  const int32_t prefix = p.prefix_lens[b];
  const KeySrc ks = key_src<false>(p, b, prefix);
  float sink2[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int32_t hh = w * MB + m;
    sink2[m] = (p.sinks && hh < p.ghead) ? p.sinks[hq0 + hh] * kLog2e : 0.f;
  }

  // gfx950 counts global loads and stores on one counter that retires in
  // issue order, so a wait for a load also waits for every store issued before
  // it, and the compiler cannot count stores that sit in a branch (it then
  // waits for them as well).  A steady tile waits for memory at its top, where
  // the band block, slots and queries issued one tile earlier arrive together,
  // and stores its output at its end, outside any branch when every head of
  // the wavefronts is valid (ALLH): the waits of the next tile are for loads
  // issued before these stores, so the stores stay in flight.  With one wavefront per SIMD (MB >= 2) a stall is not hidden by
  // another wavefront, so this matters: storing each tile's output at the top
  // of the next one instead (inside a branch) was 6% slower.  (With two
  // workgroups per CU it was the other way round, and two workgroups were no
  // faster than one.)
  int32_t qt = qt_begin;
  while (qt < qt_end) {
    Tile tl = tile_at<false>(p, ks, qo0, qt, prefix, n_new, seq);
    if (!tl.steady) {
      ++qt;
      continue;
    }
    // ---- a stretch of steady tiles starts: fill the ring with the whole band
    // of its first tile (slots 0..8), all 18 loads in flight before the first
    // LDS write waits for one (at two heads per wavefront; at one, two
    // wavefronts per SIMD leave too few registers, and the compiler pairs each
    // load with its write).
    uint4 qraw[MB][4];
    load_q<MB>(p, static_cast<int64_t>(tl.row0) + kr, hq0, w, lq, qraw);
    bool next_steady = qt + 1 < qt_end && tile_at<false>(p, ks, qo0, qt + 1, prefix, n_new, seq).steady;
    int32_t nslot;  // slot of this thread's row of the next tile's band block 8
    {
      int32_t sl[kKB];
#pragma unroll
      for (int i = 0; i < kKB; ++i) sl[i] = slot_in(ks, tl.kj0 + 16 * i + row);
      // (a position that is not needed re-reads one inside this band: no branch)
      nslot = slot_in(ks, next_steady ? tl.kj0 + kBand + row : tl.kj0 + row);
      lds_barrier();  // other waves may still read an earlier band
      uint4 kreg[kKB], vreg[kKB];
#pragma unroll
      for (int i = 0; i < kKB; ++i) fetch_piece(p, sl[i], g, kreg[i], vreg[i]);
#pragma unroll
      for (int i = 0; i < kKB; ++i) put_piece(ktile, vtile, 16 * i + row, kreg[i], vreg[i]);
      __builtin_amdgcn_sched_group_barrier(0x020, 2 * kKB, 0);  // the 18 global loads first,
      __builtin_amdgcn_sched_group_barrier(0x200, 2 * kKB, 0);  // then the 18 LDS writes
      lds_barrier();
    }
    // ---- stream: this tile, then the next while it is steady.  Each tile
    // waits for memory only at its top, where the block, slots and queries
    // issued one tile earlier arrive together.
    int32_t q0 = 0;  // ring slot of band block 0
    bool first = true;
    uint4 nk = make_uint4(0, 0, 0, 0), nv = make_uint4(0, 0, 0, 0);
    for (;;) {
      if (!first) {
        lds_barrier();  // every wave is done with the previous tile: its band block 0 slot is free
        put_piece(ktile, vtile, ring_slot(q0, kKB - 1) * 16 + row, nk, nv);  // this tile's band block 8
        lds_barrier();
      }
      first = false;
      // ---- in flight during this tile: the next tile's band block 8, the
      // slots of the one after, and the next tile's queries
      uint4 qn[MB][4];
      if (next_steady) {
        fetch_piece(p, nslot, g, nk, nv);
        const bool next2 = qt + 2 < qt_end && tile_at<false>(p, ks, qo0, qt + 2, prefix, n_new, seq).steady;
        nslot = slot_in(ks, next2 ? tl.kj0 + 16 + kBand + row : tl.kj0 + row);
        load_q<MB>(p, static_cast<int64_t>(tl.row0) + kTQ + kr, hq0, w, lq, qn);
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        int32_t slot[kKB];
#pragma unroll
        for (int j = 0; j < kKB; ++j) slot[j] = ring_slot(q0, j);
        bf16x8_t qop[MB][4];
        q_operands<MB>(qraw, qop);
        f32x4_t s0[kKB];
        uint32_t pw0[kKB][2];
        float m0, l0;
        f32x4_t acc0[8];
        typename HeadOut<OUT_BF16>::type o0;
        if constexpr (MB == 2) {
          f32x4_t s1[kKB];
          uint32_t pw1[kKB][2];
          float m1, l1;
          f32x4_t acc1[8];
          typename HeadOut<OUT_BF16>::type o1;
          head_scores(ktile, slot, qop[0], s0);
          head_scores(ktile, slot, qop[1], s1);
          head_weights(p.scale2, s0, pw0, m0, l0);
          head_pv(vtile, slot, pw0, acc0);
          head_weights(p.scale2, s1, pw1, m1, l1);
          head_pv(vtile, slot, pw1, acc1);
          finish_head<OUT_BF16>(p, acc0, m0, l0, sink2[0], o0);
          write_head<OUT_BF16>(p, o0, hq0 + 2 * w, tl.row0 + kr);
          finish_head<OUT_BF16>(p, acc1, m1, l1, sink2[1], o1);
          write_head<OUT_BF16>(p, o1, hq0 + 2 * w + 1, tl.row0 + kr);
        } else {
          head_scores(ktile, slot, qop[0], s0);
          head_weights(p.scale2, s0, pw0, m0, l0);
          head_pv(vtile, slot, pw0, acc0);
          finish_head<OUT_BF16>(p, acc0, m0, l0, sink2[0], o0);
          if (ALLH || w < p.ghead) write_head<OUT_BF16>(p, o0, hq0 + w, tl.row0 + kr);
        }
      }
      ++qt;
      if (!next_steady) break;
      tl = tile_at<false>(p, ks, qo0, qt, prefix, n_new, seq);
      next_steady = qt + 1 < qt_end && tile_at<false>(p, ks, qo0, qt + 1, prefix, n_new, seq).steady;
      q0 = q0 + 1 < kKB ? q0 + 1 : 0;
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int c = 0; c < 4; ++c) qraw[m][c] = qn[m][c];
    }
  }
}

template <int MB, bool OUT_BF16, bool CHUNKED, bool ALLH>
__device__ __forceinline__ void run_general(const ExtendParams &p, uint16_t *ktile, uint16_t *vtile, int32_t b,
                                           int32_t g, int32_t hq0, int32_t qt_begin, int32_t qt_end) {
  const int32_t lane = threadIdx.x & 63;
  const int32_t w = threadIdx.x >> 6;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;

  // Everything the tile loop needs from memory about the request (and the
  // sinks of this wave's heads) is read once here: a load inside the loop
  // would make the wave wait for all of its older memory operations, i.e. the
  // previous tile's output stores and the prefetches.
  const QoRows qrows = qo_rows(p, b);
  const int32_t n_new = qrows.n;
  const int32_t qo0 = qrows.qo0;
  int32_t seq = p.seq_lens[b];
  if (seq > p.r2t_stride) seq = static_cast<int32_t>(p.r2t_stride);
  const int32_t prefix = p.prefix_lens[b];
  const KeySrc ks = key_src<CHUNKED>(p, b, prefix);
  float sink2[MB];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int32_t hh = w * MB + m;
    sink2[m] = (p.sinks && hh < p.ghead) ? p.sinks[hq0 + hh] * kLog2e : 0.f;
  }

  for (int32_t qt = qt_begin; qt < qt_end; ++qt) {
    const Tile tl = tile_at<CHUNKED>(p, ks, qo0, qt, prefix, n_new, seq);
    if (tl.steady) continue;
    const bool qvalid = (qt * kTQ + kr) < n_new && static_cast<int64_t>(tl.row0) + kr < p.total_q;
    f32x4_t acc[MB][8];
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[MB], l_run[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      m_run[m] = kNegBig;
      l_run[m] = 0.f;
    }
    // rows past the request (last partial tile) read a real row; never stored
    uint4 qr[MB][4];
    load_q<MB>(p, qvalid ? static_cast<int64_t>(tl.row0) + kr : static_cast<int64_t>(tl.row0), hq0, w, lq, qr);
    bf16x8_t qop[MB][4];
    q_operands<MB>(qr, qop);
    tile_general<MB, CHUNKED>(p, ks, tl, qop, g, ktile, vtile, acc, m_run, l_run);
    // sink once, normalise (every lane: the bf16 packing swaps rows), store
    TileOut<MB, OUT_BF16> o;
    finish_tile<MB, OUT_BF16>(p, acc, m_run, l_run, sink2, o);
    write_tile<MB, OUT_BF16, ALLH>(p, o, hq0, tl.row0, qvalid);
  }
}

// Run r of the numbering (request, kv head, run of T tiles, q-head group);
// b = -1 past the end.  The groups of one kv head's run are neighbours, so
// they read the same K/V blocks at about the same time.  hq0: the group's
// first q head.
struct Run {
  int32_t b, g, hq0, qt_begin, qt_end;
};

__device__ __forceinline__ Run run_of(const ExtendParams &p, int32_t T, int32_t r) {
  int32_t t = r, b = 0, ntile = 0, nrun = 0;
  for (; b < p.batch; ++b) {
    ntile = (new_count(p, b) + kTQ - 1) / kTQ;
    nrun = (ntile + T - 1) / T;
    const int32_t tb = nrun * p.kv_heads * p.halves;
    if (t < tb) break;
    t -= tb;
  }
  Run run{-1, 0, 0, 0, 0};
  if (b >= p.batch) return run;
  const int32_t half = t % p.halves;
  t /= p.halves;
  run.b = b;
  run.g = t / nrun;
  run.hq0 = run.g * p.group + half * p.ghead;
  run.qt_begin = (t % nrun) * T;
  run.qt_end = run.qt_begin + T < ntile ? run.qt_begin + T : ntile;
  return run;
}

// Persistent grid (one or two workgroups per CU): the runs, numbered
// (request, kv head, run, q-head group), are split into 8 contiguous ranges, one per XCD
// (workgroup i runs on XCD i % 8), so neighbouring runs, which share band
// blocks, meet in one L2; the workgroups of an XCD stride through its range.
// CHUNKED: chunked local attention (p.chunk > 0), a separate instantiation so
// the window-only code carries none of it.
template <int MB, bool OUT_BF16, bool CHUNKED, bool ALLH>
__global__ void __launch_bounds__(kNW * 64, MB >= 2 ? 1 : 2) extend_kernel(ExtendParams p) {
  static_assert(MB == 1 || MB == 2, "one or two q heads per wavefront");
  static_assert(MB == 1 || ALLH, "two heads per wavefront only for groups of 8");
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kKB * 16 * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t vtile[kKB * 16 * kVRow];
  const int32_t T = p.run_tiles;
  int32_t total = 0;
  for (int32_t b = 0; b < p.batch; ++b)
    total += (new_count(p, b) + kTQ * T - 1) / (kTQ * T) * p.kv_heads * p.halves;
  const int32_t per_xcd = gridDim.x / 8;  // the grid is a multiple of 8
  const int32_t x = blockIdx.x % 8;
  const int32_t r_lo = static_cast<int32_t>(static_cast<int64_t>(total) * x / 8);
  const int32_t r_hi = static_cast<int32_t>(static_cast<int64_t>(total) * (x + 1) / 8);
  const int32_t r0 = r_lo + static_cast<int32_t>(blockIdx.x / 8);
  if constexpr (!CHUNKED) {  // steady tiles exist only without chunks
    for (int32_t r = r0; r < r_hi; r += per_xcd) {
      const Run run = run_of(p, T, r);
      if (run.b < 0) break;
      run_steady<MB, OUT_BF16, ALLH>(p, ktile, vtile, run.b, run.g, run.hq0, run.qt_begin, run.qt_end);
    }
  }
  for (int32_t r = r0; r < r_hi; r += per_xcd) {
    const Run run = run_of(p, T, r);
    if (run.b < 0) break;
    run_general<MB, OUT_BF16, CHUNKED, ALLH>(p, ktile, vtile, run.b, run.g, run.hq0, run.qt_begin, run.qt_end);
  }
}

template <int MB, bool ALLH>
hipError_t launch_mb(const ExtendParams &p, uint32_t grid, bool out_bf16, hipStream_t stream) {
  if (p.chunk > 0) {
    if (out_bf16)
      hipLaunchKernelGGL((extend_kernel<MB, true, true, ALLH>), dim3(grid), dim3(kNW * 64), 0, stream, p);
    else
      hipLaunchKernelGGL((extend_kernel<MB, false, true, ALLH>), dim3(grid), dim3(kNW * 64), 0, stream, p);
  } else if (out_bf16) {
    hipLaunchKernelGGL((extend_kernel<MB, true, false, ALLH>), dim3(grid), dim3(kNW * 64), 0, stream, p);
  } else {
    hipLaunchKernelGGL((extend_kernel<MB, false, false, ALLH>), dim3(grid), dim3(kNW * 64), 0, stream, p);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Long-band kernel: windows of 256 keys or more, and full attention (W = -1).
// There a query sees hundreds to thousands of keys, the work per query is
// O(W) MFMA and the kernel is bound by the matrix cores, not by HBM.
//   * a tile is 256 q rows: the group's q heads x (256 / heads) consecutive
//     queries of one request, in 16 row blocks of 16 queries x one head; each
//     wavefront owns RB row blocks, so each K / V fragment it reads from LDS
//     feeds RB MFMAs (LDS bandwidth per flop falls as 1 / RB);
//   * the band [first key of the first query, last query] is walked in blocks
//     of 64 keys through three LDS stages: while block j is computed the rows
//     of block j + 1 are in flight in registers and the slots of block j + 2
//     are read, and the odd wavefronts still read block j - 1's V rows; one
//     workgroup barrier per block;
//   * online softmax in base 2 that rescales lazily: the running max of a row
//     moves only when a block's max exceeds it by more than 8, so a row's
//     weights stay below 2^8 (well inside f16's range) and,
//     past the first blocks, the accumulators are almost never rescaled;
//   * tiles are numbered (request, kv head, tile, q-head group) and dealt to
//     the XCDs in contiguous ranges: neighbouring tiles share most of their
//     band, so they meet in one L2.
// ---------------------------------------------------------------------------
constexpr int kBK = 64;                                  // keys per band block
// The A operand of all ones (f16 1.0): an MFMA of it with a block's packed
// weights P^T gives each query's sum of those weights in every output row, so
// the normaliser is summed on the matrix cores from exactly the weights that
// enter P.V, and the VALU (the busier pipe here) does not add them.
constexpr bf16x8_t kOnes = {0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00, 0x3C00};
constexpr int kBandStage = kBK * (kKRow + kVRow);        // elements of one LDS stage (K rows, then V rows)
constexpr int32_t kBandMinWindow = 256;                  // windows at least this long use the band kernel
constexpr float kRescaleSlack = 8.f;                     // log2 of the largest weight before a rescale

struct BandTile {
  int32_t b, g, hq0, tile;  // request, kv head, first q head of the group, tile of the request
};

// Tile t of the numbering (request, kv head, tile, q-head group); b = -1 past the end.
__device__ __forceinline__ BandTile band_tile(const ExtendParams &p, int32_t TQ, int32_t t) {
  BandTile bt{-1, 0, 0, 0};
  int32_t b = 0, ntile = 0;
  for (; b < p.batch; ++b) {
    ntile = (new_count(p, b) + TQ - 1) / TQ;
    const int32_t n = ntile * p.kv_heads * p.halves;
    if (t < n) break;
    t -= n;
  }
  if (b >= p.batch) return bt;
  const int32_t half = t % p.halves;
  t /= p.halves;
  bt.b = b;
  bt.g = t / ntile;
  bt.tile = t % ntile;
  bt.hq0 = bt.g * p.group + half * p.ghead;
  return bt;
}

// Everything a tile's block loop needs, fixed per tile.
struct BandCtx {
  KeySrc ks;
  int32_t g;       // kv head
  int32_t i0;      // position of the tile's first query
  int32_t i_last;  // position of its last valid query
  int32_t kj0;     // first key of the band
  int32_t nkeys;   // keys in the band
  int32_t nblk;    // 64-key blocks
};

// Per-request fields of the band kernel, read once per workgroup into LDS (for
// batches of up to kBandTabReqs requests and up to kBandTabHeads q heads), so
// that a tile's context is found with LDS reads instead of a walk over the
// batch's qo_indptr (one dependent global round trip per request) followed by
// the request's own lengths and table range.
constexpr int kBandTabReqs = 1024;
constexpr int kBandTabHeads = 256;
struct BandReq {
  int64_t src_off;    // key source: entry 0 is src_off past the window table (or req_to_token)
  int64_t src_hi;     // entries in the key source
  int32_t pos_base;   // position of entry 0
  int32_t qo0, n;     // query rows
  int32_t prefix;     // cached positions
  int32_t seq;        // sequence length, clamped to the req_to_token stride
  int32_t tiles;      // tiles of the request (all kv heads and q-head groups)
  int32_t tile0;      // tiles of the requests before it
};

template <int NW>
struct BandStage {
  static constexpr int kRowsPerPass = NW * 64 / 16;   // 16 threads per 256-byte row
  static constexpr int kPasses = kBK / kRowsPerPass;  // K and V pieces per thread per block
};

// The band's blocks for this wave's RB row blocks (query positions q_of[i] +
// kr): S^T = K Q^T, masks on edge blocks, softmax with lazy rescaling, O^T +=
// V^T P^T (weights and V rows in f16).
//
// Two wavefronts share each SIMD.  The odd wavefronts run one block behind in
// their P.V: in the iteration of block j they first do P.V of block j - 1, then
// QK^T and the softmax of block j, so the two wavefronts of a SIMD more often
// sit in different phases (one issuing MFMAs while the other issues the
// softmax's VALU work).  Measured at the C3 shape with W = 4096: 1128 us against
// 1139 us with no wavefront behind, and 1208 us with the upper four behind
// (waves 2k and 2k + 1 appear to share a SIMD).  That P.V reads the V rows of
// block j - 1 while block j + 1 is written, hence three LDS stages.
template <int RB, int NW>
__device__ __forceinline__ void band_blocks(const ExtendParams &p, const BandCtx &c, uint16_t *lds,
                                            const bf16x8_t (&qop)[RB][4], const int32_t (&q_of)[RB],
                                            f32x4_t (&acc)[RB][8], float (&m_run)[RB], f32x4_t (&l_acc)[RB]) {
  constexpr int kPasses = BandStage<NW>::kPasses;
  constexpr int kRowsPerPass = BandStage<NW>::kRowsPerPass;
  const int32_t lane = threadIdx.x & 63;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  const int32_t srow = threadIdx.x >> 4;   // K / V row this thread stages (plus kRowsPerPass * pass)
  const int32_t spiece = threadIdx.x & 15;
  const int32_t W = p.window;
  const bool lag = (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & 1) != 0;  // wave-uniform

  // Slots of block j for this thread's rows.  Band key k (position kj0 + k) is
  // entry k - lo of sbase when lo <= k < lo + span; every other row (past the
  // band, or outside the key source) loads the first entry instead, an
  // unconditional in-bounds read, and its row is zeroed or masked later.  A
  // band with no source entry at all reads nothing and takes slot 0.
  const int64_t rel0 = static_cast<int64_t>(c.kj0) - c.ks.pos_base;  // source index of band key 0
  const int64_t lo64 = rel0 < 0 ? -rel0 : 0;
  const int64_t hi64 = c.ks.hi - rel0 < c.nkeys ? c.ks.hi - rel0 : c.nkeys;
  const bool has_src = hi64 > lo64;  // workgroup-uniform
  const int32_t lo = static_cast<int32_t>(lo64);
  const uint32_t span = has_src ? static_cast<uint32_t>(hi64 - lo64) : 0u;
  const int32_t *sbase = has_src ? c.ks.src + (rel0 + lo64) : c.ks.src;
  auto block_slots = [&](int32_t j, int32_t (&sl)[kPasses]) {
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int32_t k = kBK * j + srow + kRowsPerPass * ps - lo;
      sl[ps] = has_src ? sbase[static_cast<uint32_t>(k) < span ? k : 0] : 0;
    }
  };
  // This thread's 16 bytes of kv head c.g in a token row: row s starts s *
  // row_elems elements past the head's base (one 32 x 32 -> 64-bit multiply-add
  // per slot; a slot outside the pool reads row 0).
  const uint16_t *kbase = p.k + c.g * kD + 8 * spiece;
  const uint16_t *vbase = p.v + c.g * kD + 8 * spiece;
  const uint32_t row_elems = static_cast<uint32_t>(p.kv_heads) * kD;
  // every int32 slot in [0, rows) is below this bound and every negative one is not
  const uint32_t nrows = p.rows < (int64_t(1) << 31) ? static_cast<uint32_t>(p.rows) : 0x80000000u;
  auto block_fetch = [&](const int32_t (&sl)[kPasses], uint4 (&kv)[kPasses], uint4 (&vv)[kPasses]) {
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const uint32_t su = static_cast<uint32_t>(sl[ps]);
      const uint64_t off = static_cast<uint64_t>(su < nrows ? su : 0u) * row_elems;
      kv[ps] = *reinterpret_cast<const uint4 *>(kbase + off);
      vv[ps] = *reinterpret_cast<const uint4 *>(vbase + off);
    }
  };
  // Rows past the band (only in a tile's last block) hold slot 0's row and are
  // written as zeros; every other block is written as loaded.
  auto block_put = [&](int32_t j, uint16_t *stage, const uint4 (&kv)[kPasses], const uint4 (&vv)[kPasses]) {
    if (kBK * (j + 1) <= c.nkeys) {  // workgroup-uniform
#pragma unroll
      for (int ps = 0; ps < kPasses; ++ps) {
        const int32_t row = srow + kRowsPerPass * ps;
        *reinterpret_cast<uint4 *>(stage + row * kKRow + 8 * spiece) = kv[ps];
        *reinterpret_cast<uint4 *>(stage + kBK * kKRow + row * kVRow + 8 * spiece) = bf16x8_to_f16x8(vv[ps]);
      }
    } else {
#pragma unroll
      for (int ps = 0; ps < kPasses; ++ps) {
        const int32_t row = srow + kRowsPerPass * ps;
        const bool ok = kBK * j + row < c.nkeys;
        *reinterpret_cast<uint4 *>(stage + row * kKRow + 8 * spiece) = ok ? kv[ps] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(stage + kBK * kKRow + row * kVRow + 8 * spiece) =
            ok ? bf16x8_to_f16x8(vv[ps]) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  const int32_t voff = (4 * lq + (kr >> 2)) * kVRow + 4 * (kr & 3);
  // O^T += V^T P^T over the key-tile pairs (0, 1) and (2, 3) of the block whose V rows are at vt
  auto pv = [&](const uint16_t *vt, const bf16x8_t (&pop)[RB][2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint16_t *va = vt + (32 * u) * kVRow + voff;
      const uint16_t *vb = va + 16 * kVRow;
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const i16x4_t lo = lds_read_tr16(va + 16 * n);
        const i16x4_t hi = lds_read_tr16(vb + 16 * n);
        const bf16x8_t vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          acc[i][n] = mfma_f16(vop, pop[i][u], acc[i][n]);
        }
      }
    }
  };

  int32_t sl[kPasses];
  uint4 kv[kPasses], vv[kPasses];
  bf16x8_t pop[RB][2];  // the weights of the last softmax (the lagging half's next P.V)
  block_slots(0, sl);
  block_fetch(sl, kv, vv);
  block_slots(1, sl);
  lds_barrier();  // the previous tile's last blocks are consumed
  block_put(0, lds, kv, vv);
  lds_barrier();
  uint16_t *cur = lds, *prev = lds + 2 * kBandStage, *next = lds + kBandStage;  // stages of blocks j, j - 1, j + 1
  for (int32_t j = 0; j < c.nblk; ++j) {
    const bool more = j + 1 < c.nblk;  // workgroup-uniform
    if (more) {
      block_fetch(sl, kv, vv);  // block j + 1 in flight during block j
      block_slots(j + 2, sl);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (lag && j > 0) pv(prev + kBK * kKRow, pop);  // the lagging half: P.V of block j - 1
    const uint16_t *vt_base = cur + kBK * kKRow;
    const int32_t kb = c.kj0 + kBK * j;  // position of the block's first key
    // ---- S^T = K Q^T: key tile kt (16 keys), lane holds keys 4lq..4lq+3 of query kr
    f32x4_t s[RB][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      bf16x8_t kop[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) __builtin_memcpy(&kop[cc], cur + (16 * kt + kr) * kKRow + 32 * cc + 8 * lq, 16);
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        s[i][kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) s[i][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[cc], qop[i][cc], s[i][kt], 0, 0, 0);
      }
    }
    // ---- masks on blocks that touch the band's edges or its end (workgroup-uniform test)
    const bool interior = kb + kBK - 1 <= c.i0 && (W < 0 || kb >= c.i_last - W) && kBK * (j + 1) <= c.nkeys;
    if (!interior) {
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int32_t q = q_of[i] + kr;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int32_t key = kb + 16 * kt + 4 * lq + r;
            const bool ok = key <= q && (W < 0 || key >= q - W) && key - c.kj0 < c.nkeys;
            s[i][kt][r] = ok ? s[i][kt][r] : -INFINITY;
          }
      }
    }
    // ---- softmax: block max per row, lazy rescale, weights packed to f16 (the
    // normaliser sums the same rounded weights)
    // A row's max is the largest of its four lanes' maxima, so a wavefront
    // whose lanes all stay within the slack has no row that grew: the
    // cross-lane max is only taken in the (rare) rescale.
    float ml[RB];
    bool grow = false;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      float m = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, s[i][kt][r]);
      ml[i] = m;
      grow = grow || m * p.scale2 > m_run[i] + kRescaleSlack;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const float m_new = fmaxf(m_run[i], wave_max_q(ml[i]) * p.scale2);
        const float alpha = __builtin_amdgcn_exp2f(m_run[i] - m_new);
        m_run[i] = m_new;
        l_acc[i] *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[i][n] *= alpha;
      }
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[i][kt][r] = __builtin_amdgcn_exp2f(fmaf(s[i][kt][r], p.scale2, -m_run[i]));
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const f32x4_t &e0 = s[i][2 * u], &e1 = s[i][2 * u + 1];
        const uint32_t u4[4] = {pack_f16x2_hw(e0[0], e0[1]), pack_f16x2_hw(e0[2], e0[3]),
                                pack_f16x2_hw(e1[0], e1[1]), pack_f16x2_hw(e1[2], e1[3])};
        __builtin_memcpy(&pop[i][u], u4, 16);
        l_acc[i] = mfma_f16(kOnes, pop[i][u], l_acc[i]);
      }
    }
    if (!lag) pv(vt_base, pop);  // the leading half: P.V of block j now
    if (more) block_put(j + 1, next, kv, vv);
    lds_barrier();
    uint16_t *t = prev;
    prev = cur;
    cur = next;
    next = t;
  }
  if (lag) pv(prev + kBK * kKRow, pop);  // the last block's P.V (its stage is not rewritten before a barrier)
}

// A tile is RB * NW row blocks of 16 q rows (heads x queries); WGS
// workgroups share a CU.
template <int RB, int NW, int WGS, bool OUT_BF16>
__global__ void __launch_bounds__(NW * 64, WGS) band_kernel(ExtendParams p) {
  constexpr int kRowBlocks = RB * NW;
  __shared__ __attribute__((aligned(16))) uint16_t lds[3 * kBandStage];
  __shared__ BandReq reqs[kBandTabReqs];
  __shared__ float sinks_tab[kBandTabHeads];
  __shared__ int32_t total_tab;
  const int32_t lane = threadIdx.x & 63;
  const int32_t w = threadIdx.x >> 6;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  const int32_t TQ = kRowBlocks * 16 / p.ghead;  // queries per tile
  const int32_t nsub = TQ / 16;                  // 16-query sub-blocks per head
  const int32_t W = p.window;

  const bool tab = p.batch <= kBandTabReqs && p.q_heads <= kBandTabHeads;  // uniform
  int32_t total = 0;
  if (tab) {
    for (int32_t b = threadIdx.x; b < p.batch; b += NW * 64) {
      BandReq rq;
      const QoRows qrows = qo_rows(p, b);
      rq.qo0 = qrows.qo0;
      rq.n = qrows.n;
      rq.seq = p.seq_lens[b];
      if (rq.seq > p.r2t_stride) rq.seq = static_cast<int32_t>(p.r2t_stride);
      rq.prefix = p.prefix_lens[b];
      const KeySrc ks = key_src<false>(p, b, rq.prefix);
      rq.src_off = ks.src - (p.indptr ? p.table : p.r2t);
      rq.src_hi = ks.hi;
      rq.pos_base = ks.pos_base;
      rq.tiles = (rq.n + TQ - 1) / TQ * p.kv_heads * p.halves;
      reqs[b] = rq;
    }
    for (int32_t h = threadIdx.x; h < p.q_heads; h += NW * 64) sinks_tab[h] = p.sinks ? p.sinks[h] * kLog2e : 0.f;
    __syncthreads();
    if (w == 0) {  // exclusive prefix of the tile counts, 64 requests at a time
      int32_t run = 0;
      for (int32_t base = 0; base < p.batch; base += 64) {
        const int32_t b = base + lane;
        const int32_t cnt = b < p.batch ? reqs[b].tiles : 0;
        int32_t inc = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int32_t y = __shfl_up(inc, d);
          if (lane >= d) inc += y;
        }
        if (b < p.batch) reqs[b].tile0 = run + inc - cnt;
        run += __shfl(inc, 63);
      }
      if (lane == 0) total_tab = run;
    }
    __syncthreads();
    total = total_tab;
  } else {
    for (int32_t b = 0; b < p.batch; ++b) total += (new_count(p, b) + TQ - 1) / TQ * p.kv_heads * p.halves;
  }
  const int32_t per_xcd = gridDim.x / 8;  // the grid is a multiple of 8
  const int32_t x = blockIdx.x % 8;
  const int32_t t_lo = static_cast<int32_t>(static_cast<int64_t>(total) * x / 8);
  const int32_t t_hi = static_cast<int32_t>(static_cast<int64_t>(total) * (x + 1) / 8);

  int32_t b_from = 0;  // a workgroup's tiles increase, so their requests do too
  for (int32_t t = t_lo + static_cast<int32_t>(blockIdx.x / 8); t < t_hi; t += per_xcd) {
    BandTile bt;
    QoRows qrows;
    int32_t seq, prefix;
    BandCtx c;
    if (tab) {
      // the request holding tile t: the first from b_from whose tiles end past t
      int32_t b = -1;
      for (int32_t base = b_from; base < p.batch; base += 64) {
        const int32_t bb = base + lane;
        const bool hit = bb < p.batch && reqs[bb].tile0 + reqs[bb].tiles > t;
        const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
        if (m != 0) {
          b = base + static_cast<int32_t>(__builtin_ctzll(m));
          break;
        }
      }
      if (b < 0) break;
      b_from = b;
      const BandReq &rq = reqs[b];
      const int32_t ntile = __builtin_amdgcn_readfirstlane((rq.n + TQ - 1) / TQ);
      int32_t tl = __builtin_amdgcn_readfirstlane(t - rq.tile0);
      const int32_t half = tl % p.halves;
      tl /= p.halves;
      bt.b = b;
      bt.g = tl / ntile;
      bt.tile = tl % ntile;
      bt.hq0 = bt.g * p.group + half * p.ghead;
      qrows.qo0 = __builtin_amdgcn_readfirstlane(rq.qo0);
      qrows.n = __builtin_amdgcn_readfirstlane(rq.n);
      seq = __builtin_amdgcn_readfirstlane(rq.seq);
      prefix = __builtin_amdgcn_readfirstlane(rq.prefix);
      // 64-bit fields made wave-uniform half by half; the source pointer is
      // rebuilt from a kernel argument so that it stays a global pointer
      auto uni64 = [](int64_t v) {
        const uint64_t u = static_cast<uint64_t>(v);
        return static_cast<int64_t>(
            (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32))) << 32) |
            static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u))));
      };
      c.ks.src = (p.indptr ? p.table : p.r2t) + uni64(rq.src_off);
      c.ks.hi = uni64(rq.src_hi);
      c.ks.pos_base = __builtin_amdgcn_readfirstlane(rq.pos_base);
    } else {
      bt = band_tile(p, TQ, t);
      if (bt.b < 0) break;
      qrows = qo_rows(p, bt.b);
      seq = p.seq_lens[bt.b];
      if (seq > p.r2t_stride) seq = static_cast<int32_t>(p.r2t_stride);
      prefix = p.prefix_lens[bt.b];
      c.ks = key_src<false>(p, bt.b, prefix);
    }
    c.g = bt.g;
    c.i0 = prefix + bt.tile * TQ;
    c.i_last = c.i0 + TQ - 1;
    if (c.i_last > prefix + qrows.n - 1) c.i_last = prefix + qrows.n - 1;
    if (c.i_last > seq - 1) c.i_last = seq - 1;
    c.kj0 = W < 0 ? 0 : c.i0 - W;
    if (c.kj0 < 0) c.kj0 = 0;
    c.nkeys = c.i_last >= c.kj0 ? c.i_last - c.kj0 + 1 : 0;
    c.nblk = (c.nkeys + kBK - 1) / kBK;

    // this wave's row blocks: head hh, 16-query sub-block qs
    int32_t hh[RB], qi0[RB], q_of[RB];
    float sink2[RB];
    bf16x8_t qop[RB][4];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      const int32_t r = RB * w + i;
      hh[i] = r / nsub;
      qi0[i] = bt.tile * TQ + 16 * (r % nsub);  // first query index (within the request) of the block
      q_of[i] = prefix + qi0[i];
      const int32_t qi = qi0[i] + kr;
      const int64_t qrow = qrows.qo0 + (qi < qrows.n ? qi : 0);
      const uint16_t *qp = p.q + (qrow * p.q_heads + bt.hq0 + hh[i]) * kD + 8 * lq;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const uint4 raw = *reinterpret_cast<const uint4 *>(qp + 32 * cc);
        __builtin_memcpy(&qop[i][cc], &raw, 16);
      }
      sink2[i] = tab ? sinks_tab[bt.hq0 + hh[i]] : (p.sinks ? p.sinks[bt.hq0 + hh[i]] * kLog2e : 0.f);
    }

    f32x4_t acc[RB][8];
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[i][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m_run[RB];
    f32x4_t l_acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      m_run[i] = kNegBig;
      l_acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (c.nblk > 0) {
      band_blocks<RB, NW>(p, c, lds, qop, q_of, acc, m_run, l_acc);
    }
    // ---- sink once, normalise, store the valid query rows
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      typename HeadOut<OUT_BF16>::type o;
      // every lane of query kr holds the whole row sum: a quarter from each of the
      // four lanes that finish_head adds (exact: scaling by 1/4 and adding four
      // equal values round nothing)
      finish_head<OUT_BF16>(p, acc[i], m_run[i], 0.25f * l_acc[i][0], sink2[i], o);
      const int32_t qi = qi0[i] + kr;
      if (qi < qrows.n) write_head<OUT_BF16>(p, o, bt.hq0 + hh[i], qrows.qo0 + qi);
    }
  }
}

template <int RB, int NW, int WGS>
hipError_t launch_band(const ExtendParams &p, int64_t total_q, int32_t batch, bool out_bf16, hipStream_t stream) {
  const int64_t tq = RB * NW * 16 / p.ghead;
  const int64_t tiles = ((total_q + tq - 1) / tq + batch) * p.kv_heads * p.halves;
  int64_t grid = tiles < 256 * WGS ? tiles : 256 * WGS;  // at most WGS per CU
  grid = (grid + 7) / 8 * 8;
  if (out_bf16)
    hipLaunchKernelGGL((band_kernel<RB, NW, WGS, true>), dim3(static_cast<uint32_t>(grid)), dim3(NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((band_kernel<RB, NW, WGS, false>), dim3(static_cast<uint32_t>(grid)), dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

// Workgroups of the persistent grid: two per CU of the 256 on MI355X for one
// head per wavefront (the LDS ring allows two); one per CU for MB >= 2, whose
// wavefronts then have the whole register file (measured as fast as two per
// CU, and faster once the output stores leave their branch).
constexpr int64_t kResidentGroups = 512;

}  // namespace

hipError_t launch_extend(const ExtendArgs &a, hipStream_t stream) {
  if (a.idx.batch == 0 || a.total_q == 0) return hipSuccess;
  ExtendParams p{};
  p.q = static_cast<const uint16_t *>(a.q);
  p.k = static_cast<const uint16_t *>(a.layer.k);
  p.v = static_cast<const uint16_t *>(a.layer.v);
  p.rows = a.layer.rows;
  p.kv_heads = a.layer.kv_heads;
  p.q_heads = a.q_heads;
  p.group = a.q_heads / a.layer.kv_heads;
  p.batch = a.idx.batch;
  p.qo_indptr = a.qo_indptr;
  p.prefix_lens = a.prefix_lens;
  p.total_q = a.total_q;
  p.r2t = a.idx.req_to_token;
  p.r2t_rows = a.idx.r2t_rows;
  p.r2t_stride = a.idx.r2t_stride;
  p.req_idx = a.idx.req_pool_idx;
  p.seq_lens = a.idx.seq_lens;
  p.table = a.table;
  p.indptr = a.indptr;
  p.capacity = a.capacity;
  p.window = a.window;
  p.chunk = a.chunk;
  p.sinks = a.sinks;
  p.scale2 = a.sm_scale * kLog2e;
  p.out = a.out;
  // Tiles: every request adds at most one partial tile.  Runs of T tiles, about
  // one run per workgroup of the persistent grid (each run fills its ring once,
  // so fewer, longer runs are cheaper; more runs than workgroups would leave
  // some workgroups a second run while others idle).
  // G = 16 runs as two groups of 8 q heads per kv head on the two-heads-per-
  // wavefront kernel: K/V is read twice (mostly from L2, the two groups being
  // neighbours), but four heads per wavefront spill registers.
  p.halves = p.group >= 16 ? 2 : 1;
  p.ghead = p.group / p.halves;
  const int32_t mb = p.ghead >= 8 ? 2 : 1;  // ghead is 1, 2, 4 or 8
  const int64_t resident = mb >= 2 ? kResidentGroups / 2 : kResidentGroups;  // G >= 8: one per CU
  const int64_t tiles = ((a.total_q + kTQ - 1) / kTQ + a.idx.batch) * a.layer.kv_heads * p.halves;
  int64_t T = tiles / resident;
  if (T < 1) T = 1;
  if (T > 64) T = 64;
  p.run_tiles = static_cast<int32_t>(T);
  int64_t grid = (tiles + T - 1) / T + static_cast<int64_t>(a.idx.batch) * a.layer.kv_heads * p.halves;
  if (grid > resident) grid = resident;
  grid = (grid + 7) / 8 * 8;
  const uint32_t runs = static_cast<uint32_t>(grid);
  const bool out_bf16 = a.out_dtype == SWA_BF16;
  if (a.chunk == 0 && (a.window < 0 || a.window >= kBandMinWindow))
    return launch_band<SWA_BAND_RB, SWA_BAND_NW, SWA_BAND_WGS>(p, a.total_q, a.idx.batch, out_bf16, stream);
  if (mb == 2) {
    if (p.ghead != kNW * 2) return hipErrorInvalidValue;
    return launch_mb<2, true>(p, runs, out_bf16, stream);
  }
  if (p.ghead == kNW) return launch_mb<1, true>(p, runs, out_bf16, stream);
  return launch_mb<1, false>(p, runs, out_bf16, stream);
}

}  // namespace swa
