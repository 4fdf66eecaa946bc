// Windowed-causal extend (chunked prefill) over a cached prefix.
//
// SWA note (zdszero.github.io/swa.html): each query i attends to keys
// [max(0, i - W), i] (opening paragraph and section 实现; W excludes the current
// token, -1 = full attention), with an optional per-head sink (section 设计);
// section 运行时 describes chunked prefill, where the chunk's K/V are written to
// the pool and the chunk's queries read the prefix's last window plus the chunk.
//
// MI355X design (not the pages' kernels):
//   * one workgroup = 16 consecutive queries x the G query heads of one kv head
//     (GQA packed into the M side), so each K/V row staged in LDS serves G heads;
//   * the key range of a tile is only the band [i0 - W, i0 + 15]: blocks of 16
//     keys entirely outside the band are never loaded or multiplied (at W = 128:
//     9 blocks, two of them partially masked);
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 with fp32
//     accumulation; P is rounded to bf16 for the second product and never leaves
//     registers (the first product's accumulator layout is the second's B
//     operand layout); the V^T operand is read from a row-major LDS tile with
//     gfx950's transposing ds_read_b64_tr_b16; online softmax in base 2 over
//     chunks of up to 9 blocks, masks computed only on band-edge blocks;
//   * tiles are numbered (request, kv head, query tile) and dealt to the 8 XCDs
//     in contiguous runs, so the 9 tiles that share a K/V block run on one XCD
//     and hit its L2.
#include "common.hpp"

namespace swa {
namespace {

constexpr int kD = 128;
constexpr int kNW = 4;       // wavefronts per workgroup
constexpr int kTQ = 16;      // queries per tile
constexpr int kKB = 9;       // key blocks (of 16) per chunk
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
};

__device__ __forceinline__ float wave_max_q(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float wave_sum_q(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Queries of request b: count and first position.
__device__ __forceinline__ int32_t new_count(const ExtendParams &p, int32_t b) {
  int32_t n = p.qo_indptr[b + 1] - p.qo_indptr[b];
  return n > 0 ? n : 0;
}

// Steady-state tile: 16 valid queries, band [i0 - W, i0 + 15] not clipped at
// position 0, W = 16 * (NB - 1).  Then the band is exactly NB blocks of 16
// keys (key offset k from i0 - W): block 0 is the band's lower edge (query kr
// sees k >= kr), block NB-1 the diagonal (k <= W + kr), the rest are inside
// the band for every query.  Compile-time structure, no per-key position math.
template <int NB, int MB>
__device__ __forceinline__ void tile_fast(const ExtendParams &p, uint16_t *ktile, uint16_t *vtile,
                                          const bf16x8_t (&qop)[MB][4], const int32_t *key_slots, int32_t g,
                                          f32x4_t (&acc)[MB][8], float (&m_run)[MB], float (&l_run)[MB]) {
  const int32_t lane = threadIdx.x & 63;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  // ---- stage the NB blocks (16 threads per 256-byte row); all loads first
  {
    const int32_t piece = threadIdx.x & 15;
    int32_t slot[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) slot[i] = key_slots[(threadIdx.x >> 4) + 16 * i];
    int64_t off[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t sl = (slot[i] < 0 || slot[i] >= p.rows) ? 0 : static_cast<int64_t>(slot[i]);
      off[i] = row_elem(sl, p.kv_heads, g, kD) + 8 * piece;
    }
    uint4 kreg[NB], vreg[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) kreg[i] = *reinterpret_cast<const uint4 *>(p.k + off[i]);
#pragma unroll
    for (int i = 0; i < NB; ++i) vreg[i] = *reinterpret_cast<const uint4 *>(p.v + off[i]);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int32_t key = (threadIdx.x >> 4) + 16 * i;
      *reinterpret_cast<uint4 *>(ktile + key * kKRow + 8 * piece) = kreg[i];
      *reinterpret_cast<uint4 *>(vtile + key * kVRow + 8 * piece) = vreg[i];
    }
  }
  __syncthreads();
  // ---- S^T = K Q^T
  f32x4_t sacc[MB][NB];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
    bf16x8_t kop[4];
    const uint16_t *kp = ktile + (kb * 16 + kr) * kKRow + 32 * lq;
#pragma unroll
    for (int c = 0; c < 4; ++c) __builtin_memcpy(&kop[c], kp + 8 * c, 16);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      sacc[m][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c)
        sacc[m][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[c], qop[m][c], sacc[m][kb], 0, 0, 0);
    }
  }
  // ---- band edges: block 0 keeps k >= kr, block NB-1 keeps k <= W + kr
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int32_t k = 4 * lq + r;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      if (NB == 1) {
        sacc[m][0][r] = (k == kr) ? sacc[m][0][r] : -INFINITY;
      } else {
        sacc[m][0][r] = (k >= kr) ? sacc[m][0][r] : -INFINITY;
        sacc[m][NB - 1][r] = (k <= kr) ? sacc[m][NB - 1][r] : -INFINITY;
      }
    }
  }
  // ---- softmax (one chunk: no rescaling of acc needed)
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[m][kb][r]);
    const float m_new = wave_max_q(mx) * p.scale2;  // finite: every query sees its own key
    m_run[m] = m_new;
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[m][kb][r], p.scale2, -m_new));
        sacc[m][kb][r] = e;
        ps += e;
      }
    l_run[m] = ps;
  }
  // ---- O^T = V^T P^T over block pairs; V^T via transposing LDS reads
  const uint16_t *vrow = vtile + (4 * lq + (kr >> 2)) * kVRow + 4 * (kr & 3);
#pragma unroll
  for (int u = 0; u < (NB + 1) / 2; ++u) {
    constexpr int kLast = NB - 1;
    const bool second = 2 * u + 1 < NB;  // compile-time after unrolling
    const int kb1 = second ? 2 * u + 1 : kLast;
    bf16x8_t pop[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      uint32_t u4[4] = {pack_bf16x2_hw(sacc[m][2 * u][0], sacc[m][2 * u][1]),
                        pack_bf16x2_hw(sacc[m][2 * u][2], sacc[m][2 * u][3]),
                        second ? pack_bf16x2_hw(sacc[m][kb1][0], sacc[m][kb1][1]) : 0u,
                        second ? pack_bf16x2_hw(sacc[m][kb1][2], sacc[m][kb1][3]) : 0u};
      __builtin_memcpy(&pop[m], u4, 16);
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const i16x4_t lo = lds_read_tr16(vrow + (32 * u) * kVRow + 16 * n);
      i16x4_t hi = {0, 0, 0, 0};
      if (second) hi = lds_read_tr16(vrow + (32 * u + 16) * kVRow + 16 * n);
      const bf16x8_t vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int m = 0; m < MB; ++m)
        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[m], acc[m][n], 0, 0, 0);
    }
  }
}

template <int MB, bool OUT_BF16>
__global__ void __launch_bounds__(kNW * 64, 2) extend_kernel(ExtendParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kKB * 16 * kKRow];
  __shared__ __attribute__((aligned(16))) uint16_t vtile[kKB * 16 * kVRow];

  // ---- which tile: XCD-contiguous numbering of (request, kv head, query tile)
  const int32_t per_xcd = gridDim.x / 8;  // the grid is a multiple of 8
  int32_t t = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  int32_t b = 0;
  int32_t ntile = 0;
  for (; b < p.batch; ++b) {
    ntile = (new_count(p, b) + kTQ - 1) / kTQ;
    const int32_t tb = ntile * p.kv_heads;
    if (t < tb) break;
    t -= tb;
  }
  if (b >= p.batch) return;
  const int32_t g = t / ntile;
  const int32_t qt = t % ntile;

  const int32_t lane = threadIdx.x & 63;
  const int32_t w = threadIdx.x >> 6;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  const int32_t G = p.group;
  const int32_t W = p.window;

  const int32_t n_new = new_count(p, b);
  int32_t seq = p.seq_lens[b];
  if (seq > p.r2t_stride) seq = static_cast<int32_t>(p.r2t_stride);
  const int32_t prefix = p.prefix_lens[b];
  const int32_t row0 = p.qo_indptr[b] + qt * kTQ;      // first q row of the tile
  const int32_t i0 = prefix + qt * kTQ;                 // its position
  int32_t i_last = i0 + kTQ - 1;                        // last position of the tile
  if (i_last > prefix + n_new - 1) i_last = prefix + n_new - 1;
  if (i_last > seq - 1) i_last = seq - 1;
  int32_t kj0 = W < 0 ? 0 : i0 - W;                     // first key position of the band
  if (kj0 < 0) kj0 = 0;
  const int32_t nkeys = i_last >= kj0 ? i_last - kj0 + 1 : 0;

  // key position -> slot
  const int32_t *src = nullptr;
  int64_t src_hi = 0;  // valid index range into src: [0, src_hi)
  int32_t pos_base = 0;  // position of src[0]
  if (p.indptr) {
    int64_t lo = p.indptr[b], hi = p.indptr[b + 1];
    if (lo < 0) lo = 0;
    if (hi > p.capacity) hi = p.capacity;
    src = p.table + lo;
    src_hi = hi > lo ? hi - lo : 0;
    pos_base = W < 0 ? 0 : prefix - W;
    if (pos_base < 0) pos_base = 0;
  } else {
    int64_t row = p.req_idx[b];
    if (row < 0 || row >= p.r2t_rows) row = 0;
    src = p.r2t + row * p.r2t_stride;
    src_hi = p.r2t_stride;
  }

  // ---- Q^T operands: query kr of the tile, heads w*MB + m, dims 32lq..32lq+31.
  // Rows past the request (last partial tile) and padding heads read a real
  // row; their columns are never stored.
  const bool qvalid = (qt * kTQ + kr) < n_new && static_cast<int64_t>(row0) + kr < p.total_q;
  const int64_t qrow = qvalid ? static_cast<int64_t>(row0) + kr : static_cast<int64_t>(row0);
  bf16x8_t qop[MB][4];
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int32_t hh = w * MB + m;
    const uint4 *qp = reinterpret_cast<const uint4 *>(p.q + (qrow * p.q_heads + g * G + (hh < G ? hh : 0)) * kD +
                                                      32 * lq);
    uint4 raw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = qp[c];
#pragma unroll
    for (int c = 0; c < 4; ++c) __builtin_memcpy(&qop[m][c], &raw[c], 16);
  }

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
  const int32_t qpos = i0 + kr;  // position of the query in this lane's column

  // steady-state tile (see tile_fast): W = 128, 16 valid queries, band inside
  // the request and inside its key source
  const bool fast = W == 16 * (kKB - 1) && i0 - W >= 0 && qt * kTQ + kTQ <= n_new && i_last == i0 + kTQ - 1 &&
                    static_cast<int64_t>(kj0) - pos_base >= 0 &&
                    static_cast<int64_t>(kj0) - pos_base + 16 * kKB <= src_hi;
  if (fast) {
    tile_fast<kKB, MB>(p, ktile, vtile, qop, src + (kj0 - pos_base), g, acc, m_run, l_run);
  } else
  for (int32_t c0 = 0; c0 < nkeys; c0 += kKB * 16) {
    const int32_t nbk = min(kKB, (nkeys - c0 + 15) / 16);
    const int32_t chunk_pos = kj0 + c0;  // position of key 0 of the chunk

    // ---- stage K and V rows of the chunk in LDS (16 threads per 256-byte row).
    // Every thread issues all its loads before writing any (no control flow
    // between loads); keys past the band re-read the chunk's first key and are
    // zeroed when written to LDS.
    __syncthreads();  // previous chunk fully consumed
    {
      const int32_t piece = threadIdx.x & 15;
      int32_t slot[kKB];
      if (src_hi > 0) {  // workgroup-uniform
#pragma unroll
        for (int i = 0; i < kKB; ++i) {
          const int32_t key = (threadIdx.x >> 4) + 16 * i;
          const bool kv_ok = i < nbk && c0 + key < nkeys;
          const int64_t si = static_cast<int64_t>(chunk_pos + (kv_ok ? key : 0)) - pos_base;
          slot[i] = src[si >= 0 && si < src_hi ? si : 0];
        }
      } else {
#pragma unroll
        for (int i = 0; i < kKB; ++i) slot[i] = 0;
      }
      int64_t off[kKB];
#pragma unroll
      for (int i = 0; i < kKB; ++i) {
        const int64_t sl = (slot[i] < 0 || slot[i] >= p.rows) ? 0 : static_cast<int64_t>(slot[i]);
        off[i] = row_elem(sl, p.kv_heads, g, kD) + 8 * piece;
      }
      uint4 kreg[kKB], vreg[kKB];
#pragma unroll
      for (int i = 0; i < kKB; ++i) kreg[i] = *reinterpret_cast<const uint4 *>(p.k + off[i]);
#pragma unroll
      for (int i = 0; i < kKB; ++i) vreg[i] = *reinterpret_cast<const uint4 *>(p.v + off[i]);
#pragma unroll
      for (int i = 0; i < kKB; ++i) {
        const int32_t key = (threadIdx.x >> 4) + 16 * i;
        const bool kv_ok = i < nbk && c0 + key < nkeys;
        const uint4 kz = kv_ok ? kreg[i] : make_uint4(0, 0, 0, 0);
        const uint4 vz = kv_ok ? vreg[i] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(ktile + key * kKRow + 8 * piece) = kz;
        *reinterpret_cast<uint4 *>(vtile + key * kVRow + 8 * piece) = vz;
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
        const uint16_t *kp = ktile + (kb * 16 + kr) * kKRow + 32 * lq;
#pragma unroll
        for (int c = 0; c < 4; ++c) __builtin_memcpy(&kop[c], kp + 8 * c, 16);
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            sacc[m][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[c], qop[m][c], sacc[m][kb], 0, 0, 0);
      }
    }

    // ---- mask: only blocks that touch the band's edges or the chunk end need
    // a per-key test (a block is inside the band for every query of the tile
    // when its last key <= i0 and its first key >= i_last - W).
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const int32_t j0 = chunk_pos + kb * 16;
      const bool interior = kb < nbk && c0 + kb * 16 + 15 < nkeys && j0 + 15 <= i0 && (W < 0 || j0 >= i_last - W);
      if (!interior) {  // workgroup-uniform
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t j = j0 + 4 * lq + r;
          const bool ok = kb < nbk && (c0 + kb * 16 + 4 * lq + r) < nkeys && j <= qpos && (W < 0 || j >= qpos - W);
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
      float ps = 0.f;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[m][kb][r], p.scale2, -m_new));
          sacc[m][kb][r] = e;
          ps += e;
        }
      l_run[m] = l_run[m] * alpha + ps;
      if (c0 > 0) {
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] *= alpha;
      }
    }

    // ---- O^T += V^T P^T over block pairs (2u, 2u+1).  The V^T operand comes
    // straight from the row-major tile with transposing LDS reads: lane (kr, lq)
    // gets V[4lq + e][16n + kr], e = 0..3, of each block of the pair.
    const uint16_t *vrow = vtile + (4 * lq + (kr >> 2)) * kVRow + 4 * (kr & 3);
#pragma unroll
    for (int u = 0; u < (kKB + 1) / 2; ++u) {
      if (2 * u < nbk) {
        const bool second = 2 * u + 1 < nbk;
        bf16x8_t pop[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
          const int kb1 = (2 * u + 1) < kKB ? 2 * u + 1 : 2 * u;
          uint32_t u4[4] = {pack_bf16x2_hw(sacc[m][2 * u][0], sacc[m][2 * u][1]),
                            pack_bf16x2_hw(sacc[m][2 * u][2], sacc[m][2 * u][3]),
                            second ? pack_bf16x2_hw(sacc[m][kb1][0], sacc[m][kb1][1]) : 0u,
                            second ? pack_bf16x2_hw(sacc[m][kb1][2], sacc[m][kb1][3]) : 0u};
          __builtin_memcpy(&pop[m], u4, 16);
        }
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          i16x4_t lo = lds_read_tr16(vrow + (32 * u) * kVRow + 16 * n);
          i16x4_t hi = {0, 0, 0, 0};
          if (second) hi = lds_read_tr16(vrow + (32 * u + 16) * kVRow + 16 * n);
          bf16x8_t vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
          for (int m = 0; m < MB; ++m)
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[m], acc[m][n], 0, 0, 0);
        }
      }
    }
  }

  // ---- finalize: sink once, normalise, store
#pragma unroll
  for (int m = 0; m < MB; ++m) {
    const int32_t hh = w * MB + m;
    const float l = wave_sum_q(l_run[m]);
    if (hh >= G || !qvalid) continue;
    const int32_t h = g * G + hh;
    float M = m_run[m];
    float L = l;
    if (p.sinks) {
      const float sig2 = p.sinks[h] * kLog2e;
      const float Mn = fmaxf(M, sig2);
      L = L * exp2f(M - Mn) + exp2f(sig2 - Mn);
      const float a = exp2f(M - Mn);
#pragma unroll
      for (int n = 0; n < 8; ++n) acc[m][n] *= a;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int64_t obase = ((static_cast<int64_t>(row0) + kr) * p.q_heads + h) * kD + 4 * lq;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const float o0 = acc[m][n][0] * inv, o1 = acc[m][n][1] * inv, o2 = acc[m][n][2] * inv,
                  o3 = acc[m][n][3] * inv;
      if (OUT_BF16) {
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + obase + 16 * n) =
            make_uint2(pack_bf16x2_hw(o0, o1), pack_bf16x2_hw(o2, o3));
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + obase + 16 * n) = make_float4(o0, o1, o2, o3);
      }
    }
  }
}

template <int MB>
hipError_t launch_mb(const ExtendParams &p, uint32_t grid, bool out_bf16, hipStream_t stream) {
  if (out_bf16)
    hipLaunchKernelGGL((extend_kernel<MB, true>), dim3(grid), dim3(kNW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((extend_kernel<MB, false>), dim3(grid), dim3(kNW * 64), 0, stream, p);
  return hipGetLastError();
}

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
  p.sinks = a.sinks;
  p.scale2 = a.sm_scale * kLog2e;
  p.out = a.out;
  // Upper bound of the tile count: every request adds at most one partial tile.
  int64_t tiles = ((a.total_q + kTQ - 1) / kTQ + a.idx.batch) * a.layer.kv_heads;
  tiles = (tiles + 7) / 8 * 8;
  if (tiles > 0x7FFFFFF8LL) return hipErrorInvalidValue;
  const bool out_bf16 = a.out_dtype == SWA_BF16;
  const int32_t mb = p.group >= 16 ? 4 : (p.group >= 8 ? 2 : 1);
  if (mb == 4) return launch_mb<4>(p, static_cast<uint32_t>(tiles), out_bf16, stream);
  if (mb == 2) return launch_mb<2>(p, static_cast<uint32_t>(tiles), out_bf16, stream);
  return launch_mb<1>(p, static_cast<uint32_t>(tiles), out_bf16, stream);
}

}  // namespace swa
