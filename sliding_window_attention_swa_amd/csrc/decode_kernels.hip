// Windowed decode attention over a paged pool (one query per request).
//
// What is computed (SWA note, zdszero.github.io/swa.html: opening paragraph —
// each query attends to the most recent window; section 实现 — the configured
// window excludes the current token and -1 means full attention; section 设计 —
// a learnable per-head sink logit):
//   query position i = seq_len - 1, keys j in [max(0, i - W), i]
//   s_j = sm_scale * q_h . k_j       (kv head g = h / G)
//   o_h = sum_j e^{s_j - m} v_j / (sum_j e^{s_j - m} + e^{sink_h - m})
//
// Work decomposition (MI355X-specific, not the pages' kernels):
//   * the G query heads that share a kv head are always computed together, so
//     each K/V row is read from HBM exactly once per layer;
//   * window layers (one split): one workgroup per (kv head, request); its
//     four wavefronts take 16-key blocks of the window, all loads in flight
//     at once, and are merged through LDS;
//   * full layers (split-K): one workgroup per (key split, four kv heads,
//     request), one wavefront per kv head streaming its split with a two-deep
//     load pipeline, so a workgroup reads whole token rows page by page; each
//     wavefront writes its (max, sum, acc) partial and a merge kernel
//     combines the splits;
//   * online softmax in base 2; the sink enters exactly once, where the final
//     normalisation happens.
//
// bf16 / e4m3 K/V path: S^T = K Q^T (v_mfma_f32_16x16x32_bf16) and
// O^T = V^T P^T (v_mfma_f32_16x16x32_f16, P rounded to f16) on the CDNA4
// matrix cores.  With keys as the M dimension of the
// first product, its accumulator layout (lane = head column, 4 keys per lane)
// is exactly the B-operand layout the second product needs for P^T, so P
// never leaves registers.  The head dimension is permuted identically in Q and
// K so that each load instruction reads whole runs of K rows (the four lane
// groups of a key read neighbouring 16-byte pieces).  V is staged through LDS
// (whole rows per load instruction, padded LDS rows, conflict-free transposed
// reads with ds_read_b64_tr_b16) because the key index must be the per-lane
// contraction index of the second product; it is converted to f16 on the way
// (exact for bf16 values of magnitude 2^-14 .. 65504).  e4m3 K bytes are
// widened to bf16 and e4m3 V bytes to f16, both exactly; the per-tensor scales
// are folded into the logit scale and the output.
//
// f32 path: plain VALU; 16 keys per wavefront step, 4 lanes per key row.
#include <mutex>

#include "common.hpp"

namespace swa {
namespace {

// Split-K partials of swa_decode_noalloc: a static device array of
// kStaticScratchBytes on every GPU the library runs on, held until the process
// ends.  Host code never uses its name as an address: it reads the array's
// device address with hipGetSymbolAddress (static_scratch below).
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kD = 128;           // head_dim handled by these kernels
constexpr int kMaxG = 16;         // q heads per kv head (MFMA N = 16)

struct DecodeParams {
  const void *q;
  const void *k;
  const void *v;
  int64_t rows;
  int32_t kv_heads;
  int32_t q_heads;
  int32_t group;
  float k_scale;
  float v_scale;
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
  float scale2;  // sm_scale * k_scale * log2(e)
  void *out;
  int32_t num_splits;
  float *ws_m;
  float *ws_l;
  float *ws_acc;
  // fused store of the current token (window kernel only): bf16 rows
  // (batch, kv_heads, head_dim) and their pool slots
  const uint16_t *k_new;
  const uint16_t *v_new;
  const int64_t *new_loc;
};

// Keys of request b for this layer, as [first, first + n) of either the window
// table (table mode) or positions of the request row (req_to_token mode).
struct KeySource {
  const int32_t *src;  // slot of key k is src[k]
  int32_t n;
};

__device__ __forceinline__ KeySource key_source(const DecodeParams &p, int32_t b) {
  KeySource ks{p.table, 0};
  if (p.indptr) {
    int64_t lo = p.indptr[b];
    int64_t hi = p.indptr[b + 1];
    if (lo < 0) lo = 0;
    if (hi > p.capacity) hi = p.capacity;
    ks.src = p.table + lo;
    ks.n = hi > lo ? static_cast<int32_t>(hi - lo) : 0;
    return ks;
  }
  int32_t L = p.seq_lens[b];
  if (L > p.r2t_stride) L = static_cast<int32_t>(p.r2t_stride);
  if (L <= 0) {
    ks.src = p.r2t;
    return ks;
  }
  const int32_t i = L - 1;
  int32_t lo = p.window < 0 ? 0 : i - p.window;
  if (lo < 0) lo = 0;
  int64_t row = p.req_idx[b];
  if (row < 0 || row >= p.r2t_rows) row = 0;
  ks.src = p.r2t + row * p.r2t_stride + lo;
  ks.n = L - lo;
  return ks;
}

__device__ __forceinline__ int64_t safe_slot(int32_t s, int64_t rows) {
  return (s < 0 || s >= rows) ? 0 : static_cast<int64_t>(s);
}

__device__ __forceinline__ float wave_max_q(float x) { return rows_max(x); }  // lanes l, l^16, l^32, l^48
__device__ __forceinline__ float wave_sum_q(float x) { return rows_sum(x); }
__device__ __forceinline__ float wave_sum_all(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Split of request keys handled by workgroup `s`: a multiple of 16 keys.
__device__ __forceinline__ void split_range(int32_t n, int32_t s, int32_t splits, int32_t *k0, int32_t *k1) {
  int32_t per = (n + splits - 1) / splits;
  per = (per + 15) & ~15;
  int32_t a = s * per;
  int32_t e = a + per;
  if (a > n) a = n;
  if (e > n) e = n;
  *k0 = a;
  *k1 = e;
}

// --------------------------------------------------------------------------
// Shared epilogue: combine NW wavefront partials held in LDS and either write
// the final output (one split) or this split's partial to the workspace.
// red_m / red_l: [NW][kMaxG] (base-2 logit domain); red_acc: [NW][G][kD].
// --------------------------------------------------------------------------
template <bool OUT_BF16>
__device__ void merge_waves_and_store(const DecodeParams &p, int NW, const float *red_m, const float *red_l,
                                      const float *red_acc, int32_t b, int32_t g, int32_t s) {
  const int32_t G = p.group;
  const bool final = p.num_splits == 1;
  // each thread produces 4 consecutive dims of one head
  for (int32_t t = threadIdx.x; t < G * (kD / 4); t += blockDim.x) {
    const int32_t hh = t / (kD / 4);
    const int32_t d4 = (t % (kD / 4)) * 4;
    const int32_t h = g * G + hh;
    float M = kNegBig;
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w * kMaxG + hh]);
    float sig2 = -INFINITY;
    if (final && p.sinks) {
      sig2 = p.sinks[h] * kLog2e;
      M = fmaxf(M, sig2);
    }
    float L = 0.f;
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    for (int w = 0; w < NW; ++w) {
      const float a = exp2f(red_m[w * kMaxG + hh] - M);
      L += red_l[w * kMaxG + hh] * a;
      const float4 v = *reinterpret_cast<const float4 *>(red_acc + (w * G + hh) * kD + d4);
      o0 += v.x * a;
      o1 += v.y * a;
      o2 += v.z * a;
      o3 += v.w * a;
    }
    if (final) {
      if (p.sinks) L += exp2f(sig2 - M);
      const float inv = L > 0.f ? p.v_scale / L : 0.f;
      o0 *= inv;
      o1 *= inv;
      o2 *= inv;
      o3 *= inv;
      const int64_t off = (static_cast<int64_t>(b) * p.q_heads + h) * kD + d4;
      if (OUT_BF16) {
        uint2 pk = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + off) = pk;
      } else {
        *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + off) = make_float4(o0, o1, o2, o3);
      }
    } else {
      const int64_t pi = (static_cast<int64_t>(b) * p.q_heads + h) * p.num_splits + s;
      if (d4 == 0) {
        p.ws_m[pi] = M;
        p.ws_l[pi] = L;
      }
      *reinterpret_cast<float4 *>(p.ws_acc + pi * kD + d4) = make_float4(o0, o1, o2, o3);
    }
  }
}

// --------------------------------------------------------------------------
// MFMA path (bf16 q; bf16 or e4m3 K/V)
// --------------------------------------------------------------------------
template <typename KV>
struct KvLoad;

template <>
struct KvLoad<uint16_t> {  // bf16: the four 16-B K loads are the four contraction blocks
  __device__ static void to_bf16(const uint4 *raw, bf16x8_t *ops) {
#pragma unroll
    for (int c = 0; c < 4; ++c) __builtin_memcpy(&ops[c], &raw[c], 16);
  }
};

template <>
struct KvLoad<uint8_t> {  // e4m3: each 16-B K load widens (exactly) to two contraction blocks
  __device__ static void to_bf16(const uint4 *raw, bf16x8_t *ops) {
    uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w, raw[1].x, raw[1].y, raw[1].z, raw[1].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * c], 1.0f, false);
      bf16x2_t bq = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * c], 1.0f, true);
      bf16x2_t cc = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * c + 1], 1.0f, false);
      bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * c + 1], 1.0f, true);
      uint32_t u[4];
      __builtin_memcpy(&u[0], &a, 4);
      __builtin_memcpy(&u[1], &bq, 4);
      __builtin_memcpy(&u[2], &cc, 4);
      __builtin_memcpy(&u[3], &d, 4);
      __builtin_memcpy(&ops[c], u, 16);
    }
  }
};

// Global-load layouts.  K rows feed S^T = K Q^T straight from registers: for
// contraction block c (32 dims) lane (key kr, group lq) holds 8 dims of key kr
// (an MFMA operand needs them in one lane).  Which 8 dims is our choice (Q is
// permuted identically); it is made so that in every load instruction the
// four lane groups of one key read one contiguous run of its row, i.e. the
// loads are row-coalesced.  V rows only pass through LDS, so they are read
// 16 B per lane with each row covered by neighbouring lanes (16 lanes per
// bf16 row, 8 per e4m3 row): every instruction reads whole rows.
template <typename KV>
struct Layout;

template <>
struct Layout<uint16_t> {
  static constexpr int kKLoads = 4;  // 16-B K loads per key per lane
  static constexpr int kVLoads = 4;  // 16-B V loads per 16-key block per lane
  __device__ static int k_off(int c, int lq) { return 32 * c + 8 * lq; }   // element offset of K load c
  __device__ static int qk_dim(int c, int lq) { return 32 * c + 8 * lq; }  // dims of contraction block c
  __device__ static int v_key(int j, int lane) { return 4 * j + (lane >> 4); }
  __device__ static int v_off(int lane) { return 8 * (lane & 15); }
};

template <>
struct Layout<uint8_t> {
  static constexpr int kKLoads = 2;  // one 16-B load = 16 dims = two contraction blocks
  static constexpr int kVLoads = 2;
  __device__ static int k_off(int c, int lq) { return 64 * c + 16 * lq; }
  __device__ static int qk_dim(int c, int lq) { return 64 * (c >> 1) + 16 * lq + 8 * (c & 1); }
  __device__ static int v_key(int j, int lane) { return 8 * j + (lane >> 3); }
  __device__ static int v_off(int lane) { return 16 * (lane & 7); }
};

constexpr int kSVRow = kD + 16;  // LDS V row: 288 bytes (transposed reads are conflict-free)

// Q^T operand of head h for lane group lq, in the contraction order of Layout<KV>.
template <typename KV>
__device__ __forceinline__ void load_q(const DecodeParams &p, int32_t b, int32_t h, int32_t lq, uint4 (&qraw)[4]) {
  const uint16_t *qrow = static_cast<const uint16_t *>(p.q) + (static_cast<int64_t>(b) * p.q_heads + h) * kD;
#pragma unroll
  for (int c = 0; c < 4; ++c) qraw[c] = *reinterpret_cast<const uint4 *>(qrow + Layout<KV>::qk_dim(c, lq));
}

// The K loads of one key row (slot) for lane group lq.
template <typename KV>
__device__ __forceinline__ void load_k(const DecodeParams &p, int32_t slot, int32_t g, int32_t lq,
                                       uint4 (&raw)[Layout<KV>::kKLoads]) {
  const KV *row = static_cast<const KV *>(p.k) + row_elem(safe_slot(slot, p.rows), p.kv_heads, g, kD);
#pragma unroll
  for (int c = 0; c < Layout<KV>::kKLoads; ++c)
    raw[c] = *reinterpret_cast<const uint4 *>(row + Layout<KV>::k_off(c, lq));
}

// The V loads of one 16-key block whose slots are held by lanes 0..15 (lane
// kr holds the slot of key kr in `slot`).
template <typename KV>
__device__ __forceinline__ void load_v(const DecodeParams &p, int32_t slot, int32_t g, int32_t lane,
                                       uint4 (&raw)[Layout<KV>::kVLoads]) {
#pragma unroll
  for (int j = 0; j < Layout<KV>::kVLoads; ++j) {
    const int32_t s = __shfl(slot, Layout<KV>::v_key(j, lane));
    const KV *row = static_cast<const KV *>(p.v) + row_elem(safe_slot(s, p.rows), p.kv_heads, g, kD);
    raw[j] = *reinterpret_cast<const uint4 *>(row + Layout<KV>::v_off(lane));
  }
}

// 16 e4m3 bytes -> 16 f16 (exact: every e4m3 value, subnormals included, is
// an f16 normal).
__device__ __forceinline__ void fp8x16_to_f16(const uint4 &x, uint4 (&out)[2]) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t u[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f16x2v_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, false);
    f16x2v_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[i], 1.0f, true);
    __builtin_memcpy(&u[2 * i], &a, 4);
    __builtin_memcpy(&u[2 * i + 1], &c, 4);
  }
  out[0] = make_uint4(u[0], u[1], u[2], u[3]);
  out[1] = make_uint4(u[4], u[5], u[6], u[7]);
}

// This lane's raw bf16 pieces of request b's new K and V rows (kv head g), in
// the lane layout of Layout<KV> (bf16 pieces as they are; each e4m3 piece from
// two bf16 pieces).
template <typename KV>
__device__ __forceinline__ void load_new_rows(const DecodeParams &p, int32_t b, int32_t g, int32_t lane,
                                              uint4 (&kn_raw)[4], uint4 (&vn_raw)[2]) {
  const int32_t lq = lane >> 4;
  const uint16_t *krow = p.k_new + (static_cast<int64_t>(b) * p.kv_heads + g) * kD;
  const uint16_t *vrow = p.v_new + (static_cast<int64_t>(b) * p.kv_heads + g) * kD;
  if constexpr (sizeof(KV) == 2) {
#pragma unroll
    for (int c = 0; c < 4; ++c) kn_raw[c] = *reinterpret_cast<const uint4 *>(krow + Layout<KV>::k_off(c, lq));
    vn_raw[0] = *reinterpret_cast<const uint4 *>(vrow + Layout<KV>::v_off(lane));
  } else {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      kn_raw[2 * c] = *reinterpret_cast<const uint4 *>(krow + Layout<KV>::k_off(c, lq));
      kn_raw[2 * c + 1] = *reinterpret_cast<const uint4 *>(krow + Layout<KV>::k_off(c, lq) + 8);
    }
    vn_raw[0] = *reinterpret_cast<const uint4 *>(vrow + Layout<KV>::v_off(lane));
    vn_raw[1] = *reinterpret_cast<const uint4 *>(vrow + Layout<KV>::v_off(lane) + 8);
  }
}

// Component-wise select (a ternary on the vector struct goes through memory).
__device__ __forceinline__ uint4 sel4(bool c, const uint4 &a, const uint4 &b) {
  return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
}

// 16 bf16 -> 16 e4m3 bytes (nearest even, saturating; the pool encoding).
__device__ __forceinline__ uint4 bf16x16_to_fp8(const uint4 &lo, const uint4 &hi) {
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint16_t h = static_cast<uint16_t>(w[e >> 1] >> ((e & 1) * 16));
    o[e >> 2] |= static_cast<uint32_t>(f32_to_e4m3_rne(bf16_to_f32(h))) << ((e & 3) * 8);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// This lane's pieces of the new token's K / V head rows in the pool format,
// from their raw bf16 pieces (loaded per Layout<KV>: bf16 pieces as they are,
// each e4m3 piece from two bf16 pieces).
template <typename KV>
__device__ __forceinline__ void new_pieces(const uint4 (&kn_raw)[4], const uint4 (&vn_raw)[2],
                                           uint4 (&knew)[Layout<KV>::kKLoads], uint4 &vnew) {
  if constexpr (sizeof(KV) == 2) {
#pragma unroll
    for (int c = 0; c < 4; ++c) knew[c] = kn_raw[c];
    vnew = vn_raw[0];
  } else {
#pragma unroll
    for (int c = 0; c < 2; ++c) knew[c] = bf16x16_to_fp8(kn_raw[2 * c], kn_raw[2 * c + 1]);
    vnew = bf16x16_to_fp8(vn_raw[0], vn_raw[1]);
  }
}

// One block's V rows into its 16-row LDS tile as f16 (the P.V operand type;
// kSVRow stride); rows of keys at or past k_end are written as zeros (their
// slots may hold anything).
template <typename KV>
__device__ __forceinline__ void v_to_lds(const uint4 (&raw)[Layout<KV>::kVLoads], uint16_t *tile, int32_t lane,
                                         int32_t key_base, int32_t k_end) {
#pragma unroll
  for (int j = 0; j < Layout<KV>::kVLoads; ++j) {
    const int32_t key = Layout<KV>::v_key(j, lane);
    const bool ok = key_base + key < k_end;
    uint4 *d = reinterpret_cast<uint4 *>(tile + key * kSVRow + Layout<KV>::v_off(lane));
    if constexpr (sizeof(KV) == 2) {
      d[0] = ok ? bf16x8_to_f16x8(raw[j]) : make_uint4(0, 0, 0, 0);
    } else {
      uint4 w2[2];
      fp8x16_to_f16(raw[j], w2);
      d[0] = ok ? w2[0] : make_uint4(0, 0, 0, 0);
      d[1] = ok ? w2[1] : make_uint4(0, 0, 0, 0);
    }
  }
}

// O^T += V^T P^T for a pair of 16-key blocks whose rows start at `pair` in the
// LDS tile (the second block absent when !SECOND); pop holds P^T of the pair.
template <bool SECOND>
__device__ __forceinline__ void pv_pair(const uint16_t *pair, int32_t kr, int32_t lq, const bf16x8_t &pop,
                                        f32x4_t (&acc)[8]) {
  const uint16_t *vrow = pair + (4 * lq + (kr >> 2)) * kSVRow + 4 * (kr & 3);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const i16x4_t lo = lds_read_tr16(vrow + 16 * c);
    const i16x4_t hi = SECOND ? lds_read_tr16(vrow + 16 * kSVRow + 16 * c) : i16x4_t{0, 0, 0, 0};
    const bf16x8_t vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    acc[c] = mfma_f16(vop, pop, acc[c]);
  }
}

// O^T += V^T P^T for one 16-key block whose rows start at `blk` in the LDS
// tile (16x16x16 MFMA); pop holds P^T of the block (keys 4lq..4lq+3, head kr).
__device__ __forceinline__ void pv_single(const uint16_t *blk, int32_t kr, int32_t lq, const i16x4_t &pop,
                                          f32x4_t (&acc)[8]) {
  const uint16_t *vrow = blk + (4 * lq + (kr >> 2)) * kSVRow + 4 * (kr & 3);
  f16x4v_t b;
  __builtin_memcpy(&b, &pop, 8);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const i16x4_t v = lds_read_tr16(vrow + 16 * c);
    f16x4v_t a;
    __builtin_memcpy(&a, &v, 8);
    acc[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, acc[c], 0, 0, 0);
  }
}

// Streaming kernel (long key ranges: full layers, split-K).  Each wavefront
// walks the blocks w, w+4, w+8, ... of its workgroup's key range (the four
// wavefronts read neighbouring blocks at the same time), two blocks per round,
// in a two-stage software pipeline: the slots of round r+2 and the K/V rows of
// round r+1 are in flight while round r is computed.  All loads are
// unconditional (keys past the range re-read the range's first key and are
// masked).  V goes through a per-wavefront LDS tile and is read back with the
// transposing ds_read_b64_tr_b16, so P^T and V^T never need register shuffles.
constexpr int kStreamWaves = 4;

template <typename KV>
struct StreamRound {
  uint4 k[2][Layout<KV>::kKLoads];
  uint4 v[2][Layout<KV>::kVLoads];
};

template <typename KV>
__device__ __forceinline__ void stream_issue(const DecodeParams &p, const int32_t (&sl)[2], int32_t g, int32_t lane,
                                             StreamRound<KV> &r) {
#pragma unroll
  for (int u = 0; u < 2; ++u) load_k<KV>(p, sl[u], g, lane >> 4, r.k[u]);
#pragma unroll
  for (int u = 0; u < 2; ++u) load_v<KV>(p, sl[u], g, lane, r.v[u]);
}

template <typename KV>
__device__ __forceinline__ void stream_compute(const DecodeParams &p, const StreamRound<KV> &r, int32_t key_base0,
                                               int32_t key_base1, int32_t k1, const bf16x8_t (&qop)[4], uint16_t *vt,
                                               int32_t lane, f32x4_t (&acc)[8], float &m_run, float &l_run) {
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  // S^T for the two blocks (lane: keys 4lq..4lq+3 of head kr)
  float sc[2][4];
  float mb = -INFINITY;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    bf16x8_t kk[4];
    KvLoad<KV>::to_bf16(r.k[u], kk);
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[c], qop[c], sacc, 0, 0, 0);
    const int32_t kb = u == 0 ? key_base0 : key_base1;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      sc[u][rr] = (kb + 4 * lq + rr < k1) ? sacc[rr] : -INFINITY;
      mb = fmaxf(mb, sc[u][rr]);
    }
  }
  // V rows -> LDS (bf16): block u at rows 16u..16u+15
  v_to_lds<KV>(r.v[0], vt, lane, key_base0, k1);
  v_to_lds<KV>(r.v[1], vt + 16 * kSVRow, lane, key_base1, k1);
  // online softmax (base 2, scale folded into the exponent)
  const float m_new = fmaxf(m_run, wave_max_q(mb) * p.scale2);
  const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
  m_run = m_new;
  float pv[8];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    pv[rr] = __builtin_amdgcn_exp2f(fmaf(sc[0][rr], p.scale2, -m_new));
    pv[4 + rr] = __builtin_amdgcn_exp2f(fmaf(sc[1][rr], p.scale2, -m_new));
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] *= alpha;
  bf16x8_t pop;
  {
    uint32_t u4[4] = {pack_f16x2_hw(pv[0], pv[1]), pack_f16x2_hw(pv[2], pv[3]), pack_f16x2_hw(pv[4], pv[5]),
                      pack_f16x2_hw(pv[6], pv[7])};
    // the normaliser sums the rounded weights that enter P.V
    l_run = f16x2_acc(u4[3], f16x2_acc(u4[2], f16x2_acc(u4[1], f16x2_acc(u4[0], l_run * alpha))));
    __builtin_memcpy(&pop, u4, 16);
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's V rows are in LDS
  __builtin_amdgcn_wave_barrier();
  pv_pair<true>(vt, kr, lq, pop, acc);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next round rewrites the tile
}

// One workgroup per (key split, group of up to 4 kv heads, request): wavefront
// w handles kv head 4 * blockIdx.y + w over the whole split, so the four
// wavefronts together read whole token rows (all kv heads of a slot are
// contiguous) and each page of the paged pool is visited once per split.
// A wavefront owns its heads completely: it writes its split partial (or,
// with one split, the final output with the sink) without any LDS merge.
template <typename KV, bool OUT_BF16>
__global__ void __launch_bounds__(kStreamWaves * 64, 1) decode_stream_kernel(DecodeParams p) {
  constexpr int NW = kStreamWaves;
  __shared__ __attribute__((aligned(16))) uint16_t vtiles[NW * 32 * kSVRow];

  const int32_t s = blockIdx.x;
  const int32_t b = blockIdx.z;
  const int32_t lane = threadIdx.x & 63;
  const int32_t w = threadIdx.x >> 6;
  const int32_t g = blockIdx.y * NW + w;
  if (g >= p.kv_heads) return;  // wave-uniform; no workgroup barrier below
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  const int32_t G = p.group;

  const KeySource ks = key_source(p, b);
  int32_t k0, k1;
  split_range(ks.n, s, p.num_splits, &k0, &k1);
  const int32_t nblk = (k1 - k0 + 15) >> 4;
  const int32_t nround = (nblk + 1) / 2;

  uint4 qraw[4];
  load_q<KV>(p, b, g * G + (kr < G ? kr : 0), lq, qraw);

  f32x4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig;
  float l_run = 0.f;
  uint16_t *vt = vtiles + w * 32 * kSVRow;

  if (nround > 0) {
    auto key_of = [&](int32_t j) { return k0 + 16 * j; };
    auto slots_of = [&](int32_t round, int32_t (&sl)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int32_t key = key_of(2 * round + u) + kr;
        sl[u] = ks.src[key < k1 ? key : k0];
      }
    };
    bf16x8_t qop[4];
    KvLoad<uint16_t>::to_bf16(qraw, qop);
    // Loads retire in issue order, so a wait for a round's slots also waits
    // for everything issued before them.  Each step therefore loads the slots
    // of the round after next before it issues the next round's K/V rows: the
    // wait for those slots, one step later, leaves that round's rows in flight
    // (two rounds of rows in flight per wavefront).  Both are issued
    // unconditionally (past the split's end, slots_of gives every lane the
    // split's first key, so such a round re-reads one cached row): under a
    // branch, each round's waits would also wait for the loads issued after.
    int32_t slA[2], slB[2];
    StreamRound<KV> A, B;
    slots_of(0, slA);
    slots_of(1, slB);
    __builtin_amdgcn_sched_barrier(0);
    stream_issue<KV>(p, slA, g, lane, A);
    __builtin_amdgcn_sched_barrier(0);
    for (int32_t r = 0; r < nround; r += 2) {
      slots_of(r + 2, slA);
      __builtin_amdgcn_sched_barrier(0);
      stream_issue<KV>(p, slB, g, lane, B);
      __builtin_amdgcn_sched_barrier(0);
      stream_compute<KV>(p, A, key_of(2 * r), key_of(2 * r + 1), k1, qop, vt, lane, acc, m_run, l_run);
      if (r + 1 >= nround) break;
      slots_of(r + 3, slB);
      __builtin_amdgcn_sched_barrier(0);
      stream_issue<KV>(p, slA, g, lane, A);
      __builtin_amdgcn_sched_barrier(0);
      stream_compute<KV>(p, B, key_of(2 * r + 2), key_of(2 * r + 3), k1, qop, vt, lane, acc, m_run, l_run);
    }
  }
  l_run = wave_sum_q(l_run);
  if (kr >= G) return;
  const int32_t h = g * G + kr;
  if (p.num_splits == 1) {
    float M = m_run, L = l_run, a = 1.f;
    if (p.sinks) {
      const float sig2 = p.sinks[h] * kLog2e;
      const float Mn = fmaxf(M, sig2);
      a = __builtin_amdgcn_exp2f(M - Mn);
      L = L * a + __builtin_amdgcn_exp2f(sig2 - Mn);
    }
    const float inv = L > 0.f ? a * p.v_scale / L : 0.f;
    const int64_t off = (static_cast<int64_t>(b) * p.q_heads + h) * kD + 4 * lq;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float o0 = acc[c][0] * inv, o1 = acc[c][1] * inv, o2 = acc[c][2] * inv, o3 = acc[c][3] * inv;
      if (OUT_BF16)
        *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + off + 16 * c) =
            make_uint2(pack_bf16x2_hw(o0, o1), pack_bf16x2_hw(o2, o3));
      else
        *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + off + 16 * c) = make_float4(o0, o1, o2, o3);
    }
  } else {
    const int64_t pi = (static_cast<int64_t>(b) * p.q_heads + h) * p.num_splits + s;
    if (lq == 0) {
      p.ws_m[pi] = m_run;
      p.ws_l[pi] = l_run;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c)
      *reinterpret_cast<float4 *>(p.ws_acc + pi * kD + 16 * c + 4 * lq) =
          make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
  }
}

// --------------------------------------------------------------------------
// Window kernel (SWA layers, one split).  The window's 16-key blocks are dealt
// to 4 wavefronts, at most MAXB blocks each (3 at W = 128), and every K/V row
// of the window is requested before any arithmetic starts: the registers of a
// CU (512 KB) hold far more bytes in flight than its LDS, so the whole batch is
// resident in one round and the kernel is one dependent chain deep:
//   slot table -> K/V rows -> MFMA -> wavefront merge -> output.
// (Plain loads: measured on MI355X, non-temporal loads made this gather ~50%
// slower.)
// --------------------------------------------------------------------------
constexpr int kWinWaves = 4;

// Workgroup -> (kv head g, request b) of the window kernel (grid: 1 x kv heads x
// requests).  Workgroups go to the 8 XCDs round-robin by linear id, so with the
// plain mapping (id = g + kv_heads * b) and 8 kv heads, XCD g would read only
// head g's piece of every token row.  When the batch is a multiple of 8 the ids
// are relabelled so that XCD x serves every kv head of requests x, x + 8, ...
// and reads whole token rows (measured about 1.5% faster on a 64-request batch).
__device__ __forceinline__ void window_item(int32_t &g, int32_t &b) {
  const int32_t H = static_cast<int32_t>(gridDim.y);
  g = static_cast<int32_t>(blockIdx.y);
  b = static_cast<int32_t>(blockIdx.z);
  if ((gridDim.z & 7u) == 0) {
    const int32_t i = g + H * b;  // linear id (gridDim.x == 1)
    const int32_t j = i >> 3;
    g = j % H;
    b = (i & 7) + 8 * (j / H);
  }
}

template <typename KV, int MAXB, bool OUT_BF16, bool FUSED>
__global__ void __launch_bounds__(kWinWaves * 64) decode_window_kernel(DecodeParams p) {
  // each wavefront stages one pair of blocks (32 V rows) at a time
  constexpr int NW = kWinWaves;
  constexpr int kStageRows = 32;
  constexpr int kTileBytes = NW * kStageRows * kSVRow * 2;
  constexpr int kRedBytes = NW * kMaxG * kD * 4;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kTileBytes > kRedBytes ? kTileBytes : kRedBytes];
  __shared__ float red_m[NW * kMaxG];
  __shared__ float red_l[NW * kMaxG];
  int32_t g, b;
  window_item(g, b);
  const int32_t lane = threadIdx.x & 63;
  const int32_t w = threadIdx.x >> 6;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  const int32_t G = p.group;
  constexpr int kKL = Layout<KV>::kKLoads;
  constexpr int kVL = Layout<KV>::kVLoads;

  // ---- key source (window table or req_to_token row).  A window holds at
  // most W + 1 keys: only the last W + 1 entries are used.
  // In table mode the slots are first read speculatively at the offset a full
  // window per request would have (b * (W + 1)), at the same time as the
  // table offsets, which removes one dependent memory hop; they are re-read in
  // the rare case the offsets disagree (a short request earlier in the batch).
  int32_t sl[MAXB];
  int64_t spec_base = 0;
  if (p.indptr && p.capacity > 0) {
    spec_base = static_cast<int64_t>(b) * (p.window + 1);
#pragma unroll
    for (int u = 0; u < MAXB; ++u) {
      // keys past the window re-read its last entry (one row, cached)
      const int32_t key = 16 * (w + NW * u) + kr;
      int64_t idx = spec_base + (key < p.window ? key : p.window);
      idx = idx < p.capacity ? idx : p.capacity - 1;
      sl[u] = p.table[idx < 0 ? 0 : idx];
    }
  }
  // Q^T operand (head g*G + kr).  Lanes of padding heads (kr >= G) read a
  // real head: their columns are never stored.
  uint4 qraw[4];
  load_q<KV>(p, b, g * G + (kr < G ? kr : 0), lq, qraw);
  // Fused store: the current token (window key n - 1) is attended from the new
  // rows, converted to the pool format exactly as they are stored.  Only the
  // wavefront that holds key n - 1 needs them.  It is known once the window
  // length is; the wavefront that holds it in a full window (n = W + 1, every
  // request at least W + 1 long) loads them now, with the other first-hop
  // loads, and another owner loads them after the window length arrives.
  const int32_t wu = __builtin_amdgcn_readfirstlane(w);  // w, known to the compiler as wave-uniform
  const int32_t full_owner = (p.window >> 4) % NW;
  uint4 kn_raw[4], vn_raw[2];
  int64_t new_loc = -1;
  if constexpr (FUSED) {
    new_loc = p.new_loc[b];
    if (wu == full_owner) load_new_rows<KV>(p, b, g, lane, kn_raw, vn_raw);
  }
  __builtin_amdgcn_sched_barrier(0);

  const KeySource ks = key_source(p, b);
  const int32_t n = ks.n < p.window + 1 ? ks.n : p.window + 1;
  const int32_t *src = ks.src + (ks.n - n);
  const int32_t nblk = (n + 15) >> 4;  // <= NW * MAXB for this instantiation
  const bool spec_ok = p.indptr && p.capacity > 0 && src == p.table + spec_base;
  const int32_t owner = ((n > 0 ? n - 1 : 0) >> 4) % NW;  // wavefront holding key n - 1
  const int32_t last = n - 1;
  uint4 knew[kKL], vnew;  // (fused store) the new rows in the pool format, owner wave only

  f32x4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig;
  float l_run = 0.f;
  uint16_t *vt = reinterpret_cast<uint16_t *>(lds) + w * kStageRows * kSVRow;

  if (wu < nblk) {  // this wavefront owns at least one block
    // All row loads are unconditional (no control flow between them, so none
    // of them waits for another); rows of keys past the end are masked out
    // below.  The phases are fenced with scheduling barriers so that the
    // compiler cannot pull arithmetic into the load phase (its in-order vmcnt
    // waits would make later rows wait for earlier ones).
    if (!spec_ok) {
#pragma unroll
      for (int u = 0; u < MAXB; ++u) {
        const int32_t key = 16 * (w + NW * u) + kr;
        sl[u] = src[key < n ? key : 16 * w];
      }
    }
    if constexpr (FUSED) {
      // a short window's owner: the new rows go out ahead of its K/V rows
      if (wu == owner && owner != full_owner) load_new_rows<KV>(p, b, g, lane, kn_raw, vn_raw);
    }
    __builtin_amdgcn_sched_barrier(0);
    // every K row first, then every V row: the scores only wait for K
    uint4 kraw[MAXB][kKL], vraw[MAXB][kVL];
#pragma unroll
    for (int u = 0; u < MAXB; ++u) load_k<KV>(p, sl[u], g, lq, kraw[u]);
#pragma unroll
    for (int u = 0; u < MAXB; ++u) load_v<KV>(p, sl[u], g, lane, vraw[u]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FUSED) {
      // The owner converts the new rows (they were issued before its K/V rows,
      // so this waits for them only).  They replace key n - 1's K just before
      // its block's scores and its V just before the block is staged, so
      // nothing here waits for the pool rows; the owner stores them at the
      // kernel's end (below).
      if (wu == owner) new_pieces<KV>(kn_raw, vn_raw, knew, vnew);
    }
    bf16x8_t qop[4];
    KvLoad<uint16_t>::to_bf16(qraw, qop);

    // ---- S^T = K Q^T for every block (lane: keys 4lq..4lq+3 of head kr)
    float sc[MAXB][4];
    float mb = -INFINITY;
#pragma unroll
    for (int u = 0; u < MAXB; ++u) {
      const int32_t t = w + NW * u;
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (FUSED) {
        if (wu == owner) {
#pragma unroll
          for (int c = 0; c < kKL; ++c) kraw[u][c] = sel4(16 * t + kr == last, knew[c], kraw[u][c]);
        }
      }
      bf16x8_t kk[4];
      KvLoad<KV>::to_bf16(kraw[u], kk);
#pragma unroll
      for (int c = 0; c < 4; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[c], qop[c], sacc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[u][r] = (16 * t + 4 * lq + r < n) ? sacc[r] * p.scale2 : -INFINITY;
        mb = fmaxf(mb, sc[u][r]);
      }
    }
    // ---- one softmax over the wavefront's keys (no rescaling needed)
    m_run = fmaxf(kNegBig, wave_max_q(mb));
    constexpr int kPairsN = (MAXB + 1) / 2;
    bf16x8_t pop[kPairsN];
#pragma unroll
    for (int u2 = 0; u2 < kPairsN; ++u2) {
      float pv[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pv[r] = __builtin_amdgcn_exp2f(sc[2 * u2][r] - m_run);
        pv[4 + r] =
            (2 * u2 + 1 < MAXB) ? __builtin_amdgcn_exp2f(sc[(2 * u2 + 1) < MAXB ? 2 * u2 + 1 : 0][r] - m_run) : 0.f;
      }
      uint32_t u4[4] = {pack_f16x2_hw(pv[0], pv[1]), pack_f16x2_hw(pv[2], pv[3]), pack_f16x2_hw(pv[4], pv[5]),
                        pack_f16x2_hw(pv[6], pv[7])};
      // the normaliser sums the rounded weights that enter P.V
      l_run = f16x2_acc(u4[3], f16x2_acc(u4[2], f16x2_acc(u4[1], f16x2_acc(u4[0], l_run))));
      __builtin_memcpy(&pop[u2], u4, 16);
    }
    // ---- O^T = V^T P^T over block pairs (2u2, 2u2+1), each pair's V rows
    // staged in this wave's 32-row LDS tile
#pragma unroll
    for (int u2 = 0; u2 < kPairsN; ++u2) {
      const int32_t u0 = 2 * u2;
      if constexpr (FUSED) {
        if (wu == owner) {
#pragma unroll
          for (int u = u0; u < u0 + 2 && u < MAXB; ++u) {
            const int32_t kb = 16 * (w + NW * u);
#pragma unroll
            for (int j = 0; j < kVL; ++j)
              vraw[u][j] = sel4(kb + Layout<KV>::v_key(j, lane) == last, vnew, vraw[u][j]);
          }
        }
      }
      v_to_lds<KV>(vraw[u0], vt, lane, 16 * (w + NW * u0), n);
      if (u0 + 1 < MAXB)
        v_to_lds<KV>(vraw[u0 + 1 < MAXB ? u0 + 1 : u0], vt + 16 * kSVRow, lane, 16 * (w + NW * (u0 + 1)), n);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's V rows are in LDS
      __builtin_amdgcn_wave_barrier();
      if (u0 + 1 < MAXB)
        pv_pair<true>(vt, kr, lq, pop[u2], acc);
      else
        pv_pair<false>(vt, kr, lq, pop[u2], acc);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the tile is rewritten
    }
  }
  l_run = wave_sum_q(l_run);

  __syncthreads();  // all V tiles consumed: the LDS is reused for the merge
  float *red_acc = reinterpret_cast<float *>(lds);
  if (kr < G) {
    if (lq == 0) {
      red_m[w * kMaxG + kr] = m_run;
      red_l[w * kMaxG + kr] = l_run;
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float4 v = make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
      *reinterpret_cast<float4 *>(red_acc + (w * G + kr) * kD + 16 * c + 4 * lq) = v;
    }
  }
  __syncthreads();
  merge_waves_and_store<OUT_BF16>(p, NW, red_m, red_l, red_acc, b, g, 0);
  if constexpr (FUSED) {
    // The owner's kv-head slice of the new rows goes to the pool last.  Stores
    // share the in-order counter with loads, so stores issued earlier would
    // make the owner's last V wait (and the merge's sink load) wait for their
    // write acknowledgements too: C2 12.6 -> 12.4 us.  No other workgroup
    // reads this slice, and the rows this workgroup reads there belong to
    // masked keys.
    if (wu < nblk && wu == owner && new_loc >= 0 && new_loc < p.rows) {
      KV *kdst = static_cast<KV *>(const_cast<void *>(p.k)) + row_elem(new_loc, p.kv_heads, g, kD);
      KV *vdst = static_cast<KV *>(const_cast<void *>(p.v)) + row_elem(new_loc, p.kv_heads, g, kD);
      if (kr == 0) {
#pragma unroll
        for (int c = 0; c < kKL; ++c) *reinterpret_cast<uint4 *>(kdst + Layout<KV>::k_off(c, lq)) = knew[c];
      }
      if (Layout<KV>::v_key(0, lane) == 0) *reinterpret_cast<uint4 *>(vdst + Layout<KV>::v_off(lane)) = vnew;
    }
  }
}

// --------------------------------------------------------------------------
// One-wavefront window kernel (e4m3 pools, windows of at most 9 blocks, big
// batches).  Each wavefront owns one (kv head, request) and holds its whole
// window in flight in registers: the e4m3 rows are small enough (9 blocks x 4
// loads) that no split over wavefronts, and so no cross-wavefront merge and no
// duplicated accumulator, is needed.  178 registers give two wavefronts
// per SIMD: 2048 items are resident at once, where the four-wavefront kernel
// (whose accumulators sit in every wavefront) runs such a batch in two rounds.
// At 256 requests x 8 kv heads (W = 128, e4m3): 22.1 -> 20.7 us per launch.  A
// loads-only probe of the same rows takes 13.4 us (head slices) and 12.7 us
// (whole rows), and delaying the loads of half the workgroups made the launch
// slower, not faster: what remains is the time for the rows to arrive.
// A workgroup holds four wavefronts, four kv heads of one request (half of an
// e4m3 token row at 8 kv heads); with a batch of a multiple of 8 the two
// workgroups of a request are placed on one XCD.
// --------------------------------------------------------------------------
constexpr int kOneWaveBlocks = 9;

__device__ __forceinline__ void wave_item(int32_t kv_heads, int32_t batch, int32_t w, int32_t &g, int32_t &b) {
  const int32_t per_req = kv_heads / 4;                        // workgroups per request (kv_heads % 4 == 0)
  int32_t i = static_cast<int32_t>(blockIdx.x);
  if ((batch & 7) == 0) {                                       // XCD i % 8 serves requests x, x + 8, ...
    const int32_t x = i & 7, j = i >> 3;
    i = (x + 8 * (j / per_req)) * per_req + j % per_req;
  }
  b = i / per_req;
  g = 4 * (i % per_req) + w;
}

template <bool OUT_BF16>
__global__ void __launch_bounds__(256, 2) decode_wave_kernel(DecodeParams p) {
  using KV = uint8_t;
  constexpr int NB = kOneWaveBlocks;
  constexpr int kKL = Layout<KV>::kKLoads;
  constexpr int kVL = Layout<KV>::kVLoads;
  __shared__ __attribute__((aligned(16))) uint16_t vtiles[4 * 16 * kSVRow];
  const int32_t lane = threadIdx.x & 63;
  const int32_t w = threadIdx.x >> 6;
  const int32_t kr = lane & 15;
  const int32_t lq = lane >> 4;
  const int32_t G = p.group;
  int32_t g, b;
  wave_item(p.kv_heads, static_cast<int32_t>(gridDim.x) * 4 / p.kv_heads, w, g, b);

  // slots (read speculatively at b * (W + 1), as in the window kernel) and Q
  int32_t sl[NB];
  int64_t spec_base = 0;
  if (p.indptr && p.capacity > 0) {
    spec_base = static_cast<int64_t>(b) * (p.window + 1);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int32_t key = 16 * u + kr;
      int64_t idx = spec_base + (key < p.window ? key : p.window);
      idx = idx < p.capacity ? idx : p.capacity - 1;
      sl[u] = p.table[idx < 0 ? 0 : idx];
    }
  }
  uint4 qraw[4];
  load_q<KV>(p, b, g * G + (kr < G ? kr : 0), lq, qraw);
  __builtin_amdgcn_sched_barrier(0);
  const KeySource ks = key_source(p, b);
  const int32_t n = ks.n < p.window + 1 ? ks.n : p.window + 1;
  const int32_t *src = ks.src + (ks.n - n);
  const bool spec_ok = p.indptr && p.capacity > 0 && src == p.table + spec_base;
  if (!spec_ok) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int32_t key = 16 * u + kr;
      sl[u] = n > 0 ? src[key < n ? key : 0] : 0;  // an empty window reads nothing from the table
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  // every K row, then every V row, unconditionally (keys past n are masked)
  uint4 kraw[NB][kKL], vraw[NB][kVL];
#pragma unroll
  for (int u = 0; u < NB; ++u) load_k<KV>(p, sl[u], g, lq, kraw[u]);
#pragma unroll
  for (int u = 0; u < NB; ++u) load_v<KV>(p, sl[u], g, lane, vraw[u]);
  __builtin_amdgcn_sched_barrier(0);
  bf16x8_t qop[4];
  KvLoad<uint16_t>::to_bf16(qraw, qop);
  // ---- S^T = K Q^T for every block, one softmax over the window
  float sc[NB][4];
  float mb = -INFINITY;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
    bf16x8_t kk[4];
    KvLoad<KV>::to_bf16(kraw[u], kk);
#pragma unroll
    for (int c = 0; c < 4; ++c) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[c], qop[c], sacc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[u][r] = (16 * u + 4 * lq + r < n) ? sacc[r] * p.scale2 : -INFINITY;
      mb = fmaxf(mb, sc[u][r]);
    }
  }
  const float m_run = fmaxf(kNegBig, wave_max_q(mb));
  float l_run = 0.f;
  f32x4_t acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // ---- O^T += V^T P^T block by block (16x16x16 MFMA), V through this wave's LDS tile
  uint16_t *vt = vtiles + w * 16 * kSVRow;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    uint32_t u2[2] = {pack_f16x2_hw(__builtin_amdgcn_exp2f(sc[u][0] - m_run), __builtin_amdgcn_exp2f(sc[u][1] - m_run)),
                      pack_f16x2_hw(__builtin_amdgcn_exp2f(sc[u][2] - m_run), __builtin_amdgcn_exp2f(sc[u][3] - m_run))};
    l_run = f16x2_acc(u2[1], f16x2_acc(u2[0], l_run));  // the normaliser sums the rounded weights
    i16x4_t pop;
    __builtin_memcpy(&pop, u2, 8);
    v_to_lds<KV>(vraw[u], vt, lane, 16 * u, n);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's V rows are in LDS
    __builtin_amdgcn_wave_barrier();
    pv_single(vt, kr, lq, pop, acc);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the tile is rewritten
  }
  l_run = wave_sum_q(l_run);
  // ---- sink once, normalise, store head g * G + kr
  if (kr >= G) return;
  const int32_t h = g * G + kr;
  float M = m_run, L = l_run, a = 1.f;
  if (p.sinks) {
    const float sig2 = p.sinks[h] * kLog2e;
    const float Mn = fmaxf(M, sig2);
    a = __builtin_amdgcn_exp2f(M - Mn);
    L = L * a + __builtin_amdgcn_exp2f(sig2 - Mn);
  }
  const float inv = L > 0.f ? a * p.v_scale / L : 0.f;
  const int64_t off = (static_cast<int64_t>(b) * p.q_heads + h) * kD + 4 * lq;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const float o0 = acc[c][0] * inv, o1 = acc[c][1] * inv, o2 = acc[c][2] * inv, o3 = acc[c][3] * inv;
    if (OUT_BF16)
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.out) + off + 16 * c) =
          make_uint2(pack_bf16x2_hw(o0, o1), pack_bf16x2_hw(o2, o3));
    else
      *reinterpret_cast<float4 *>(static_cast<float *>(p.out) + off + 16 * c) = make_float4(o0, o1, o2, o3);
  }
}

// --------------------------------------------------------------------------
// f32 VALU path (f32 q, f32 K/V).  A wavefront takes 16 keys at a time:
// lane (key kr = lane / 4, quarter c = lane % 4) holds dims 32c..32c+31 of
// that key's K and V rows, so a score needs 32 FMAs and a 4-lane sum.  The
// chunk's probabilities and V rows go through this wavefront's LDS slice and
// lane l then accumulates dims 2l, 2l+1 of every head.  The rows of the next
// chunk are loaded (unconditionally: keys past the split re-read its first
// row and get probability 0) while the current one is computed.
// --------------------------------------------------------------------------
constexpr int kF32Waves = 4;
constexpr int kF32Chunk = 16;

struct F32Rows {
  float4 k[8], v[8];
};

__device__ __forceinline__ void f32_issue(const DecodeParams &p, int32_t slot, int32_t g, int32_t c, F32Rows &r) {
  const int64_t off = row_elem(safe_slot(slot, p.rows), p.kv_heads, g, kD) + 32 * c;
  const float4 *kp = reinterpret_cast<const float4 *>(static_cast<const float *>(p.k) + off);
  const float4 *vp = reinterpret_cast<const float4 *>(static_cast<const float *>(p.v) + off);
#pragma unroll
  for (int i = 0; i < 8; ++i) r.k[i] = kp[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) r.v[i] = vp[i];
}

// NW wavefronts per workgroup: 4, or 8 when the grid is too small to fill the
// chip (each wavefront then walks half as many chunks of the window).
template <int G, bool OUT_BF16, int NW>
__global__ void __launch_bounds__(NW * 64) decode_f32_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) float q_lds[kMaxG * kD];
  // per-wavefront V chunk during the loop; the cross-wavefront partials after it
  __shared__ __attribute__((aligned(16))) float big[NW * kMaxG * kD];
  __shared__ float p_lds[NW * kF32Chunk * kMaxG];
  __shared__ float red_m[NW * kMaxG];
  __shared__ float red_l[NW * kMaxG];
  static_assert(NW * kF32Chunk * kD <= NW * kMaxG * kD, "V chunk must fit the partials buffer");

  const int32_t s = blockIdx.x;
  const int32_t g = blockIdx.y;
  const int32_t b = blockIdx.z;
  const int32_t lane = threadIdx.x & 63;
  const int32_t w = threadIdx.x >> 6;
  const int32_t kr = lane >> 2;
  const int32_t c = lane & 3;

  const KeySource ks = key_source(p, b);
  int32_t k0, k1;
  split_range(ks.n, s, p.num_splits, &k0, &k1);

  float m_run[G], l_run[G];
  float2 acc[G];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    m_run[hh] = kNegBig;
    l_run[hh] = 0.f;
    acc[hh] = make_float2(0.f, 0.f);
  }
  float *vc = big + w * kF32Chunk * kD;
  float *pc = p_lds + w * kF32Chunk * kMaxG;

  auto chunk_base = [&](int32_t j) { return k0 + kF32Chunk * (w + NW * j); };
  auto slot_of = [&](int32_t j) {
    const int32_t key = chunk_base(j) + kr;
    return ks.src[key < k1 ? key : k0];
  };

  // Slots run two chunks ahead of the rows, rows one chunk ahead of the
  // arithmetic; the query rows are fetched while the first slots are in flight.
  const bool any = chunk_base(0) < k1;  // wavefront-uniform; implies k0 < k1
  int32_t sl0 = 0, sl1 = 0;
  if (any) {
    sl0 = slot_of(0);
    sl1 = slot_of(1);
  }
  constexpr int kQVec = (G * kD / 4 + NW * 64 - 1) / (NW * 64);
  float4 qr[kQVec];
  const float4 *qsrc = reinterpret_cast<const float4 *>(static_cast<const float *>(p.q) +
                                                        (static_cast<int64_t>(b) * p.q_heads + g * G) * kD);
#pragma unroll
  for (int i = 0; i < kQVec; ++i) {
    const int32_t t = threadIdx.x + i * NW * 64;
    if (t < G * kD / 4) qr[i] = qsrc[t];
  }
  F32Rows cur, nxt;
  if (any) f32_issue(p, sl0, g, c, cur);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kQVec; ++i) {
    const int32_t t = threadIdx.x + i * NW * 64;
    if (t < G * kD / 4) reinterpret_cast<float4 *>(q_lds)[t] = qr[i];
  }
  __syncthreads();

  if (any) {
    for (int32_t j = 0; chunk_base(j) < k1; ++j) {
      const bool more = chunk_base(j + 1) < k1;  // wavefront-uniform
      if (more) {
        f32_issue(p, sl1, g, c, nxt);
        sl1 = slot_of(j + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
      const bool valid = chunk_base(j) + kr < k1;
      // V chunk to LDS (row kr, dims 32c..32c+31)
#pragma unroll
      for (int i = 0; i < 8; ++i) reinterpret_cast<float4 *>(vc + kr * kD + 32 * c)[i] = cur.v[i];
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float4 *qh = reinterpret_cast<const float4 *>(q_lds + hh * kD + 32 * c);
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float4 qv = qh[i];
          d0 = fmaf(qv.x, cur.k[i].x, d0);
          d1 = fmaf(qv.y, cur.k[i].y, d1);
          d0 = fmaf(qv.z, cur.k[i].z, d0);
          d1 = fmaf(qv.w, cur.k[i].w, d1);
        }
        float dot = d0 + d1;
        dot += __shfl_xor(dot, 1);
        dot += __shfl_xor(dot, 2);
        const float sc = valid ? dot * p.scale2 : -INFINITY;
        float cm = sc;
        cm = fmaxf(cm, __shfl_xor(cm, 4));
        cm = rows_max(fmaxf(cm, __shfl_xor(cm, 8)));
        const float m_new = fmaxf(m_run[hh], cm);
        const float alpha = exp2f(m_run[hh] - m_new);
        const float pj = exp2f(sc - m_new);
        float ps = pj;
        ps += __shfl_xor(ps, 4);
        ps = rows_sum(ps + __shfl_xor(ps, 8));
        m_run[hh] = m_new;
        l_run[hh] = l_run[hh] * alpha + ps;
        acc[hh].x *= alpha;
        acc[hh].y *= alpha;
        if (c == 0) pc[kr * kMaxG + hh] = pj;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's V rows and probabilities are in LDS
      __builtin_amdgcn_wave_barrier();
#pragma unroll 4
      for (int32_t r = 0; r < kF32Chunk; ++r) {
        const float2 v2 = reinterpret_cast<const float2 *>(vc + r * kD)[lane];
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float pr = pc[r * kMaxG + hh];
          acc[hh].x = fmaf(pr, v2.x, acc[hh].x);
          acc[hh].y = fmaf(pr, v2.y, acc[hh].y);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next chunk overwrites the slice
      __builtin_amdgcn_wave_barrier();
      if (!more) break;
      cur = nxt;
    }
  }
  __syncthreads();  // every wavefront is done with its V slice before `big` holds partials
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    if (lane == 0) {
      red_m[w * kMaxG + hh] = m_run[hh];
      red_l[w * kMaxG + hh] = l_run[hh];
    }
    reinterpret_cast<float2 *>(big + (w * G + hh) * kD)[lane] = acc[hh];
  }
  __syncthreads();
  merge_waves_and_store<OUT_BF16>(p, NW, red_m, red_l, big, b, g, s);
}

// --------------------------------------------------------------------------
// Split merge: one workgroup of 128 threads (one per dim) per (request, q head).
//   M = max(max_s m_s, sink), L = sum_s l_s 2^{m_s - M} + 2^{sink - M}
//   o = v_scale * sum_s acc_s 2^{m_s - M} / L
// --------------------------------------------------------------------------
template <bool OUT_BF16>
__global__ void __launch_bounds__(kD) decode_merge_kernel(DecodeParams p) {
  const int32_t h = blockIdx.x;
  const int32_t b = blockIdx.y;
  const int32_t d = threadIdx.x;
  const int64_t base = (static_cast<int64_t>(b) * p.q_heads + h) * p.num_splits;
  float M = kNegBig;
  for (int32_t s = 0; s < p.num_splits; ++s) M = fmaxf(M, p.ws_m[base + s]);
  float sig2 = -INFINITY;
  if (p.sinks) {
    sig2 = p.sinks[h] * kLog2e;
    M = fmaxf(M, sig2);
  }
  float L = p.sinks ? exp2f(sig2 - M) : 0.f;
  float o = 0.f;
  for (int32_t s = 0; s < p.num_splits; ++s) {
    const float a = exp2f(p.ws_m[base + s] - M);
    L += p.ws_l[base + s] * a;
    o += p.ws_acc[(base + s) * kD + d] * a;
  }
  o = L > 0.f ? o * (p.v_scale / L) : 0.f;
  const int64_t off = (static_cast<int64_t>(b) * p.q_heads + h) * kD + d;
  if (OUT_BF16)
    static_cast<uint16_t *>(p.out)[off] = f32_to_bf16_rne(o);
  else
    static_cast<float *>(p.out)[off] = o;
}

template <bool OUT_BF16>
hipError_t launch_f32(const DecodeParams &p, dim3 grid, hipStream_t stream) {
  // fewer workgroups than half the CUs: twice the wavefronts per workgroup
  const bool wide = static_cast<int64_t>(grid.x) * grid.y * grid.z < 128;
  const dim3 block((wide ? 8 : kF32Waves) * 64);
#define SWA_F32_LAUNCH(GG)                                                                                  \
  if (wide)                                                                                                 \
    hipLaunchKernelGGL((decode_f32_kernel<GG, OUT_BF16, 8>), grid, block, 0, stream, p);                    \
  else                                                                                                      \
    hipLaunchKernelGGL((decode_f32_kernel<GG, OUT_BF16, kF32Waves>), grid, block, 0, stream, p);
  switch (p.group) {  // validated on the host: 1, 2, 4, 8 or 16
    case 1: SWA_F32_LAUNCH(1) break;
    case 2: SWA_F32_LAUNCH(2) break;
    case 4: SWA_F32_LAUNCH(4) break;
    case 8: SWA_F32_LAUNCH(8) break;
    case 16: SWA_F32_LAUNCH(16) break;
    default: return hipErrorInvalidValue;
  }
#undef SWA_F32_LAUNCH
  return hipGetLastError();
}

template <typename KV, int MAXB>
hipError_t launch_window_b(const DecodeParams &p, dim3 grid, bool out_bf16, hipStream_t stream) {
  const dim3 block(kWinWaves * 64);
  if (p.new_loc) {
    if (out_bf16)
      hipLaunchKernelGGL((decode_window_kernel<KV, MAXB, true, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((decode_window_kernel<KV, MAXB, false, true>), grid, block, 0, stream, p);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((decode_window_kernel<KV, MAXB, true, false>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((decode_window_kernel<KV, MAXB, false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

// Workgroups of four wavefronts that are resident at once (four per CU of the
// 256, by their LDS); a bigger grid runs in rounds.
constexpr int64_t kWindowResident = 1024;

// Blocks per wavefront for a window of W + 1 keys over kWinWaves wavefronts.
template <typename KV>
hipError_t launch_window(const DecodeParams &p, dim3 grid, int window, bool out_bf16, hipStream_t stream) {
  const int blocks = (window + 1 + 15) / 16;
  const int64_t items = static_cast<int64_t>(grid.y) * grid.z;
  if (sizeof(KV) == 1 && !p.new_loc && items > kWindowResident && blocks <= kOneWaveBlocks && p.kv_heads % 4 == 0) {
    const dim3 wgrid(static_cast<uint32_t>(items / 4));
    if (out_bf16)
      hipLaunchKernelGGL((decode_wave_kernel<true>), wgrid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_wave_kernel<false>), wgrid, dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  const int maxb = (blocks + kWinWaves - 1) / kWinWaves;
  if (maxb <= 1) return launch_window_b<KV, 1>(p, grid, out_bf16, stream);
  if (maxb == 2) return launch_window_b<KV, 2>(p, grid, out_bf16, stream);
  if (maxb == 3) return launch_window_b<KV, 3>(p, grid, out_bf16, stream);
  return launch_window_b<KV, 4>(p, grid, out_bf16, stream);
}

template <typename KV>
hipError_t launch_stream(const DecodeParams &p, dim3 grid0, bool out_bf16, hipStream_t stream) {
  // grid: (splits, groups of kStreamWaves kv heads, requests)
  const dim3 grid(grid0.x, (p.kv_heads + kStreamWaves - 1) / kStreamWaves, grid0.z);
  if (out_bf16)
    hipLaunchKernelGGL((decode_stream_kernel<KV, true>), grid, dim3(kStreamWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_stream_kernel<KV, false>), grid, dim3(kStreamWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t static_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  static void *addr[kMaxDevices];
  static hipError_t err[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(once[dev], [dev] { err[dev] = hipGetSymbolAddress(&addr[dev], HIP_SYMBOL(scratch)); });
  if (err[dev] != hipSuccess) return err[dev];
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream) {
  if (a.idx.batch == 0) return hipSuccess;
  DecodeParams p{};
  p.q = a.q;
  p.k = a.layer.k;
  p.v = a.layer.v;
  p.rows = a.layer.rows;
  p.kv_heads = a.layer.kv_heads;
  p.q_heads = a.q_heads;
  p.group = a.q_heads / a.layer.kv_heads;
  const bool fp8 = a.layer.dtype == SWA_FP8_E4M3;
  p.k_scale = fp8 ? a.layer.k_scale : 1.f;
  p.v_scale = fp8 ? a.layer.v_scale : 1.f;
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
  p.scale2 = a.sm_scale * p.k_scale * kLog2e;
  p.out = a.out;
  p.num_splits = a.num_splits;
  if (a.num_splits > 1) {
    const int64_t parts = static_cast<int64_t>(a.idx.batch) * a.q_heads * a.num_splits;
    p.ws_m = a.ws;
    p.ws_l = a.ws + parts;
    p.ws_acc = a.ws + 2 * parts;
  }
  p.k_new = static_cast<const uint16_t *>(a.k_new);
  p.v_new = static_cast<const uint16_t *>(a.v_new);
  p.new_loc = a.new_loc;
  const bool out_bf16 = a.out_dtype == SWA_BF16;
  const dim3 grid(static_cast<uint32_t>(a.num_splits), static_cast<uint32_t>(a.layer.kv_heads),
                  static_cast<uint32_t>(a.idx.batch));
  const bool window_path = a.num_splits == 1 && a.window >= 0 && a.window < 16 * kWinWaves * 4;
  // the fused store exists in the window kernel only (bf16 / e4m3 pools)
  if (a.new_loc && (!window_path || a.layer.dtype == SWA_F32)) return hipErrorInvalidValue;
  hipError_t e;
  if (a.layer.dtype == SWA_F32) {
    e = out_bf16 ? launch_f32<true>(p, grid, stream) : launch_f32<false>(p, grid, stream);
  } else if (window_path) {
    // SWA layer: the whole window in flight at once (up to 4 blocks per wavefront)
    e = a.layer.dtype == SWA_BF16 ? launch_window<uint16_t>(p, grid, a.window, out_bf16, stream)
                                  : launch_window<uint8_t>(p, grid, a.window, out_bf16, stream);
  } else if (a.layer.dtype == SWA_BF16) {
    e = launch_stream<uint16_t>(p, grid, out_bf16, stream);
  } else {
    e = launch_stream<uint8_t>(p, grid, out_bf16, stream);
  }
  if (e != hipSuccess || a.num_splits == 1) return e;
  const dim3 mgrid(static_cast<uint32_t>(a.q_heads), static_cast<uint32_t>(a.idx.batch));
  if (out_bf16)
    hipLaunchKernelGGL((decode_merge_kernel<true>), mgrid, dim3(kD), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_merge_kernel<false>), mgrid, dim3(kD), 0, stream, p);
  return hipGetLastError();
}

}  // namespace swa
