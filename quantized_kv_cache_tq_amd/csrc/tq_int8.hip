// tq_int8.hip -- prompt attention over a paged int8 K/V cache.
//
// [QSA1821] What / Change: the Turing kernel walks 32-cell chunks whose int8
// K and V rows are scattered in memory, prefetching the next chunk while the
// current one computes.  On CDNA4 the same walk becomes 64-key tiles (two
// pages) gathered through the page table straight into LDS, converted to
// float16 on the way (int8 is exact in float16; K and V both stored [key][d],
// V read transposed for its product), and multiplied on the matrix cores:
//   S^T[key][qrow] = K[key][:] . Q[qrow][:]      (then x k_scale[key])
//   O^T[d][qrow]  += V^T[d][key] P^T[key][qrow]   (P already x v_scale[key])
// The float32 query and P are each split into a high and a low float16 part
// (x = hi + lo to ~22 bits) and both parts go through the matrix cores, so the
// result stays within float32-level error of the exact attention.
// The output depends only on the logical key order: physical page placement
// changes which bytes are read, never the arithmetic.
//
// Workgroup: 128 qrows (128/n_rep queries x n_rep heads of one kv head),
// eight waves = 4 qrow quarters x 2 key halves of each tile, merged at the
// end.  Each key tile is gathered and converted once for all 128 qrows (with
// 64 qrows per workgroup the conversion and the gather addressing were a
// quarter of the loop's vector instructions).  For few queries the key range
// is split over workgroups and merged by a second kernel.
#include "tq_common.h"
#include "tq_launch.h"

namespace tq {

namespace i8 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kQBlocks = 4;              // 32-qrow blocks per workgroup
constexpr int kWaves = 2 * kQBlocks;     // x 2 key halves
constexpr int kThreads = 64 * kWaves;
constexpr int kD = 128;
constexpr int kQRows = 32 * kQBlocks;
constexpr int kKT = 64;              // keys per tile (two 32-cell pages)
constexpr int kPage = 32;
constexpr int kKsStride = kD + 8;    // halves per K row
constexpr int kVsStride = kD + 16;   // halves per V row (288 B: a transposing read's four rows hit distinct banks)
constexpr int kPartStride = kD + 4;  // o[128], m, l, pad
constexpr float kPTop = 15.f;         // P = p * scale stays below 2^kPTop
constexpr float kPSet = 9.f;          // a moved reference puts the tile's top at 2^kPSet

struct Args {
  const float *q;
  const int8_t *k;
  const int8_t *v;
  const uint16_t *ks;
  const uint16_t *vs;
  const int32_t *pt;
  float *out;
  float *ws;
  int64_t n_q, ctx_len, q_pos0, n_phys_pages;
  int n_q_heads, n_kv, n_rep, bq, n_split, tiles_per_split;
  float qscale;
};

__device__ __forceinline__ int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }

// 16 signed bytes -> 16 float16 values, in order.  With every byte's top bit
// flipped (b ^ 0x80 = b + 128 as an unsigned byte), the float16 bit pattern
// 0x64 : (b ^ 0x80) is 1024 + b + 128, exact, so subtracting 1152 leaves b
// exactly.  A byte permute places two flipped bytes under 0x64 high bytes.
__device__ __forceinline__ void bytes16_to_halves(const u32x4_t &x, uint32_t (&h)[8]) {
  const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t y = x[w] ^ 0x80808080u;
    const uint32_t p0 = __builtin_amdgcn_perm(0x64646464u, y, 0x04010400u);   // bytes 0, 1
    const uint32_t p1 = __builtin_amdgcn_perm(0x64646464u, y, 0x04030402u);   // bytes 2, 3
    h[2 * w] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p0) - bias);
    h[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p1) - bias);
  }
}

// Four 16-bit values by a transposing LDS read: within each 16-lane group,
// lane j gives the address of four consecutive values of row j / 4 of a
// 4 x 16 block (columns 4 (j % 4) .. + 3), and lane i receives column i of
// the block's four rows.
__device__ __forceinline__ s16x4_t read_tr16(const _Float16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)p);
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

struct TileRaw {
  u32x4_t k;          // K: key t>>3, bytes 16*(t&7) .. +15
  u32x4_t v;          // V: key t>>3, bytes 16*(t&7) .. +15
  uint16_t scl;       // scale: t < 64 -> K of key t, 64 <= t < 128 -> V of key t-64
  bool page_ok;       // this thread's scale key's page exists
};

// The two pages of key tile kt (wave-uniform, so the page-table entries are
// scalar loads): tile key kk (0..63, clamped to the last key) sits on page
// p[(kk' >> 5)] at row p * 32 + (kk' & 31); ok = that entry is in range.
struct TilePages {
  int64_t base[2];   // first physical row of each page (0 for an entry out of range)
  bool ok[2];
  int last_rel;      // last valid key of the tile, relative to its first key
};

__device__ __forceinline__ TilePages tile_pages(const Args &a, int64_t kt) {
  const int64_t last = a.ctx_len - 1, lastpg = last >> 5;
  TilePages t;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int32_t pg = a.pt[lmin(2 * kt + h, lastpg)];
    t.ok[h] = pg >= 0 && pg < a.n_phys_pages;
    t.base[h] = (int64_t)(t.ok[h] ? pg : 0) * kPage;
  }
  const int64_t rel = last - kt * kKT;
  t.last_rel = rel < kKT - 1 ? (int)rel : kKT - 1;
  return t;
}

// Row index (cell * n_kv + g) of tile key kk for kv head g, and its byte
// offset in the K / V planes (32-bit arithmetic when the whole cache is below
// 2^32 bytes, which the host checks).
template <bool kOff32>
__device__ __forceinline__ int64_t key_row(const Args &a, const TilePages &t, int g, int kk, bool &ok) {
  const int j = kk < t.last_rel ? kk : t.last_rel;
  const int h = j >> 5;
  ok = h ? t.ok[1] : t.ok[0];
  const int64_t cell = (h ? t.base[1] : t.base[0]) + (j & (kPage - 1));
  if constexpr (kOff32) return (int64_t)((uint32_t)cell * (uint32_t)a.n_kv + (uint32_t)g);
  return cell * a.n_kv + g;
}
template <bool kOff32>
__device__ __forceinline__ int64_t row_bytes(int64_t row) {
  if constexpr (kOff32) return (int64_t)((uint32_t)row * (uint32_t)kD);
  return row * kD;
}

template <bool kOff32>
__device__ __forceinline__ void load_tile(const Args &a, int g, int64_t kt, int tid, TileRaw &r) {
  const TilePages t = tile_pages(a, kt);
  bool ok;
  {
    const int64_t e = key_row<kOff32>(a, t, g, tid >> 3, ok);
    r.k = *reinterpret_cast<const u32x4_t *>(a.k + row_bytes<kOff32>(e) + 16 * (tid & 7));
  }
  {
    const int64_t e = key_row<kOff32>(a, t, g, tid >> 3, ok);
    r.v = *reinterpret_cast<const u32x4_t *>(a.v + row_bytes<kOff32>(e) + 16 * (tid & 7));
  }
  if (tid < 2 * kKT) {
    const int64_t e = key_row<kOff32>(a, t, g, tid & 63, ok);
    r.page_ok = ok;
    r.scl = (tid < kKT) ? a.ks[e] : a.vs[e];
  }
}

__device__ __forceinline__ void store_tile(const Args &a, int64_t kt, int tid, const TileRaw &r,
                                           _Float16 *ksm, _Float16 *vt, float (*skq)[kKT], float *sv,
                                           float *ve_max, int *kval, const int *qexp_s) {
  // K and V rows alike: [key][d], 16 bytes -> 16 halves per thread
  {
    uint32_t h[8];
    bytes16_to_halves(r.k, h);
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(ksm + (tid >> 3) * kKsStride + 16 * (tid & 7));
    dst[0] = u32x4_t{h[0], h[1], h[2], h[3]};
    dst[1] = u32x4_t{h[4], h[5], h[6], h[7]};
  }
  {
    uint32_t h[8];
    bytes16_to_halves(r.v, h);
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(vt + (tid >> 3) * kVsStride + 16 * (tid & 7));
    dst[0] = u32x4_t{h[0], h[1], h[2], h[3]};
    dst[1] = u32x4_t{h[4], h[5], h[6], h[7]};
  }
  if (tid < 2 * kKT) {
    const int64_t j = kt * kKT + (tid & 63);
    const bool ok = j < a.ctx_len && r.page_ok;
    const float s = ok ? half_to_float(r.scl) : 0.f;
    if (tid < kKT) {
      // the K scale times each row block's 2^-qexp (exact: a power of two)
#pragma unroll
      for (int q = 0; q < kQBlocks; ++q) skq[q][tid] = __builtin_amdgcn_ldexpf(s, -qexp_s[q]);
      kval[tid] = ok ? 1 : 0;
    } else {
      sv[tid - kKT] = s;
      // the tile's largest binary exponent of a V scale (every s < 2^e)
      float e = (float)__builtin_amdgcn_frexp_expf(s);
      e = fmaxf(e, xor_lane<1>(e));
      e = fmaxf(e, xor_lane<2>(e));
      e = fmaxf(e, xor_lane<4>(e));
      e = fmaxf(e, xor_lane<8>(e));
      e = fmaxf(e, xor_lane<16>(e));
      e = fmaxf(e, xor_lane<32>(e));
      if (tid == kKT) *ve_max = e;
    }
  }
}

__device__ __forceinline__ void split_hl(float x, _Float16 &hi, _Float16 &lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

template <bool kOff32>
__global__ __launch_bounds__(kThreads, 2) void int8_prompt_kernel(Args a) {
  constexpr int kTileHalves = kKT * kKsStride + kKT * kVsStride;
  constexpr int kMergeHalves = kQBlocks * 4 * 16 * 64 * 2;   // o of the key-half-1 waves, float32
  constexpr int kArenaHalves = kTileHalves > kMergeHalves ? kTileHalves : kMergeHalves;
  __shared__ __align__(16) _Float16 arena[kArenaHalves];
  __shared__ __align__(16) float skq[kQBlocks][kKT], sv[kKT];
  __shared__ float ve_max;                  // largest binary exponent of the tile's V scales
  __shared__ int qexp_s[kQBlocks];
  __shared__ float mstat[kQBlocks][32], lstat[kQBlocks][32];
  __shared__ int kval[kKT];   // key exists (in context, page in range)
  _Float16 *ksm = arena;
  _Float16 *vt = arena + kKT * kKsStride;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qblk = wave & (kQBlocks - 1), khalf = wave / kQBlocks;
  const int qt = blockIdx.x, split = blockIdx.y, g = blockIdx.z;
  const int ql = lane & 31, hl = lane >> 5;
  const int qrow = 32 * qblk + ql;
  const int head_local = qrow / a.bq, row_local = qrow % a.bq;
  const int head = g * a.n_rep + head_local;
  const int64_t q0 = (int64_t)qt * a.bq;
  const int64_t qi = q0 + row_local;                         // this column's query
  const int64_t qi_c = lmin(qi, a.n_q - 1);
  const int64_t last_q = lmin(q0 + a.bq, a.n_q) - 1;
  const int64_t kend = lmin(a.ctx_len, a.q_pos0 + last_q + 1);
  const int64_t n_kt_all = ceil_div<int64_t>(kend, kKT);
  const int64_t kt0 = (int64_t)split * a.tiles_per_split;
  const int64_t kt1 = lmin(kt0 + a.tiles_per_split, n_kt_all);
  const int64_t pos = a.q_pos0 + qi_c;

  // query operand: d = 16t + 8hl + i, high and low float16 parts of
  // q * qscale * 2^qexp, the power of two putting the largest element of the
  // wave's 32 rows just under 2^14 (no float16 overflow; the low parts keep
  // an absolute error of at most 2^-25 of that scale); the K scales stored
  // for this row block carry the 2^-qexp back
  half8_t qhi[8], qlo[8];
  int qexp;
  {
    const float *qr = a.q + (qi_c * a.n_q_heads + head) * kD + 8 * hl;
    float x[8][8];
    float amax = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float4 f0 = *reinterpret_cast<const float4 *>(qr + 16 * t);
      const float4 f1 = *reinterpret_cast<const float4 *>(qr + 16 * t + 4);
      const float y[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x[t][i] = y[i] * a.qscale;
        amax = fmaxf(amax, fabsf(x[t][i]));
      }
    }
    amax = fmaxf(amax, xor_lane<1>(amax));
    amax = fmaxf(amax, xor_lane<2>(amax));
    amax = fmaxf(amax, xor_lane<4>(amax));
    amax = fmaxf(amax, xor_lane<8>(amax));
    amax = fmaxf(amax, xor_lane<16>(amax));
    amax = fmaxf(amax, xor_lane<32>(amax));
    qexp = 14 - __builtin_amdgcn_frexp_expf(amax);   // amax * 2^qexp < 2^14
    if (khalf == 0 && lane == 0) qexp_s[qblk] = qexp;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        _Float16 h, l;
        split_hl(__builtin_amdgcn_ldexpf(x[t][i], qexp), h, l);
        qhi[t][i] = h;
        qlo[t][i] = l;
      }
  }

  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) o[dt][rr] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  __syncthreads();   // qexp_s
  TileRaw raw;
  if (kt0 < kt1) load_tile<kOff32>(a, g, kt0, tid, raw);
  for (int64_t kt = kt0; kt < kt1; ++kt) {
    store_tile(a, kt, tid, raw, ksm, vt, skq, sv, &ve_max, kval, qexp_s);
    if (kt + 1 < kt1) load_tile<kOff32>(a, g, kt + 1, tid, raw);
    __syncthreads();

    // one chain of products over the high and low query parts (two chains
    // and their sum cost 16 more registers and vector additions per tile,
    // which measured slower)
    f32x16_t s;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) s[rr] = 0.f;
    const _Float16 *krow = ksm + (32 * khalf + ql) * kKsStride + 8 * hl;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const half8_t av = *reinterpret_cast<const half8_t *>(krow + 16 * t);
      s = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, qhi[t], s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, qlo[t], s, 0, 0, 0);
    }
    const int64_t lim64 = pos - (kt * kKT + 32 * khalf);   // keys past lim are masked
    const int lim = lim64 > 64 ? 64 : (int)lim64;
    // m_run is a reference, not the running maximum: p = exp2(s - m_run)
    // and P = p * (V scale) goes to float16 as a high and a low part.  With
    // e the largest binary exponent of the tile's V scales,
    // P < 2^(s + e - m_run); the reference moves only when some key could
    // reach 2^kPTop, and then to put the tile's bound at 2^kPSet.  So P never overflows, its parts stay clear
    // of float16 subnormals, and the accumulators are rescaled rarely.
    // Softmax does not depend on the reference.
    // a tile whose 64 keys all exist (in context, pages in range) and whose
    // key half no column's causal limit cuts needs no per-key test; the test
    // is taken wave-uniformly, so the fast path reads no existence flags
    const TilePages tp = tile_pages(a, kt);
    const bool whole = tp.last_rel == kKT - 1 && tp.ok[0] && tp.ok[1] && __all(lim >= 31);
    float tref = -INFINITY;
    auto scale_scores = [&](auto mask_tag) {
      constexpr bool kMask = decltype(mask_tag)::value;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int k0 = 8 * g4 + 4 * hl;   // keys k0 .. k0+3 of the half <-> registers 4 g4 .. 4 g4 + 3
        const float4 sk4 = *reinterpret_cast<const float4 *>(&skq[qblk][32 * khalf + k0]);
        const float skv[4] = {sk4.x, sk4.y, sk4.z, sk4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int rr = 4 * g4 + i, kk = k0 + i;
          float v = s[rr] * skv[i];
          if (kMask && (kk > lim || !kval[32 * khalf + kk])) v = -INFINITY;  // causal / no such key
          s[rr] = v;
          tref = fmaxf(tref, v);
        }
      }
    };
    if (whole)
      scale_scores(std::false_type{});
    else
      scale_scores(std::true_type{});
    tref = fmaxf(tref, xor_lane<32>(tref)) + ve_max;
    const float m_new = tref > m_run + kPTop ? tref - kPSet : m_run;
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    half8_t phi[2], plo[2];
    float psum = 0.f;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 sv4 = *reinterpret_cast<const float4 *>(&sv[32 * khalf + 8 * g4 + 4 * hl]);
      const float svv[4] = {sv4.x, sv4.y, sv4.z, sv4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 4 * g4 + i;
        const float p = __builtin_amdgcn_exp2f(s[rr] - m_use);
        psum += p;
        // P = p * (V scale) split into float16 parts straight from the exact
        // product: hi = RN(P), lo = RN(P - hi) (fused multiply-adds with a
        // float16 result, no float32 rounding of P in between)
        const _Float16 h = (_Float16)__builtin_fmaf(p, svv[i], 0.f);
        const _Float16 l = (_Float16)__builtin_fmaf(p, svv[i], -(float)h);
        phi[rr >> 3][rr & 7] = h;
        plo[rr >> 3][rr & 7] = l;
      }
    }
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.0f)) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) o[dt][rr] *= alpha;
    }
    // products in the order (key step, P part, d-tile): consecutive ones
    // update different accumulators.  The V^T operand (d = 32 dt + ql, k-slots
    // 8 hl + i <-> keys 16 ga + 8 (i >> 2) + 4 hl + (i & 3), as P's) is two
    // transposing reads of the [key][d] tile: lane j of 16-lane group gq
    // points at d 16 (gq & 1) + 4 (j & 3) of key 4 hl + (j >> 2), so lane i
    // of the group receives d 16 (gq & 1) + i, that is ql, of four keys
    const int gq = lane >> 4, tj = lane & 15;
    const _Float16 *vtr = vt + (32 * khalf + 4 * hl + (tj >> 2)) * kVsStride + 16 * (gq & 1) + 4 * (tj & 3);
#pragma unroll
    for (int ga = 0; ga < 2; ++ga) {
      half8_t av[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const _Float16 *vr = vtr + 16 * ga * kVsStride + 32 * dt;
        const s16x4_t lo = read_tr16(vr);                    // keys 16 ga + 4 hl + 0..3
        const s16x4_t hi = read_tr16(vr + 8 * kVsStride);    // keys 16 ga + 8 + 4 hl + 0..3
        av[dt] = __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[dt], phi[ga], o[dt], 0, 0, 0);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[dt], plo[ga], o[dt], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- merge the key halves
  l_run += xor_lane<32>(l_run);
  float *mbuf = reinterpret_cast<float *>(arena);
  if (khalf == 1) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mbuf[((qblk * 4 + dt) * 16 + rr) * 64 + lane] = o[dt][rr];
    if (hl == 0) {
      mstat[qblk][ql] = m_run;
      lstat[qblk][ql] = l_run;
    }
  }
  __syncthreads();
  if (khalf != 0) return;
  const float m2 = mstat[qblk][ql], l2 = lstat[qblk][ql];
  const float M = fmaxf(m_run, m2);
  const float f1 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
  const float f2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
  const float L = l_run * f1 + l2 * f2;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      o[dt][rr] = o[dt][rr] * f1 + mbuf[((qblk * 4 + dt) * 16 + rr) * 64 + lane] * f2;
  if (qi >= a.n_q) return;
  // O^T register rr of tile dt <-> d = 32dt + 8(rr/4) + 4hl + rr%4
  if (a.n_split == 1) {
    const float r = 1.0f / L;
    float *orow = a.out + (qi * a.n_q_heads + head) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<float4 *>(orow + 32 * dt + 8 * rq + 4 * hl) =
            make_float4(o[dt][4 * rq] * r, o[dt][4 * rq + 1] * r, o[dt][4 * rq + 2] * r,
                        o[dt][4 * rq + 3] * r);
  } else {
    float *prow = a.ws + ((qi * a.n_q_heads + head) * (int64_t)a.n_split + split) * kPartStride;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<float4 *>(prow + 32 * dt + 8 * rq + 4 * hl) =
            make_float4(o[dt][4 * rq], o[dt][4 * rq + 1], o[dt][4 * rq + 2], o[dt][4 * rq + 3]);
    if (hl == 0) *reinterpret_cast<float2 *>(prow + kD) = make_float2(M, L);
  }
}

// Merge split partials of one output row (query, head): 32 lanes x 4 elements.
__global__ __launch_bounds__(64) void int8_merge_kernel(const float *__restrict__ ws, int n_split,
                                                        int64_t n_rows, float *__restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 5);
  const int j = threadIdx.x & 31;
  if (row >= n_rows) return;
  const float *p = ws + row * n_split * kPartStride;
  float mg = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < n_split; ++s) {
    const float2 ml = *reinterpret_cast<const float2 *>(p + s * kPartStride + kD);
    if (ml.x == -INFINITY) continue;
    const float4 v = reinterpret_cast<const float4 *>(p + s * kPartStride)[j];
    const float mn = fmaxf(mg, ml.x);
    const float al = __builtin_amdgcn_exp2f(mg - mn);
    const float w = __builtin_amdgcn_exp2f(ml.x - mn);
    L = L * al + w * ml.y;
    acc.x = acc.x * al + w * v.x;
    acc.y = acc.y * al + w * v.y;
    acc.z = acc.z * al + w * v.z;
    acc.w = acc.w * al + w * v.w;
    mg = mn;
  }
  const float r = 1.0f / L;
  reinterpret_cast<float4 *>(out + row * kD)[j] = make_float4(acc.x * r, acc.y * r, acc.z * r, acc.w * r);
}

}  // namespace i8

hipError_t plan_int8(int64_t n_q, int32_t n_q_heads, int32_t n_kv_heads, int64_t ctx_len,
                     Int8Plan *p) {
  const int n_rep = n_q_heads / n_kv_heads;
  if (n_rep < 1 || i8::kQRows % n_rep != 0) return hipErrorNotSupported;
  int n_cu = 0;
  hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  p->queries_per_tile = i8::kQRows / n_rep;
  const int64_t q_tiles = ceil_div<int64_t>(n_q, p->queries_per_tile);
  if (q_tiles > 0x7fffffff) return hipErrorInvalidValue;
  p->n_q_tiles = (int)q_tiles;
  const int64_t max_tiles = ceil_div<int64_t>(ctx_len, i8::kKT);
  // one workgroup fills a compute unit (two waves per SIMD): split the key
  // range so that there is a workgroup for every compute unit, or, with more
  // workgroups than compute units, until their last round is 85% full
  const int64_t wgs = q_tiles * n_kv_heads;
  int64_t n_split = 1;
  if (wgs < n_cu) {
    n_split = ceil_div<int64_t>(n_cu, wgs);
  } else {
    while (n_split < 16) {
      const int64_t w = wgs * n_split, rounds = ceil_div<int64_t>(w, n_cu);
      if (w * 100 >= rounds * n_cu * 85) break;
      ++n_split;
    }
  }
  if (n_split > max_tiles) n_split = max_tiles;
  if (n_split > 65535) n_split = 65535;
  const int64_t tps = ceil_div<int64_t>(max_tiles, n_split);
  n_split = ceil_div<int64_t>(max_tiles, tps);
  p->keys_per_split = (int)(tps * i8::kKT);
  p->n_split = (int)n_split;
  p->workspace_bytes = n_split > 1 ? (((size_t)n_q * n_q_heads * n_split * i8::kPartStride *
                                       sizeof(float)) + 255) & ~(size_t)255
                                   : 0;
  return hipSuccess;
}

hipError_t launch_int8(const float *q, int64_t n_q, int32_t n_q_heads, const int8_t *k,
                       const int8_t *v, const uint16_t *k_scale, const uint16_t *v_scale,
                       int32_t n_kv_heads, const int32_t *page_table, int64_t n_phys_pages,
                       int64_t ctx_len, int64_t q_pos0, float scale, float *out, void *workspace,
                       const Int8Plan &p, hipStream_t stream) {
  i8::Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.ks = k_scale;
  a.vs = v_scale;
  a.pt = page_table;
  a.out = out;
  a.ws = reinterpret_cast<float *>(workspace);
  a.n_q = n_q;
  a.ctx_len = ctx_len;
  a.q_pos0 = q_pos0;
  a.n_phys_pages = n_phys_pages;
  a.n_q_heads = n_q_heads;
  a.n_kv = n_kv_heads;
  a.n_rep = n_q_heads / n_kv_heads;
  a.bq = p.queries_per_tile;
  a.n_split = p.n_split;
  a.tiles_per_split = p.keys_per_split / i8::kKT;
  a.qscale = scale * 1.4426950408889634f;  // log2 domain
  if (n_kv_heads > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)p.n_q_tiles, (unsigned)p.n_split, (unsigned)n_kv_heads);
  // element offsets of rows fit 32 bits when the whole paged cache does
  const bool off32 = (uint64_t)n_phys_pages * i8::kPage * (uint64_t)n_kv_heads * i8::kD < (1ull << 32);
  if (off32)
    hipLaunchKernelGGL(i8::int8_prompt_kernel<true>, grid, dim3(i8::kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(i8::int8_prompt_kernel<false>, grid, dim3(i8::kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  const int64_t rows = n_q * n_q_heads;
  hipLaunchKernelGGL(i8::int8_merge_kernel, dim3((unsigned)ceil_div<int64_t>(rows, 2)), dim3(64), 0,
                     stream, a.ws, p.n_split, rows, out);
  return hipGetLastError();
}

}  // namespace tq
