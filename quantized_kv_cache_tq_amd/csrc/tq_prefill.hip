// tq_prefill.hip -- causal multi-row attention over a turbo cache with the
// codes dequantized inside the tile load.
//
// [PR28] "Inline-dequant TILE prefill": the earlier path materialized the
// whole cache as float16 temporaries on every step; the fast path decodes the
// 3-bit K/V codes while loading each tile into shared memory.  Here each
// 64-key tile is decoded through the LDS pair table straight into two LDS
// tiles, K and V both as [key][d], as float16 values level * norm / 16: the
// group norm is folded
// into the tile, so the products need no per-key scaling.  Such a value is at
// most 2.8 * 65504 / 16 in magnitude, so it never overflows float16.  Nothing
// is written back to global memory but the output.
//
// Scales: the rotated coordinate of a group is level * norm / sqrt(128), and
// the query is rotated with the unnormalized transform H (sqrt(128) times the
// orthonormal one), so score = H(s.q) . Ktile / 8 and the output group is
// s . H(sum_k p_k Vtile_k) / (8 sum_k p_k).
//
// Products (v_mfma_f32_32x32x16_f16, fp32 accumulate):
//   S^T[key][qrow] = K[key][:] . Qrot[qrow][:]   A = K tile, B = rotated query
//   O^T[d][qrow]  += V^T[d][key] P^T[key][qrow]  A = V^T, B = P
// The V^T operand comes from the [key][d] tile by transposing LDS reads
// (ds_read_b64_tr_b16: within 16 lanes, lane j points at four consecutive d
// of one key and lane i receives d0 + i of four consecutive keys).
// A "qrow" is one (query row, query head) pair; the accumulator layout of S^T
// (one query column per lane pair) is the B-operand layout P needs, so the
// softmax never leaves registers.
//
// Workgroup: 64 qrows (64/n_rep query rows x n_rep heads of one kv head) and
// eight waves in two roles, one of each per SIMD:
//   * matrix waves 0-3 (qrow half x key half of every tile): scores, softmax,
//     P.V.  The scores of tile t+1 are issued together with the softmax of
//     tile t, so the exponentials overlap the matrix products.
//   * decode waves 4-7: turn the codes of later tiles into the float16 tiles
//     in the phase that does not read them (V looked up one tile ahead into
//     registers, the codes of each tile loaded two tiles ahead).
// Two barriers per tile separate the phases; each tile buffer is single:
//   A(t): matrix: S(t+1) from K, softmax(t)   decode: write V(t), look up V(t+1)
//   B(t): matrix: O += V(t) P(t)              decode: decode K(t+2) into K
// Causal balance: workgroup p processes query tiles p and T-1-p, so every
// workgroup sees about the same number of key tiles; when that grid would
// not give every compute unit a workgroup, each tile takes its own
// workgroup instead (one pass: the passes' fixed costs then outweigh the
// imbalance).  After the key loop all
// eight waves merge the two key halves and apply the inverse rotation.
#include "tq_common.h"
#include "tq_launch.h"

namespace tq {

namespace pf {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHalf = kThreads / 2;   // matrix threads; the rest decode
constexpr int kQRows = 64;            // qrows per workgroup
constexpr int kKT = 64;               // keys per tile
// key-half merge: per qrow half [d-tile][4 regs][64 lanes][4], d-tile
// stride padded by 16 floats so the reads of four d-tiles hit distinct banks
constexpr int kEDt = 16 * 64 + 16;
constexpr float kLazy = 8.f;          // the reference moves only past 2^8

// Sizes that follow the head dimension KD (256 or 128: one or two groups).
template <int KD>
struct Dims {
  static_assert(KD == 128 || KD == 256, "head_dim 128 or 256");
  static constexpr int NG = KD / 128;              // groups per key
  static constexpr int KsStride = KD + 8;          // halves per K row and per query row
  // halves per V row: 80 B of padding puts consecutive rows 20 banks apart.
  // The decode waves' row writes (one row per lane, 16 rows served together)
  // then hit distinct banks, and a transposing read's four rows overlap at
  // most pairwise, as they did 8 banks apart (32 B of padding), where the
  // writes conflicted pairwise too
  static constexpr int VsStride = KD + 40;
  static constexpr int KsHalves = kKT * KsStride;
  static constexpr int VsHalves = kKT * VsStride;
  static constexpr int QsHalves = kQRows * KsStride;
  static constexpr int TileHalves = KsHalves + VsHalves + QsHalves;
  static constexpr int NS = KD / 16;               // products per score tile
  static constexpr int ND = KD / 32;               // 32-row d-tiles of the output
  static constexpr int EK = KD / 4;                // K elements per decode thread (one key)
  static constexpr int EQ = KD / 4;                // query elements per matrix thread
  static constexpr int EE = KD / 8;                // output elements per thread
  static constexpr int EWave = ND * kEDt;          // merge floats per qrow half
  static_assert(2 * EWave * 4 <= TileHalves * 2, "merge buffer must fit in the tile buffers");
  static_assert(KsHalves <= VsHalves, "K tile 0 is staged in the V buffer");
  static_assert(kQRows * (KD + 4) * 4 <= TileHalves * 2, "the output staging must fit in the tile buffers");
};

// 32 sign bits of a group starting at element 32w (w = 0..3).
__device__ __forceinline__ uint32_t sign_word32(int w) {
  return (uint32_t)(((w >> 1) ? kSignWord1 : kSignWord0) >> (32 * (w & 1)));
}

__device__ __forceinline__ int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }

// Pair table: entry e (two B-bit codes, the first in the low bits) holds
// their two float16 levels, in C = 32 copies with copy c of entry e at dword
// 32e + c.  Lane l reads copy l % 32; an LDS 32-bit read serves 32 lanes at
// a time, so the lanes served together read distinct copies and hit distinct
// banks whatever their indices (measured as fast as 64 copies).  2 / 8 /
// 32 KB for 2 / 3 / 4-bit codes.
template <int B>
struct PfTable {
  static constexpr int C = 32;
  static constexpr int N = 1 << (2 * B);
  static constexpr int WORDS = N * C;
};

template <int B, int NT>
__device__ __forceinline__ void build_pf_table(uint32_t *tab, int tid) {
  using T = PfTable<B>;
  constexpr uint32_t CM = (1u << B) - 1u;
  static_assert(T::WORDS % NT == 0, "pair table fill");
#pragma unroll
  for (int j = 0; j < T::WORDS / NT; ++j) {
    const uint32_t e = (uint32_t)(tid + NT * j) / T::C;
    tab[tid + NT * j] = level_pair<B>(e & CM, e >> B);
  }
}

// A lane's view of the pair table: the table base and the byte offset of the
// lane's copy (4 c, below 128).  The byte offset of entry e in that copy,
// 128 e + 4 c, is formed with an OR: the 2B-bit code field (pos, NB
// compile-time after unrolling) is shifted straight to bit 7 and masked,
// then OR'ed with the lane's offset, two instructions per lookup.
struct TabRef {
  const uint32_t *base;
  uint32_t lane_off;
};

// Byte offset of the entry whose index is the nb-bit field at bit pos of dw.
template <int NB>
__device__ __forceinline__ uint32_t entry_off(const uint32_t *dw, int pos, uint32_t lane_off) {
  constexpr uint32_t M = ((1u << NB) - 1u) << 7;
  const int w = pos >> 5, sh = pos & 31;
  uint32_t x;
  if (sh + NB <= 32)
    x = sh >= 7 ? dw[w] >> (sh - 7) : dw[w] << (7 - sh);
  else
    x = __builtin_amdgcn_alignbit(dw[w + 1], dw[w], sh - 7);   // sh > 32 - NB >= 24
  return (x & M) | lane_off;
}

// The pair-table entry at byte offset off, scaled by the float16 pair n2 (the
// group norm / 16 in both halves).
__device__ __forceinline__ uint32_t pair_scaled(const TabRef &tab, uint32_t off, uint32_t n2) {
  const uint32_t lv = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const char *>(tab.base) + off);
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, lv) * __builtin_bit_cast(half2_t, n2));
}

// norm / 16 as float16, in both halves.
__device__ __forceinline__ uint32_t norm_pair(uint16_t h) {
  const _Float16 n = __builtin_bit_cast(_Float16, h) * (_Float16)0.0625f;
  const uint32_t b = __builtin_bit_cast(uint16_t, n);
  return b | (b << 16);
}

// Codes of one key tile (K or V) for a decode thread dt (0..255): key
// dt & 63, elements EK q .. EK q + EK - 1 with q = dt >> 6 (its decode wave).
template <int B, int KD>
struct KRaw {
  uint32_t c[KD * B / 128];
  uint16_t n;
};

struct Args {
  const uint8_t *kcodes;
  const uint16_t *knorms;
  const uint8_t *vcodes;
  const uint16_t *vnorms;
  int64_t n_cells, kv_len, n_rows, q_pos0;
  const void *q;
  float *out;
  int n_q, n_rep, bq, n_qtiles;
  int n_live;                 // live qrows per tile: n_rep * bq (<= 64)
  int paired;                 // 1: workgroup p also takes query tile n_qtiles - 1 - p
  // key splits (kSplit): workgroup z takes key tiles [z ks_tiles, (z+1) ks_tiles)
  // of each of its query tiles and writes partials [row][q head][split][KD + 4]
  // (16 * unnormalized rotated output, then the log2-domain maximum and the
  // weight sum) for the decode merge kernel
  int ks_tiles, n_split;
  float *ws;
  float qscale;
};

// Per-head code and norm bases (wave-uniform); key offsets from them are
// 32-bit (the host checks that a head's codes span less than 4 GiB).
struct HeadPtrs {
  const uint8_t *kc, *vc;
  const uint16_t *kn, *vn;
};

// Global loads (keys clamped to the last valid one: tiles past the end load
// valid rows, and their scores are masked).  A key's codes are its groups'
// codes back to back, so element e of the key starts at bit e * B.
template <int B, int KD>
__device__ __forceinline__ void load_row(const uint8_t *codes, const uint16_t *norms, int last, int kt, int dt,
                                         KRaw<B, KD> &r) {
  using D = Dims<KD>;
  const int q = dt >> 6;
  const uint32_t key = (uint32_t)min(kt * kKT + (dt & 63), last);
  const uint8_t *src = codes + key * (16u * B * D::NG) + (D::EK * B / 8) * q;
  if constexpr (KD == 256) {
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const u32x2_t v = reinterpret_cast<const u32x2_t *>(src)[i];
      r.c[2 * i] = v.x;
      r.c[2 * i + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < B; ++i) r.c[i] = reinterpret_cast<const uint32_t *>(src)[i];
  }
  r.n = norms[key * (uint32_t)D::NG + (D::EK * q) / 128];
}

// Rows of one tile (K or V): EK elements of one key, every pair-table read
// first (held in h), then written as 16-byte stores at row stride `stride`.
template <int B, int KD>
__device__ __forceinline__ void lookup_row(const KRaw<B, KD> &r, const TabRef &tab,
                                           uint32_t (&h)[Dims<KD>::EK / 2]) {
  using D = Dims<KD>;
  const uint32_t n2 = norm_pair(r.n);
#pragma unroll
  for (int j = 0; j < D::EK / 2; ++j) h[j] = pair_scaled(tab, entry_off<2 * B>(r.c, 2 * B * j, tab.lane_off), n2);
}

template <int KD>
__device__ __forceinline__ void write_row(const uint32_t (&h)[Dims<KD>::EK / 2], int dt, _Float16 *buf, int stride) {
  using D = Dims<KD>;
  u32x4_t *dst = reinterpret_cast<u32x4_t *>(buf + (dt & 63) * stride + D::EK * (dt >> 6));
#pragma unroll
  for (int v = 0; v < D::EK / 8; ++v) dst[v] = u32x4_t{h[4 * v], h[4 * v + 1], h[4 * v + 2], h[4 * v + 3]};
}

template <int B, int KD>
__device__ __forceinline__ void store_k(const KRaw<B, KD> &r, int dt, const TabRef &tab, _Float16 *ks) {
  uint32_t h[Dims<KD>::EK / 2];
  lookup_row<B, KD>(r, tab, h);
  write_row<KD>(h, dt, ks, Dims<KD>::KsStride);
}

// Four 16-bit values by a transposing LDS read (see the header).
__device__ __forceinline__ s16x4_t read_tr16(const _Float16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t *)p);
}

// S^T of this wave's 32 keys x 32 qrows over all KD dimensions.
template <int KD>
__device__ __forceinline__ f32x16_t scores(const _Float16 *krow, const _Float16 *qrow) {
  f32x16_t s;
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) s[rr] = 0.f;
#pragma unroll
  for (int t = 0; t < KD / 16; ++t)
    s = __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const half8_t *>(krow + 16 * t),
                                               *reinterpret_cast<const half8_t *>(qrow + 16 * t), s, 0, 0, 0);
  return s;
}

// One unnormalized 128-point transform step inside a thread's 2^L elements
// (stage h: pairs (i, i + h) for i with bit h clear).
template <int N>
__device__ __forceinline__ void wht_in_regs(float (&x)[N]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (!(i & h)) {
        const float u = x[i], v = x[i + h];
        x[i] = u + v;
        x[i + h] = u - v;
      }
}

template <int B, int KD, bool QBF16, bool kSplit>
__global__ __launch_bounds__(kThreads) void prefill_kernel(Args a) {
  using D = Dims<KD>;
  // (aligned to its size, which places it first, at LDS address 0: a
  // lookup's address is then its byte offset, with nothing added)
  __shared__ __align__(PfTable<B>::WORDS * 4) uint32_t ptab[PfTable<B>::WORDS];
  // the K tile, the V^T tile, the rotated query rows; after the key loop the
  // same bytes hold the key-half merge
  __shared__ __align__(16) _Float16 tiles[D::TileHalves];
  __shared__ float mst[2][kQRows], lst[2][kQRows];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = blockIdx.y;
  const int64_t head_base = (int64_t)g * a.n_cells;
  _Float16 *kbuf = tiles;
  _Float16 *vbuf = tiles + D::KsHalves;
  _Float16 *qbuf = vbuf + D::VsHalves;
  float *ebuf = reinterpret_cast<float *>(tiles);
  const TabRef tab = {ptab, 4u * (uint32_t)(lane % PfTable<B>::C)};   // this lane's pair-table copy

  build_pf_table<B, kThreads>(ptab, tid);
  __syncthreads();

  for (int pass = 0; pass < 2; ++pass) {
    const int qt = pass == 0 ? (int)blockIdx.x : a.n_qtiles - 1 - (int)blockIdx.x;
    if (pass == 1 && (!a.paired || qt == (int)blockIdx.x)) break;
    const int64_t row0 = (int64_t)qt * a.bq;
    const int64_t last_row = lmin(row0 + a.bq, a.n_rows) - 1;
    const int64_t kend = lmin(a.kv_len, a.q_pos0 + last_row + 1);
    const int n_kt = (int)ceil_div<int64_t>(kend, kKT);
    // tiles past this key need the causal mask (the first row sees keys <= pos_min)
    const int64_t pos_min = lmin(a.q_pos0 + row0, a.kv_len - 1);
    // this workgroup's key tiles [kt0, kt1)
    const int kt0 = kSplit ? (int)blockIdx.z * a.ks_tiles : 0;
    const int kt1 = kSplit ? min(kt0 + a.ks_tiles, n_kt) : n_kt;
    if (kSplit && kt0 >= kt1) {
      // no key of this range: an empty partial (maximum -inf, weight 0) per row
      constexpr int EE = D::EE, PE = 128 / EE;
      const int j = tid % PE, c = (tid / PE) & 63, grp = tid / (PE * 64);
      const int64_t r = row0 + c % a.bq;
      if (r < a.n_rows && c < a.n_live) {
        float *pr = a.ws + ((r * a.n_q + g * a.n_rep + c / a.bq) * a.n_split + blockIdx.z) * (KD + 4);
#pragma unroll
        for (int v = 0; v < EE / 4; ++v)
          reinterpret_cast<float4 *>(pr + 128 * grp + EE * j)[v] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j == 0 && grp == 0) *reinterpret_cast<float2 *>(pr + KD) = make_float2(-INFINITY, 0.f);
      }
      continue;
    }

    if (wave < 4) {
      // ================================================= matrix waves
      const int qhalf = wave & 1, khalf = wave >> 1;
      const int ql = lane & 31, hl = lane >> 5;
      {
        // ---- rotated query rows: thread (pi, c, grp) owns elements
        //      EQ pi .. EQ pi + EQ - 1 of group grp of qrow c
        constexpr int EQ = D::EQ, PP = 128 / EQ;
        const int pi = tid % PP, c = (tid / PP) & 63, grp = tid / (PP * 64);
        // (a qrow past the last live one, when n_rep does not divide 64, reads
        // a live head's row and its result is never stored)
        const int hq = min(c / a.bq, a.n_rep - 1), rq = c % a.bq;
        const int64_t rr = lmin(row0 + rq, a.n_rows - 1);
        const int64_t off = (rr * a.n_q + g * a.n_rep + hq) * KD + 128 * grp + EQ * pi;
        float x[EQ];
        if constexpr (QBF16) {
          const u32x4_t *src = reinterpret_cast<const u32x4_t *>(reinterpret_cast<const uint16_t *>(a.q) + off);
#pragma unroll
          for (int v = 0; v < EQ / 8; ++v) {
            const u32x4_t b = src[v];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              x[8 * v + 2 * k] = __uint_as_float(b[k] << 16);
              x[8 * v + 2 * k + 1] = __uint_as_float(b[k] & 0xffff0000u);
            }
          }
        } else {
          const float4 *src = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.q) + off);
#pragma unroll
          for (int v = 0; v < EQ / 4; ++v) {
            const float4 f = src[v];
            x[4 * v] = f.x; x[4 * v + 1] = f.y; x[4 * v + 2] = f.z; x[4 * v + 3] = f.w;
          }
        }
        uint32_t sw[EQ / 32];
#pragma unroll
        for (int w = 0; w < EQ / 32; ++w) sw[w] = sign_word32((EQ / 32) * pi + w);
        // opaque, so the sign masks are formed here and not hoisted out of
        // the pass loop (where they would be spilled)
#pragma unroll
        for (int w = 0; w < EQ / 32; ++w) asm volatile("" : "+v"(sw[w]));
#pragma unroll
        for (int e = 0; e < EQ; ++e) x[e] = flip_sign(x[e], (sw[e >> 5] >> (e & 31)) & 1u);
        wht_in_regs<EQ>(x);
#pragma unroll
        for (int e = 0; e < EQ; ++e) x[e] = bfly_lane<1>(x[e], (pi & 1) != 0);
        if constexpr (PP > 2) {
#pragma unroll
          for (int e = 0; e < EQ; ++e) x[e] = bfly_lane<2>(x[e], (pi & 2) != 0);
        }
        u32x4_t *dst = reinterpret_cast<u32x4_t *>(qbuf + c * D::KsStride + 128 * grp + EQ * pi);
#pragma unroll
        for (int v = 0; v < EQ / 8; ++v) {
          uint32_t w[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const _Float16 lo = (_Float16)(x[8 * v + 2 * k] * a.qscale);
            const _Float16 hi = (_Float16)(x[8 * v + 2 * k + 1] * a.qscale);
            w[k] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
          dst[v] = u32x4_t{w[0], w[1], w[2], w[3]};
        }
      }
      const int qrow = 32 * qhalf + ql;
      const int64_t r = row0 + qrow % a.bq;
      const int64_t pos = lmin(a.q_pos0 + r, a.kv_len - 1);   // last key this column sees
      const _Float16 *qrow_p = qbuf + qrow * D::KsStride + 8 * hl;
      const int koff = (32 * khalf + ql) * D::KsStride + 8 * hl;
      __syncthreads();   // query rows, K tiles 0 (in the V buffer) and 1 ready
      f32x16_t sa = scores<KD>(vbuf + koff, qrow_p), sb;
      __syncthreads();   // K tile 0 read: the V buffer may take V tile 0

      constexpr int ND = D::ND, NS = D::NS;
      f32x16_t o[ND];
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[dt][rr] = 0.f;
      float m_run = -INFINITY, l_run = 0.f;

      auto step = [&](int kt, const f32x16_t &cur, f32x16_t &nxt) {
        half8_t pb[2];
        float alpha = 1.f;
        // phase A: scores of tile kt+1 (past the end: unused) with the
        // softmax of tile kt
        auto phase_a = [&](auto mask_tag) {
          constexpr bool kMask = decltype(mask_tag)::value;
          // distinct markers keep the two variants from sharing (and hoisting
          // above the branch) their operand reads
          if constexpr (kMask)
            asm volatile("; masked tile" ::: "memory");
          else
            asm volatile("; full tile" ::: "memory");
          // scores of tile kt+1: operands three products ahead in a 4-slot
          // ring, two accumulators (even/odd d-steps) so consecutive products
          // do not wait on each other; the softmax of tile kt runs in NS
          // slices between the products (maxima, then exponentials)
          constexpr int HS = NS / 2, PER = 16 / HS;
          const _Float16 *kb = kbuf + koff;
          half8_t ka[4], qa[4];
#pragma unroll
          for (int i = 0; i < 3; ++i) {
            ka[i] = *reinterpret_cast<const half8_t *>(kb + 16 * i);
            qa[i] = *reinterpret_cast<const half8_t *>(qrow_p + 16 * i);
          }
          f32x16_t s0, s1;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) { s0[rr] = 0.f; s1[rr] = 0.f; }
          // register rr <-> key 8(rr/4) + 4hl + rr%4 of this wave's half
          const int64_t lim64 = pos - ((int64_t)kt * kKT + 32 * khalf);
          const int lim = lim64 > 64 ? 64 : (int)lim64;
          float v[16], tmax = -INFINITY, m_use = 0.f, psum = 0.f;
#pragma unroll
          for (int t = 0; t < NS; ++t) {
            if (t + 3 < NS) {
              ka[(t + 3) & 3] = *reinterpret_cast<const half8_t *>(kb + 16 * (t + 3));
              qa[(t + 3) & 3] = *reinterpret_cast<const half8_t *>(qrow_p + 16 * (t + 3));
            }
            if (t & 1)
              s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[t & 3], qa[t & 3], s1, 0, 0, 0);
            else
              s0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[t & 3], qa[t & 3], s0, 0, 0, 0);
            if (t < HS) {
#pragma unroll
              for (int e = PER * t; e < PER * t + PER; ++e) {
                v[e] = cur[e];
                if (kMask && 8 * (e >> 2) + 4 * hl + (e & 3) > lim) v[e] = -INFINITY;
              }
#pragma unroll
              for (int e = PER * t; e < PER * t + PER; e += 2) tmax = fmaxf(tmax, fmaxf(v[e], v[e + 1]));
            }
            if (t == HS - 1) {
              tmax = max_xor32(tmax);
              // lazy reference: it moves only when a score passes it by
              // 2^kLazy, so P <= 2^kLazy and rescales are rare
              const float m_new = tmax > m_run + kLazy ? tmax : m_run;
              m_use = m_new == -INFINITY ? 0.f : m_new;
              alpha = __builtin_amdgcn_exp2f(m_run - m_use);
              m_run = m_new;
            }
            if (t >= HS) {
#pragma unroll
              for (int e = PER * (t - HS); e < PER * (t - HS) + PER; e += 2) {
                const float p0 = __builtin_amdgcn_exp2f(v[e] - m_use);
                const float p1 = __builtin_amdgcn_exp2f(v[e + 1] - m_use);
                psum += p0 + p1;
                pb[e >> 3][e & 7] = (_Float16)p0;
                pb[e >> 3][(e & 7) + 1] = (_Float16)p1;
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
          l_run = l_run * alpha + psum;
          nxt = s0 + s1;
        };
        if ((int64_t)kt * kKT + kKT - 1 > pos_min)
          phase_a(std::true_type{});
        else
          phase_a(std::false_type{});
        if (__builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
          for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) o[dt][rr] *= alpha;
        }
        __syncthreads();   // V tile kt written; K tile kt+1 read
        // phase B: O^T += V^T P^T; k-slot (hl, i) of step ga <-> key
        // 16ga + 8(i>>2) + 4hl + (i&3).  Products in the order (ga, dt), so
        // no two consecutive ones share an accumulator; V^T operands three
        // products ahead.  An operand is two transposing reads of the
        // [key][d] tile: lane j of each 16-lane group points at d 16 (g & 1)
        // + 4 (j & 3) .. + 3 of key 4 hl + (j >> 2) (g = lane >> 4), so lane
        // i of the group receives d 16 (g & 1) + i, that is ql, of the four
        // keys of its k-slots 4r .. 4r + 3
        const int trg = lane >> 4, trj = lane & 15;
        const _Float16 *vtr =
            vbuf + (32 * khalf + 4 * hl + (trj >> 2)) * D::VsStride + 16 * (trg & 1) + 4 * (trj & 3);
        auto vop = [&](int idx) {
          const _Float16 *vr = vtr + 16 * (idx / ND) * D::VsStride + 32 * (idx % ND);
          const s16x4_t lo = read_tr16(vr);                      // keys 16 ga + 4 hl + 0..3
          const s16x4_t hi = read_tr16(vr + 8 * D::VsStride);    // keys 16 ga + 8 + 4 hl + 0..3
          return __builtin_bit_cast(half8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        half8_t va[4];
#pragma unroll
        for (int i = 0; i < 3; ++i) va[i] = vop(i);
#pragma unroll
        for (int idx = 0; idx < 2 * ND; ++idx) {
          if (idx + 3 < 2 * ND) va[(idx + 3) & 3] = vop(idx + 3);
          o[idx % ND] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[idx & 3], pb[idx / ND], o[idx % ND], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();   // V tile kt consumed; K tile kt+2 written
      };
      for (int kt = kt0; kt < kt1; kt += 2) {
        step(kt, sa, sb);
        if (kt + 1 < kt1) step(kt + 1, sb, sa);
      }

      // ---- merge the key halves: khalf 1 hands its partial output to
      //      khalf 0, which writes the normalized sum back in place
      l_run += xor_lane<32>(l_run);
      float *ew = ebuf + qhalf * D::EWave + lane * 4;
      if (hl == 0) {
        mst[khalf][qrow] = m_run;
        lst[khalf][qrow] = l_run;
      }
      if (khalf == 1) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq)
            *reinterpret_cast<float4 *>(ew + dt * kEDt + rq * 256) =
                float4{o[dt][4 * rq], o[dt][4 * rq + 1], o[dt][4 * rq + 2], o[dt][4 * rq + 3]};
      }
      __syncthreads();   // partial outputs and statistics in shared memory
      if (khalf == 0) {
        const float m2 = mst[1][qrow], l2 = lst[1][qrow];
        const float M = fmaxf(m_run, m2);
        const float f1 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
        const float f2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
        // a split keeps 16 x the unnormalized sum and its statistics (the
        // merge divides by 128 L: the output's 1 / (8 L))
        float g1, g2;
        if constexpr (kSplit) {
          g1 = 16.f * f1;
          g2 = 16.f * f2;
          if (hl == 0) {
            mst[0][qrow] = M;
            lst[0][qrow] = l_run * f1 + l2 * f2;
          }
        } else {
          const float rinv = 1.0f / (8.0f * (l_run * f1 + l2 * f2));
          g1 = f1 * rinv;
          g2 = f2 * rinv;
        }
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            float4 *ptr = reinterpret_cast<float4 *>(ew + dt * kEDt + rq * 256);
            const float4 u = *ptr;
            *ptr = float4{o[dt][4 * rq] * g1 + u.x * g2, o[dt][4 * rq + 1] * g1 + u.y * g2,
                          o[dt][4 * rq + 2] * g1 + u.z * g2, o[dt][4 * rq + 3] * g1 + u.w * g2};
          }
      }
    } else {
      // ================================================= decode waves
      const int dt = tid - kHalf;
      int last = (int)(a.kv_len - 1);
      asm volatile("" : "+s"(last));   // keeps tile addresses in the pass (not hoisted, spilled)
      HeadPtrs hp;
      hp.kc = a.kcodes + head_base * (16 * B * D::NG);
      hp.vc = a.vcodes + head_base * (16 * B * D::NG);
      hp.kn = a.knorms + head_base * D::NG;
      hp.vn = a.vnorms + head_base * D::NG;
      // raw codes in three register sets per cache that rotate roles every
      // tile (the loop runs three tiles per trip): a tile's codes are loaded
      // two tiles before their lookups, and a load never targets registers
      // whose previous contents are still to be used (with one set, the
      // compiler issued each load into fresh registers and copied them back
      // at the end of the phase, which waited for the load there).  Loads
      // retire in order; the issue order V(j), K(j+1), V(j+1), ... lets each
      // phase wait for its own tile's codes with the next two tiles' loads
      // still in flight
      KRaw<B, KD> ka, kb, kc, va, vb, vc;
      uint32_t vw[D::EK / 2];
      load_row<B, KD>(hp.kc, hp.kn, last, kt0, dt, ka);
      load_row<B, KD>(hp.kc, hp.kn, last, min(kt0 + 1, kt1 - 1), dt, kb);
      load_row<B, KD>(hp.vc, hp.vn, last, kt0, dt, va);
      store_k<B, KD>(ka, dt, tab, vbuf);   // K tile 0 goes where V tile 0 will
      store_k<B, KD>(kb, dt, tab, kbuf);
      lookup_row<B, KD>(va, tab, vw);
      // loads are unconditional (tile index clamped): a conditional load
      // would merge into the loop-carried registers through copies that wait
      // for the data
      load_row<B, KD>(hp.vc, hp.vn, last, min(kt0 + 1, kt1 - 1), dt, va);
      load_row<B, KD>(hp.kc, hp.kn, last, min(kt0 + 2, kt1 - 1), dt, ka);
      load_row<B, KD>(hp.vc, hp.vn, last, min(kt0 + 2, kt1 - 1), dt, vb);
      load_row<B, KD>(hp.kc, hp.kn, last, min(kt0 + 3, kt1 - 1), dt, kb);
      __syncthreads();   // query rows, K tiles 0 (in the V buffer) and 1 ready
      __syncthreads();   // K tile 0 read: the V buffer may take V tile 0
      // one tile: vcur holds V tile kt+1, kcur K tile kt+2; vnew and knew
      // receive V tile kt+3 and K tile kt+4
      auto tile = [&](int kt, KRaw<B, KD> &vcur, KRaw<B, KD> &vnew, KRaw<B, KD> &kcur, KRaw<B, KD> &knew) {
        // phase A: V tile kt into the buffer, look up V tile kt+1
        write_row<KD>(vw, dt, vbuf, D::VsStride);
        lookup_row<B, KD>(vcur, tab, vw);   // past the end: never written
        load_row<B, KD>(hp.vc, hp.vn, last, min(kt + 3, kt1 - 1), dt, vnew);
        __syncthreads();   // V tile kt written; K tile kt+1 read
        // phase B: K tile kt+2 into the (now free) K buffer
        if (kt + 2 < kt1) store_k<B, KD>(kcur, dt, tab, kbuf);
        load_row<B, KD>(hp.kc, hp.kn, last, min(kt + 4, kt1 - 1), dt, knew);
        __syncthreads();   // V tile kt consumed; K tile kt+2 written
      };
      // whole trips only, so the loop is entered and re-entered with the
      // same loads in flight in the same order (the wait before each lookup
      // then leaves the later tiles' loads outstanding); then the 0-2 tiles
      // left
      int kt = kt0;
      for (; kt + 3 <= kt1; kt += 3) {
        tile(kt, va, vc, ka, kc);
        tile(kt + 1, vb, va, kb, ka);
        tile(kt + 2, vc, vb, kc, kb);
      }
      if (kt < kt1) {
        tile(kt, va, vc, ka, kc);
        if (kt + 1 < kt1) tile(kt + 1, vb, va, kb, ka);
      }
      __syncthreads();   // partial outputs and statistics in shared memory
    }
    __syncthreads();   // merged output in shared memory

    // ---- merge, normalize, inverse transform: thread (j, c, grp) owns
    //      elements EE j .. EE j + EE - 1 of group grp of qrow c
    {
      constexpr int EE = D::EE, PE = 128 / EE;
      const int j = tid % PE, c = (tid / PE) & 63, grp = tid / (PE * 64);
      const int qh = c >> 5, ql = c & 31;
      const int d0 = 128 * grp + EE * j;   // first element (its d-tile: d0 / 32)
      const float *e0 = ebuf + qh * D::EWave + (d0 >> 5) * kEDt + ((d0 & 31) >> 3) * 256;
      float x[EE];
#pragma unroll
      for (int rq = 0; rq < EE / 8; ++rq)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          // element 8rq + 4hh + i of the d-tile <-> register 4rq + i of lane
          // ql + 32hh
          const float4 u = *reinterpret_cast<const float4 *>(e0 + rq * 256 + (ql + 32 * hh) * 4);
          x[8 * rq + 4 * hh + 0] = u.x;
          x[8 * rq + 4 * hh + 1] = u.y;
          x[8 * rq + 4 * hh + 2] = u.z;
          x[8 * rq + 4 * hh + 3] = u.w;
        }
      if constexpr (kSplit) {
        const int64_t r = row0 + c % a.bq;
        if (r < a.n_rows && c < a.n_live) {
          float *pr = a.ws + ((r * a.n_q + g * a.n_rep + c / a.bq) * a.n_split + blockIdx.z) * (KD + 4);
#pragma unroll
          for (int v = 0; v < EE / 4; ++v)
            reinterpret_cast<float4 *>(pr + 128 * grp + EE * j)[v] =
                make_float4(x[4 * v], x[4 * v + 1], x[4 * v + 2], x[4 * v + 3]);
          if (j == 0 && grp == 0) *reinterpret_cast<float2 *>(pr + KD) = make_float2(mst[0][c], lst[0][c]);
        }
        __syncthreads();   // merge buffer read: the tiles may be overwritten
        continue;
      }
      wht_in_regs<EE>(x);
#pragma unroll
      for (int e = 0; e < EE; ++e) x[e] = bfly_lane<1>(x[e], (j & 1) != 0);
#pragma unroll
      for (int e = 0; e < EE; ++e) x[e] = bfly_lane<2>(x[e], (j & 2) != 0);
      if constexpr (PE > 4) {
#pragma unroll
        for (int e = 0; e < EE; ++e) x[e] = bfly_lane<4>(x[e], (j & 4) != 0);
      }
      // the finished rows go through LDS ([qrow][KD + 4] floats over the
      // tile buffers) so that each store instruction writes whole output
      // rows: stored straight from this layout, an instruction covered 16
      // rows in 16-byte pieces 128 bytes apart (measured: the output stores
      // cost 10 us of a 2048-row call)
      __syncthreads();   // every thread has read its part of the merge buffer
      constexpr int SS = KD + 4;   // staging row stride (floats)
      float *stg = reinterpret_cast<float *>(tiles);
      {
        uint32_t sw = sign_word32((EE * j) >> 5) >> ((EE * j) & 31);
        asm volatile("" : "+v"(sw));   // formed here, not hoisted and spilled
        float4 *dst = reinterpret_cast<float4 *>(stg + c * SS + d0);
#pragma unroll
        for (int v = 0; v < EE / 4; ++v) {
          float4 f;
          f.x = flip_sign(x[4 * v + 0], (sw >> (4 * v + 0)) & 1u);
          f.y = flip_sign(x[4 * v + 1], (sw >> (4 * v + 1)) & 1u);
          f.z = flip_sign(x[4 * v + 2], (sw >> (4 * v + 2)) & 1u);
          f.w = flip_sign(x[4 * v + 3], (sw >> (4 * v + 3)) & 1u);
          dst[v] = f;
        }
      }
      __syncthreads();   // staged rows complete
      // wave w stores qrows 8w .. 8w + 7, RPI rows per instruction
      constexpr int RPI = 256 / KD, LPR = 64 / RPI;
#pragma unroll
      for (int i = 0; i < 8 / RPI; ++i) {
        const int cc = 8 * wave + RPI * i + lane / LPR;
        const int64_t rr = row0 + cc % a.bq;
        if (rr < a.n_rows && cc < a.n_live) {
          const float4 f = *reinterpret_cast<const float4 *>(stg + cc * SS + 4 * (lane % LPR));
          reinterpret_cast<float4 *>(a.out + (rr * a.n_q + g * a.n_rep + cc / a.bq) * KD)[lane % LPR] = f;
        }
      }
    }
    __syncthreads();   // merge buffer read: the tiles may be overwritten
  }
}

}  // namespace pf

hipError_t plan_prefill(const tq_cache &k, int64_t n_rows, int32_t n_q_heads, int64_t kv_len,
                        PrefillPlan *p) {

  const int n_rep = n_q_heads / k.n_kv_heads;
  if (n_rep < 1 || n_rep > 8) return hipErrorNotSupported;
  // key offsets inside one head are 32-bit
  if (k.n_cells > (int64_t)(0xffffffffu / (32u * 4))) return hipErrorNotSupported;
  // query rows per tile: the tile's 64 qrows hold bq rows of n_rep heads;
  // when n_rep does not divide 64 the last 64 - n_rep bq qrows are idle
  p->rows_per_tile = pf::kQRows / n_rep;
  const int64_t tiles = ceil_div<int64_t>(n_rows, p->rows_per_tile);
  if (tiles > 0x3fffffff) return hipErrorInvalidValue;
  p->n_row_tiles = (int)tiles;
  int n_cu = 0;
  const hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  p->paired = ceil_div<int64_t>(tiles, 2) * k.n_kv_heads >= n_cu ? 1 : 0;
  p->keys_per_split = 0;
  p->max_splits = 1;
  p->workspace_bytes = 0;
  // Key splits when the grid leaves most compute units idle and the rows see
  // many key tiles (rows after a long prefix): each split takes a
  // power-of-two number (>= 8) of key tiles, partials merged by a second
  // kernel; sized for kv_len and capped at 256 MiB of partials.
  const int64_t base = (p->paired ? ceil_div<int64_t>(tiles, 2) : tiles) * k.n_kv_heads;
  const int64_t max_kt = ceil_div<int64_t>(kv_len, pf::kKT);
  if (2 * base <= n_cu && max_kt >= 16) {
    int64_t want = n_cu / base;   // the split grid stays one round
    if (want > max_kt / 8) want = max_kt / 8;
    int64_t ks = 8;
    while (ks * want < max_kt) ks *= 2;
    const size_t per_split = (size_t)n_rows * (size_t)n_q_heads * (size_t)(k.head_dim + 4) * sizeof(float);
    int64_t n_split = ceil_div<int64_t>(max_kt, ks);
    while (n_split > 1 && (size_t)n_split * per_split > (size_t(256) << 20)) {
      ks *= 2;
      n_split = ceil_div<int64_t>(max_kt, ks);
    }
    if (n_split > 1 && n_split <= 65535) {
      p->keys_per_split = (int)(ks * pf::kKT);
      p->max_splits = (int)n_split;
      p->workspace_bytes = ((size_t)n_split * per_split + 255) & ~(size_t)255;
    }
  }
  return hipSuccess;
}

hipError_t launch_prefill(const tq_cache &k, const tq_cache &v, int64_t kv_len, const void *q,
                          int q_dtype, int64_t n_rows, int32_t n_q_heads, int64_t q_pos0,
                          float scale, float *out, void *workspace, const PrefillPlan &p,
                          hipStream_t stream) {

  pf::Args a;
  a.kcodes = k.codes;
  a.knorms = k.norms;
  a.vcodes = v.codes;
  a.vnorms = v.norms;
  a.n_cells = k.n_cells;
  a.kv_len = kv_len;
  a.n_rows = n_rows;
  a.q_pos0 = q_pos0;
  a.q = q;
  a.out = out;
  a.n_q = n_q_heads;
  a.n_rep = n_q_heads / k.n_kv_heads;
  a.bq = p.rows_per_tile;
  a.n_live = a.n_rep * a.bq;
  a.n_qtiles = p.n_row_tiles;
  a.paired = p.paired;
  const bool split = p.max_splits > 1;
  a.n_split = p.max_splits;
  a.ks_tiles = split ? p.keys_per_split / pf::kKT : 0;
  a.ws = reinterpret_cast<float *>(workspace);
  // log2 domain; 1/8 for the transform and tile scales (score = H(s.q) . K / 8)
  a.qscale = scale * 1.4426950408889634f / 8.0f;
  dim3 grid((unsigned)(p.paired ? ceil_div(p.n_row_tiles, 2) : p.n_row_tiles), (unsigned)k.n_kv_heads,
            (unsigned)p.max_splits);
  dim3 block(pf::kThreads);
#define TQ_PF_Q(B, KD, QB)                                                                        \
  do {                                                                                            \
    if (split)                                                                                    \
      hipLaunchKernelGGL((pf::prefill_kernel<B, KD, QB, true>), grid, block, 0, stream, a);      \
    else                                                                                          \
      hipLaunchKernelGGL((pf::prefill_kernel<B, KD, QB, false>), grid, block, 0, stream, a);     \
  } while (0)
#define TQ_PF(B, KD)                       \
  do {                                     \
    if (q_dtype == TQ_BF16)                \
      TQ_PF_Q(B, KD, true);                \
    else                                   \
      TQ_PF_Q(B, KD, false);               \
  } while (0)
#define TQ_PF_TYPES(KD)                  \
  switch (k.type) {                      \
    case TQ_TURBO2: TQ_PF(2, KD); break; \
    case TQ_TURBO3: TQ_PF(3, KD); break; \
    case TQ_TURBO4: TQ_PF(4, KD); break; \
    default: return hipErrorNotSupported; \
  }
  if (k.head_dim == 256)
    TQ_PF_TYPES(256)
  else if (k.head_dim == 128)
    TQ_PF_TYPES(128)
  else
    return hipErrorNotSupported;
#undef TQ_PF_TYPES
#undef TQ_PF
#undef TQ_PF_Q
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  return launch_split_merge(a.ws, p.max_splits, __builtin_ctz((unsigned)p.keys_per_split), k.head_dim,
                            n_rows * n_q_heads, out, stream);
}

}  // namespace tq
