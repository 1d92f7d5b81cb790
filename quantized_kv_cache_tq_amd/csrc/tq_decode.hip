// tq_decode.hip -- decode attention (one query row) over a turbo cache.
//
// [PR36] (c) decodes with a per-query-head Q x centroid table in shared
// memory (one shared read per element and head).  With eight query heads per
// kv head that is eight table reads per cache element, far more LDS traffic
// than the packed stream itself.  On CDNA4 the eight heads are one dense
// contraction instead: every packed code is decoded ONCE per kv head into
// the float16 hi and lo parts of its level through a table in LDS (indexed
// by the concatenated codes of 2 neighbouring elements, so one LDS read
// yields both parts of 2 levels), and the matrix cores do Q.K^T and P.V for
// all heads of the kv head at once.
//
// One 16-key tile in a wave (v_mfma_f32_16x16x32_f16 for scores,
// v_mfma_f32_16x16x16_f16 for values):
//   scores  S^T[key][col] = K[key][:] . Qcol[:]; column c < 8 is the high
//           float16 half of head c's rotated query, column 8 + c its low half
//           (q = hi + lo keeps ~22 bits of the float32 query);
//   values  O[row][d] += P[row][key] V[key][d]; rows < 8 hold the high half of
//           p * vnorm, rows >= 8 the low half.  V's 8 d-tiles take element
//           8n + t in column n of tile t, so a lane decodes 8 consecutive
//           elements of 4 keys.
// A level (a float32 value) enters both products as its float16 hi and lo
// parts, one product each into the same accumulator, so every operand
// carries about 22 bits and the roundings that matter are float32
// accumulation and the exponential.
//
// Work split ([PR36] (d) raised occupancy to hide load latency; on MI355X the
// split-K grid and up-front loads do that job): workgroup (split s, kv head g)
// owns keys [s*KPS, (s+1)*KPS).  At entry every thread issues all its global
// loads (K and V codes as 16-byte chunks, norms, the level table, the query),
// so one HBM round trip covers the whole tile; K is staged to LDS and scored
// while the V loads are still in flight.  The eight waves score every key,
// take one workgroup-wide max per head (no rescaling), then accumulate
// values.  decode_merge_kernel merges the splits and rotates back.
#include "tq_common.h"
#include "tq_launch.h"

namespace tq {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecWaves = 8;
constexpr int kDecThreads = 64 * kDecWaves;
// A split partial is o[head width], m, l, pad: head width + 4 floats
// (16-byte rows).
__host__ __device__ constexpr int part_stride(int dv) { return dv + 4; }


// Bits [pos, pos+nbits) of a little-endian dword array (pos and nbits are
// compile-time after unrolling; the field spans at most two dwords).
__device__ __forceinline__ uint32_t bits_at(const uint32_t *dw, int pos, int nbits) {
  const int w = pos >> 5, sh = pos & 31;
  uint32_t x = dw[w] >> sh;
  if (sh + nbits > 32) x |= dw[w + 1] << (32 - sh);
  return nbits == 32 ? x : (x & ((1u << nbits) - 1u));
}

// Decode NEL consecutive elements held in dw (first element in bit 0)
// through the pair table into float16 pairs: hi[0 .. NEL/2) and lo[0 ..
// NEL/2) hold the hi and lo parts of the levels.  tab points at this lane's
// copy (8-byte slot lane % 32 of the table).
template <int B, int NEL>
__device__ __forceinline__ void decode_pairs_hl(const uint32_t *dw, const u32x2_t *tab, uint32_t *hi,
                                                uint32_t *lo) {
  constexpr int PB = 2 * B;
#pragma unroll
  for (int j = 0; j < NEL / 2; ++j) {
    const u32x2_t v = tab[bits_at(dw, PB * j, PB) * PairCfg<B>::COPIES];
    hi[j] = v.x;
    lo[j] = v.y;
  }
}
// One part only (tab: this lane's hi dword, or lo dword, of the table).
template <int B, int NEL>
__device__ __forceinline__ void decode_pairs(const uint32_t *dw, const uint32_t *tab, uint32_t *out) {
  constexpr int PB = 2 * B;
#pragma unroll
  for (int j = 0; j < NEL / 2; ++j) out[j] = tab[bits_at(dw, PB * j, PB) * (2 * PairCfg<B>::COPIES)];
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }

// Keeps the compiler from moving LDS accesses across this point; LDS
// operations of one wave execute in order, so other lanes' earlier writes
// are visible to later reads of the same wave.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Four int8 codes (one dword, first in the low byte) -> four exact float16
// values as two half2 dwords: byte ^ 0x80 is code + 128 in [0, 255]; placed
// under the exponent bits of 1024 it reads 1024 + code + 128, and
// subtracting 1152 leaves the code.
__device__ __forceinline__ u32x2_t i8x4_to_half4(uint32_t w) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const uint32_t x = w ^ 0x80808080u;
  const h2_t bias = {(_Float16)1152.f, (_Float16)1152.f};
  const h2_t lo = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, x, 0x04010400u)) - bias;
  const h2_t hi = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, x, 0x04030402u)) - bias;
  return u32x2_t{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// The cells of sequence z: [start, start + len) of every kv head.  Without
// arrays, one sequence of kv_len cells from cell 0; with them, the entries
// are clamped so that no access leaves the cache (start into [0, n_cells],
// len into [0, min(max_len, n_cells - start)]).
struct SeqExtent {
  int64_t start, len;
};
__device__ __forceinline__ SeqExtent seq_extent(const int64_t *seq_start, const int32_t *seq_len, int z,
                                                int64_t kv_len, int64_t n_cells) {
  if (!seq_len) return SeqExtent{0, kv_len};
  int64_t a = seq_start[z], n = seq_len[z];
  a = a < 0 ? 0 : (a > n_cells ? n_cells : a);
  const int64_t cap = kv_len < n_cells - a ? kv_len : n_cells - a;
  n = n < 0 ? 0 : (n > cap ? cap : n);
  return SeqExtent{a, n};
}

// Workgroup (split s, kv head g): eight waves, four key ranges of KPW = 16T
// keys.  Waves 0-3 ("key waves") score their range and turn the scores into
// the matrix-core operand P; waves 4-7 ("value waves") meanwhile decode the
// V codes of the same ranges into B operands held in registers.  After one
// barrier every value wave runs its value products; the four partial
// outputs are merged in shared memory and written as one split partial.
// K rows hold GK and V rows GV 128-element groups (head widths 128 GK and
// 128 GV, which may differ): a score sums its K groups' products, each
// scaled by that group's norm, and P has one operand per V group (p times
// that group's norm), the V groups taking their products one after another.
// The HP (8 or 16) heads of a workgroup are (query row, q head) pairs:
// sequence z = blockIdx.z has n_rows query rows, row r seeing the sequence's
// cells j <= len - n_rows + r, and a kv head's n_rows * n_rep pairs are cut
// into head groups of HP (blockIdx.y = kv head * n_hg + head group).  Sixteen
// pairs form two column sets of eight that share one decode of the K and V
// codes, each set with its own score and value products.  Splits past the
// sequence's length exit at once and write nothing.
// KQ8: K in the 8-bit block format ([PR36] (b): an asymmetric cache's K in
// 8-bit blocks beside the turbo V of type B).  Such K is not rotated, so the
// query is not either; a key row's 32-element blocks map onto the 32 k-slots
// of one product each (k-slot (lane >> 4, i) of K-step st <-> element 32 st +
// 8 (lane >> 4) + i), and each product is scaled by its block's scale.
template <int B, int T, int GK, int GV, bool QBF16, bool KQ8, int HP>
__global__ __launch_bounds__(kDecThreads, 2) void decode_split_kernel(
    const uint8_t *__restrict__ kcodes, const uint16_t *__restrict__ knorms,
    const uint8_t *__restrict__ vcodes, const uint16_t *__restrict__ vnorms, int64_t n_cells,
    const int64_t *__restrict__ seq_start, const int32_t *__restrict__ seq_len, int64_t kv_len,
    const void *__restrict__ q, int n_q, int n_rep, int n_rows, int n_hg, float qscale, float tau,
    float *__restrict__ ws, int n_split) {
  constexpr int DV = kGroup * GV;              // output width
  constexpr int KPW = 16 * T;                  // keys per range
  constexpr int KPS = 4 * KPW;                 // keys per split
  constexpr int GW = 4 * B;                    // code dwords per group
  constexpr int ROWP = GV * GW + 1;            // padded LDS V row
  constexpr int RPL = ceil_div(KPW, 64);       // V rows per lane
  constexpr int NNORM = ceil_div(KPW, 64);
  constexpr int PSTRIDE = DV + 4;              // floats per split partial
  constexpr int NS = HP / 8;                   // column sets of eight (row, head) pairs
  // One block of shared memory for the V rows of the four ranges (plus one
  // spare dword: a lane's two-dword read of a row may touch the dword after
  // it), the P operands [GV][4][T][NS][64] and the range outputs [4][HP][DV].
  // With two V groups or sixteen pairs the outputs reuse the bytes of the
  // rows and operands, dead by then, so that two workgroups still fit one
  // compute unit.
  constexpr int kRowWords = (4 * KPW * ROWP + 1 + 3) & ~3;
  constexpr int kPWords = GV * 4 * T * NS * 64 * 2;
  constexpr int kOutWords = 4 * HP * DV;
  constexpr bool kReuse = GV > 1 || HP == 16;
  constexpr int kOutOff = kReuse ? 0 : kRowWords + kPWords;
  constexpr int kBlockWords = kReuse ? (kRowWords + kPWords > kOutWords ? kRowWords + kPWords : kOutWords)
                                     : kRowWords + kPWords + kOutWords;
  // 256-byte aligned: a lookup address is the entry offset OR the lane offset
  __shared__ __align__(256) uint32_t ptab[PairCfg<B>::WORDS];   // pair table, 32 copies
  __shared__ __align__(16) uint32_t block[kBlockWords];
  __shared__ __align__(16) float nk[GK][4][KPW * (KQ8 ? 4 : 1)];   // K norms, or 4 block scales per key
  __shared__ __align__(16) float nv[GV][4][KPW];
  __shared__ __align__(16) uint32_t qbuf[NS][GK][4 * 64 * 4];   // query operand, [t][lane][8 halves]
  __shared__ float wm[4][HP], wl[4][HP];
  uint32_t *vrows = block;
  u32x2_t *pbuf = reinterpret_cast<u32x2_t *>(block + kRowWords);
  float *obuf = reinterpret_cast<float *>(block + kOutOff);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 3;                     // key range of this wave
  const bool kwave = wave < 4;
  const int col = lane & 15, quad = lane >> 4;
  const int s = blockIdx.x, z = blockIdx.z;
  // (divisions only where there are several head groups or rows: they sit
  // in front of the first loads)
  const int g = n_hg == 1 ? (int)blockIdx.y : (int)blockIdx.y / n_hg;
  const int hg = (int)blockIdx.y - g * n_hg;
  const SeqExtent ext = seq_extent(seq_start, seq_len, z, kv_len, n_cells);
  if ((int64_t)s * KPS >= ext.len) return;     // uniform: the whole workgroup
  const int n_vh = n_rows * n_rep;             // (row, head) pairs of a kv head
  // keys [w0, w0 + wkeys) of range rg (relative to the sequence start);
  // addressing is relative to row0, a valid key row, with lane offsets
  // clamped to the range's last key
  const int64_t w0 = (int64_t)s * KPS + (int64_t)rg * KPW;
  const int64_t left = ext.len - w0;
  const int wkeys = (int)(left < 0 ? 0 : (left < KPW ? left : KPW));
  const int wlast = wkeys > 0 ? wkeys - 1 : 0;
  const int64_t row0 = (int64_t)g * n_cells + ext.start + (wkeys > 0 ? w0 : ext.len - 1);

  if (kwave) {
    // ---------------- key wave: loads first (query, norms, K codes)
    constexpr int KRB = KQ8 ? kGroup * GK : 16 * B * GK;   // K bytes per key row
    constexpr int KNS = KQ8 ? 4 : 1;                          // K scales per group
    constexpr int KDW = KQ8 ? 8 : B;                          // K dwords per lane, tile and group
    const uint8_t *kb = kcodes + row0 * KRB;
    const uint16_t *knb = knorms + row0 * (KNS * GK), *vnb = vnorms + row0 * GV;
    // this lane's query head in column set ns: pair HP hg + 8 ns + qh
    const int qh = 2 * rg + (lane >> 5), qj = lane & 31;
    float qv[NS][GK][4];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      const int vq = imin(HP * hg + 8 * ns + qh, n_vh - 1);   // (row, head) pair of this lane's head
      const int vr = n_rows == 1 ? 0 : vq / n_rep;
      const int64_t qbase = (((int64_t)z * n_rows + vr) * n_q + (int64_t)g * n_rep + (vq - vr * n_rep)) *
                                (kGroup * GK) + 4 * qj;
#pragma unroll
      for (int gk = 0; gk < GK; ++gk) {
        if constexpr (QBF16) {
          const u32x2_t b = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(q) + qbase +
                                                               kGroup * gk);
          qv[ns][gk][0] = __uint_as_float(b.x << 16);
          qv[ns][gk][1] = __uint_as_float(b.x & 0xffff0000u);
          qv[ns][gk][2] = __uint_as_float(b.y << 16);
          qv[ns][gk][3] = __uint_as_float(b.y & 0xffff0000u);
        } else {
          const float4 f = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(q) + qbase +
                                                             kGroup * gk);
          qv[ns][gk][0] = f.x; qv[ns][gk][1] = f.y; qv[ns][gk][2] = f.z; qv[ns][gk][3] = f.w;
        }
      }
    }
    uint16_t kn[NNORM][GK][KNS], vn[NNORM][GV];
#pragma unroll
    for (int i = 0; i < NNORM; ++i) {
      const uint32_t kk = (uint32_t)imin(lane + 64 * i, wlast);
#pragma unroll
      for (int gk = 0; gk < GK; ++gk) {
        if constexpr (KQ8) {
          const u32x2_t w = *reinterpret_cast<const u32x2_t *>(knb + (kk * GK + gk) * 4);
          kn[i][gk][0] = (uint16_t)w.x; kn[i][gk][1] = (uint16_t)(w.x >> 16);
          kn[i][gk][2] = (uint16_t)w.y; kn[i][gk][3] = (uint16_t)(w.y >> 16);
        } else {
          kn[i][gk][0] = knb[kk * GK + gk];
        }
      }
#pragma unroll
      for (int gv = 0; gv < GV; ++gv) vn[i][gv] = vnb[kk * GV + gv];
    }
    // lane (col, quad) of tile t reads key 16t + col: turbo, dwords B*quad ..
    // B*quad+B-1 of each group; 8-bit blocks, bytes 8quad .. 8quad+7 of each
    // of the group's four blocks
    uint32_t kd[T][GK][KDW];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int gk = 0; gk < GK; ++gk) {
        const uint32_t key = (uint32_t)imin(16 * t + col, wlast);
        if constexpr (KQ8) {
          const uint8_t *row = kb + key * (uint32_t)KRB + kGroup * gk + 8 * quad;
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const u32x2_t w = *reinterpret_cast<const u32x2_t *>(row + 32 * st);
            kd[t][gk][2 * st] = w.x;
            kd[t][gk][2 * st + 1] = w.y;
          }
        } else {
          const uint32_t *row = reinterpret_cast<const uint32_t *>(kb + key * (uint32_t)KRB + 16u * B * gk + 4u * B * quad);
#pragma unroll
          for (int i = 0; i < B; ++i) kd[t][gk][i] = row[i];
        }
      }

    build_pair_table<B, kDecThreads>(ptab, tid);
    // rotate (turbo K) + split heads 2rg, 2rg+1, group by group: thread holds
    // d = 4qj .. 4qj+3 of head qh; in the MFMA B operand they are slots
    // i = 4(qj&1) .. +3 of K-step t = (qj>>1)&3 in lane 16*(qj>>3) + qh (high
    // half) and 16*(qj>>3) + 8 + qh (low half); for 8-bit block K, of K-step
    // qj>>3 in lanes 16*((qj>>1)&3) + qh and + 8 (each column set its own
    // operand)
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int gk = 0; gk < GK; ++gk) {
        if constexpr (!KQ8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) qv[ns][gk][i] = flip_sign(qv[ns][gk][i], sign_bit_of(4 * qj + i));
          wht128_half(qv[ns][gk], qj);
        }
        const bool live = HP * hg + 8 * ns + qh < n_vh;
        uint32_t hw[2], lw[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const float x0 = live ? qv[ns][gk][2 * p] * qscale : 0.f;
          const float x1 = live ? qv[ns][gk][2 * p + 1] * qscale : 0.f;
          const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
          const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
          hw[p] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
          lw[p] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
        }
        const int t = KQ8 ? qj >> 3 : (qj >> 1) & 3, qd = KQ8 ? (qj >> 1) & 3 : qj >> 3;
        const int half_off = 2 * (qj & 1);
        *reinterpret_cast<u32x2_t *>(qbuf[ns][gk] + (t * 64 + 16 * qd + qh) * 4 + half_off) = u32x2_t{hw[0], hw[1]};
        *reinterpret_cast<u32x2_t *>(qbuf[ns][gk] + (t * 64 + 16 * qd + 8 + qh) * 4 + half_off) =
            u32x2_t{lw[0], lw[1]};
      }
    __syncthreads();   // table and query operand complete

    // norms of the range (this wave's own slice)
#pragma unroll
    for (int i = 0; i < NNORM; ++i) {
      const int kk = lane + 64 * i;
      if (kk < KPW) {
        const bool ok = kk < wkeys;
#pragma unroll
        for (int gk = 0; gk < GK; ++gk)
#pragma unroll
          for (int b = 0; b < KNS; ++b) nk[gk][rg][KNS * kk + b] = ok ? half_to_float(kn[i][gk][b]) : 0.f;
#pragma unroll
        for (int gv = 0; gv < GV; ++gv) nv[gv][rg][kk] = ok ? half_to_float(vn[i][gv]) : 0.f;
      }
    }
    // Query operand: column n = lane & 15 -> head n & 7 of the set, high
    // (n < 8) or low half; k-slot (lane >> 4, i) of K-step t <-> element
    // d = 32*(lane>>4) + 8t + i.
    half8_t qb[NS][GK][4];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int gk = 0; gk < GK; ++gk)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          qb[ns][gk][t] = __builtin_bit_cast(half8_t, reinterpret_cast<const u32x4_t *>(qbuf[ns][gk])[t * 64 + lane]);
    wave_lds_fence();

    // ---- scores: S^T[key][col] over the range, tile by tile; every column
    //      set takes the same decoded K operand
    const u32x2_t *tab = reinterpret_cast<const u32x2_t *>(ptab) + (lane & 31);
    float sc[T][NS][4];
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int gk = 0; gk < GK; ++gk) {
        if constexpr (KQ8) {
          // one product per 32-element block, each times its block's scale
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) {
            float4_t acc[4];
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              const u32x2_t a0 = i8x4_to_half4(kd[t][gk][2 * st]);
              const u32x2_t a1 = i8x4_to_half4(kd[t][gk][2 * st + 1]);
              const u32x4_t av = {a0.x, a0.y, a1.x, a1.y};
              acc[st] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[ns][gk][st],
                                                              float4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float4 d4 = *reinterpret_cast<const float4 *>(&nk[gk][rg][4 * (16 * t + 4 * quad + i)]);
              const float y = acc[0][i] * d4.x + acc[1][i] * d4.y + acc[2][i] * d4.z + acc[3][i] * d4.w;
              const float x = y + xor_lane<8>(y);
              sc[t][ns][i] = gk == 0 ? x : sc[t][ns][i] + x;
            }
          }
        } else {
          // the level's hi and lo parts in two products over the same query
          // operand: (Kh + Kl) (Qh + Ql)
          uint32_t a16[16], l16[16];
          decode_pairs_hl<B, 32>(kd[t][gk], tab, a16, l16);
          float4_t acc[NS];
#pragma unroll
          for (int ns = 0; ns < NS; ++ns) acc[ns] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const u32x4_t av = {a16[4 * st], a16[4 * st + 1], a16[4 * st + 2], a16[4 * st + 3]};
            const u32x4_t al = {l16[4 * st], l16[4 * st + 1], l16[4 * st + 2], l16[4 * st + 3]};
#pragma unroll
            for (int ns = 0; ns < NS; ++ns) {
              acc[ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[ns][gk][st],
                                                               acc[ns], 0, 0, 0);
              acc[ns] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, al), qb[ns][gk][st],
                                                               acc[ns], 0, 0, 0);
            }
          }
          const float4 n4 = *reinterpret_cast<const float4 *>(&nk[gk][rg][16 * t + 4 * quad]);
          const float nkv[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
          for (int ns = 0; ns < NS; ++ns)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x = (acc[ns][i] + xor_lane<8>(acc[ns][i])) * nkv[i];
              sc[t][ns][i] = gk == 0 ? x : sc[t][ns][i] + x;
            }
        }
      }
    }
    // causal limit of this lane's column (pair HP hg + 8 ns + (col & 7)):
    // the key (relative to the range) of its row's last visible cell; only
    // ranges reaching past the first row's limit mask (wave-uniform)
    if (w0 + KPW - 1 > ext.len - n_rows) {
#pragma unroll
      for (int ns = 0; ns < NS; ++ns) {
        const int vc = HP * hg + 8 * ns + (col & 7);
        const int64_t lim64 = ext.len - n_rows + (vc < n_vh && n_rows > 1 ? vc / n_rep : 0) - w0;
        const int lim = lim64 < -1 ? -1 : (lim64 > KPW ? KPW : (int)lim64);
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * t + 4 * quad + i > lim) sc[t][ns][i] = -INFINITY;
      }
    }
    // range max per head (log2 domain); -inf for a range without keys
    float mx[NS], msafe[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      float m = -INFINITY;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, sc[t][ns][i]);
      m = fmaxf(m, xor_lane<16>(m));
      mx[ns] = max_xor32(m);
      msafe[ns] = mx[ns] == -INFINITY ? 0.f : mx[ns];
    }

    // ---- P operands: the score layout (lane = column + 16 * key quad) is
    //      the A-operand layout of the value product.  Rows < 8 carry the
    //      float16 high part of p * vnorm, rows >= 8 the low part:
    //      x - hi * lo_sel (lo_sel = 1 on low rows, 0 on high rows) is exact
    //      in float32 and rounds once to float16.  Sparse V ([PR36] (d) item
    //      3): a key whose weight against the range maximum (<= the true
    //      maximum) is below tau leaves the value sum but stays in lsum.
    const float lo_sel = col >= 8 ? 1.f : 0.f;
    float lsum[NS];
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) lsum[ns] = 0.f;
    // every tile's V norms read up front, so the reads' latencies overlap
    float4 nvq[T][GV];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int gv = 0; gv < GV; ++gv) nvq[t][gv] = *reinterpret_cast<const float4 *>(&nv[gv][rg][16 * t + 4 * quad]);
    // (the dense form without the threshold test when tau is 0: wave-uniform)
    auto p_tiles = [&](auto sparse_tag) {
      constexpr bool kSparse = decltype(sparse_tag)::value;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[i] = __builtin_amdgcn_exp2f(sc[t][ns][i] - msafe[ns]);
            lsum[ns] += p[i];
          }
#pragma unroll
          for (int gv = 0; gv < GV; ++gv) {
            const float4 n4 = nvq[t][gv];
            const float nvv[4] = {n4.x, n4.y, n4.z, n4.w};
            half4_t pa;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x = kSparse && p[i] < tau ? 0.f : p[i] * nvv[i];
              const _Float16 h = (_Float16)x;
              pa[i] = (_Float16)__builtin_fmaf(-(float)h, lo_sel, x);
            }
            pbuf[(((gv * 4 + rg) * T + t) * NS + ns) * 64 + lane] = __builtin_bit_cast(u32x2_t, pa);
          }
        }
    };
    if (tau > 0.f)
      p_tiles(std::true_type{});
    else
      p_tiles(std::false_type{});
#pragma unroll
    for (int ns = 0; ns < NS; ++ns) {
      float l = lsum[ns] + xor_lane<16>(lsum[ns]);
      l = sum_xor32(l);
      if (lane < 8) {
        wm[rg][8 * ns + lane] = mx[ns];
        wl[rg][8 * ns + lane] = l;
      }
    }
    __syncthreads();   // P operands complete
    if constexpr (kReuse) __syncthreads();   // V rows and P operands consumed
    __syncthreads();   // value products done (partial outputs in obuf)
  } else {
    // ---------------- value wave: the range's V rows are contiguous; lane
    //                  l loads 16-byte chunks l, l + 64, ... of them, so each
    //                  load instruction covers 1 KB of consecutive bytes
    constexpr int CH = GV * B;                 // 16-byte chunks per row
    constexpr int NCH = KPW * CH;
    constexpr int CPL = ceil_div(NCH, 64);     // chunks per lane
    const uint8_t *vb = vcodes + row0 * (16 * B * GV);
    u32x4_t vraw[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = imin(lane + 64 * j, NCH - 1);
      const int r = c / CH, part = c - r * CH;
      vraw[j] = *reinterpret_cast<const u32x4_t *>(vb + (uint32_t)imin(r, wlast) * (16u * B * GV) + 16u * part);
    }
    build_pair_table<B, kDecThreads>(ptab, tid);
    __syncthreads();   // table and query operand complete

    uint32_t *vr = vrows + rg * KPW * ROWP;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (NCH % 64 == 0 || c < NCH) {
        const int r = c / CH, part = c - r * CH;
        uint32_t *d = vr + r * ROWP + 4 * part;
        d[0] = vraw[j].x;
        d[1] = vraw[j].y;
        d[2] = vraw[j].z;
        d[3] = vraw[j].w;
      }
    }
    wave_lds_fence();
    // B operands: lane (n, quad) of tile t holds keys 16t + 4quad + j
    // (j = 0..3) at d = 8n + dt of d-tile dt; it decodes the 8 elements
    // 8n .. 8n+7 of each of its four keys and regroups them by element.
    constexpr int VBITS = 8 * B;
    const int vpos = VBITS * col;
    const int vw0 = vpos >> 5, vsh = vpos & 31;
    // this lane's hi dword of the pair table (its lo dword follows)
    const uint32_t *tabw = ptab + 2 * (lane & 31);
    // after the swap, lanes 0-31 hold d-tiles 0-3 and lanes 32-63 d-tiles
    // 4-7, each as high + low; row (head) 4*((lane&31)>>4) + i
    const int qd = (lane & 31) >> 4, dhi = lane >> 5;
    // B operands of tile t from one part of the levels (tb: the hi or lo
    // dword of this lane's table copy)
    auto v_tile = [&](const uint32_t *vlane, int t, const uint32_t *tb, u32x2_t (&ops)[8]) {
      uint32_t vv[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t *row = vlane + (16 * t + i) * ROWP;
        const uint32_t run[1] = {__builtin_amdgcn_alignbit(row[1], row[0], vsh)};
        decode_pairs<B, 8>(run, tb, vv[i]);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int w = dt >> 1;
        const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;
        ops[dt] = u32x2_t{__builtin_amdgcn_perm(vv[1][w], vv[0][w], sel),
                          __builtin_amdgcn_perm(vv[3][w], vv[2][w], sel)};
      }
    };
    float4 res[NS][GV][4];
#pragma unroll
    for (int gv = 0; gv < GV; ++gv) {
      const uint32_t *vlane = vr + 4 * quad * ROWP + GW * gv + vw0;
      // hi parts of every tile before the barrier; lo parts tile pair by
      // tile pair beside the products
      u32x2_t vbop[T][8];
#pragma unroll
      for (int t = 0; t < T; ++t) v_tile(vlane, t, tabw, vbop[t]);
      if (gv == 0) __syncthreads();   // P operands complete

      // each column set takes the same decoded V operands; the products run
      // (Ph + Pl)(Vh + Vl) as two products per d-tile into one accumulator
      float4_t o[NS][8];
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[ns][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
      // tiles in pairs on the 32-deep product: k-slots (quad, 0..3) hold
      // the first tile's keys 4 quad + i and (quad, 4..7) the second's, in
      // both operands, so the sum runs over the same 32 keys; an odd last
      // tile takes the 16-deep product
#pragma unroll
      for (int t = 0; t + 1 < T; t += 2) {
        u32x2_t l0[8], l1[8];
        v_tile(vlane, t, tabw + 1, l0);
        v_tile(vlane, t + 1, tabw + 1, l1);
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const u32x2_t p0 = pbuf[(((gv * 4 + rg) * T + t) * NS + ns) * 64 + lane];
          const u32x2_t p1 = pbuf[(((gv * 4 + rg) * T + t + 1) * NS + ns) * 64 + lane];
          const half8_t pa = __builtin_bit_cast(half8_t, u32x4_t{p0.x, p0.y, p1.x, p1.y});
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            const u32x4_t vh = {vbop[t][dt].x, vbop[t][dt].y, vbop[t + 1][dt].x, vbop[t + 1][dt].y};
            const u32x4_t vl = {l0[dt].x, l0[dt].y, l1[dt].x, l1[dt].y};
            o[ns][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, __builtin_bit_cast(half8_t, vh), o[ns][dt], 0, 0, 0);
            o[ns][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, __builtin_bit_cast(half8_t, vl), o[ns][dt], 0, 0, 0);
          }
        }
      }
      if constexpr (T & 1) {
        u32x2_t l0[8];
        v_tile(vlane, T - 1, tabw + 1, l0);
#pragma unroll
        for (int ns = 0; ns < NS; ++ns) {
          const half4_t pa =
              __builtin_bit_cast(half4_t, pbuf[(((gv * 4 + rg) * T + T - 1) * NS + ns) * 64 + lane]);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) {
            o[ns][dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, __builtin_bit_cast(half4_t, vbop[T - 1][dt]),
                                                             o[ns][dt], 0, 0, 0);
            o[ns][dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, __builtin_bit_cast(half4_t, l0[dt]),
                                                             o[ns][dt], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int ns = 0; ns < NS; ++ns)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float oc[4];
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[ns][dt][i]),
                                                            __float_as_uint(o[ns][dt + 4][i]), false, false);
            oc[dt] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
          }
          res[ns][gv][i] = make_float4(oc[0], oc[1], oc[2], oc[3]);
        }
    }
    if constexpr (kReuse) __syncthreads();   // V rows and P operands consumed
#pragma unroll
    for (int ns = 0; ns < NS; ++ns)
#pragma unroll
      for (int gv = 0; gv < GV; ++gv)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4 *>(
              &obuf[(rg * HP + 8 * ns + 4 * qd + i) * DV + kGroup * gv + 8 * col + 4 * dhi]) = res[ns][gv][i];
    __syncthreads();   // value products done (partial outputs in obuf)
  }

  // ---- merge the four ranges: obuf[r][h][128gv + 8c + t] holds element
  //      8c + t of group gv of head h, relative to the range's own max;
  //      512 / HP threads per head, EPT elements of each group per thread
  {
    constexpr int TPH = kDecThreads / HP, EPT = kGroup / TPH;
    const int h = tid / TPH, d = EPT * (tid % TPH);
    const int vh = HP * hg + h;
    if (vh < n_vh) {
      const float M = fmaxf(fmaxf(wm[0][h], wm[1][h]), fmaxf(wm[2][h], wm[3][h]));
      float f[4], L = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mr = wm[r][h];
        f[r] = mr == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mr - M);
        L += f[r] * wl[r][h];
      }
      // partial of (sequence z, row, q head), split s
      const int vr = n_rows == 1 ? 0 : vh / n_rep;
      const int64_t qrow = ((int64_t)z * n_rows + vr) * n_q + (int64_t)g * n_rep + (vh - vr * n_rep);
      float *ph = ws + (qrow * n_split + s) * PSTRIDE;
#pragma unroll
      for (int gv = 0; gv < GV; ++gv) {
        if constexpr (EPT == 2) {
          float a0 = 0.f, a1 = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float2 v = *reinterpret_cast<const float2 *>(&obuf[(r * HP + h) * DV + kGroup * gv + d]);
            a0 += f[r] * v.x;
            a1 += f[r] * v.y;
          }
          *reinterpret_cast<float2 *>(ph + kGroup * gv + d) = make_float2(a0, a1);
        } else {
          float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float4 v = *reinterpret_cast<const float4 *>(&obuf[(r * HP + h) * DV + kGroup * gv + d]);
            a.x += f[r] * v.x;
            a.y += f[r] * v.y;
            a.z += f[r] * v.z;
            a.w += f[r] * v.w;
          }
          *reinterpret_cast<float4 *>(ph + kGroup * gv + d) = a;
        }
      }
      if (d == 0) *reinterpret_cast<float2 *>(ph + DV) = make_float2(M, L);
    }
  }
}

// ---------------------------------------------------------------- fused decode
//
// decode_fused_kernel: the single-group (128-wide K and V, both turbo) decode
// with at most eight (query row, q head) pairs per kv head.  Workgroup
// (split s, kv head g) has eight waves; wave w takes the blocks of KPB = 16 TB
// keys numbered 8b + w (b = 0 .. nb-1) of the split and runs each block
// through the whole chain itself: scores, the running maximum, P kept in
// registers (the score accumulator's lane layout is the A-operand layout of
// the value product), the V rows staged in the wave's own LDS rows, and the
// value products.  No barrier separates the waves until the eight partial
// results are merged into the split partial, so the waves take their blocks
// as their loads arrive; with nb > 1 each wave loads its next block while it
// computes the current one, and the running maximum rescales the
// accumulators (wave-uniform test) when it moves.
//
// Operand layouts (v_mfma_f32_16x16x32_f16; a level enters as its float16 hi
// and lo parts, the query and P as theirs):
//   scores  K-step st (0..7), lane (col, quad): k-slots hold hi(e0) hi(e1)
//           lo(e0) lo(e1) hi(e2) hi(e3) lo(e2) lo(e3) of the key's elements
//           e = 32 quad + 4 st + 0..3, i.e. two pair-table entries read as
//           they are; the query operand repeats each element twice (column
//           c < 8: the high part of pair c's rotated query, 8 + c its low part)
//   values  per 16-key tile and d-tile dt, lane (n, quad): k-slots hold
//           keys 4 quad + (0, 1) hi, (0, 1) lo, (2, 3) hi, (2, 3) lo of element
//           8n + dt; P repeats each key twice (rows < 8: the high part of
//           p * vnorm, rows >= 8 the low part).
// Sparse V ([PR36] (d) item 3): P entries below tau become 0, and a tile whose
// entries are all 0 skips its value decode and products.
template <int B>
__device__ __forceinline__ uint32_t pair_field_at8(const uint32_t *dw, int pos) {
  // the 2B-bit field at bit pos of dw (pos compile-time), moved to bit 8
  const int w = pos >> 5, sh = pos & 31;
  if (sh >= 8)
    return sh + 2 * B <= 32 ? dw[w] >> (sh - 8) : __builtin_amdgcn_alignbit(dw[w + 1], dw[w], sh - 8);
  return w == 0 ? dw[0] << (8 - sh) : __builtin_amdgcn_alignbit(dw[w], dw[w - 1], 24 + sh);
}
// Byte offset of a pair-table entry (in bits 8 .. 8 + 2B of x) in this
// lane's copy: entry e, copy c at byte 256 e + 8 c.
template <int B>
__device__ __forceinline__ uint32_t pair_byte(uint32_t x, uint32_t lane8) {
  return (x & (((1u << (2 * B)) - 1u) << 8)) | lane8;
}
__device__ __forceinline__ u32x2_t lds_u32x2(const uint32_t *base, uint32_t byte) {
  return *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const char *>(base) + byte);
}

// PF: the next block's loads are issued before the current block is
// computed (waves with several blocks); without it a block is loaded when
// its turn comes.
template <int B, int TB, bool QBF16, bool PF>
__global__ __launch_bounds__(kDecThreads, 2) void decode_fused_kernel(
    const uint8_t *__restrict__ kcodes, const uint16_t *__restrict__ knorms,
    const uint8_t *__restrict__ vcodes, const uint16_t *__restrict__ vnorms, int64_t n_cells,
    const int64_t *__restrict__ seq_start, const int32_t *__restrict__ seq_len, int64_t kv_len,
    const void *__restrict__ q, int n_q, int n_rep, int n_rows, int n_hg, int nb, float qscale, float tau,
    float *__restrict__ ws, int n_split) {
  constexpr int KPB = 16 * TB;                 // keys per wave block
  constexpr int GW = 4 * B;                    // code dwords per key row
  constexpr int ROWP = GW + 1;                 // padded LDS V row
  constexpr int NCH = KPB * B;                 // 16-byte V chunks per block
  constexpr int CPL = ceil_div(NCH, 64);       // chunks per lane
  constexpr int PSTRIDE = kGroup + 4;
  constexpr int kVstWords = (KPB * ROWP + 1 + 3) & ~3;   // + a spare dword (two-dword row reads)
  constexpr int kStageWords = 8 * (kVstWords + 2 * KPB);
  constexpr int kOutWords = 8 * 8 * kGroup;
  constexpr int kBlockWords = kStageWords > kOutWords ? kStageWords : kOutWords;
  __shared__ __align__(256) uint32_t ptab[PairCfg<B>::WORDS];   // pair table, 32 copies
  __shared__ __align__(16) uint32_t qbuf[8 * 64 * 4];            // query operand [st][lane][8 halves]
  // per wave: V rows and the block's K and V norms; after the last block the
  // same bytes take the eight waves' outputs [wave][pair][128]
  __shared__ __align__(16) uint32_t blk[kBlockWords];
  __shared__ float wm[8][8], wl[8][8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, quad = lane >> 4;
  const int s = blockIdx.x, z = blockIdx.z;
  const int g = (int)blockIdx.y / n_hg, hg = (int)blockIdx.y - g * n_hg;   // kv head, pair group
  const SeqExtent ext = seq_extent(seq_start, seq_len, z, kv_len, n_cells);
  const int64_t kps = (int64_t)8 * nb * KPB;
  if ((int64_t)s * kps >= ext.len) return;     // uniform: the whole workgroup
  // (row, head) pairs 8 hg .. 8 hg + n_vh - 1 of the kv head's n_rows n_rep
  const int p0 = 8 * hg;
  const int n_vh = imin(8, n_rows * n_rep - p0);
  const int64_t kbase = (int64_t)g * n_cells + ext.start;
  uint32_t *vst = blk + wave * (kVstWords + 2 * KPB);
  float *nk = reinterpret_cast<float *>(vst + kVstWords), *nv = nk + KPB;

  // raw global loads of block b: K codes of the lane's 32 elements (lane
  // (col, quad) of tile t: dwords B quad .. B quad + B - 1 of key 16t + col),
  // V rows as consecutive 16-byte chunks, one norm of each per lane (key =
  // lane)
  struct Raw {
    uint32_t k[TB][B];
    u32x4_t v[CPL];
    uint16_t kn, vn;
  };
  auto block_keys = [&](int b, int64_t &w0) {
    w0 = (int64_t)s * kps + (int64_t)(b * 8 + wave) * KPB;
    const int64_t left = ext.len - w0;
    return (int)(left <= 0 ? 0 : (left < KPB ? left : KPB));
  };
  auto load = [&](int b, Raw &r) {
    int64_t w0;
    const int wk = block_keys(b, w0);
    const int wlast = wk > 0 ? wk - 1 : 0;
    const int64_t row0 = kbase + (wk > 0 ? w0 : ext.len - 1);
    const uint8_t *kb = kcodes + row0 * (16 * B);
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const uint32_t key = (uint32_t)imin(16 * t + col, wlast);
      const uint32_t *row = reinterpret_cast<const uint32_t *>(kb + key * (16u * B) + 4u * B * quad);
#pragma unroll
      for (int i = 0; i < B; ++i) r.k[t][i] = row[i];
    }
    const uint8_t *vb = vcodes + row0 * (16 * B);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = imin(lane + 64 * j, NCH - 1);
      const int rr = c / B, part = c - rr * B;
      r.v[j] = *reinterpret_cast<const u32x4_t *>(vb + (uint32_t)imin(rr, wlast) * (16u * B) + 16u * part);
    }
    const uint32_t kk = (uint32_t)imin(lane, wlast);
    r.kn = knorms[row0 + kk];
    r.vn = vnorms[row0 + kk];
  };

  // rotate + split the query of pairs 2w, 2w+1 (waves 0-3): thread (qh, qj)
  // holds d = 4qj .. 4qj+3 of pair qh, which is the element chunk of quad
  // qj >> 3 and K-step qj & 7: it writes that chunk's high parts to lane
  // 16 (qj >> 3) + qh and its low parts to lane 16 (qj >> 3) + 8 + qh.
  // The query load is issued before the block's K/V loads: loads retire in
  // order, so issued after them it could only be used once they had all
  // arrived, and the rotation would wait for the whole block
  const int qh = 2 * wave + (lane >> 5), qj = lane & 31;
  u32x4_t qraw = {0u, 0u, 0u, 0u};   // the lane's 4 query values as loaded (bf16 pairs or fp32)
  if (wave < 4) {
    const int vq = p0 + imin(qh, n_vh - 1);
    const int vr = n_rows == 1 ? 0 : vq / n_rep;
    const int64_t qbase =
        (((int64_t)z * n_rows + vr) * n_q + (int64_t)g * n_rep + (vq - vr * n_rep)) * kGroup + 4 * qj;
    if constexpr (QBF16) {
      const u32x2_t bw = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(q) + qbase);
      qraw.x = bw.x;
      qraw.y = bw.y;
    } else {
      qraw = *reinterpret_cast<const u32x4_t *>(reinterpret_cast<const float *>(q) + qbase);
    }
  }
  Raw cur;
  load(0, cur);
  build_pair_table<B, kDecThreads>(ptab, tid);
  if (wave < 4) {
    float qv[4];
    if constexpr (QBF16) {
      qv[0] = __uint_as_float(qraw.x << 16);
      qv[1] = __uint_as_float(qraw.x & 0xffff0000u);
      qv[2] = __uint_as_float(qraw.y << 16);
      qv[3] = __uint_as_float(qraw.y & 0xffff0000u);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) qv[i] = __uint_as_float(qraw[i]);
    }
    const uint32_t sn = sign_nibble(qj);
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[i] = flip_sign(qv[i], (sn >> i) & 1u);
    wht128_half(qv, qj);
    const bool live = qh < n_vh;
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const float x0 = live ? qv[2 * p] * qscale : 0.f;
      const float x1 = live ? qv[2 * p + 1] * qscale : 0.f;
      const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
      const _Float16 l0 = (_Float16)(x0 - (float)h0), l1 = (_Float16)(x1 - (float)h1);
      hw[p] = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
      lw[p] = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
    }
    const int st = qj & 7, qd = qj >> 3;
    reinterpret_cast<u32x4_t *>(qbuf)[st * 64 + 16 * qd + qh] = u32x4_t{hw[0], hw[0], hw[1], hw[1]};
    reinterpret_cast<u32x4_t *>(qbuf)[st * 64 + 16 * qd + 8 + qh] = u32x4_t{lw[0], lw[0], lw[1], lw[1]};
  }
  __syncthreads();   // pair table and query operand complete
  half8_t qb[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) qb[st] = __builtin_bit_cast(half8_t, reinterpret_cast<const u32x4_t *>(qbuf)[st * 64 + lane]);

  const uint32_t lane8 = 8u * (uint32_t)(lane & 31);   // this lane's table copy
  // this lane's score column: pair col & 7 -> causal offset of its row
  const int vcol = col & 7;
  const int row_off = vcol < n_vh && n_rows > 1 ? (p0 + vcol) / n_rep : 0;
  const float lo_sel = col >= 8 ? 1.f : 0.f;
  // V: lane (n, quad) of tile t decodes elements 8n .. 8n+7 of keys
  // 16t + 4quad + i (i = 0..3), the 8B-bit run at bit 8Bn of each row
  const int vpos = 8 * B * col;
  const int vw0 = vpos >> 5, vsh = vpos & 31;
  const uint32_t *vlane = vst + 4 * quad * ROWP + vw0;

  float4_t o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;   // of this lane's column

  for (int b = 0; b < nb; ++b) {
    int64_t w0;
    const int wk = block_keys(b, w0);
    if (wk == 0) break;                        // wave-uniform: later blocks are empty too
    if (!PF && b > 0) load(b, cur);
    // stage the V rows and norms of the block in the wave's own LDS
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if (NCH % 64 == 0 || c < NCH) {
        const int rr = c / B, part = c - rr * B;
        uint32_t *d = vst + rr * ROWP + 4 * part;
        d[0] = cur.v[j].x;
        d[1] = cur.v[j].y;
        d[2] = cur.v[j].z;
        d[3] = cur.v[j].w;
      }
    }
    if (lane < KPB) {
      nk[lane] = lane < wk ? half_to_float(cur.kn) : 0.f;
      nv[lane] = lane < wk ? half_to_float(cur.vn) : 0.f;
    }
    uint32_t kr[TB][B];
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int i = 0; i < B; ++i) kr[t][i] = cur.k[t][i];
    if (PF && b + 1 < nb) load(b + 1, cur);     // the next block's loads fly over this one
    wave_lds_fence();

    // ---- scores of the block's tiles
    float sc[TB][4];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      u32x2_t lv[16];   // (hi pair, lo pair) of the lane's element pairs 2j, 2j+1
#pragma unroll
      for (int j = 0; j < 16; ++j) lv[j] = lds_u32x2(ptab, pair_byte<B>(pair_field_at8<B>(kr[t], 2 * B * j), lane8));
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4_t av = {lv[2 * st].x, lv[2 * st].y, lv[2 * st + 1].x, lv[2 * st + 1].y};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[st], acc, 0, 0, 0);
      }
      const float4 n4 = *reinterpret_cast<const float4 *>(nk + 16 * t + 4 * quad);
      const float nkv[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[t][i] = (acc[i] + xor_lane<8>(acc[i])) * nkv[i];
      // (keeps the next tile's lookups below this one's products)
      __builtin_amdgcn_sched_barrier(0);
    }
    // causal limit of this lane's column (relative to the block), only for
    // blocks reaching past the first row's last cell (wave-uniform)
    if (w0 + KPB - 1 > ext.len - n_rows) {
      const int64_t lim64 = ext.len - n_rows + row_off - w0;
      const int lim = lim64 < -1 ? -1 : (lim64 > KPB ? KPB : (int)lim64);
#pragma unroll
      for (int t = 0; t < TB; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * t + 4 * quad + i > lim) sc[t][i] = -INFINITY;
    }
    // running maximum of the column (log2 domain)
    float mb = -INFINITY;
#pragma unroll
    for (int t = 0; t < TB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mb = fmaxf(mb, sc[t][i]);
    mb = fmaxf(mb, xor_lane<16>(mb));
    mb = max_xor32(mb);
    const float m_new = fmaxf(m_run, mb);
    if (b > 0 && __builtin_amdgcn_ballot_w64(m_new > m_run) != 0) {
      // rescale: the factor of pair c lives in lanes c, c + 8 (any quad);
      // value row 4 quad + i is pair 4 (quad & 1) + i
      const float a = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
      l_run *= a;
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ar[i] = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * (4 * (quad & 1) + i), __float_as_int(a)));
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[dt][i] *= ar[i];
    }
    m_run = m_new;
    const float msafe = m_new == -INFINITY ? 0.f : m_new;

    // ---- P in registers (rows < 8: high part of p * vnorm, rows >= 8: low
    //      part), then the value products tile by tile
    auto tiles = [&](auto sparse_tag) {
      constexpr bool kSparse = decltype(sparse_tag)::value;
#pragma unroll
      for (int t = 0; t < TB; ++t) {
        const float4 n4 = *reinterpret_cast<const float4 *>(nv + 16 * t + 4 * quad);
        const float nvv[4] = {n4.x, n4.y, n4.z, n4.w};
        bool any = false;
        uint32_t pw[2];
#pragma unroll
        for (int i2 = 0; i2 < 2; ++i2) {
          _Float16 ph[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int i = 2 * i2 + e;
            const float p = __builtin_amdgcn_exp2f(sc[t][i] - msafe);
            l_run += p;
            const float x = kSparse && p < tau ? 0.f : p * nvv[i];
            any |= x != 0.f;
            const _Float16 h = (_Float16)x;
            ph[e] = (_Float16)__builtin_fmaf(-(float)h, lo_sel, x);
          }
          pw[i2] = (uint32_t)__builtin_bit_cast(uint16_t, ph[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, ph[1]) << 16);
        }
        if (kSparse && __builtin_amdgcn_ballot_w64(any) == 0) continue;   // wave-uniform
        const half8_t pp = __builtin_bit_cast(half8_t, u32x4_t{pw[0], pw[0], pw[1], pw[1]});
        // the (hi pair, lo pair) of elements 8n + 2j, +1 of the lane's four keys
        u32x2_t hl[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t *row = vlane + (16 * t + i) * ROWP;
          const uint32_t run = __builtin_amdgcn_alignbit(row[1], row[0], vsh);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t x = 2 * B * j >= 8 ? run >> (2 * B * j - 8) : run << (8 - 2 * B * j);
            hl[i][j] = lds_u32x2(ptab, pair_byte<B>(x, lane8));
          }
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const int w = dt >> 1;
          const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;
          const u32x4_t vb = {__builtin_amdgcn_perm(hl[1][w].x, hl[0][w].x, sel),
                              __builtin_amdgcn_perm(hl[1][w].y, hl[0][w].y, sel),
                              __builtin_amdgcn_perm(hl[3][w].x, hl[2][w].x, sel),
                              __builtin_amdgcn_perm(hl[3][w].y, hl[2][w].y, sel)};
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pp, __builtin_bit_cast(half8_t, vb), o[dt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    if (tau > 0.f)
      tiles(std::true_type{});
    else
      tiles(std::false_type{});
    wave_lds_fence();   // the block's V rows read before the next block overwrites them
  }

  // ---- merge the eight waves: value row 4 quad + i holds pair (4quad+i) & 7,
  //      high rows in lanes 0-31 and low rows in lanes 32-63; after the swap
  //      lanes 0-31 hold d-tiles 0-3 and lanes 32-63 d-tiles 4-7 of pair
  //      4((lane&31)>>4) + i as high + low
  float l = l_run + xor_lane<16>(l_run);
  l = sum_xor32(l);
  float4 res[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float oc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[dt][i]), __float_as_uint(o[dt + 4][i]),
                                                      false, false);
      oc[dt] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    res[i] = make_float4(oc[0], oc[1], oc[2], oc[3]);
  }
  __syncthreads();   // every wave is done with its LDS rows: they take the outputs now
  float *obuf = reinterpret_cast<float *>(blk);
  const int qd = (lane & 31) >> 4, dhi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<float4 *>(&obuf[(wave * 8 + 4 * qd + i) * kGroup + 8 * col + 4 * dhi]) = res[i];
  if (lane < 8) {
    wm[wave][lane] = m_run;
    wl[wave][lane] = l;
  }
  __syncthreads();
  // the weight of wave w's partial of pair h, exp2(m_w - M_h), once per
  // (w, h) by the first wave (wm then holds the weights, wl[0] L and
  // wl[1] M)
  if (wave == 0) {
    const int h = lane & 7, w = lane >> 3;
    float M = wm[0][h];
#pragma unroll
    for (int v = 1; v < 8; ++v) M = fmaxf(M, wm[v][h]);
    const float mw = wm[w][h];
    const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
    float fl = f * wl[w][h];
    fl += __shfl_xor(fl, 8);
    fl += __shfl_xor(fl, 16);
    fl += __shfl_xor(fl, 32);
    wave_lds_fence();
    wm[w][h] = f;
    if (w == 0) {
      wl[0][h] = fl;
      wl[1][h] = M;
    }
  }
  __syncthreads();
  {
    const int h = tid >> 6, d = 2 * (tid & 63);
    if (h < n_vh) {
      const float L = wl[0][h], M = wl[1][h];
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float f = wm[w][h];
        const float2 v = *reinterpret_cast<const float2 *>(&obuf[(w * 8 + h) * kGroup + d]);
        a0 += f * v.x;
        a1 += f * v.y;
      }
      const int gh = p0 + h;
      const int vr = n_rows == 1 ? 0 : gh / n_rep;
      const int64_t qrow = ((int64_t)z * n_rows + vr) * n_q + (int64_t)g * n_rep + (gh - vr * n_rep);
      float *ph = ws + (qrow * n_split + s) * PSTRIDE;
      *reinterpret_cast<float2 *>(ph + d) = make_float2(a0, a1);
      if (d == 0) *reinterpret_cast<float2 *>(ph + kGroup) = make_float2(M, L);
    }
  }
}

// ---------------------------------------------------------------- LUT decode
//
// decode_lut_kernel: the decode of [PR36] (c), a Q x centroid lookup table
// in LDS built once per split, for one query row, 128-wide turbo2/turbo3
// heads and NREP (1..8) q heads per kv head.  The table is indexed by the
// code pair of two neighbouring elements: lut[h][dp][e] = q[2dp] c[e0] +
// q[2dp+1] c[e1] (float32, q the rotated query of head h, e0 and e1 the two
// codes packed in e, c the float32 levels), so a key's score is 64 table
// reads per head.  Workgroup (split s, kv head g), 256 threads, 256 keys:
//   scores  thread j takes key j; every thread reads row dp of the table at
//           the same time, so the lanes of a read hit distinct banks or
//           broadcast one dword (no conflict, no padding needed);
//   values  thread (slot, d) accumulates p * vnorm * c[code] of element d
//           over the keys (V code rows staged in LDS): slot = key half for
//           one head, else the head parity;
// and the split partial (unnormalized rotated sum, log2 maximum, weight sum)
// goes to the merge kernel like the other decode paths' partials.
template <int B, int NREP, bool QBF16>
__global__ __launch_bounds__(256) void decode_lut_kernel(
    const uint8_t *__restrict__ kcodes, const uint16_t *__restrict__ knorms,
    const uint8_t *__restrict__ vcodes, const uint16_t *__restrict__ vnorms, int64_t n_cells,
    int64_t kv_len, const void *__restrict__ q, int n_q, int n_rep, float qscale, float tau,
    float *__restrict__ ws, int n_split) {
  constexpr int NE = 1 << (2 * B);             // code-pair entries
  constexpr int KPS = 256;                     // keys per split
  constexpr int RW = 4 * B;                    // code dwords per row
  constexpr int RWP = RW + 1;                  // padded LDS row
  constexpr int PSTRIDE = kGroup + 4;
  constexpr int CM = (1 << B) - 1;
  __shared__ float lut[NREP][64][NE];
  __shared__ float qr[NREP][kGroup];
  __shared__ uint32_t vrow[KPS * RWP + 1];
  __shared__ float pv[NREP][KPS];
  __shared__ float lvl[1 << B];
  __shared__ float red_m[4][NREP], red_l[4][NREP];
  __shared__ float obuf2[NREP == 1 ? kGroup : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x, g = blockIdx.y;
  const int64_t w0 = (int64_t)s * KPS;
  if (w0 >= kv_len) return;
  const int nk = (int)(kv_len - w0 < KPS ? kv_len - w0 : KPS);
  const int64_t row0 = (int64_t)g * n_cells + w0;
  const int key = imin(tid, nk - 1);

  // loads: this thread's K and V rows (16-byte chunks) and norms
  uint32_t kw[RW], vw[RW];
#pragma unroll
  for (int c = 0; c < B; ++c) {
    const u32x4_t a = reinterpret_cast<const u32x4_t *>(kcodes + (row0 + key) * (16 * B))[c];
    const u32x4_t b = reinterpret_cast<const u32x4_t *>(vcodes + (row0 + key) * (16 * B))[c];
    kw[4 * c] = a.x; kw[4 * c + 1] = a.y; kw[4 * c + 2] = a.z; kw[4 * c + 3] = a.w;
    vw[4 * c] = b.x; vw[4 * c + 1] = b.y; vw[4 * c + 2] = b.z; vw[4 * c + 3] = b.w;
  }
  const float kn = half_to_float(knorms[row0 + key]);
  const float vn = half_to_float(vnorms[row0 + key]);
  // rotated query of the NREP heads: lanes 0-31 / 32-63 of wave w hold heads
  // 2w / 2w + 1, lane j elements 4j .. 4j+3
  if (wave < (NREP + 1) / 2) {
    const int h = 2 * wave + (lane >> 5), j = lane & 31;
    if (h < NREP) {
      const int64_t qb = ((int64_t)g * n_rep + h) * kGroup + 4 * j;
      float x[4];
      if constexpr (QBF16) {
        const u32x2_t bw = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(q) + qb);
        x[0] = __uint_as_float(bw.x << 16);
        x[1] = __uint_as_float(bw.x & 0xffff0000u);
        x[2] = __uint_as_float(bw.y << 16);
        x[3] = __uint_as_float(bw.y & 0xffff0000u);
      } else {
        const float4 f = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(q) + qb);
        x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
      }
      const uint32_t sn = sign_nibble(j);
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = flip_sign(x[i], (sn >> i) & 1u);
      wht128_half(x, j);
#pragma unroll
      for (int i = 0; i < 4; ++i) qr[h][4 * j + i] = x[i];
    }
  }
  if (tid <= CM) lvl[tid] = code_value<B>(tid);
#pragma unroll
  for (int w = 0; w < RW; ++w) vrow[tid * RWP + w] = vw[w];
  __syncthreads();
  // the table: entry e of dim pair dp packs the codes of elements 2dp (low
  // bits) and 2dp + 1
#pragma unroll 4
  for (int i = tid; i < NREP * 64 * NE; i += 256) {
    const int h = i / (64 * NE), dp = (i / NE) % 64, e = i % NE;
    lut[h][dp][e] = qr[h][2 * dp] * lvl[e & CM] + qr[h][2 * dp + 1] * lvl[e >> B];
  }
  __syncthreads();

  // ---- scores (log2 domain): key tid
  float sc[NREP];
#pragma unroll
  for (int h = 0; h < NREP; ++h) sc[h] = 0.f;
#pragma unroll
  for (int dp = 0; dp < 64; ++dp) {
    const int pos = 2 * B * dp, w = pos >> 5, sh = pos & 31;
    const uint32_t x = sh + 2 * B <= 32 ? kw[w] >> sh : __builtin_amdgcn_alignbit(kw[w + 1], kw[w], sh);
    const int e = (int)(x & (NE - 1));
#pragma unroll
    for (int h = 0; h < NREP; ++h) sc[h] += lut[h][dp][e];
  }
#pragma unroll
  for (int h = 0; h < NREP; ++h) sc[h] = tid < nk ? sc[h] * kn * qscale : -INFINITY;
  // split maximum and weight sum per head
  float M[NREP];
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    float m = sc[h];
    m = fmaxf(m, xor_lane<1>(m));
    m = fmaxf(m, xor_lane<2>(m));
    m = fmaxf(m, xor_lane<4>(m));
    m = fmaxf(m, xor_lane<8>(m));
    m = fmaxf(m, xor_lane<16>(m));
    m = max_xor32(m);
    if (lane == 0) red_m[wave][h] = m;
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < NREP; ++h) M[h] = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    const float p = __builtin_amdgcn_exp2f(sc[h] - M[h]);   // 0 for a masked key
    pv[h][tid] = tau > 0.f && p < tau ? 0.f : p * vn;
    float l = p;
    l += xor_lane<1>(l);
    l += xor_lane<2>(l);
    l += xor_lane<4>(l);
    l += xor_lane<8>(l);
    l += xor_lane<16>(l);
    l = sum_xor32(l);
    if (lane == 0) red_l[wave][h] = l;
  }
  __syncthreads();

  // ---- values: thread (slot, d), element d's code at bit B d of each row
  const int d = tid & (kGroup - 1), slot = tid >> 7;
  const int vwi = (B * d) >> 5, vsh = (B * d) & 31;
  auto code_of = [&](int j) {
    const uint32_t *r = vrow + j * RWP + vwi;
    const uint32_t x = vsh + B <= 32 ? r[0] >> vsh : __builtin_amdgcn_alignbit(r[1], r[0], vsh);
    return (int)(x & CM);
  };
  if constexpr (NREP == 1) {
    // one head: the two slots take the two key halves
    float o = 0.f;
    const int j0 = slot * (KPS / 2), j1 = imin(j0 + KPS / 2, nk);
#pragma unroll 4
    for (int j = j0; j < j1; ++j) o += pv[0][j] * lvl[code_of(j)];
    if (slot == 1) obuf2[d] = o;
    __syncthreads();
    if (slot == 0) {
      o += obuf2[d];
      const float L = (red_l[0][0] + red_l[1][0]) + (red_l[2][0] + red_l[3][0]);
      float *ph = ws + (((int64_t)g * n_rep) * n_split + s) * PSTRIDE;
      ph[d] = o;
      if (d == 0) *reinterpret_cast<float2 *>(ph + kGroup) = make_float2(M[0], L);
    }
  } else {
    for (int h = slot; h < NREP; h += 2) {
      float o = 0.f;
#pragma unroll 4
      for (int j = 0; j < nk; ++j) o += pv[h][j] * lvl[code_of(j)];
      const float L = (red_l[0][h] + red_l[1][h]) + (red_l[2][h] + red_l[3][h]);
      float *ph = ws + (((int64_t)g * n_rep + h) * n_split + s) * PSTRIDE;
      ph[d] = o;
      if (d == 0) *reinterpret_cast<float2 *>(ph + kGroup) = make_float2(M[h], L);
    }
  }
}

// Merge the split partials of one 128-element group (blockIdx.y) of one
// output row (blockIdx.x: (sequence, query row, q head)), undo the rotation
// and write that part of the float32 row: out = s (.) H O / (128 L).  Only
// the splits that hold the sequence's cells are read.  NTH / 32 lane groups
// of 32 share the splits (s = group mod NTH / 32), each with its own running
// max; lane j owns elements 4j..4j+3.  NTH = 256 up to 64 splits (eight per
// group), else 512: at 64 splits 256 threads measured 0.14 us less per call,
// at 128 splits 0.3-0.45 us more.  dv is the output width (128 x gridDim.y);
// a split holds 2^split_log2 cells.
// A row that sees no cell (all its splits' maxima -inf) is written as zeros.
// kRowsMasked: several query rows per sequence, so a split may hold no cell
// that a row sees (maximum -inf); one-row calls never have such splits and
// keep the unguarded chain of running maxima.
template <bool kRowsMasked, int NTH>
__global__ __launch_bounds__(NTH) void decode_merge_kernel(
    const float *__restrict__ ws, int n_split, int split_log2, int dv, const int64_t *__restrict__ seq_start,
    const int32_t *__restrict__ seq_len, int64_t kv_len, int64_t n_cells, int rows_per_seq,
    float *__restrict__ out) {
  constexpr int kMergeGroups = NTH / 32;
  __shared__ float4 obuf[kMergeGroups][32];
  __shared__ float lbuf[kMergeGroups], mbuf[kMergeGroups];
  const int h = blockIdx.x, og = blockIdx.y, tid = threadIdx.x;
  const int grp = tid >> 5, j = tid & 31;
  const int pstride = part_stride(dv);
  const SeqExtent ext = seq_extent(seq_start, seq_len, h / rows_per_seq, kv_len, n_cells);
  const int n_valid = (int)((ext.len + (1 << split_log2) - 1) >> split_log2);   // splits holding its cells
  const float *part = ws + (int64_t)h * n_split * pstride;
  float mg = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // batches of 8 splits per group, every load of a batch issued before the
  // first use: the partials come from other compute units' writes, so each
  // dependent round costs a full memory latency
  constexpr int kBatch = 8;
  for (int s0 = grp; s0 < n_valid; s0 += kBatch * kMergeGroups) {
    float2 ml[kBatch];
    float4 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int s = s0 + i * kMergeGroups;
      if (s < n_valid) {
        const float *p = part + (int64_t)s * pstride;
        ml[i] = *reinterpret_cast<const float2 *>(p + dv);
        v[i] = reinterpret_cast<const float4 *>(p + kGroup * og)[j];
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (s0 + i * kMergeGroups >= n_valid) break;
      const float mn = fmaxf(mg, ml[i].x);
      float a = __builtin_amdgcn_exp2f(mg - mn);
      float w = __builtin_amdgcn_exp2f(ml[i].x - mn);
      if constexpr (kRowsMasked) {
        // both maxima -inf: nothing seen yet, and -inf - -inf is NaN
        a = mg == -INFINITY ? 0.f : a;
        w = ml[i].x == -INFINITY ? 0.f : w;
      }
      L = L * a + w * ml[i].y;
      acc.x = acc.x * a + w * v[i].x;
      acc.y = acc.y * a + w * v[i].y;
      acc.z = acc.z * a + w * v[i].z;
      acc.w = acc.w * a + w * v[i].w;
      mg = mn;
    }
  }
  obuf[grp][j] = acc;
  if (j == 0) {
    lbuf[grp] = L;
    mbuf[grp] = mg;
  }
  __syncthreads();
  if (tid >= 32) return;
  float M = mbuf[0];
#pragma unroll
  for (int gq = 1; gq < kMergeGroups; ++gq) M = fmaxf(M, mbuf[gq]);
  float u[4] = {0.f, 0.f, 0.f, 0.f};
  float Lt = 0.f;
#pragma unroll
  for (int gq = 0; gq < kMergeGroups; ++gq) {
    const float w = mbuf[gq] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mbuf[gq] - M);
    const float4 v = obuf[gq][j];
    u[0] += w * v.x; u[1] += w * v.y; u[2] += w * v.z; u[3] += w * v.w;
    Lt += w * lbuf[gq];
  }
  wht128_half(u, j);
  const float r = Lt > 0.f ? 1.0f / (128.0f * Lt) : 0.f;
  float4 res;
  res.x = flip_sign(u[0] * r, sign_bit_of(4 * j + 0));
  res.y = flip_sign(u[1] * r, sign_bit_of(4 * j + 1));
  res.z = flip_sign(u[2] * r, sign_bit_of(4 * j + 2));
  res.w = flip_sign(u[3] * r, sign_bit_of(4 * j + 3));
  reinterpret_cast<float4 *>(out + (int64_t)h * dv + kGroup * og)[j] = res;
}

#ifndef TQ_DECODE_FUSED_BLOCK4_TU
// ---------------------------------------------------------------- host side

// The one-block fused variants (64-key blocks, no prefetch) are compiled in
// tq_decode_fused4.hip, with another instruction scheduling strategy.
#define TQ_FUSED_PARAMS                                                                                     \
  const uint8_t *, const uint16_t *, const uint8_t *, const uint16_t *, int64_t, const int64_t *,        \
      const int32_t *, int64_t, const void *, int, int, int, int, int, float, float, float *, int
extern template __global__ void decode_fused_kernel<2, 4, true, false>(TQ_FUSED_PARAMS);
extern template __global__ void decode_fused_kernel<2, 4, false, false>(TQ_FUSED_PARAMS);
extern template __global__ void decode_fused_kernel<3, 4, true, false>(TQ_FUSED_PARAMS);
extern template __global__ void decode_fused_kernel<3, 4, false, false>(TQ_FUSED_PARAMS);
extern template __global__ void decode_fused_kernel<4, 4, true, false>(TQ_FUSED_PARAMS);
extern template __global__ void decode_fused_kernel<4, 4, false, false>(TQ_FUSED_PARAMS);
#undef TQ_FUSED_PARAMS

hipError_t device_cu_count(int *n_cu) {
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && cache[dev] > 0) {
    *n_cu = cache[dev];
    return hipSuccess;
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (n < 1) n = 1;
  if (dev >= 0 && dev < 64) cache[dev] = n;
  *n_cu = n;
  return hipSuccess;
}

hipError_t launch_split_merge(const float *ws, int n_split, int split_log2, int dv, int64_t rows_out,
                              float *out, hipStream_t stream) {
  if (n_split < 1 || rows_out < 1 || rows_out > 0x7fffffff || dv % kGroup) return hipErrorInvalidValue;
  const dim3 mgrid((unsigned)rows_out, dv / kGroup);
  // every split is read (length n_split << split_log2 from cell 0); empty
  // ones carry maximum -inf, which the masked chain skips
  const int64_t len = (int64_t)n_split << split_log2;
  if (n_split <= 64)
    hipLaunchKernelGGL((decode_merge_kernel<true, 256>), mgrid, dim3(256), 0, stream, ws, n_split, split_log2, dv,
                       nullptr, nullptr, len, len, 1, out);
  else
    hipLaunchKernelGGL((decode_merge_kernel<true, 512>), mgrid, dim3(512), 0, stream, ws, n_split, split_log2, dv,
                       nullptr, nullptr, len, len, 1, out);
  return hipGetLastError();
}

// Most q heads per kv head for which automatic routing takes the Q x
// centroid table kernel: none.  Measured on one MI355X (turbo3, graph
// replay, us per call, matrix path against table path): 1 q / 1 kv head
// over 256 cells 6.9 / 18.1; over 32768 cells 8 q / 8 kv 18.9 / 27.4, 16 q /
// 8 kv 19.1 / 63.2, 32 q / 4 kv 14.5 / 227.5.  The table path stays
// available by request (TQ_DECODE_TABLE).
constexpr int kTableMaxRepAuto = 0;

hipError_t plan_decode(const tq_cache &k, const tq_cache &v, int64_t max_len, int32_t n_q_heads,
                       int n_rows, int n_seq, DecodePlan *p, int path) {
  int n_cu = 0;
  hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  const int n_rep = n_q_heads / k.n_kv_heads;
  p->n_rows = n_rows;
  p->n_seq = n_seq;
  // (row, q head) pairs per workgroup: 16 (two column sets over one decode
  // of the cells) when a kv head has more than eight pairs and both caches
  // are turbo with 128-wide heads, else 8
  const int n_pairs = n_rows * n_rep;
  p->pairs = n_pairs > 8 && k.type != TQ_Q8 && k.head_dim == kGroup && v.head_dim == kGroup ? 16 : 8;
  p->head_groups = ceil_div(n_pairs, p->pairs);
  // a split covers 4 ranges of 16 * tiles keys.  Tiles per range: the most
  // (1, 2, 4 or 8) with at most 16 group-tiles per range (tiles x (K groups
  // + V groups)) that still give every compute unit a workgroup; 8 only
  // while its grid is a single round (8-tile workgroups hold one compute
  // unit each).  Measured: fewer, larger workgroups cost less setup and
  // fewer split partials in one round; over several rounds two 4-tile
  // workgroups per compute unit hide each other's memory latency (20% faster
  // for 8 sequences of 2 rows).
  const int groups = k.head_dim / kGroup + v.head_dim / kGroup;
  const int64_t wg_per_split = (int64_t)k.n_kv_heads * p->head_groups * n_seq;
  // (sixteen pairs hold two column sets of value accumulators beside the
  // tiles' hi operands: at most 4 tiles fit the registers)
  int tpw = p->pairs == 16 ? 4 : 8;
  while (tpw > 1) {
    const int64_t splits = ceil_div<int64_t>(max_len, 64LL * tpw);
    if (tpw * groups <= 16 && splits * wg_per_split >= n_cu) {
      if (tpw == 8 && splits * wg_per_split > n_cu) tpw = 4;
      break;
    }
    tpw >>= 1;
  }
  p->tiles_per_wave = tpw;
  p->keys_per_split = 64 * tpw;
  p->fused = 0;
  p->nb = 1;
  p->lut = 0;
  const bool table_ok = n_rows == 1 && n_seq == 1 && n_rep <= 8 && (k.type == TQ_TURBO2 || k.type == TQ_TURBO3) &&
                        k.type == v.type && k.head_dim == kGroup && v.head_dim == kGroup;
  if (path == TQ_DECODE_TABLE && !table_ok) return hipErrorNotSupported;
  if (path != TQ_DECODE_AUTO && path != TQ_DECODE_MATRIX && path != TQ_DECODE_TABLE) return hipErrorInvalidValue;
  if (table_ok && (path == TQ_DECODE_TABLE || (path == TQ_DECODE_AUTO && n_rep <= kTableMaxRepAuto))) {
    p->lut = 1;
    p->pairs = n_rep;
    p->head_groups = 1;
    p->tiles_per_wave = 1;
    p->keys_per_split = 256;
  } else
  // One 128-wide group each way, both caches turbo, and at most eight
  // (row, q head) pairs per kv head or a single sequence: the fused kernel,
  // eight waves of blocks of 16 tb keys, eight pairs per workgroup (more
  // pairs take more pair groups over the same cells).  tb: the most (4, 2,
  // 1) that still gives every compute unit a workgroup; nb blocks per wave:
  // as many (a power of two) as keep the grid at least one full round, so
  // long sequences stream through one round of workgroups (then with blocks
  // of at most 2 tiles, the next block's loads in flight beside the current
  // one).  Batches of several sequences with more than eight pairs keep the
  // sixteen-pair split kernel: the fused kernel holds a compute unit per
  // workgroup, and when the batch's lengths (which live on the device) are
  // mixed, the split kernel's two workgroups per compute unit overlap its
  // several rounds.  Measured, 8 sequences x 2 rows, 32 q / 4 kv heads,
  // graph replay, us per call, split kernel against fused pair groups:
  // lengths 2000 - 32768 (131,072 cells) 77.0 / 84.0; all 16384: 63.3 / 48.2
  // (with the fused grid sized for one sequence of max_len cells instead of
  // all of them: 105 / 69).
  if (k.type != TQ_Q8 && k.type == v.type && k.head_dim == kGroup && v.head_dim == kGroup &&
      (n_pairs <= 8 || n_seq == 1)) {
    const int n_hg = ceil_div(n_pairs, 8);
    const int64_t wg = (int64_t)k.n_kv_heads * n_hg * n_seq;
    int tb = 4;
    while (tb > 1 && ceil_div<int64_t>(max_len, 128LL * tb) * wg < n_cu) tb >>= 1;
    int64_t per = ceil_div<int64_t>(max_len, 128LL * tb) * wg;
    if (tb == 4 && per >= 2 * n_cu) {
      tb = 2;
      per = ceil_div<int64_t>(max_len, 256LL) * wg;
    }
    int nb = 1;
    while (nb < (1 << 20) && (int64_t)nb * 2 * n_cu <= per) nb *= 2;
    p->fused = 1;
    p->pairs = 8;
    p->head_groups = n_hg;
    p->tiles_per_wave = tb;
    p->nb = nb;
    p->keys_per_split = 128 * tb * nb;
  }
  const int64_t n_split = ceil_div<int64_t>(max_len, p->keys_per_split);
  if (n_split > 0x7fffffff || (int64_t)k.n_kv_heads * p->head_groups > 65535 || n_seq > 65535)
    return hipErrorInvalidValue;
  p->n_split = (int)n_split;
  const size_t bytes = (size_t)n_seq * (size_t)n_rows * (size_t)n_q_heads * (size_t)n_split *
                       part_stride(v.head_dim) * sizeof(float);
  p->workspace_bytes = (bytes + 255) & ~(size_t)255;
  return hipSuccess;
}

namespace {

struct SplitArgs {
  const tq_cache *k, *v;
  const int64_t *seq_start;
  const int32_t *seq_len;
  int64_t kv_len;
  const void *q;
  int n_q, n_rep, n_rows, n_hg;
  float qs, tau;
  float *ws;
  int n_split;
};

// Tile counts the plan can choose for GK + GV groups (8 only for one turbo
// group each: the ranges of wider heads would not fit the registers and LDS).
template <int B, int GK, int GV, bool QBF, bool KQ8>
hipError_t launch_split(int tpw, int pairs, dim3 grid, hipStream_t st, const SplitArgs &a) {
  dim3 block(kDecThreads);
#define TQ_DEC(T, HP)                                                                                  \
  hipLaunchKernelGGL((decode_split_kernel<B, T, GK, GV, QBF, KQ8, HP>), grid, block, 0, st, a.k->codes, \
                     a.k->norms, a.v->codes, a.v->norms, a.k->n_cells, a.seq_start, a.seq_len,         \
                     a.kv_len, a.q, a.n_q, a.n_rep, a.n_rows, a.n_hg, a.qs, a.tau, a.ws, a.n_split)
  if (pairs == 16) {
    // 16 pairs: one turbo group each way, up to 4 tiles
    if constexpr (GK + GV == 2 && !KQ8) {
      switch (tpw) {
        case 1: TQ_DEC(1, 16); break;
        case 2: TQ_DEC(2, 16); break;
        case 4: TQ_DEC(4, 16); break;
        default: return hipErrorNotSupported;
      }
      return hipSuccess;
    } else {
      return hipErrorNotSupported;
    }
  }
  switch (tpw) {
    case 1: TQ_DEC(1, 8); break;
    case 2: TQ_DEC(2, 8); break;
    case 4: TQ_DEC(4, 8); break;
    case 8:
      if constexpr (GK + GV == 2) {
        TQ_DEC(8, 8);
        break;
      } else {
        return hipErrorNotSupported;
      }
    default: return hipErrorNotSupported;
  }
#undef TQ_DEC
  return hipSuccess;
}

template <int B, int GK, int GV>
hipError_t launch_split_q(int qbf, int kq8, int tpw, int pairs, dim3 grid, hipStream_t st, const SplitArgs &a) {
  if (kq8)
    return qbf ? launch_split<B, GK, GV, true, true>(tpw, pairs, grid, st, a)
               : launch_split<B, GK, GV, false, true>(tpw, pairs, grid, st, a);
  return qbf ? launch_split<B, GK, GV, true, false>(tpw, pairs, grid, st, a)
             : launch_split<B, GK, GV, false, false>(tpw, pairs, grid, st, a);
}

template <int B>
hipError_t launch_split_dims(int gk, int gv, int qbf, int kq8, int tpw, int pairs, dim3 grid, hipStream_t st,
                             const SplitArgs &a) {
  if (gk == 1 && gv == 1) return launch_split_q<B, 1, 1>(qbf, kq8, tpw, pairs, grid, st, a);
  if (gk == 2 && gv == 2) return launch_split_q<B, 2, 2>(qbf, kq8, tpw, pairs, grid, st, a);
  if (gk == 2) return launch_split_q<B, 2, 1>(qbf, kq8, tpw, pairs, grid, st, a);
  return launch_split_q<B, 1, 2>(qbf, kq8, tpw, pairs, grid, st, a);
}

template <int B, bool QBF>
hipError_t launch_fused_tb(int tb, dim3 grid, hipStream_t st, const SplitArgs &a, int nb) {
  dim3 block(kDecThreads);
#define TQ_FUSED(TB, PF)                                                                               \
  hipLaunchKernelGGL((decode_fused_kernel<B, TB, QBF, PF>), grid, block, 0, st, a.k->codes, a.k->norms, \
                     a.v->codes, a.v->norms, a.k->n_cells, a.seq_start, a.seq_len, a.kv_len, a.q, a.n_q, \
                     a.n_rep, a.n_rows, a.n_hg, nb, a.qs, a.tau, a.ws, a.n_split)
  // several blocks per wave: prefetching variants (at most 2 tiles per
  // block, the prefetch registers beside them)
  if (nb > 1) {
    switch (tb) {
      case 1: TQ_FUSED(1, true); break;
      case 2: TQ_FUSED(2, true); break;
      default: return hipErrorNotSupported;
    }
  } else {
    switch (tb) {
      case 1: TQ_FUSED(1, false); break;
      case 2: TQ_FUSED(2, false); break;
      case 4: TQ_FUSED(4, false); break;
      default: return hipErrorNotSupported;
    }
  }
#undef TQ_FUSED
  return hipSuccess;
}

template <int B, int R, bool QBF>
hipError_t launch_lut_r(dim3 grid, hipStream_t st, const SplitArgs &a) {
  hipLaunchKernelGGL((decode_lut_kernel<B, R, QBF>), grid, dim3(256), 0, st, a.k->codes, a.k->norms,
                     a.v->codes, a.v->norms, a.k->n_cells, a.kv_len, a.q, a.n_q, a.n_rep, a.qs, a.tau, a.ws,
                     a.n_split);
  return hipSuccess;
}

template <int B, bool QBF>
hipError_t launch_lut_b(int n_rep, dim3 grid, hipStream_t st, const SplitArgs &a) {
  switch (n_rep) {
    case 1: return launch_lut_r<B, 1, QBF>(grid, st, a);
    case 2: return launch_lut_r<B, 2, QBF>(grid, st, a);
    case 3: return launch_lut_r<B, 3, QBF>(grid, st, a);
    case 4: return launch_lut_r<B, 4, QBF>(grid, st, a);
    case 5: return launch_lut_r<B, 5, QBF>(grid, st, a);
    case 6: return launch_lut_r<B, 6, QBF>(grid, st, a);
    case 7: return launch_lut_r<B, 7, QBF>(grid, st, a);
    case 8: return launch_lut_r<B, 8, QBF>(grid, st, a);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_lut(int type, int n_rep, int qbf, dim3 grid, hipStream_t st, const SplitArgs &a) {
  switch (type) {
    case TQ_TURBO2: return qbf ? launch_lut_b<2, true>(n_rep, grid, st, a) : launch_lut_b<2, false>(n_rep, grid, st, a);
    case TQ_TURBO3: return qbf ? launch_lut_b<3, true>(n_rep, grid, st, a) : launch_lut_b<3, false>(n_rep, grid, st, a);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_fused(int type, int tb, int qbf, dim3 grid, hipStream_t st, const SplitArgs &a, int nb) {
  switch (type) {
    case TQ_TURBO2: return qbf ? launch_fused_tb<2, true>(tb, grid, st, a, nb) : launch_fused_tb<2, false>(tb, grid, st, a, nb);
    case TQ_TURBO3: return qbf ? launch_fused_tb<3, true>(tb, grid, st, a, nb) : launch_fused_tb<3, false>(tb, grid, st, a, nb);
    case TQ_TURBO4: return qbf ? launch_fused_tb<4, true>(tb, grid, st, a, nb) : launch_fused_tb<4, false>(tb, grid, st, a, nb);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

hipError_t launch_decode(const tq_cache &k, const tq_cache &v, const int64_t *seq_start,
                         const int32_t *seq_len, int64_t kv_len, const void *q, int q_dtype,
                         int32_t n_q_heads, float scale, float sparse_v_tau, float *out,
                         void *workspace, const DecodePlan &p, hipStream_t stream) {
  const int gk = k.head_dim / kGroup, gv = v.head_dim / kGroup;
  const int kq8 = k.type == TQ_Q8 ? 1 : 0;
  if (gk < 1 || gk > 2 || gv < 1 || gv > 2 || (!kq8 && k.type != v.type) || v.type == TQ_Q8)
    return hipErrorNotSupported;
  SplitArgs a;
  a.k = &k;
  a.v = &v;
  a.seq_start = seq_start;
  a.seq_len = seq_len;
  a.kv_len = kv_len;
  a.q = q;
  a.n_q = n_q_heads;
  a.n_rep = n_q_heads / k.n_kv_heads;
  a.n_rows = p.n_rows;
  a.n_hg = p.head_groups;
  // scores in the log2 domain: scale * log2(e), and for turbo K 1/128 for
  // the two 1/sqrt(128) factors of the rotated query and the rotated levels
  a.qs = scale * 1.4426950408889634f / (kq8 ? 1.0f : 128.0f);
  a.tau = sparse_v_tau;
  a.ws = reinterpret_cast<float *>(workspace);
  a.n_split = p.n_split;
  dim3 grid(p.n_split, k.n_kv_heads * p.head_groups, p.n_seq);
  const int qbf = q_dtype == TQ_BF16 ? 1 : 0;
  hipError_t e;
  if (p.lut) {
    if (seq_start || seq_len) return hipErrorInvalidValue;
    e = launch_lut(v.type, a.n_rep, qbf, dim3(p.n_split, k.n_kv_heads, 1), stream, a);
  } else if (p.fused) {
    e = launch_fused(v.type, p.tiles_per_wave, qbf, grid, stream, a, p.nb);
  } else {
  switch (v.type) {
    case TQ_TURBO2: e = launch_split_dims<2>(gk, gv, qbf, kq8, p.tiles_per_wave, p.pairs, grid, stream, a); break;
    case TQ_TURBO3: e = launch_split_dims<3>(gk, gv, qbf, kq8, p.tiles_per_wave, p.pairs, grid, stream, a); break;
    default: e = launch_split_dims<4>(gk, gv, qbf, kq8, p.tiles_per_wave, p.pairs, grid, stream, a); break;
  }
  }
  if (e != hipSuccess) return e;
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows_out = (int64_t)p.n_seq * p.n_rows * n_q_heads;
  const dim3 mgrid((unsigned)rows_out, gv);
  const int split_log2 = __builtin_ctz((unsigned)p.keys_per_split);
#define TQ_MERGE(MASKED, NTH)                                                                        \
  hipLaunchKernelGGL((decode_merge_kernel<MASKED, NTH>), mgrid, dim3(NTH), 0, stream, a.ws, p.n_split,     \
                     split_log2, v.head_dim, seq_start, seq_len, kv_len, k.n_cells, p.n_rows * n_q_heads, out)
  const bool narrow = p.n_split <= 64;
  if (p.n_rows > 1) {
    if (narrow) TQ_MERGE(true, 256); else TQ_MERGE(true, 512);
  } else {
    if (narrow) TQ_MERGE(false, 256); else TQ_MERGE(false, 512);
  }
#undef TQ_MERGE
  return hipGetLastError();
}

#endif  // TQ_DECODE_FUSED_BLOCK4_TU

}  // namespace tq
