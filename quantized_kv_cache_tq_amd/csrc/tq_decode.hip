// tq_decode.hip -- decode attention (one query row) over a turbo cache.
//
// [PR36] (c) decodes with a per-query-head Q x centroid table in shared
// memory (one shared read per element and head).  With eight query heads per
// kv head that is eight table reads per cache element, far more LDS traffic
// than the packed stream itself.  On CDNA4 the eight heads are one dense
// contraction instead: every packed code is decoded ONCE per kv head into a
// float16 level through a table in LDS (indexed by the concatenated codes of
// 2 or 4 neighbouring elements, so one LDS read yields 2-4 levels), and the
// matrix cores do Q.K^T and P.V for all heads of the kv head at once.
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
// The levels are float16-exact, so the only roundings are float32
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
constexpr int kD = 128;              // head_dim handled by this kernel
constexpr int kPartStride = kD + 4;  // o[128], m, l, pad (floats; 16-byte rows)


// Bits [pos, pos+nbits) of a little-endian dword array (pos and nbits are
// compile-time after unrolling; the field spans at most two dwords).
__device__ __forceinline__ uint32_t bits_at(const uint32_t *dw, int pos, int nbits) {
  const int w = pos >> 5, sh = pos & 31;
  uint32_t x = dw[w] >> sh;
  if (sh + nbits > 32) x |= dw[w + 1] << (32 - sh);
  return nbits == 32 ? x : (x & ((1u << nbits) - 1u));
}

// Decode NEL consecutive elements held in dw (first element in bit 0) into
// float16 pairs out[0 .. NEL/2) through the pair table; tab points at this
// lane's copy (dword lane of the table).
template <int B, int NEL>
__device__ __forceinline__ void decode_pairs(const uint32_t *dw, const uint32_t *tab,
                                             uint32_t *out) {
  constexpr int PB = 2 * B;
#pragma unroll
  for (int j = 0; j < NEL / 2; ++j) out[j] = tab[bits_at(dw, PB * j, PB) * 64];
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

// Workgroup (split s, kv head g): eight waves, four key ranges of KPW = 16T
// keys.  Waves 0-3 ("key waves") score their range and turn the scores into
// the matrix-core operand P; waves 4-7 ("value waves") meanwhile decode the
// V codes of the same ranges into B operands held in registers.  After one
// barrier every value wave runs its T x 8 value products; the four partial
// outputs are merged in shared memory and written as one split partial.
template <int B, int T, bool QBF16>
__global__ __launch_bounds__(kDecThreads, 2) void decode_split_kernel(
    const uint8_t *__restrict__ kcodes, const uint16_t *__restrict__ knorms,
    const uint8_t *__restrict__ vcodes, const uint16_t *__restrict__ vnorms, int64_t n_cells,
    int64_t kv_len, const void *__restrict__ q, int n_rep, float qscale, float tau,
    float *__restrict__ ws, int n_split) {
  constexpr int KPW = 16 * T;                  // keys per range
  constexpr int KPS = 4 * KPW;                 // keys per split
  constexpr int ROWW = 4 * B;                  // code dwords per key
  constexpr int ROWP = ROWW + 1;               // padded LDS row
  constexpr int RPL = ceil_div(KPW, 64);       // V rows per lane
  constexpr int NNORM = ceil_div(KPW, 64);
  __shared__ __align__(16) uint32_t ptab[PairCfg<B>::WORDS];   // pair table, 64 copies
  // V rows of the four ranges, plus one spare dword (a lane's two-dword
  // read of a row may touch the dword after it)
  __shared__ __align__(16) uint32_t vrows[4 * KPW * ROWP + 1];
  __shared__ __align__(16) u32x2_t pbuf[4][T][64];          // P operands, per lane
  __shared__ __align__(16) float nk[4][KPW];
  __shared__ __align__(16) float nv[4][KPW];
  __shared__ __align__(16) uint32_t qbuf[4 * 64 * 4];       // query operand, [t][lane][8 halves]
  __shared__ __align__(16) float obuf[4][8 * kD];
  __shared__ float wm[4][8], wl[4][8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & 3;                     // key range of this wave
  const bool kwave = wave < 4;
  const int col = lane & 15, quad = lane >> 4;
  const int s = blockIdx.x, g = blockIdx.y;
  // keys [w0, w0 + wkeys) of range rg; addressing is relative to row0, a
  // valid key row, with lane offsets clamped to the range's last key
  const int64_t w0 = (int64_t)s * KPS + (int64_t)rg * KPW;
  const int64_t left = kv_len - w0;
  const int wkeys = (int)(left < 0 ? 0 : (left < KPW ? left : KPW));
  const int wlast = wkeys > 0 ? wkeys - 1 : 0;
  const int64_t row0 = (int64_t)g * n_cells + (wkeys > 0 ? w0 : kv_len - 1);

  if (kwave) {
    // ---------------- key wave: loads first (query, norms, K codes)
    const uint8_t *kb = kcodes + row0 * (16 * B);
    const uint16_t *knb = knorms + row0, *vnb = vnorms + row0;
    const int qh = 2 * rg + (lane >> 5), qj = lane & 31;
    const int64_t qbase = ((int64_t)g * n_rep + imin(qh, n_rep - 1)) * kD + 4 * qj;
    float qv[4];
    if constexpr (QBF16) {
      const u32x2_t b = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(q) + qbase);
      qv[0] = __uint_as_float(b.x << 16);
      qv[1] = __uint_as_float(b.x & 0xffff0000u);
      qv[2] = __uint_as_float(b.y << 16);
      qv[3] = __uint_as_float(b.y & 0xffff0000u);
    } else {
      const float4 f = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(q) + qbase);
      qv[0] = f.x; qv[1] = f.y; qv[2] = f.z; qv[3] = f.w;
    }
    uint16_t kn[NNORM], vn[NNORM];
#pragma unroll
    for (int i = 0; i < NNORM; ++i) {
      const uint32_t kk = (uint32_t)imin(lane + 64 * i, wlast);
      kn[i] = knb[kk];
      vn[i] = vnb[kk];
    }
    // lane (col, quad) of tile t reads key 16t + col, dwords B*quad .. B*quad+B-1
    uint32_t kd[T][B];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const uint32_t off = (uint32_t)imin(16 * t + col, wlast) * (4u * ROWW) + 4u * B * quad;
      const uint32_t *row = reinterpret_cast<const uint32_t *>(kb + off);
#pragma unroll
      for (int i = 0; i < B; ++i) kd[t][i] = row[i];
    }

    build_pair_table<B, kDecThreads>(ptab, tid);
    // rotate + split heads 2rg, 2rg+1: thread holds d = 4qj .. 4qj+3 of head
    // qh; in the MFMA B operand they are slots i = 4(qj&1) .. +3 of K-step
    // t = (qj>>1)&3 in lane 16*(qj>>3) + qh (high half) and
    // 16*(qj>>3) + 8 + qh (low half)
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[i] = flip_sign(qv[i], sign_bit_of(4 * qj + i));
    wht128_half(qv, qj);
    {
      const bool live = qh < n_rep;
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
      const int t = (qj >> 1) & 3, qd = qj >> 3, half_off = 2 * (qj & 1);
      *reinterpret_cast<u32x2_t *>(qbuf + (t * 64 + 16 * qd + qh) * 4 + half_off) = u32x2_t{hw[0], hw[1]};
      *reinterpret_cast<u32x2_t *>(qbuf + (t * 64 + 16 * qd + 8 + qh) * 4 + half_off) = u32x2_t{lw[0], lw[1]};
    }
    __syncthreads();   // table and query operand complete

    // norms of the range (this wave's own slice)
#pragma unroll
    for (int i = 0; i < NNORM; ++i) {
      const int kk = lane + 64 * i;
      if (kk < KPW) {
        const bool ok = kk < wkeys;
        nk[rg][kk] = ok ? half_to_float(kn[i]) : 0.f;
        nv[rg][kk] = ok ? half_to_float(vn[i]) : 0.f;
      }
    }
    // Query operand: column n = lane & 15 -> head n & 7, high (n < 8) or low
    // half; k-slot (lane >> 4, i) of K-step t <-> element d = 32*(lane>>4) + 8t + i.
    half8_t qb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      qb[t] = __builtin_bit_cast(half8_t, reinterpret_cast<const u32x4_t *>(qbuf)[t * 64 + lane]);
    wave_lds_fence();

    // ---- scores: S^T[key][col] over the range, tile by tile
    const uint32_t *tab = ptab + lane;
    float sc[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      uint32_t a16[16];
      decode_pairs<B, 32>(kd[t], tab, a16);
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const u32x4_t av = {a16[4 * st], a16[4 * st + 1], a16[4 * st + 2], a16[4 * st + 3]};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[st], acc,
                                                    0, 0, 0);
      }
      const float4 n4 = *reinterpret_cast<const float4 *>(&nk[rg][16 * t + 4 * quad]);
      const float nkv[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[t][i] = (acc[i] + xor_lane<8>(acc[i])) * nkv[i];
    }
    if (wkeys < KPW) {   // wave-uniform: only a ragged last range masks
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * t + 4 * quad + i >= wkeys) sc[t][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[t][i]);
    // range max per head (log2 domain); -inf for a range without keys
    mx = fmaxf(mx, xor_lane<16>(mx));
    mx = max_xor32(mx);
    const float msafe = mx == -INFINITY ? 0.f : mx;

    // ---- P operand: the score layout (lane = column + 16 * key quad) is the
    //      A-operand layout of the value product.  Rows < 8 carry the
    //      float16 high part of p * vnorm, rows >= 8 the low part:
    //      x - hi * lo_sel (lo_sel = 1 on low rows, 0 on high rows) is exact
    //      in float32 and rounds once to float16.  Sparse V ([PR36] (d) item
    //      3): a key whose weight against the range maximum (<= the true
    //      maximum) is below tau leaves the value sum but stays in lsum.
    const float lo_sel = col >= 8 ? 1.f : 0.f;
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const float4 n4 = *reinterpret_cast<const float4 *>(&nv[rg][16 * t + 4 * quad]);
      const float nvv[4] = {n4.x, n4.y, n4.z, n4.w};
      half4_t pa;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(sc[t][i] - msafe);
        lsum += p;
        const float x = p < tau ? 0.f : p * nvv[i];
        const _Float16 h = (_Float16)x;
        pa[i] = (_Float16)__builtin_fmaf(-(float)h, lo_sel, x);
      }
      pbuf[rg][t][lane] = __builtin_bit_cast(u32x2_t, pa);
    }
    lsum += xor_lane<16>(lsum);
    lsum = sum_xor32(lsum);
    if (lane < 8) {
      wm[rg][lane] = mx;
      wl[rg][lane] = lsum;
    }
    __syncthreads();   // P operands complete
    __syncthreads();   // value products done (partial outputs in obuf)
  } else {
    // ---------------- value wave: V rows (lane r loads rows r, r + 64, ...)
    const uint8_t *vb = vcodes + row0 * (16 * B);
    u32x4_t vraw[RPL][B];
#pragma unroll
    for (int j = 0; j < RPL; ++j)
#pragma unroll
      for (int i = 0; i < B; ++i)
        vraw[j][i] = *reinterpret_cast<const u32x4_t *>(
            vb + (uint32_t)imin(lane + 64 * j, wlast) * (16u * B) + 16u * i);
    build_pair_table<B, kDecThreads>(ptab, tid);
    __syncthreads();   // table and query operand complete

    uint32_t *vr = vrows + rg * KPW * ROWP;
#pragma unroll
    for (int j = 0; j < RPL; ++j) {
      const int r = lane + 64 * j;
      if (r < KPW) {
        uint32_t *d = vr + r * ROWP;
#pragma unroll
        for (int i = 0; i < B; ++i) {
          d[4 * i] = vraw[j][i].x;
          d[4 * i + 1] = vraw[j][i].y;
          d[4 * i + 2] = vraw[j][i].z;
          d[4 * i + 3] = vraw[j][i].w;
        }
      }
    }
    wave_lds_fence();
    // B operands: lane (n, quad) of tile t holds keys 16t + 4quad + j
    // (j = 0..3) at d = 8n + dt of d-tile dt; it decodes the 8 elements
    // 8n .. 8n+7 of each of its four keys and regroups them by element.
    constexpr int VBITS = 8 * B;
    const int vpos = VBITS * col;
    const int vw0 = vpos >> 5, vsh = vpos & 31;
    const uint32_t *vlane = vr + 4 * quad * ROWP + vw0;
    const uint32_t *tab = ptab + lane;
    u32x2_t vbop[T][8];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      uint32_t vv[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t *row = vlane + (16 * t + i) * ROWP;
        const uint32_t run[1] = {__builtin_amdgcn_alignbit(row[1], row[0], vsh)};
        decode_pairs<B, 8>(run, tab, vv[i]);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int w = dt >> 1;
        const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;
        vbop[t][dt] = u32x2_t{__builtin_amdgcn_perm(vv[1][w], vv[0][w], sel),
                              __builtin_amdgcn_perm(vv[3][w], vv[2][w], sel)};
      }
    }
    __syncthreads();   // P operands complete

    float4_t o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const half4_t pa = __builtin_bit_cast(half4_t, pbuf[rg][t][lane]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, __builtin_bit_cast(half4_t, vbop[t][dt]),
                                                     o[dt], 0, 0, 0);
    }
    // combine high/low rows: after the swap, lanes 0-31 hold d-tiles 0-3 and
    // lanes 32-63 d-tiles 4-7, each as high + low; row (head) 4*((lane&31)>>4) + i
    const int qd = (lane & 31) >> 4, dhi = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float oc[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[dt][i]),
                                                        __float_as_uint(o[dt + 4][i]), false, false);
        oc[dt] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
      *reinterpret_cast<float4 *>(&obuf[rg][(4 * qd + i) * kD + 8 * col + 4 * dhi]) =
          make_float4(oc[0], oc[1], oc[2], oc[3]);
    }
    __syncthreads();   // value products done (partial outputs in obuf)
  }

  // ---- merge the four ranges: obuf[r][h][8c + t] holds element d = 8c + t
  //      of head h, relative to the range's own max
  float *part = ws + ((int64_t)g * n_rep * n_split + s) * kPartStride;
  {
    const int h = tid >> 6, d = 2 * (tid & 63);
    if (h < n_rep) {
      const float M = fmaxf(fmaxf(wm[0][h], wm[1][h]), fmaxf(wm[2][h], wm[3][h]));
      float a0 = 0.f, a1 = 0.f, L = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float mr = wm[r][h];
        const float f = mr == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mr - M);
        const float2 v = *reinterpret_cast<const float2 *>(&obuf[r][h * kD + d]);
        a0 += f * v.x;
        a1 += f * v.y;
        L += f * wl[r][h];
      }
      float *ph = part + (int64_t)h * n_split * kPartStride;
      *reinterpret_cast<float2 *>(ph + d) = make_float2(a0, a1);
      if (d == 0) *reinterpret_cast<float2 *>(ph + kD) = make_float2(M, L);
    }
  }
}

// Merge the split partials of one query head, undo the rotation and write the
// float32 output row: out = s (.) H O / (128 L).  Sixteen 32-lane groups
// share the splits (s = group mod 16), each with its own running max; lane j
// owns elements 4j..4j+3.
constexpr int kMergeThreads = 512;
constexpr int kMergeGroups = kMergeThreads / 32;
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const float *__restrict__ ws,
                                                                     int n_split,
                                                                     float *__restrict__ out) {
  __shared__ float4 obuf[kMergeGroups][32];
  __shared__ float lbuf[kMergeGroups], mbuf[kMergeGroups];
  const int h = blockIdx.x, tid = threadIdx.x;
  const int grp = tid >> 5, j = tid & 31;
  const float *part = ws + (int64_t)h * n_split * kPartStride;
  float mg = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // batches of 8 splits per group, every load of a batch issued before the
  // first use: the partials come from other compute units' writes, so each
  // dependent round costs a full memory latency
  constexpr int kBatch = 8;
  for (int s0 = grp; s0 < n_split; s0 += kBatch * kMergeGroups) {
    float2 ml[kBatch];
    float4 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int s = s0 + i * kMergeGroups;
      if (s < n_split) {
        const float *p = part + (int64_t)s * kPartStride;
        ml[i] = *reinterpret_cast<const float2 *>(p + kD);
        v[i] = reinterpret_cast<const float4 *>(p)[j];
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (s0 + i * kMergeGroups >= n_split) break;
      const float mn = fmaxf(mg, ml[i].x);
      const float a = __builtin_amdgcn_exp2f(mg - mn);
      const float w = __builtin_amdgcn_exp2f(ml[i].x - mn);
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
  const float r = 1.0f / (128.0f * Lt);
  float4 res;
  res.x = flip_sign(u[0] * r, sign_bit_of(4 * j + 0));
  res.y = flip_sign(u[1] * r, sign_bit_of(4 * j + 1));
  res.z = flip_sign(u[2] * r, sign_bit_of(4 * j + 2));
  res.w = flip_sign(u[3] * r, sign_bit_of(4 * j + 3));
  reinterpret_cast<float4 *>(out + (int64_t)h * kD)[j] = res;
}

// ---------------------------------------------------------------- host side

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

hipError_t plan_decode(const tq_cache &k, int64_t kv_len, int32_t n_q_heads, DecodePlan *p) {
  int n_cu = 0;
  hipError_t e = device_cu_count(&n_cu);
  if (e != hipSuccess) return e;
  // largest tile count (<= 4 per key range) that still gives every compute
  // unit two workgroups; a split covers 4 ranges of 16 * tiles keys
  int tpw = 4;
  while (tpw > 1) {
    const int64_t splits = ceil_div<int64_t>(kv_len, 64LL * tpw);
    if (splits * k.n_kv_heads >= 2LL * n_cu) break;
    tpw >>= 1;
  }
  p->tiles_per_wave = tpw;
  p->keys_per_split = 64 * tpw;
  const int64_t n_split = ceil_div<int64_t>(kv_len, p->keys_per_split);
  if (n_split > 0x7fffffff) return hipErrorInvalidValue;
  p->n_split = (int)n_split;
  const size_t bytes = (size_t)n_q_heads * (size_t)n_split * kPartStride * sizeof(float);
  p->workspace_bytes = (bytes + 255) & ~(size_t)255;
  return hipSuccess;
}

template <int B, bool QBF>
static void launch_split(int tpw, dim3 grid, hipStream_t st, const tq_cache &k,
                         const tq_cache &v, int64_t kv_len, const void *q, int n_rep, float qs,
                         float tau, float *ws, int n_split) {
  dim3 block(kDecThreads);
#define TQ_DEC(T)                                                                             \
  hipLaunchKernelGGL((decode_split_kernel<B, T, QBF>), grid, block, 0, st, k.codes, k.norms, \
                     v.codes, v.norms, k.n_cells, kv_len, q, n_rep, qs, tau, ws, n_split)
  switch (tpw) {
    case 1: TQ_DEC(1); break;
    case 2: TQ_DEC(2); break;
    case 4: TQ_DEC(4); break;
    default: TQ_DEC(8); break;
  }
#undef TQ_DEC
}

template <int B>
static void launch_split_q(int qbf, int tpw, dim3 grid, hipStream_t st, const tq_cache &k,
                           const tq_cache &v, int64_t kv_len, const void *q, int n_rep, float qs,
                           float tau, float *ws, int n_split) {
  if (qbf) launch_split<B, true>(tpw, grid, st, k, v, kv_len, q, n_rep, qs, tau, ws, n_split);
  else launch_split<B, false>(tpw, grid, st, k, v, kv_len, q, n_rep, qs, tau, ws, n_split);
}

hipError_t launch_decode(const tq_cache &k, const tq_cache &v, int64_t kv_len, const void *q,
                         int q_dtype, int32_t n_q_heads, float scale, float sparse_v_tau,
                         float *out, void *workspace, const DecodePlan &p, hipStream_t stream) {
  const int n_rep = n_q_heads / k.n_kv_heads;
  // scores in the log2 domain: scale * log2(e), and 1/128 for the two
  // 1/sqrt(128) factors of the rotated query and the rotated levels
  const float qs = scale * 1.4426950408889634f / 128.0f;
  float *ws = reinterpret_cast<float *>(workspace);
  dim3 grid(p.n_split, k.n_kv_heads);
  const int qbf = q_dtype == TQ_BF16 ? 1 : 0;
  switch (k.type) {
    case TQ_TURBO2: launch_split_q<2>(qbf, p.tiles_per_wave, grid, stream, k, v, kv_len, q, n_rep, qs, sparse_v_tau, ws, p.n_split); break;
    case TQ_TURBO3: launch_split_q<3>(qbf, p.tiles_per_wave, grid, stream, k, v, kv_len, q, n_rep, qs, sparse_v_tau, ws, p.n_split); break;
    default: launch_split_q<4>(qbf, p.tiles_per_wave, grid, stream, k, v, kv_len, q, n_rep, qs, sparse_v_tau, ws, p.n_split); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(n_q_heads), dim3(kMergeThreads), 0, stream, ws,
                     p.n_split, out);
  return hipGetLastError();
}

}  // namespace tq
