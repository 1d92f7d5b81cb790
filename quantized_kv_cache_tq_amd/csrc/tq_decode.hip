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

__device__ const LevelTable<2> kLevels2;
__device__ const LevelTable<3> kLevels3;
__device__ const LevelTable<4> kLevels4;

template <int B>
__device__ __forceinline__ const uint32_t *level_table() {
  if constexpr (B == 2) return kLevels2.w;
  else if constexpr (B == 3) return kLevels3.w;
  else return kLevels4.w;
}

// Bits [pos, pos+nbits) of a little-endian dword array (pos and nbits are
// compile-time after unrolling; the field spans at most two dwords).
__device__ __forceinline__ uint32_t bits_at(const uint32_t *dw, int pos, int nbits) {
  const int w = pos >> 5, sh = pos & 31;
  uint32_t x = dw[w] >> sh;
  if (sh + nbits > 32) x |= dw[w + 1] << (32 - sh);
  return nbits == 32 ? x : (x & ((1u << nbits) - 1u));
}

// Decode NEL consecutive elements held in dw (first element in bit 0) into
// float16 pairs out[0 .. NEL/2).
template <int B, int NEL>
__device__ __forceinline__ void decode_run(const uint32_t *dw, const uint32_t *lut,
                                           uint32_t *out) {
  using C = UnitCfg<B>;
#pragma unroll
  for (int u = 0; u < NEL / C::U; ++u) {
    const uint32_t idx = bits_at(dw, u * C::IBITS, C::IBITS);
    if constexpr (C::DW == 2) {
      const u32x2_t e = *reinterpret_cast<const u32x2_t *>(lut + idx * 2);
      out[2 * u] = e.x;
      out[2 * u + 1] = e.y;
    } else {
      out[u] = lut[idx];
    }
  }
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

template <int B, int TPW>
struct DecodeSmem {
  static constexpr int KPW = 16 * TPW;               // keys per wave
  static constexpr int KPS = KPW * kDecWaves;        // keys per split
  static constexpr int ROWW = 4 * B;                 // code dwords per key
  static constexpr int ROWP = ROWW + 1;              // padded LDS row (dwords)
  static constexpr int VWORDS = KPW * ROWP;          // one wave's V rows
  static constexpr int OBUF_WORDS = kDecWaves * 8 * kD;
  static constexpr int LUT_WORDS = UnitCfg<B>::WORDS;
  // after the value phase the level table and V rows are dead: the output
  // buffer reuses them
  static constexpr int BIG = LUT_WORDS + kDecWaves * VWORDS;
  static constexpr int ARENA = BIG > OBUF_WORDS ? BIG : OBUF_WORDS;
};

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }

// Float16 high part (hi lanes) or low part (lo lanes) of x: x - fp16(x) is
// exact in float32, so hi + lo carries ~22 significant bits of x.
__device__ __forceinline__ _Float16 split_half(float x, bool lo_lane) {
  const _Float16 h = (_Float16)x;
  return lo_lane ? (_Float16)(x - (float)h) : h;
}

// Keeps the compiler from moving LDS accesses across this point; LDS
// operations of one wave execute in order, so other lanes' earlier writes
// are visible to later reads of the same wave.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int B, int TPW, bool QBF16>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const uint8_t *__restrict__ kcodes, const uint16_t *__restrict__ knorms,
    const uint8_t *__restrict__ vcodes, const uint16_t *__restrict__ vnorms, int64_t n_cells,
    int64_t kv_len, const void *__restrict__ q, int n_rep, float qscale,
    float *__restrict__ ws, int n_split) {
  using C = UnitCfg<B>;
  using S = DecodeSmem<B, TPW>;
  constexpr int KPW = S::KPW, KPS = S::KPS, ROWP = S::ROWP;
  constexpr int VCH = KPW * B;                             // 16-byte V chunks per wave
  constexpr int NV = ceil_div(VCH, 64);
  constexpr int NLUT = ceil_div(C::WORDS / 4, kDecThreads);
  constexpr int NNORM = ceil_div(KPW, 64);
  __shared__ __align__(16) uint32_t arena[S::ARENA];       // level table | V rows, later obuf
  __shared__ __align__(16) float nk[kDecWaves][KPW];
  __shared__ __align__(16) float nv[kDecWaves][KPW];
  __shared__ __align__(16) uint32_t qbuf[4 * 64 * 4];      // query operand, [t][lane][8 halves]
  __shared__ float wm[kDecWaves][8], wl[kDecWaves][8];
  uint32_t *lut = arena;
  uint32_t *vrows = arena + S::LUT_WORDS + (threadIdx.x >> 6) * S::VWORDS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, quad = lane >> 4;
  const int s = blockIdx.x, g = blockIdx.y;
  const int64_t head_base = (int64_t)g * n_cells;
  const int64_t w0 = (int64_t)s * KPS + (int64_t)wave * KPW;     // first key of this wave
  const int wkeys = (int)(kv_len - w0 < 0 ? 0 : (kv_len - w0 < KPW ? kv_len - w0 : KPW));
  const int64_t wsafe = wkeys > 0 ? w0 : kv_len - 1;              // a valid row for clamping
  const int wlast = wkeys > 0 ? wkeys - 1 : 0;

  // ---- every global load, straight-line (clamped, never branched around),
  //      in the order of first use: table, query, norms, K tiles, V rows.
  u32x4_t lraw[NLUT];
  const u32x4_t *lsrc = reinterpret_cast<const u32x4_t *>(level_table<B>());
#pragma unroll
  for (int i = 0; i < NLUT; ++i) lraw[i] = lsrc[imin(tid + kDecThreads * i, C::WORDS / 4 - 1)];
  const int qh = 2 * (wave & 3) + (lane >> 5), qj = lane & 31;
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
    const int64_t key = wsafe + imin(lane + 64 * i, wlast);
    kn[i] = knorms[head_base + key];
    vn[i] = vnorms[head_base + key];
  }
  // K: lane (col, quad) of tile t reads key 16t + col, dwords B*quad .. B*quad+B-1
  uint32_t kd[TPW][B];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t key = wsafe + imin(16 * t + col, wlast);
    const uint32_t *row =
        reinterpret_cast<const uint32_t *>(kcodes + (head_base + key) * (16 * B)) + B * quad;
#pragma unroll
    for (int i = 0; i < B; ++i) kd[t][i] = row[i];
  }
  const u32x4_t *vseg = reinterpret_cast<const u32x4_t *>(vcodes + (head_base + wsafe) * (16 * B));
  u32x4_t vraw[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) vraw[i] = vseg[imin(lane + 64 * i, wkeys * B - 1 < 0 ? 0 : wkeys * B - 1)];

  // ---- level table to LDS; rotate + split the queries into the operand buffer
#pragma unroll
  for (int i = 0; i < NLUT; ++i) {
    const int c = tid + kDecThreads * i;
    if (c < C::WORDS / 4) reinterpret_cast<u32x4_t *>(lut)[c] = lraw[i];
  }
  if (wave < 4) {
    // thread holds elements d = 4qj .. 4qj+3 of head qh; in the MFMA B operand
    // they are slots i = 4(qj&1) .. +3 of K-step t = (qj>>1)&3 in lane
    // 16*(qj>>3) + qh (high half) and 16*(qj>>3) + 8 + qh (low half).
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[i] = flip_sign(qv[i], sign_bit_of(4 * qj + i));
    wht128_half(qv, qj);
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
#pragma unroll
  for (int i = 0; i < NNORM; ++i) {
    const int kk = lane + 64 * i;
    if (kk < KPW) {
      const bool ok = kk < wkeys;
      nk[wave][kk] = ok ? half_to_float(kn[i]) : 0.f;
      nv[wave][kk] = ok ? half_to_float(vn[i]) : 0.f;
    }
  }
  __syncthreads();

  // Query operand: column n = lane & 15 -> head n & 7, high (n < 8) or low half;
  // k-slot (lane >> 4, i) of K-step t <-> element d = 32*(lane>>4) + 8t + i.
  half8_t qb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
    qb[t] = __builtin_bit_cast(half8_t, reinterpret_cast<const u32x4_t *>(qbuf)[t * 64 + lane]);

  // ---- scores of this wave's keys, tile by tile as their codes arrive
  float sc[TPW][4];
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    uint32_t a16[16];
    decode_run<B, 32>(kd[t], lut, a16);
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4_t av = {a16[4 * st], a16[4 * st + 1], a16[4 * st + 2], a16[4 * st + 3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[st], acc,
                                                  0, 0, 0);
    }
    const float4 n4 = *reinterpret_cast<const float4 *>(&nk[wave][16 * t + 4 * quad]);
    const float nkv[4] = {n4.x, n4.y, n4.z, n4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = (acc[i] + xor_lane<8>(acc[i])) * nkv[i];
      if (wkeys < KPW && 16 * t + 4 * quad + i >= wkeys) v = -INFINITY;
      sc[t][i] = v;
      mx = fmaxf(mx, v);
    }
  }
  // wave max per head (log2 domain); -inf for a wave without keys
  mx = fmaxf(mx, xor_lane<16>(mx));
  mx = fmaxf(mx, xor_lane<32>(mx));
  const float msafe = mx == -INFINITY ? 0.f : mx;

  // ---- this wave's V rows to its LDS slice
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c < VCH) {
      uint32_t *d = vrows + (c / B) * ROWP + 4 * (c % B);
      d[0] = vraw[i].x; d[1] = vraw[i].y; d[2] = vraw[i].z; d[3] = vraw[i].w;
    }
  }
  wave_lds_fence();

  // ---- probabilities and values
  float4_t o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  const bool lo_lane = col >= 8;
  constexpr int VBITS = 8 * B;
  const int vpos = VBITS * col;  // value elements 8*col .. 8*col + 7
  const int vw0 = vpos >> 5, vsh = vpos & 31;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const float4 n4 = *reinterpret_cast<const float4 *>(&nv[wave][16 * t + 4 * quad]);
    const float nvv[4] = {n4.x, n4.y, n4.z, n4.w};
    half4_t pa;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(sc[t][i] - msafe);
      lsum += p;
      pa[i] = split_half(p * nvv[i], lo_lane);
    }
    uint32_t vv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t *row = vrows + (16 * t + 4 * quad + i) * ROWP + vw0;
      const uint32_t run[1] = {__builtin_amdgcn_alignbit(row[1], row[0], vsh)};
      decode_run<B, 8>(run, lut, vv[i]);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int w = dt >> 1;
      const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;
      const u32x2_t bv = {__builtin_amdgcn_perm(vv[1][w], vv[0][w], sel),
                          __builtin_amdgcn_perm(vv[3][w], vv[2][w], sel)};
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, __builtin_bit_cast(half4_t, bv), o[dt], 0,
                                                   0, 0);
    }
  }
  lsum += xor_lane<16>(lsum);
  lsum += xor_lane<32>(lsum);

  // ---- combine high/low rows: after the swap, lanes 0-31 hold d-tiles 0-3
  //      and lanes 32-63 d-tiles 4-7, each as high + low.
  float oc[4][4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[dt][i]),
                                                      __float_as_uint(o[dt + 4][i]), false, false);
      oc[dt][i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
  if (lane < 8) {
    wm[wave][lane] = mx;
    wl[wave][lane] = lsum;
  }
  __syncthreads();  // all waves are done with the table and V rows
  float *obuf = reinterpret_cast<float *>(arena);
  {
    const int qd = (lane & 31) >> 4, dhi = lane >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = make_float4(oc[0][i], oc[1][i], oc[2][i], oc[3][i]);
      *reinterpret_cast<float4 *>(obuf + (wave * 8 + 4 * qd + i) * kD + 8 * col + 4 * dhi) = v;
    }
  }
  __syncthreads();
  // obuf[wave][h][8c + t] holds d-tile t, column c, i.e. element d = 8c + t;
  // each wave's sums are relative to its own max, rescaled here.
  float *part = ws + ((int64_t)g * n_rep * n_split + s) * kPartStride;
  {
    const int h = tid >> 6, d = 2 * (tid & 63);
    if (h < n_rep) {
      float M = wm[0][h];
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, wm[w][h]);
      float a0 = 0.f, a1 = 0.f, L = 0.f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = wm[w][h];
        const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        const float2 v = *reinterpret_cast<const float2 *>(obuf + (w * 8 + h) * kD + d);
        a0 += f * v.x;
        a1 += f * v.y;
        L += f * wl[w][h];
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
#pragma unroll 4
  for (int s = grp; s < n_split; s += kMergeGroups) {
    const float *p = part + (int64_t)s * kPartStride;
    const float2 ml = *reinterpret_cast<const float2 *>(p + kD);
    const float4 v = reinterpret_cast<const float4 *>(p)[j];
    const float mn = fmaxf(mg, ml.x);
    const float a = __builtin_amdgcn_exp2f(mg - mn);
    const float w = __builtin_amdgcn_exp2f(ml.x - mn);
    L = L * a + w * ml.y;
    acc.x = acc.x * a + w * v.x;
    acc.y = acc.y * a + w * v.y;
    acc.z = acc.z * a + w * v.z;
    acc.w = acc.w * a + w * v.w;
    mg = mn;
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
  // largest tile count (<= 4) that still gives every compute unit a workgroup
  int tpw = 4;
  while (tpw > 1) {
    const int64_t splits = ceil_div<int64_t>(kv_len, 16LL * kDecWaves * tpw);
    if (splits * k.n_kv_heads >= n_cu) break;
    tpw >>= 1;
  }
  p->tiles_per_wave = tpw;
  p->keys_per_split = 16 * kDecWaves * tpw;
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
                         float *ws, int n_split) {
  dim3 block(kDecThreads);
#define TQ_DEC(T)                                                                             \
  hipLaunchKernelGGL((decode_split_kernel<B, T, QBF>), grid, block, 0, st, k.codes, k.norms, \
                     v.codes, v.norms, k.n_cells, kv_len, q, n_rep, qs, ws, n_split)
  switch (tpw) {
    case 1: TQ_DEC(1); break;
    case 2: TQ_DEC(2); break;
    default: TQ_DEC(4); break;
  }
#undef TQ_DEC
}

template <int B>
static void launch_split_q(int qbf, int tpw, dim3 grid, hipStream_t st, const tq_cache &k,
                           const tq_cache &v, int64_t kv_len, const void *q, int n_rep, float qs,
                           float *ws, int n_split) {
  if (qbf) launch_split<B, true>(tpw, grid, st, k, v, kv_len, q, n_rep, qs, ws, n_split);
  else launch_split<B, false>(tpw, grid, st, k, v, kv_len, q, n_rep, qs, ws, n_split);
}

hipError_t launch_decode(const tq_cache &k, const tq_cache &v, int64_t kv_len, const void *q,
                         int q_dtype, int32_t n_q_heads, float scale, float *out, void *workspace,
                         const DecodePlan &p, hipStream_t stream) {
  const int n_rep = n_q_heads / k.n_kv_heads;
  // scores in the log2 domain: scale * log2(e), and 1/128 for the two
  // 1/sqrt(128) factors of the rotated query and the rotated levels
  const float qs = scale * 1.4426950408889634f / 128.0f;
  float *ws = reinterpret_cast<float *>(workspace);
  dim3 grid(p.n_split, k.n_kv_heads);
  const int qbf = q_dtype == TQ_BF16 ? 1 : 0;
  switch (k.type) {
    case TQ_TURBO2: launch_split_q<2>(qbf, p.tiles_per_wave, grid, stream, k, v, kv_len, q, n_rep, qs, ws, p.n_split); break;
    case TQ_TURBO3: launch_split_q<3>(qbf, p.tiles_per_wave, grid, stream, k, v, kv_len, q, n_rep, qs, ws, p.n_split); break;
    default: launch_split_q<4>(qbf, p.tiles_per_wave, grid, stream, k, v, kv_len, q, n_rep, qs, ws, p.n_split); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(n_q_heads), dim3(kMergeThreads), 0, stream, ws,
                     p.n_split, out);
  return hipGetLastError();
}

}  // namespace tq
