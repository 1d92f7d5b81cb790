// tq_prefill.hip -- causal multi-row attention over a turbo cache with the
// codes dequantized inside the tile load.
//
// [PR28] "Inline-dequant TILE prefill": the earlier path materialized the
// whole cache as float16 temporaries on every step; the fast path decodes the
// 3-bit K/V codes while loading each tile into shared memory.  Here each
// 64-key tile is decoded through the LDS level table straight into two LDS
// tiles: K as [key][d] and V transposed as [d][key], the layouts the matrix
// cores read.  Nothing is ever written back to global memory but the output.
//
// Products (v_mfma_f32_32x32x16_f16, fp32 accumulate):
//   S^T[key][qrow] = K[key][:] . Qrot[qrow][:]   A = K tile, B = rotated query
//   O^T[d][qrow]  += V^T[d][key] P^T[key][qrow]  A = V^T tile, B = P
// A "qrow" is one (query row, query head) pair; the accumulator layout of
// S^T (one query column per lane pair) is exactly the B-operand layout P needs,
// so softmax never leaves registers.  Per-key norms scale S^T's rows (K) and
// fold into P (V); the rotation of Q happens at tile load and its inverse on
// the accumulators.
//
// Workgroup: 64 qrows (64/n_rep query rows x n_rep heads of one kv head),
// four waves = 2 qrow halves x 2 key halves of every tile; the two key halves
// are merged at the end.  Causal balance: workgroup p processes query tiles p
// and T-1-p, so every workgroup sees about the same number of key tiles.
#include "tq_common.h"
#include "tq_launch.h"

namespace tq {

namespace pf {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kD = 256;             // head_dim
constexpr int kQRows = 64;          // qrows per workgroup
constexpr int kKT = 64;             // keys per tile
constexpr int kKsStride = kD + 8;   // halves per K row (and per staged query row)
constexpr int kVtStride = kKT + 8;  // halves per V^T row
constexpr float kPTop = 15.f;       // P = p * norm stays below 2^kPTop
constexpr float kPSet = 9.f;        // a moved reference puts the tile's top at 2^kPSet

__device__ const LevelTable<2> kLevels2;
__device__ const LevelTable<3> kLevels3;
__device__ const LevelTable<4> kLevels4;
template <int B>
__device__ __forceinline__ const uint32_t *level_table() {
  if constexpr (B == 2) return kLevels2.w;
  else if constexpr (B == 3) return kLevels3.w;
  else return kLevels4.w;
}

__device__ __forceinline__ uint32_t bits_at(const uint32_t *dw, int pos, int nbits) {
  const int w = pos >> 5, sh = pos & 31;
  uint32_t x = dw[w] >> sh;
  if (sh + nbits > 32) x |= dw[w + 1] << (32 - sh);
  return x & ((1u << nbits) - 1u);
}

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

__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
__device__ __forceinline__ int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Raw codes of one key tile, prefetched into registers.
template <int B>
struct TileRaw {
  uint32_t k[2 * B];     // K: key t>>2, elements 64*(t&3) .. +63
  uint32_t v[4][2];      // V: keys 4*(t&15)+i, 16 elements from 16*(t>>4)
  uint16_t nrm;          // norms: t < 128 -> K (key (t&127)>>1, group t&1); else V
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
  float qscale;
};

template <int B>
__device__ __forceinline__ void load_tile(const Args &a, int64_t head_base, int kt, int tid,
                                          TileRaw<B> &r) {
  const int64_t last = a.kv_len - 1;
  {
    const int64_t key = lmin((int64_t)kt * kKT + (tid >> 2), last);
    const u32x2_t *src = reinterpret_cast<const u32x2_t *>(a.kcodes + (head_base + key) * (32 * B) +
                                                           8 * B * (tid & 3));
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const u32x2_t v = src[i];
      r.k[2 * i] = v.x;
      r.k[2 * i + 1] = v.y;
    }
  }
  {
    const int db = tid >> 4, m = db & 7;
    const int pos = 16 * B * m;
    const int w0 = pos >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t key = lmin((int64_t)kt * kKT + 4 * (tid & 15) + i, last);
      const uint32_t *row = reinterpret_cast<const uint32_t *>(
          a.vcodes + (head_base + key) * (32 * B) + 16 * B * (db >> 3));
      r.v[i][0] = row[w0];
      r.v[i][1] = (B == 2) ? 0u : row[w0 + 1];
    }
  }
  {
    // two float16 norms per key (one per 128-group), [key][group]
    const int64_t key = lmin((int64_t)kt * kKT + ((tid & 127) >> 1), last);
    const int64_t idx = (head_base + key) * 2 + (tid & 1);
    r.nrm = (tid < 128) ? a.knorms[idx] : a.vnorms[idx];
  }
}

template <int B>
__device__ __forceinline__ void store_tile(const Args &a, int kt, int tid, const TileRaw<B> &r,
                                           const uint32_t *lut, _Float16 *ks, _Float16 *vt,
                                           float *nk, float *nv, float *ve) {
  using C = UnitCfg<B>;
  {
    // K: 64 elements of key t>>2 -> ks row, 8 halves (16 bytes) at a time
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(ks + (tid >> 2) * kKsStride + 64 * (tid & 3));
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      uint32_t h[4];
#pragma unroll
      for (int e = 0; e < 8 / C::U; ++e) {
        const int u = v * (8 / C::U) + e;
        const uint32_t idx = bits_at(r.k, u * C::IBITS, C::IBITS);
        if constexpr (C::DW == 2) {
          const u32x2_t w = *reinterpret_cast<const u32x2_t *>(lut + idx * 2);
          h[2 * e] = w.x;
          h[2 * e + 1] = w.y;
        } else {
          h[e] = lut[idx];
        }
      }
      dst[v] = u32x4_t{h[0], h[1], h[2], h[3]};
    }
  }
  {
    // V: 4 keys x 16 elements -> V^T rows d = 16*db + j, one decode unit
    // (U elements) of all four keys at a time
    const int db = tid >> 4, m = db & 7;
    const int sh = (16 * B * m) & 31;
    uint32_t run[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (B == 2) {
        run[i][0] = r.v[i][0];
        run[i][1] = 0;
      } else {
        run[i][0] = __builtin_amdgcn_alignbit(r.v[i][1], r.v[i][0], sh);
        run[i][1] = sh ? (r.v[i][1] >> sh) : r.v[i][1];
      }
    }
    _Float16 *base = vt + (16 * db) * kVtStride + 4 * (tid & 15);
#pragma unroll
    for (int u = 0; u < 16 / C::U; ++u) {
      uint32_t pr[4][C::DW];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t idx = bits_at(run[i], u * C::IBITS, C::IBITS);
        if constexpr (C::DW == 2) {
          const u32x2_t w = *reinterpret_cast<const u32x2_t *>(lut + idx * 2);
          pr[i][0] = w.x;
          pr[i][1] = w.y;
        } else {
          pr[i][0] = lut[idx];
        }
      }
#pragma unroll
      for (int p = 0; p < C::DW; ++p) {
        const int d = u * C::U + 2 * p;  // elements d, d+1 of the 16
        const u32x2_t e = {__builtin_amdgcn_perm(pr[1][p], pr[0][p], 0x05040100u),
                           __builtin_amdgcn_perm(pr[3][p], pr[2][p], 0x05040100u)};
        const u32x2_t o = {__builtin_amdgcn_perm(pr[1][p], pr[0][p], 0x07060302u),
                           __builtin_amdgcn_perm(pr[3][p], pr[2][p], 0x07060302u)};
        *reinterpret_cast<u32x2_t *>(base + d * kVtStride) = e;
        *reinterpret_cast<u32x2_t *>(base + (d + 1) * kVtStride) = o;
      }
    }
  }
  {
    const int64_t key = (int64_t)kt * kKT + ((tid & 127) >> 1);
    const float n = key < a.kv_len ? half_to_float(r.nrm) : 0.f;
    const float n2 = fmaxf(n, xor_lane<1>(n));   // larger norm of the key's two groups
    if (tid < 2 * kKT) {
      nk[tid] = n;                         // nk[key * 2 + group]
    } else {
      nv[tid - 2 * kKT] = n;
      // binary exponent of the larger V norm: both norms are < 2^ve
      if (!(tid & 1)) ve[(tid - 2 * kKT) >> 1] = (float)__builtin_amdgcn_frexp_expf(n2);
    }
  }
}

template <int B, bool QBF16>
__global__ __launch_bounds__(kThreads) void prefill_kernel(Args a) {
  using C = UnitCfg<B>;
  constexpr int NLUT = ceil_div(C::WORDS / 4, kThreads);
  __shared__ __align__(16) uint32_t lut[C::WORDS];
  // one arena: K tile [key][d] | V^T tile [d][key]; it also stages the query
  // rows (first part) and, after the key loop, the key-half merge (64 KB)
  constexpr int kArenaHalves = kKT * kKsStride + kD * kVtStride;
  static_assert(kArenaHalves * 2 >= 2 * 8 * 16 * 64 * 4, "merge buffer must fit");
  static_assert(kQRows * kKsStride <= kKT * kKsStride, "query staging must fit");
  __shared__ __align__(16) _Float16 arena[kArenaHalves];
  _Float16 *ks = arena;
  _Float16 *vt = arena + kKT * kKsStride;
  __shared__ __align__(16) float nk[2 * kKT];   // [key][group]
  __shared__ __align__(16) float nv[2 * kKT];
  __shared__ __align__(16) float ve[kKT];       // V-norm exponent per key
  __shared__ float mstat[2][32], lstat[2][32];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qhalf = wave & 1, khalf = wave >> 1;
  const int g = blockIdx.y;
  const int64_t head_base = (int64_t)g * a.n_cells;
  const int ql = lane & 31, hl = lane >> 5;       // column (qrow within the wave), lane half
  const int qrow = 32 * qhalf + ql;               // qrow within the workgroup
  const int head_local = qrow / a.bq, row_local = qrow % a.bq;
  const int head = g * a.n_rep + head_local;

  {
    const u32x4_t *lsrc = reinterpret_cast<const u32x4_t *>(level_table<B>());
#pragma unroll
    for (int i = 0; i < NLUT; ++i) {
      const int c = tid + kThreads * i;
      if (c < C::WORDS / 4) reinterpret_cast<u32x4_t *>(lut)[c] = lsrc[c];
    }
  }

  for (int pass = 0; pass < 2; ++pass) {
    const int qt = pass == 0 ? (int)blockIdx.x : a.n_qtiles - 1 - (int)blockIdx.x;
    if (pass == 1 && qt == (int)blockIdx.x) break;
    const int64_t row0 = (int64_t)qt * a.bq;
    const int64_t last_row = lmin(row0 + a.bq, a.n_rows) - 1;
    const int64_t kend = lmin(a.kv_len, a.q_pos0 + last_row + 1);
    const int n_kt = (int)ceil_div<int64_t>(kend, kKT);
    const int64_t r = row0 + row_local;
    const int64_t pos = lmin(a.q_pos0 + r, a.kv_len - 1);   // mask bound of this column

    // ---- stage the rotated query rows (float16) in ks; (qrow, group) pairs
    //      are rotated by half-waves, 4 elements per lane
    __syncthreads();  // previous pass is done with ks
    for (int batch = 0; batch < 4; ++batch) {
      float qv[8][4];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int idx = 16 * batch + 2 * k + (lane >> 5);   // 0..63 within the wave
        const int c = 32 * qhalf + (idx >> 1);  // qrow
        const int grp = idx & 1;
        const int hq = c / a.bq, rq = c % a.bq;
        const int64_t rr = lmin(row0 + rq, a.n_rows - 1);
        const int64_t off = (rr * a.n_q + g * a.n_rep + hq) * kD + 128 * grp + 4 * (lane & 31);
        if constexpr (QBF16) {
          const u32x2_t b = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(a.q) + off);
          qv[k][0] = __uint_as_float(b.x << 16);
          qv[k][1] = __uint_as_float(b.x & 0xffff0000u);
          qv[k][2] = __uint_as_float(b.y << 16);
          qv[k][3] = __uint_as_float(b.y & 0xffff0000u);
        } else {
          const float4 f = *reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(a.q) + off);
          qv[k][0] = f.x; qv[k][1] = f.y; qv[k][2] = f.z; qv[k][3] = f.w;
        }
      }
      if (khalf == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int idx = 16 * batch + 2 * k + (lane >> 5);
          const int c = 32 * qhalf + (idx >> 1);
          const int grp = idx & 1;
          const int j = lane & 31;
#pragma unroll
          for (int i = 0; i < 4; ++i) qv[k][i] = flip_sign(qv[k][i], sign_bit_of(4 * j + i));
          wht128_half(qv[k], j);
          const _Float16 h0 = (_Float16)(qv[k][0] * a.qscale), h1 = (_Float16)(qv[k][1] * a.qscale);
          const _Float16 h2 = (_Float16)(qv[k][2] * a.qscale), h3 = (_Float16)(qv[k][3] * a.qscale);
          const u32x2_t w = {(uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16),
                             (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16)};
          *reinterpret_cast<u32x2_t *>(ks + c * kKsStride + 128 * grp + 4 * j) = w;
        }
      }
    }
    __syncthreads();
    // query operand: lane (ql, hl) holds qrow ql of this wave, d = 16t + 8hl + i
    half8_t qb[16];
#pragma unroll
    for (int t = 0; t < 16; ++t)
      qb[t] = *reinterpret_cast<const half8_t *>(ks + (32 * qhalf + ql) * kKsStride + 16 * t + 8 * hl);
    __syncthreads();  // ks is about to hold K tiles

    f32x16_t o[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) o[dt][rr] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    TileRaw<B> raw;
    load_tile<B>(a, head_base, 0, tid, raw);
    for (int kt = 0; kt < n_kt; ++kt) {
      store_tile<B>(a, kt, tid, raw, lut, ks, vt, nk, nv, ve);
      if (kt + 1 < n_kt) load_tile<B>(a, head_base, kt + 1, tid, raw);
      __syncthreads();

      // ---- scores S^T for this wave's 32 keys x 32 qrows
      // one accumulator per 128-group: each group has its own norm
      f32x16_t s, s1;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) { s[rr] = 0.f; s1[rr] = 0.f; }
      const _Float16 *krow = ks + (32 * khalf + ql) * kKsStride + 8 * hl;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const half8_t av = *reinterpret_cast<const half8_t *>(krow + 16 * t);
        s = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, qb[t], s, 0, 0, 0);
      }
#pragma unroll
      for (int t = 8; t < 16; ++t) {
        const half8_t av = *reinterpret_cast<const half8_t *>(krow + 16 * t);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, qb[t], s1, 0, 0, 0);
      }
      // register rr <-> key 8(rr/4) + 4hl + rr%4 of this wave's half; keys
      // past lim = pos - (first key of the half) are masked
      const int64_t lim64 = pos - ((int64_t)kt * kKT + 32 * khalf);
      const int lim = lim64 > 64 ? 64 : (int)lim64;
      // m_run is a reference, not the running maximum: p = exp2(s - m_run)
      // and P = p * (V norm) goes to float16.  With e the binary exponent of
      // a key's larger V norm, P < 2^(s + e - m_run); the reference moves
      // only when some key would reach 2^kPTop, and then to put the tile's
      // top at 2^kPSet.  So P never overflows, stays clear of float16
      // subnormals, and the accumulators are rescaled rarely.  Softmax does
      // not depend on the reference.
      float tref = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int kk = 8 * (rr >> 2) + 4 * hl + (rr & 3);
        const float2 nn = *reinterpret_cast<const float2 *>(nk + 2 * (32 * khalf + kk));
        float v = s[rr] * nn.x + s1[rr] * nn.y;
        if (kk > lim) v = -INFINITY;
        s[rr] = v;
        tref = fmaxf(tref, v + ve[32 * khalf + kk]);
      }
      tref = fmaxf(tref, xor_lane<32>(tref));
      const float m_new = tref > m_run + kPTop ? tref - kPSet : m_run;
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      half8_t pb[2], pb1[2];   // P of group 0 / group 1
      float psum = 0.f;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int kk = 8 * (rr >> 2) + 4 * hl + (rr & 3);
        const float p = __builtin_amdgcn_exp2f(s[rr] - m_use);
        psum += p;
        const float2 nn = *reinterpret_cast<const float2 *>(nv + 2 * (32 * khalf + kk));
        pb[rr >> 3][rr & 7] = (_Float16)(p * nn.x);
        pb1[rr >> 3][rr & 7] = (_Float16)(p * nn.y);
      }
      l_run = l_run * alpha + psum;
      if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[dt][rr] *= alpha;
      }

      // ---- O^T += V^T P^T; k-slot (hl, i) of group ga <-> key 16ga + 8(i>>2) + 4hl + (i&3)
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const _Float16 *vrow = vt + (32 * dt + ql) * kVtStride + 32 * khalf + 4 * hl;
#pragma unroll
        for (int ga = 0; ga < 2; ++ga) {
          const u32x2_t lo = *reinterpret_cast<const u32x2_t *>(vrow + 16 * ga);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t *>(vrow + 16 * ga + 8);
          const u32x4_t av = {lo.x, lo.y, hi.x, hi.y};
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, av),
                                                        dt < 4 ? pb[ga] : pb1[ga], o[dt], 0, 0, 0);
        }
      }
      __syncthreads();  // the next store_tile overwrites ks / vt
    }

    // ---- merge the two key halves (waves khalf=1 hand their state to khalf=0)
    l_run += xor_lane<32>(l_run);
    float *mbuf = reinterpret_cast<float *>(arena);  // 2 waves x 128 regs x 64 lanes = 64 KB
    if (khalf == 1) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mbuf[((qhalf * 8 + dt) * 16 + rr) * 64 + lane] = o[dt][rr];
      if (hl == 0) {
        mstat[qhalf][ql] = m_run;
        lstat[qhalf][ql] = l_run;
      }
    }
    __syncthreads();
    if (khalf == 0) {
      const float m2 = mstat[qhalf][ql], l2 = lstat[qhalf][ql];
      const float M = fmaxf(m_run, m2);
      const float f1 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
      const float f2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - M);
      const float L = l_run * f1 + l2 * f2;
      const float rinv = 1.0f / (128.0f * L);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          o[dt][rr] = (o[dt][rr] * f1 + mbuf[((qhalf * 8 + dt) * 16 + rr) * 64 + lane] * f2) * rinv;
      // inverse transform per 128-group: d = 32dt + 8(rr/4) + 4hl + rr%4.
      // Stages over d bits 0,1 (rr%4), 2 (hl: lanes 32 apart), 3,4 (rr/4),
      // 5,6 (dt&3); d bit 7 (dt>>2) selects the group.
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
        for (int hbit = 1; hbit <= 8; hbit <<= 1) {
          if (hbit == 4) continue;
          // in-register stage over register index bit: hbit 1,2 -> rr bits 0,1; 8 -> rr bit 2 (d bit 3)
          const int rb = hbit == 8 ? 4 : hbit;
#pragma unroll
          for (int rr = 0; rr < 16; ++rr)
            if (!(rr & rb)) {
              const float x = o[dt][rr], y = o[dt][rr + rb];
              o[dt][rr] = x + y;
              o[dt][rr + rb] = x - y;
            }
        }
        // d bit 4 <-> rr bit 3
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          if (!(rr & 8)) {
            const float x = o[dt][rr], y = o[dt][rr + 8];
            o[dt][rr] = x + y;
            o[dt][rr + 8] = x - y;
          }
        // d bit 2 <-> lane bit 5 (partner 32 lanes away): upper half takes partner - self
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const float p = xor_lane<32>(o[dt][rr]);
          o[dt][rr] = hl ? (p - o[dt][rr]) : (o[dt][rr] + p);
        }
      }
      // d bits 5, 6 <-> dt bits 0, 1 within each group (dt>>2)
#pragma unroll
      for (int gq = 0; gq < 2; ++gq)
#pragma unroll
        for (int b = 1; b <= 2; b <<= 1)
#pragma unroll
          for (int dl = 0; dl < 4; ++dl)
            if (!(dl & b)) {
#pragma unroll
              for (int rr = 0; rr < 16; ++rr) {
                const float x = o[4 * gq + dl][rr], y = o[4 * gq + dl + b][rr];
                o[4 * gq + dl][rr] = x + y;
                o[4 * gq + dl + b][rr] = x - y;
              }
            }
      if (r < a.n_rows) {
        float *orow = a.out + (r * a.n_q + head) * kD;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int d0 = 32 * dt + 8 * rq + 4 * hl;
            float4 v;
            v.x = flip_sign(o[dt][4 * rq + 0], sign_bit_of((d0 + 0) & 127));
            v.y = flip_sign(o[dt][4 * rq + 1], sign_bit_of((d0 + 1) & 127));
            v.z = flip_sign(o[dt][4 * rq + 2], sign_bit_of((d0 + 2) & 127));
            v.w = flip_sign(o[dt][4 * rq + 3], sign_bit_of((d0 + 3) & 127));
            *reinterpret_cast<float4 *>(orow + d0) = v;
          }
      }
    }
  }
}

}  // namespace pf

hipError_t plan_prefill(const tq_cache &k, int64_t n_rows, int32_t n_q_heads, int64_t kv_len,
                        PrefillPlan *p) {
  (void)kv_len;
  const int n_rep = n_q_heads / k.n_kv_heads;
  if (n_rep < 1 || pf::kQRows % n_rep != 0) return hipErrorNotSupported;
  p->rows_per_tile = pf::kQRows / n_rep;
  const int64_t tiles = ceil_div<int64_t>(n_rows, p->rows_per_tile);
  if (tiles > 0x3fffffff) return hipErrorInvalidValue;
  p->n_row_tiles = (int)tiles;
  p->keys_per_split = 0;
  p->max_splits = 1;
  p->workspace_bytes = 0;
  return hipSuccess;
}

hipError_t launch_prefill(const tq_cache &k, const tq_cache &v, int64_t kv_len, const void *q,
                          int q_dtype, int64_t n_rows, int32_t n_q_heads, int64_t q_pos0,
                          float scale, float *out, void *workspace, const PrefillPlan &p,
                          hipStream_t stream) {
  (void)workspace;
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
  a.n_qtiles = p.n_row_tiles;
  // log2 domain; 1/128 for the 1/sqrt(128) of the rotated query and level
  a.qscale = scale * 1.4426950408889634f / 128.0f;
  dim3 grid((unsigned)ceil_div(p.n_row_tiles, 2), (unsigned)k.n_kv_heads);
  dim3 block(pf::kThreads);
  if (k.type == TQ_TURBO3) {
    if (q_dtype == TQ_BF16)
      hipLaunchKernelGGL((pf::prefill_kernel<3, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((pf::prefill_kernel<3, false>), grid, block, 0, stream, a);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace tq
