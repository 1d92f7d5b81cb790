// tq_decode.hip -- decode attention (one query row) over a turbo cache.
//
// [PR36] (c) decodes with a per-query-head Q x centroid table in shared
// memory (one shared read per element and head).  With eight query heads per
// kv head that is eight table reads per cache element, far more LDS traffic
// than the packed stream itself.  On CDNA4 the eight heads are instead one
// dense contraction: every packed code is decoded ONCE per kv head into a
// float16 level through a table in LDS (indexed by the concatenated codes of
// 2 or 4 neighbouring elements, so one LDS read yields 2-4 levels), and the
// matrix cores do Q.K^T and P.V for all eight heads at once.
//
// Layout of one 16-key tile in a wave (v_mfma_f32_16x16x32_f16 for scores,
// v_mfma_f32_16x16x16_f16 for values):
//   scores  S^T[key][col] = K[key][:] . Qcol[:]; column c < 8 is the high
//           float16 half of head c's rotated query, column 8 + c its low half
//           (q = hi + lo keeps ~22 bits of the float32 query);
//   values  O[row][d] += P[row][key] V[key][d]; rows < 8 hold the high half of
//           p * vnorm, rows >= 8 the low half.
// The levels themselves are float16-exact, so the only roundings are float32
// accumulation and the exponential.
//
// Work split ([PR36] (d) raised occupancy to hide load latency; here the
// split-K grid does that job): workgroup (split s, kv head g) owns keys
// [s*KPS, (s+1)*KPS); its four waves compute every score first, take one
// workgroup-wide max, then accumulate values, so no rescaling is needed.
// A second small kernel merges the splits and rotates back.
#include "tq_common.h"
#include "tq_launch.h"

namespace tq {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kDecodeWaves = 4;
constexpr int kD = 128;  // head_dim handled by this kernel
constexpr int kPartialStride = kD + 2;  // o[128], m, l (floats)

// Elements per LUT index: 4 for 2/3-bit codes (8/12-bit index), 2 for 4-bit.
template <int B>
struct UnitCfg {
  static constexpr int U = (B == 4) ? 2 : 4;
  static constexpr int IBITS = U * B;
  static constexpr int N = 1 << IBITS;
  static constexpr int DW = U / 2;  // dwords per entry (two float16 per dword)
};

__device__ __forceinline__ uint32_t half_bits(float v) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}

// Fill the level table: entry idx holds the float16 levels of the U codes
// idx bits [B*u, B*u+B), u = 0..U-1, two per dword, element u in the low half
// for even u.
template <int B>
__device__ void build_unit_lut(uint32_t *lut, int tid, int nthreads) {
  using C = UnitCfg<B>;
  constexpr uint32_t mask = (1u << B) - 1u;
  for (int idx = tid; idx < C::N; idx += nthreads) {
#pragma unroll
    for (int p = 0; p < C::DW; ++p) {
      const int c0 = (idx >> (B * (2 * p))) & mask;
      const int c1 = (idx >> (B * (2 * p + 1))) & mask;
      lut[idx * C::DW + p] = half_bits(code_value<B>(c0)) | (half_bits(code_value<B>(c1)) << 16);
    }
  }
}

// Bits [pos, pos+nbits) of a little-endian dword array (pos, nbits known
// after unrolling; nbits <= 32 and the field spans at most two dwords).
__device__ __forceinline__ uint32_t bits_at(const uint32_t *dw, int pos, int nbits) {
  const int w = pos >> 5, sh = pos & 31;
  uint32_t x = dw[w] >> sh;
  if (sh + nbits > 32) x |= dw[w + 1] << (32 - sh);
  return nbits == 32 ? x : (x & ((1u << nbits) - 1u));
}

// Decode `n_el` consecutive elements held in dw (bit 0 = first element) into
// float16 pairs out[0 .. n_el/2).
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

__device__ __forceinline__ float load_q(const void *q, int q_bf16, int64_t i) {
  if (q_bf16) {
    const uint16_t b = reinterpret_cast<const uint16_t *>(q)[i];
    return __uint_as_float((uint32_t)b << 16);
  }
  return reinterpret_cast<const float *>(q)[i];
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

template <int B, int TPW>
__global__ __launch_bounds__(64 * kDecodeWaves) void decode_split_kernel(
    const uint8_t *__restrict__ kcodes, const uint16_t *__restrict__ knorms,
    const uint8_t *__restrict__ vcodes, const uint16_t *__restrict__ vnorms, int64_t n_cells,
    int64_t kv_len, const void *__restrict__ q, int q_bf16, int n_rep, float qscale,
    float *__restrict__ ws, int n_split) {
  using C = UnitCfg<B>;
  constexpr int KPS = 16 * TPW * kDecodeWaves;
  constexpr int ROWB = 16 * B;  // code bytes per key (head_dim 128)
  __shared__ __align__(16) uint32_t lut[C::N * C::DW];
  __shared__ float qrot[8][kD];
  __shared__ float nk[KPS], nv[KPS];
  __shared__ float wmax[kDecodeWaves][8], wsum[kDecodeWaves][8];
  __shared__ float obuf[kDecodeWaves][8][kD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.x, g = blockIdx.y;
  const int64_t k0 = (int64_t)s * KPS;
  const int64_t head_base = (int64_t)g * n_cells;

  // ---- setup: level table, norms, rotated queries
  build_unit_lut<B>(lut, tid, 64 * kDecodeWaves);
  for (int i = tid; i < KPS; i += 64 * kDecodeWaves) {
    const int64_t key = k0 + i;
    const bool ok = key < kv_len;
    nk[i] = ok ? half_to_float(knorms[head_base + key]) : 0.f;
    nv[i] = ok ? half_to_float(vnorms[head_base + key]) : 0.f;
  }
  for (int h = wave; h < 8; h += kDecodeWaves) {
    float a = 0.f, b = 0.f;
    if (h < n_rep) {
      const int64_t qh = ((int64_t)g * n_rep + h) * kD;
      a = load_q(q, q_bf16, qh + lane);
      b = load_q(q, q_bf16, qh + lane + 64);
      a = flip_sign(a, (uint32_t)(kSignWord0 >> lane) & 1u);
      b = flip_sign(b, (uint32_t)(kSignWord1 >> lane) & 1u);
      wht128_wave(a, b, lane);
      a *= qscale;
      b *= qscale;
    }
    qrot[h][lane] = a;
    qrot[h][lane + 64] = b;
  }
  __syncthreads();

  // Query operand: column n = lane & 15 -> head n & 7, high (n < 8) or low half;
  // k-slot (lane >> 4, i) of K-step t <-> element d = 32*(lane>>4) + 8t + i.
  const int col = lane & 15, quad = lane >> 4;
  half8_t qb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = qrot[col & 7][32 * quad + 8 * t + i];
      const _Float16 hi = (_Float16)x;
      const _Float16 lo = (_Float16)(x - (float)hi);
      qb[t][i] = col < 8 ? hi : lo;
    }
  }

  // ---- scores for all keys of this wave
  float sc[TPW][4];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int kl0 = 16 * (wave * TPW + t);  // first key of the tile, local
    const int64_t key = k0 + kl0 + col;
    const int64_t kc = key < kv_len ? key : kv_len - 1;
    const uint32_t *row =
        reinterpret_cast<const uint32_t *>(kcodes + (head_base + kc) * ROWB + 4 * B * quad);
    uint32_t dw[B];
#pragma unroll
    for (int i = 0; i < B; ++i) dw[i] = row[i];
    uint32_t a16[16];
    decode_run<B, 32>(dw, lut, a16);
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const u32x4_t av = {a16[4 * st], a16[4 * st + 1], a16[4 * st + 2], a16[4 * st + 3]};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, av), qb[st], acc,
                                                  0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float full = acc[i] + __shfl_xor(acc[i], 8, 64);
      const int kl = kl0 + 4 * quad + i;
      sc[t][i] = (k0 + kl < kv_len) ? full * nk[kl] : -INFINITY;
    }
  }

  // ---- workgroup max per head (log2 domain)
  float mx = -INFINITY;
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[t][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (lane < 8) wmax[wave][lane] = mx;
  __syncthreads();
  float m = wmax[0][col & 7];
#pragma unroll
  for (int w = 1; w < kDecodeWaves; ++w) m = fmaxf(m, wmax[w][col & 7]);

  // ---- probabilities and values
  float4_t o[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) o[t] = float4_t{0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  const int vn = col;  // value elements 8*vn .. 8*vn+7
  constexpr int VBITS = 8 * B;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int kl0 = 16 * (wave * TPW + t);
    half4_t pa;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kl = kl0 + 4 * quad + i;
      const float p = __builtin_amdgcn_exp2f(sc[t][i] - m);
      lsum += p;
      const float pv = p * nv[kl];
      const _Float16 hi = (_Float16)pv;
      const _Float16 lo = (_Float16)(pv - (float)hi);
      pa[i] = col < 8 ? hi : lo;
    }
    // value codes of keys kl0 + 4*quad + i, elements 8*vn .. 8*vn + 7
    uint32_t vv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t key = k0 + kl0 + 4 * quad + i;
      const int64_t kc = key < kv_len ? key : kv_len - 1;
      const uint32_t *row = reinterpret_cast<const uint32_t *>(vcodes + (head_base + kc) * ROWB);
      const int pos = VBITS * vn;
      const int w0 = pos >> 5, sh = pos & 31;
      uint32_t x = row[w0] >> sh;
      if (sh + VBITS > 32) x |= row[w0 + 1] << (32 - sh);
      const uint32_t run[1] = {x};
      decode_run<B, 8>(run, lut, vv[i]);
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int w = dt >> 1;
      uint32_t lo01, lo23;
      if (dt & 1) {
        lo01 = (vv[0][w] >> 16) | (vv[1][w] & 0xffff0000u);
        lo23 = (vv[2][w] >> 16) | (vv[3][w] & 0xffff0000u);
      } else {
        lo01 = (vv[0][w] & 0xffffu) | (vv[1][w] << 16);
        lo23 = (vv[2][w] & 0xffffu) | (vv[3][w] << 16);
      }
      const u32x2_t bv = {lo01, lo23};
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, __builtin_bit_cast(half4_t, bv), o[dt], 0,
                                                   0, 0);
    }
  }

  // ---- combine high/low rows, then the four waves
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (lane < 8) wsum[wave][lane] = lsum;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = o[dt][i] + __shfl_xor(o[dt][i], 32, 64);
      if (lane < 32) obuf[wave][4 * quad + i][8 * col + dt] = v;
    }
  }
  __syncthreads();
  float *part = ws + ((int64_t)g * n_rep * n_split + s) * kPartialStride;
  for (int idx = tid; idx < 8 * kD; idx += 64 * kDecodeWaves) {
    const int h = idx / kD, d = idx % kD;
    if (h >= n_rep) continue;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) acc += obuf[w][h][d];
    part[(int64_t)h * n_split * kPartialStride + d] = acc;
  }
  if (tid < n_rep) {
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) l += wsum[w][tid];
    float mm = wmax[0][tid];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) mm = fmaxf(mm, wmax[w][tid]);
    part[(int64_t)tid * n_split * kPartialStride + kD] = mm;
    part[(int64_t)tid * n_split * kPartialStride + kD + 1] = l;
  }
}

// Merge the split partials of one query head, undo the rotation and write the
// float32 output row: out = s (.) H O / (128 L).
__global__ __launch_bounds__(64) void decode_merge_kernel(const float *__restrict__ ws,
                                                          int n_split, float *__restrict__ out) {
  const int h = blockIdx.x, lane = threadIdx.x;
  const float *part = ws + (int64_t)h * n_split * kPartialStride;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, part[(int64_t)s * kPartialStride + kD]);
  float L = 0.f, a = 0.f, b = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float *p = part + (int64_t)s * kPartialStride;
    const float w = __builtin_amdgcn_exp2f(p[kD] - M);
    L += w * p[kD + 1];
    a += w * p[lane];
    b += w * p[lane + 64];
  }
  wht128_wave(a, b, lane);
  const float r = 1.0f / (128.0f * L);
  a = flip_sign(a * r, (uint32_t)(kSignWord0 >> lane) & 1u);
  b = flip_sign(b * r, (uint32_t)(kSignWord1 >> lane) & 1u);
  out[(int64_t)h * kD + lane] = a;
  out[(int64_t)h * kD + lane + 64] = b;
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
  int tpw = 8;
  while (tpw > 1) {
    const int64_t splits = ceil_div<int64_t>(kv_len, 64 * tpw);
    if (splits * k.n_kv_heads >= 2LL * n_cu) break;
    tpw >>= 1;
  }
  p->tiles_per_wave = tpw;
  p->keys_per_split = 64 * tpw;
  const int64_t n_split = ceil_div<int64_t>(kv_len, p->keys_per_split);
  if (n_split > 0x7fffffff) return hipErrorInvalidValue;
  p->n_split = (int)n_split;
  const size_t bytes = (size_t)n_q_heads * (size_t)n_split * kPartialStride * sizeof(float);
  p->workspace_bytes = (bytes + 255) & ~(size_t)255;
  return hipSuccess;
}

template <int B>
static void launch_split(int tpw, dim3 grid, hipStream_t st, const tq_cache &k,
                         const tq_cache &v, int64_t kv_len, const void *q, int qbf, int n_rep,
                         float qs, float *ws, int n_split) {
  dim3 block(64 * kDecodeWaves);
#define TQ_DEC(T)                                                                             \
  hipLaunchKernelGGL((decode_split_kernel<B, T>), grid, block, 0, st, k.codes, k.norms,      \
                     v.codes, v.norms, k.n_cells, kv_len, q, qbf, n_rep, qs, ws, n_split)
  switch (tpw) {
    case 1: TQ_DEC(1); break;
    case 2: TQ_DEC(2); break;
    case 4: TQ_DEC(4); break;
    default: TQ_DEC(8); break;
  }
#undef TQ_DEC
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
    case TQ_TURBO2: launch_split<2>(p.tiles_per_wave, grid, stream, k, v, kv_len, q, qbf, n_rep, qs, ws, p.n_split); break;
    case TQ_TURBO3: launch_split<3>(p.tiles_per_wave, grid, stream, k, v, kv_len, q, qbf, n_rep, qs, ws, p.n_split); break;
    default: launch_split<4>(p.tiles_per_wave, grid, stream, k, v, kv_len, q, qbf, n_rep, qs, ws, p.n_split); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(n_q_heads), dim3(64), 0, stream, ws, p.n_split,
                     out);
  return hipGetLastError();
}

}  // namespace tq
