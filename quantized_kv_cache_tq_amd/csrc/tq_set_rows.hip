// tq_set_rows.hip -- the SET_ROWS quantizer: float32 rows -> packed b-bit
// codes + float16 group norms.
//
// [PR36] (a), the llama-cpp-turboquant SET_ROWS butterfly commit, describes
// the kernel as a sign flip and a 128-point butterfly (h = 1..64) per group;
// the earlier CUDA kernel spread a group over several 32-wide warps and used
// block barriers for h = 32 and 64.  On CDNA4 one wave64 holds a whole group
// (lane j owns elements j and j + 64): stages h = 1..32 are cross-lane
// exchanges inside the wave and stage h = 64 is in-register, so no barrier is
// needed anywhere in the transform.
//
// Bit-exact contract (float32, no contraction): see tq_set_rows in tq.h.
#include "tq_common.h"

namespace tq {

constexpr int kSetRowsWaves = 4;  // groups per workgroup (one wave each)

template <int B>
__global__ __launch_bounds__(64 * kSetRowsWaves) void set_rows_kernel(
    uint8_t *__restrict__ codes, uint16_t *__restrict__ norms, const float *__restrict__ src,
    const int64_t *__restrict__ cell_idx, int64_t n_rows, int32_t n_kv, int32_t n_groups_per_head,
    int64_t n_cells) {
#pragma clang fp contract(off)
  __shared__ uint8_t lds_codes[kSetRowsWaves][kGroup];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t groups_per_row = (int64_t)n_kv * n_groups_per_head;
  const int64_t total = n_rows * groups_per_row;
  const int64_t gi = (int64_t)blockIdx.x * kSetRowsWaves + wave;
  const bool active = gi < total;  // uniform per wave

  int64_t row = 0, cell = -1;
  int head = 0, grp = 0;
  float a = 0.f, b = 0.f;
  if (active) {
    row = gi / groups_per_row;
    const int64_t rem = gi - row * groups_per_row;
    head = (int)(rem / n_groups_per_head);
    grp = (int)(rem - (int64_t)head * n_groups_per_head);
    cell = cell_idx[row];
    const float *x = src + gi * kGroup;
    a = x[lane];
    b = x[lane + 64];
  }

  // 1. sum of squares in the butterfly's pairing order: partials at distance
  //    1, 2, .., 32 across lanes, then the two halves (distance 64).
  float sa = a * a;
  float sb = b * b;
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    sa = sa + shfl_xor_f(sa, h);
    sb = sb + shfl_xor_f(sb, h);
  }
  const float n2 = sa + sb;
  const float norm = __builtin_sqrtf(n2);  // correctly rounded (no afn)
  const float inv = norm > 0.f ? 1.0f / norm : 0.f;  // correctly rounded division

  // 2. sign flip, 3. butterfly, 4. unit-variance coordinates
  const uint32_t neg_a = (uint32_t)(kSignWord0 >> lane) & 1u;
  const uint32_t neg_b = (uint32_t)(kSignWord1 >> lane) & 1u;
  float ua = flip_sign(a, neg_a);
  float ub = flip_sign(b, neg_b);
  wht128_wave(ua, ub, lane);
  const float ya = ua * inv;
  const float yb = ub * inv;

  // 5. nearest stored level: sign bit + magnitude index
  const float aa = __builtin_fabsf(ya);
  const float ab = __builtin_fabsf(yb);
  int qa = 0, qb = 0;
#pragma unroll
  for (int k = 1; k < (1 << (B - 1)); ++k) {
    qa += aa > threshold<B>(k) ? 1 : 0;
    qb += ab > threshold<B>(k) ? 1 : 0;
  }
  const int ca = qa | ((ya < 0.f ? 1 : 0) << (B - 1));
  const int cb = qb | ((yb < 0.f ? 1 : 0) << (B - 1));

  // 6. pack: element e's code at stream bits B*e .. B*e+B-1
  lds_codes[wave][lane] = (uint8_t)ca;
  lds_codes[wave][lane + 64] = (uint8_t)cb;
  __syncthreads();
  if (!active || cell < 0 || cell >= n_cells) return;
  constexpr int kWords = 4 * B;  // 16*B bytes per group
  const int64_t slot = ((int64_t)head * n_cells + cell) * n_groups_per_head + grp;
  if (lane < kWords) {
    const int bit0 = 32 * lane;
    const int e0 = bit0 / B;
    const int e1 = (bit0 + 31) / B;
    uint32_t word = 0;
    for (int e = e0; e <= e1; ++e) {
      const uint32_t c = lds_codes[wave][e];
      const int pos = B * e - bit0;
      word |= pos >= 0 ? (c << pos) : (c >> (-pos));
    }
    reinterpret_cast<uint32_t *>(codes + slot * (16 * B))[lane] = word;
  }
  if (lane == 0) {
    const _Float16 h16 = (_Float16)norm;
    norms[slot] = __builtin_bit_cast(uint16_t, h16);
  }
}

hipError_t launch_set_rows(const tq_cache &c, const float *src, const int64_t *cell_idx,
                           int64_t n_rows, hipStream_t stream) {
  const int32_t gph = c.head_dim / kGroup;
  const int64_t total = n_rows * (int64_t)c.n_kv_heads * gph;
  const int64_t blocks = ceil_div<int64_t>(total, kSetRowsWaves);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(64 * kSetRowsWaves);
  switch (c.type) {
    case TQ_TURBO2:
      hipLaunchKernelGGL(set_rows_kernel<2>, grid, block, 0, stream, c.codes, c.norms, src,
                         cell_idx, n_rows, c.n_kv_heads, gph, c.n_cells);
      break;
    case TQ_TURBO3:
      hipLaunchKernelGGL(set_rows_kernel<3>, grid, block, 0, stream, c.codes, c.norms, src,
                         cell_idx, n_rows, c.n_kv_heads, gph, c.n_cells);
      break;
    default:
      hipLaunchKernelGGL(set_rows_kernel<4>, grid, block, 0, stream, c.codes, c.norms, src,
                         cell_idx, n_rows, c.n_kv_heads, gph, c.n_cells);
      break;
  }
  return hipGetLastError();
}

}  // namespace tq
