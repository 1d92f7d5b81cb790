// tq_set_rows.hip -- the SET_ROWS quantizer: float32 rows -> packed b-bit
// codes + float16 group norms.
//
// [PR36] (a), the llama-cpp-turboquant SET_ROWS butterfly commit, describes
// the kernel as a sign flip and a 128-point butterfly (h = 1..64) per group;
// the CUDA kernel spread a group over several 32-wide warps and kept block
// barriers for h = 32 and 64.  On CDNA4 half a wave64 holds a whole group:
// lane j owns elements 4j..4j+3 (one 16-byte load), stages h = 1 and 2 are
// in-register and h = 4..64 are DPP / swizzle exchanges inside the 32 lanes,
// so no barrier or LDS round trip is needed anywhere in the transform.  Each
// wave quantizes 2 x kRounds groups and issues all their loads first, so
// enough bytes are in flight to stream from HBM.
//
// Bit-exact contract (float32, no contraction): see tq_set_rows in tq.h.
#include "tq_common.h"

namespace tq {

constexpr int kSrWaves = 4;
constexpr int kSrRounds = 4;                              // groups per half-wave
constexpr int kSrGroupsPerBlock = kSrWaves * 2 * kSrRounds;

// kSmall: fewer than 2^31 groups in the call, so the one division that
// places a lane's first group is 32-bit.
template <int B, bool kSmall>
__global__ __launch_bounds__(64 * kSrWaves) void set_rows_kernel(
    uint8_t *__restrict__ codes, uint16_t *__restrict__ norms, const float *__restrict__ src,
    const int64_t *__restrict__ cell_idx, int64_t n_rows, int32_t n_kv, int32_t n_groups_per_head,
    int64_t n_cells) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, j = lane & 31;
  const int64_t groups_per_row = (int64_t)n_kv * n_groups_per_head;
  const int64_t total = n_rows * groups_per_row;
  const int64_t gbase = ((int64_t)blockIdx.x * kSrWaves + wave) * (2 * kSrRounds) + half;

  // the lane's groups gbase, gbase + 2, ...: row, kv head and group of the
  // first by one division, the later ones stepped from it (the group index
  // grows by 2, so each carry loop runs at most twice)
  int64_t row;
  int head, grp;
  if constexpr (kSmall) {
    const uint32_t g32 = (uint32_t)gbase, gpr = (uint32_t)groups_per_row;
    const uint32_t r32 = g32 / gpr, rem = g32 - r32 * gpr;
    row = r32;
    head = (int)(rem / (uint32_t)n_groups_per_head);
    grp = (int)(rem - (uint32_t)head * (uint32_t)n_groups_per_head);
  } else {
    row = gbase / groups_per_row;
    const int64_t rem = gbase - row * groups_per_row;
    head = (int)(rem / n_groups_per_head);
    grp = (int)(rem - (int64_t)head * n_groups_per_head);
  }
  int64_t rrow[kSrRounds];
  int rhead[kSrRounds], rgrp[kSrRounds];
#pragma unroll
  for (int r = 0; r < kSrRounds; ++r) {
    rrow[r] = row;
    rhead[r] = head;
    rgrp[r] = grp;
    grp += 2;
    while (grp >= n_groups_per_head) {
      grp -= n_groups_per_head;
      ++head;
    }
    while (head >= n_kv) {
      head -= n_kv;
      ++row;
    }
  }
  // issue every load first
  float4 x[kSrRounds];
  int64_t cell[kSrRounds];
#pragma unroll
  for (int r = 0; r < kSrRounds; ++r) {
    const int64_t gi = gbase + 2 * r;
    if (gi < total) {
      x[r] = reinterpret_cast<const float4 *>(src + gi * kGroup)[j];
      cell[r] = cell_idx[rrow[r]];
    } else {
      x[r] = make_float4(0.f, 0.f, 0.f, 0.f);
      cell[r] = -1;
    }
  }
  uint32_t neg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) neg[i] = sign_bit_of(4 * j + i);

#pragma unroll
  for (int r = 0; r < kSrRounds; ++r) {
    const int64_t gi = gbase + 2 * r;
    float u[4] = {x[r].x, x[r].y, x[r].z, x[r].w};
    // 1. norm: sum of squares in the butterfly's pairing order
    const float n2 = sum_squares_half(u);
    const float norm = __builtin_sqrtf(n2);             // correctly rounded
    const float inv = norm > 0.f ? 1.0f / norm : 0.f;   // correctly rounded
    // 2. sign flip, 3. butterfly, 4. unit-variance coordinates, 5. codes
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = flip_sign(u[i], neg[i]);
    wht128_half(u, j);
    uint32_t field = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = u[i] * inv;
      const float a = __builtin_fabsf(y);
      uint32_t qs = 0;
#pragma unroll
      for (int k = 1; k < (1 << (B - 1)); ++k) qs += a > threshold<B>(k) ? 1u : 0u;
      const uint32_t c = qs | ((y < 0.f ? 1u : 0u) << (B - 1));
      field |= c << (B * i);
    }
    // 6. pack: lane j's 4B-bit field sits at stream bit 4B*j; lane w < 4B
    //    assembles output dword w from the (at most KMAX) fields it overlaps.
    constexpr int FB = 4 * B;
    constexpr int KMAX = (B == 4) ? 2 : 4;
    const int w = j;
    const int j0 = (32 * w) / FB;
    const int j1 = (32 * w + 31) / FB;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int jj = j0 + k;
      const int srcl = (half << 5) + (jj < 32 ? jj : 31);
      const uint32_t f = (uint32_t)__shfl((int)field, srcl, 64);
      const int pos = FB * jj - 32 * w;
      if (jj <= j1) word |= pos >= 0 ? (f << pos) : (f >> (-pos));
    }
    const int64_t c = cell[r];
    if (gi < total && c >= 0 && c < n_cells) {
      const int64_t slot = ((int64_t)rhead[r] * n_cells + c) * n_groups_per_head + rgrp[r];
      if (w < FB) reinterpret_cast<uint32_t *>(codes + slot * (16 * B))[w] = word;
      if (j == 0) {
        const _Float16 h16 = (_Float16)norm;
        norms[slot] = __builtin_bit_cast(uint16_t, h16);
      }
    }
  }
}

// The 8-bit block format (an asymmetric cache's K, [PR36] (b)): eight lanes
// per 32-element block, each with one 16-byte load of four elements; the
// block maximum is an exchange over the eight lanes, and each lane writes its
// four codes as one dword.  Rows are [n_rows][n_kv][head_dim], blocks in
// order, so consecutive lanes read and write consecutive bytes.
constexpr int kQ8Threads = 256;
constexpr int kQ8Block = 32;

__global__ __launch_bounds__(kQ8Threads) void set_rows_q8_kernel(
    int8_t *__restrict__ codes, uint16_t *__restrict__ scales, const float *__restrict__ src,
    const int64_t *__restrict__ cell_idx, int64_t n_rows, int32_t n_kv, int32_t head_dim,
    int64_t n_cells) {
#pragma clang fp contract(off)
  const int64_t quad = (int64_t)blockIdx.x * kQ8Threads + threadIdx.x;   // 4 elements
  const int64_t row_elems = (int64_t)n_kv * head_dim;
  const int64_t total = n_rows * row_elems / 4;
  const bool live = quad < total;
  const float4 x = live ? reinterpret_cast<const float4 *>(src)[quad] : make_float4(0.f, 0.f, 0.f, 0.f);
  float amax = fmaxf(fmaxf(__builtin_fabsf(x.x), __builtin_fabsf(x.y)),
                     fmaxf(__builtin_fabsf(x.z), __builtin_fabsf(x.w)));
  amax = fmaxf(amax, xor_lane<1>(amax));
  amax = fmaxf(amax, xor_lane<2>(amax));
  amax = fmaxf(amax, xor_lane<4>(amax));
  const _Float16 d16 = (_Float16)(amax / 127.0f);      // correctly rounded, then nearest-even
  const float d = (float)d16;
  const bool ok = d > 0.f && d <= 65504.f;
  const float e[4] = {x.x, x.y, x.z, x.w};
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float q = ok ? __builtin_rintf(e[i] / d) : 0.f;    // correctly rounded quotient, ties to even
    q = fminf(fmaxf(q, -127.f), 127.f);
    word |= ((uint32_t)(int32_t)q & 0xffu) << (8 * i);
  }
  if (!live) return;
  const int64_t r = (4 * quad) / row_elems;
  const int64_t rem = 4 * quad - r * row_elems;
  const int head = (int)(rem / head_dim);
  const int elem = (int)(rem - (int64_t)head * head_dim);
  const int64_t c = cell_idx[r];
  if (c < 0 || c >= n_cells) return;
  const int64_t row = (int64_t)head * n_cells + c;
  reinterpret_cast<uint32_t *>(codes + row * head_dim)[elem >> 2] = word;
  if ((elem & (kQ8Block - 1)) == 0) scales[row * (head_dim / kQ8Block) + elem / kQ8Block] = __builtin_bit_cast(uint16_t, d16);
}

hipError_t launch_set_rows(const tq_cache &c, const float *src, const int64_t *cell_idx,
                           int64_t n_rows, hipStream_t stream) {
  if (c.type == TQ_Q8) {
    const int64_t quads = n_rows * (int64_t)c.n_kv_heads * c.head_dim / 4;
    const int64_t blocks = ceil_div<int64_t>(quads, kQ8Threads);
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(set_rows_q8_kernel, dim3((unsigned)blocks), dim3(kQ8Threads), 0, stream,
                       reinterpret_cast<int8_t *>(c.codes), c.norms, src, cell_idx, n_rows, c.n_kv_heads,
                       c.head_dim, c.n_cells);
    return hipGetLastError();
  }
  const int32_t gph = c.head_dim / kGroup;
  const int64_t total = n_rows * (int64_t)c.n_kv_heads * gph;
  const int64_t blocks = ceil_div<int64_t>(total, kSrGroupsPerBlock);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(64 * kSrWaves);
  // a lane's first group index stays below total + the groups of one block
  const bool small = total + kSrGroupsPerBlock < 0x7fffffffLL;
#define TQ_SR(B)                                                                                   \
  do {                                                                                             \
    if (small)                                                                                     \
      hipLaunchKernelGGL((set_rows_kernel<B, true>), grid, block, 0, stream, c.codes, c.norms, src, \
                         cell_idx, n_rows, c.n_kv_heads, gph, c.n_cells);                          \
    else                                                                                           \
      hipLaunchKernelGGL((set_rows_kernel<B, false>), grid, block, 0, stream, c.codes, c.norms,    \
                         src, cell_idx, n_rows, c.n_kv_heads, gph, c.n_cells);                     \
  } while (0)
  switch (c.type) {
    case TQ_TURBO2: TQ_SR(2); break;
    case TQ_TURBO3: TQ_SR(3); break;
    default: TQ_SR(4); break;
  }
#undef TQ_SR
  return hipGetLastError();
}

}  // namespace tq
