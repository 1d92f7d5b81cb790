// tq_common.h -- device-side building blocks shared by the libtq kernels
// (gfx950 / CDNA4, wave64).  Host code includes it for the constant tables.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

constexpr int kGroup = 128;  // elements per quantization group

// Positive reconstruction magnitudes, ascending: the Lloyd-Max levels of a
// unit normal source with 2^b levels (computed in double precision),
// rounded to float32.  A code is qs | sign << (b-1), value
// (sign ? -1 : +1) * mag[qs].
__host__ __device__ constexpr float mag2(int i) {
  return i == 0 ? 0x1.cfa592p-2f : 0x1.82aabap+0f;
}
__host__ __device__ constexpr float mag3(int i) {
  return i == 0 ? 0x1.f5f3f0p-3f : i == 1 ? 0x1.831320p-1f : i == 2 ? 0x1.580a70p+0f : 0x1.1372f4p+1f;
}
__host__ __device__ constexpr float mag4(int i) {
  return i == 0 ? 0x1.06f3fap-3f
       : i == 1 ? 0x1.8d5c88p-2f
       : i == 2 ? 0x1.5042bcp-1f
       : i == 3 ? 0x1.e27a72p-1f
       : i == 4 ? 0x1.41985ep+0f
       : i == 5 ? 0x1.9e384ap+0f
       : i == 6 ? 0x1.08d58ep+1f
                : 0x1.5dc57ep+1f;
}
template <int B>
__host__ __device__ constexpr float magnitude(int i) {
  return B == 2 ? mag2(i) : B == 3 ? mag3(i) : mag4(i);
}
// Decision threshold between magnitudes k-1 and k (k >= 1): the midpoint of
// the two double-precision levels, rounded to float32.
__host__ __device__ constexpr float thr2(int) { return 0x1.f6941ep-1f; }
__host__ __device__ constexpr float thr3(int k) {
  return k == 1 ? 0x1.00480ep-1f : k == 2 ? 0x1.0cca00p+0f : 0x1.bf782ep+0f;
}
__host__ __device__ constexpr float thr4(int k) {
  return k == 1 ? 0x1.086b42p-2f
       : k == 2 ? 0x1.0b7880p-1f
       : k == 3 ? 0x1.995e96p-1f
       : k == 4 ? 0x1.196accp+0f
       : k == 5 ? 0x1.6fe854p+0f
       : k == 6 ? 0x1.d7f1b4p+0f
                : 0x1.334d86p+1f;
}
template <int B>
__host__ __device__ constexpr float threshold(int k) {
  return B == 2 ? thr2(k) : B == 3 ? thr3(k) : thr4(k);
}
template <int B>
__host__ __device__ constexpr bool thresholds_between_levels() {
  for (int k = 1; k < (1 << (B - 1)); ++k)
    if (!(threshold<B>(k) > magnitude<B>(k - 1) && threshold<B>(k) < magnitude<B>(k))) return false;
  return true;
}
static_assert(thresholds_between_levels<2>() && thresholds_between_levels<3>() &&
                  thresholds_between_levels<4>(),
              "each threshold lies between its two levels");
// Value of code c.
template <int B>
__host__ __device__ constexpr float code_value(int c) {
  return (c >> (B - 1)) ? -magnitude<B>(c & ((1 << (B - 1)) - 1))
                        : magnitude<B>(c & ((1 << (B - 1)) - 1));
}

// float16 bits of a finite float below 65520 in magnitude, rounded to
// nearest even (subnormal results included).
__host__ __device__ constexpr uint16_t f16_bits_rne(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const int ex = (int)((u >> 23) & 0xffu);
  if (ex == 0) return (uint16_t)sign;          // float32 zero or subnormal: below float16's range
  const int e = ex - 127;
  const uint32_t m = (u & 0x7fffffu) | 0x800000u;   // value = m * 2^(e - 23)
  const int ulp_e = e >= -14 ? e - 10 : -24;        // the float16 ulp at this magnitude
  const int sh = ulp_e - (e - 23);                  // right shift from m to float16 ulps (>= 13)
  if (sh > 25) return (uint16_t)sign;
  uint32_t q = m >> sh;
  const uint32_t rem = m & ((1u << sh) - 1u), half = 1u << (sh - 1);
  if (rem > half || (rem == half && (q & 1u))) ++q;
  // normal: the implicit bit of q adds one to the biased exponent field,
  // and a carry out of the significand moves on to the next exponent
  const uint32_t bits = e >= -14 ? ((uint32_t)(e + 14) << 10) + q : q;
  return (uint16_t)(sign | bits);
}
// float value of float16 bits (finite).
__host__ __device__ constexpr float f16_value(uint16_t h) {
  const uint32_t e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
  const float a = e == 0 ? (float)m * 0x1p-24f
                         : __builtin_bit_cast(float, ((e - 15u + 127u) << 23) | (m << 13));
  return (h & 0x8000u) ? -a : a;
}
// The matrix cores take 16-bit operands, so a level enters a product as two
// float16 parts: hi = float16(level), lo = float16(level - hi) (the
// difference is exact in float32).  hi + lo carries about 22 bits of the
// level.
template <int B>
__host__ __device__ constexpr uint16_t mag_bits(int i, bool lo) {
  return lo ? f16_bits_rne(magnitude<B>(i) - f16_value(f16_bits_rne(magnitude<B>(i))))
            : f16_bits_rne(magnitude<B>(i));
}
template <int B>
__host__ __device__ constexpr bool split_is_close() {
  for (int i = 0; i < (1 << (B - 1)); ++i) {
    const double m = magnitude<B>(i);
    const double h = f16_value(mag_bits<B>(i, false)), l = f16_value(mag_bits<B>(i, true));
    const double err = m - h - l;
    if ((err < 0 ? -err : err) > m * 0x1p-21) return false;
  }
  return true;
}
static_assert(split_is_close<2>() && split_is_close<3>() && split_is_close<4>(),
              "hi + lo float16 parts reproduce each level to 2^-21");

// float16 bits (hi or lo part) of magnitudes 2k and 2k+1 (low, high half).
template <int B, bool LO>
__host__ __device__ constexpr uint32_t mag_word(int k) {
  return (uint32_t)mag_bits<B>(2 * k, LO) |
         ((2 * k + 1 < (1 << (B - 1))) ? (uint32_t)mag_bits<B>(2 * k + 1, LO) << 16 : 0u);
}

// float16 parts (hi or lo) of the levels of codes c0 (low half) and c1 (high
// half): the magnitudes are picked by v_perm_b32 from the constant magnitude
// words (byte selector 2q, 2q+1 per half), then the sign bits are applied
// (the parts of -level are the negated parts of level).
template <int B, bool LO = false>
__device__ __forceinline__ uint32_t level_pair(uint32_t c0, uint32_t c1) {
  const uint32_t sgn = ((c0 >> (B - 1)) << 15) | ((c1 >> (B - 1)) << 31);
  const uint32_t q0 = c0 & 3u, q1 = c1 & 3u;
  const uint32_t sel = 0x01000100u + (q0 | (q1 << 16)) * 0x202u;
  if constexpr (B == 2) {
    return __builtin_amdgcn_perm(mag_word<2, LO>(0), mag_word<2, LO>(0), sel) ^ sgn;
  } else if constexpr (B == 3) {
    return __builtin_amdgcn_perm(mag_word<3, LO>(1), mag_word<3, LO>(0), sel) ^ sgn;
  } else {
    const uint32_t lo = __builtin_amdgcn_perm(mag_word<4, LO>(1), mag_word<4, LO>(0), sel);
    const uint32_t hi = __builtin_amdgcn_perm(mag_word<4, LO>(3), mag_word<4, LO>(2), sel);
    const uint32_t m = ((c0 & 4u) ? 0xffffu : 0u) | ((c1 & 4u) ? 0xffff0000u : 0u);
    return ((hi & m) | (lo & ~m)) ^ sgn;
  }
}

// Pair table for the decode kernels: entry e (the 2B-bit concatenation of
// two codes, first code in the low bits) holds the float16 hi parts of their
// two levels (first in the low half) in its first dword and the lo parts in
// its second.  It is stored in 32 copies with copy c of entry e at 8-byte
// slot 32e + c, and lane l of a wave always reads copy l % 32: the lanes an
// LDS read serves together touch distinct copies, so distinct banks,
// whatever the indices (a single-copy table's random lookups pile onto the
// same banks).  Reading only one part is a 4-byte read at dword 2(32e+c) (+1
// for lo).
template <int B>
struct PairCfg {
  static constexpr int BITS = 2 * B;
  static constexpr int N = 1 << BITS;
  static constexpr int COPIES = 32;
  static constexpr int WORDS = N * COPIES * 2;
};

template <int B, int NT>
__device__ __forceinline__ void build_pair_table(uint32_t *tab, int tid) {
  using P = PairCfg<B>;
  constexpr uint32_t CM = (1u << B) - 1u;
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  // NT threads over N entries: each thread computes entries e (its entry,
  // then e + NT / TPE, ...) once and writes CPT consecutive copies of each
  // as 16-byte stores (two copies per store)
  constexpr int TPE = NT >= P::N ? (NT / P::N < P::COPIES / 2 ? NT / P::N : P::COPIES / 2) : 1;
  constexpr int CPT = P::COPIES / TPE;                    // copies per thread
  constexpr int WORK = P::N * TPE;                        // (entry, copy run) tasks
  constexpr int EPT = (WORK + NT - 1) / NT;               // tasks per thread
  static_assert(TPE * CPT == P::COPIES && CPT % 2 == 0 && (WORK % NT == 0 || WORK < NT), "pair table fill");
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const int task = tid + NT * k;
    if (WORK < NT && task >= WORK) break;
    const uint32_t e = (uint32_t)(task / TPE);
    const uint32_t c0 = (uint32_t)(task % TPE) * CPT;
    const uint32_t hi = level_pair<B, false>(e & CM, e >> B), lo = level_pair<B, true>(e & CM, e >> B);
    u32x4_t *dst = reinterpret_cast<u32x4_t *>(tab + 2 * (P::COPIES * e + c0));
#pragma unroll
    for (int c = 0; c < CPT / 2; ++c) dst[c] = u32x4_t{hi, lo, hi, lo};
  }
}

// The fixed random sign flip: element d negated iff bit d%64 of word d/64 is
// set (the first two SplitMix64 outputs from state 0).
constexpr uint64_t kSignWord0 = 0xe220a8397b1dcdafull;
constexpr uint64_t kSignWord1 = 0x6e789e6aa1b965f4ull;

__device__ __forceinline__ uint32_t sign_bit_of(int d) {
  return (uint32_t)((d < 64 ? kSignWord0 >> d : kSignWord1 >> (d - 64)) & 1u);
}
// Sign bits of elements 4j .. 4j+3 (j < 32) as a nibble, element 4j in bit 0.
__device__ __forceinline__ uint32_t sign_nibble(int j) {
  const uint64_t w = j < 16 ? kSignWord0 : kSignWord1;
  return (uint32_t)(w >> (4 * (j & 15))) & 0xfu;
}

// ---------------------------------------------------------------- lane exchanges

// v from lane (lane ^ H).  H = 1, 2: DPP quad permutes; H = 4: half-row
// mirror (lane ^ 7) then quad reverse (^ 3); H = 8: row rotate by 8;
// H = 16: ds_swizzle in xor mode (within 32 lanes); H = 32: v_permlane32_swap.
template <int H>
__device__ __forceinline__ float xor_lane(float v) {
  const int x = __float_as_int(v);
  int r;
  if constexpr (H == 1) {
    r = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
  } else if constexpr (H == 2) {
    r = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
  } else if constexpr (H == 4) {
    const int m = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);
    r = __builtin_amdgcn_update_dpp(0, m, 0x1B, 0xF, 0xF, false);
  } else if constexpr (H == 8) {
    r = __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);
  } else if constexpr (H == 16) {
    r = __builtin_amdgcn_ds_swizzle(x, 0x401F);
  } else {
    static_assert(H == 32, "xor_lane: H must be a power of two <= 32");
    // v_permlane32_swap(a, b) trades a's upper 32 lanes for b's lower 32:
    // with a = b = x the first result holds x[l & 31], the second x[l | 32]
    const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    r = (int)((threadIdx.x & 32) ? p[0] : p[1]);
  }
  return __int_as_float(r);
}

// Sum and maximum of v over the lane pair (l, l ^ 32); both lanes get the
// same bits (the operands meet in the same order).
__device__ __forceinline__ float sum_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float flip_sign(float x, uint32_t negate) {
  return __uint_as_float(__float_as_uint(x) ^ (negate << 31));
}

// One butterfly stage between lanes at distance H/... : the lower element of
// each pair takes lower + partner, the upper one partner - upper.
template <int H>
__device__ __forceinline__ float bfly_lane(float v, bool upper) {
#pragma clang fp contract(off)
  const float p = xor_lane<H>(v);
  return upper ? (p - v) : (v + p);
}

// Unnormalized 128-point Walsh-Hadamard transform of one group held by 32
// lanes of a wave (lanes 0-31 or 32-63), lane j = lane & 31 owning elements
// 4j .. 4j+3 in u[0..3].  Stages h = 1, 2 are in-register, h = 4 .. 64 are
// exchanges with lane j ^ (h/4); in every pair the lower element becomes
// lower + upper and the upper one lower - upper, stages in ascending h.
// Each stage is one IEEE float32 add or subtract of the same two operands, so
// the result equals any other schedule of the same stages bit for bit.
__device__ __forceinline__ void wht128_half(float (&u)[4], int j) {
#pragma clang fp contract(off)
  float a0 = u[0] + u[1], a1 = u[0] - u[1];
  float a2 = u[2] + u[3], a3 = u[2] - u[3];
  u[0] = a0 + a2;
  u[2] = a0 - a2;
  u[1] = a1 + a3;
  u[3] = a1 - a3;
#define TQ_STAGE(H)                                          \
  {                                                          \
    const bool up = (j & (H)) != 0;                          \
    _Pragma("unroll") for (int i = 0; i < 4; ++i) u[i] = bfly_lane<H>(u[i], up); \
  }
  TQ_STAGE(1)
  TQ_STAGE(2)
  TQ_STAGE(4)
  TQ_STAGE(8)
  TQ_STAGE(16)
#undef TQ_STAGE
}

// Sum of squares of the group held as in wht128_half, in the butterfly's
// pairing order (neighbours first, then distances 2, 4, .., 64); the result
// is the same in all 32 lanes.
__device__ __forceinline__ float sum_squares_half(const float (&x)[4]) {
#pragma clang fp contract(off)
  const float s01 = x[0] * x[0] + x[1] * x[1];
  const float s23 = x[2] * x[2] + x[3] * x[3];
  float s = s01 + s23;
  s = s + xor_lane<1>(s);
  s = s + xor_lane<2>(s);
  s = s + xor_lane<4>(s);
  s = s + xor_lane<8>(s);
  s = s + xor_lane<16>(s);
  return s;
}

template <typename T>
__host__ __device__ constexpr T ceil_div(T a, T b) {
  return (a + b - 1) / b;
}

}  // namespace tq
