// tq_common.h -- device-side building blocks shared by the libtq kernels
// (gfx950 / CDNA4, wave64).  Host code includes it for the constant tables.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

constexpr int kGroup = 128;  // elements per quantization group

// Positive reconstruction magnitudes, ascending: the Lloyd-Max levels of a
// unit normal source with 2^b levels, rounded to float16 (so they are exact
// 16-bit matrix-core operands).  A code is qs | sign << (b-1), value
// (sign ? -1 : +1) * mag[qs].
__host__ __device__ constexpr float mag2(int i) {
  return i == 0 ? 0x1.cfcp-2f : 0x1.82cp+0f;
}
__host__ __device__ constexpr float mag3(int i) {
  return i == 0 ? 0x1.f6p-3f : i == 1 ? 0x1.83p-1f : i == 2 ? 0x1.58p+0f : 0x1.138p+1f;
}
__host__ __device__ constexpr float mag4(int i) {
  return i == 0 ? 0x1.07p-3f
       : i == 1 ? 0x1.8d4p-2f
       : i == 2 ? 0x1.504p-1f
       : i == 3 ? 0x1.e28p-1f
       : i == 4 ? 0x1.418p+0f
       : i == 5 ? 0x1.9e4p+0f
       : i == 6 ? 0x1.08cp+1f
                : 0x1.5dcp+1f;
}
template <int B>
__host__ __device__ constexpr float magnitude(int i) {
  return B == 2 ? mag2(i) : B == 3 ? mag3(i) : mag4(i);
}
// Decision threshold between magnitudes k-1 and k (k >= 1); the midpoint of
// two float16 values is exact in float32.
template <int B>
__host__ __device__ constexpr float threshold(int k) {
  return 0.5f * (magnitude<B>(k - 1) + magnitude<B>(k));
}
// Value of code c.
template <int B>
__host__ __device__ constexpr float code_value(int c) {
  return (c >> (B - 1)) ? -magnitude<B>(c & ((1 << (B - 1)) - 1))
                        : magnitude<B>(c & ((1 << (B - 1)) - 1));
}

// float16 bit pattern of a float that is an exact normal float16 value.
__host__ __device__ constexpr uint16_t f16_bits_exact(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t e = ((u >> 23) & 0xffu) - 127u + 15u;
  return (uint16_t)(sign | (e << 10) | ((u >> 13) & 0x3ffu));
}
template <int B>
__host__ __device__ constexpr bool levels_are_f16() {
  for (int i = 0; i < (1 << (B - 1)); ++i) {
    const uint32_t u = __builtin_bit_cast(uint32_t, magnitude<B>(i));
    if (u & 0x1fffu) return false;
  }
  return true;
}
static_assert(levels_are_f16<2>() && levels_are_f16<3>() && levels_are_f16<4>(),
              "levels must be exact float16 values");

// Level table for the attention kernels: entry idx decodes the U codes
// packed in idx (code u in bits [B*u, B*u+B)) to U float16 levels, two per
// dword (code 2p in the low half).  U = 4 for 2- and 3-bit codes (8/12-bit
// index), U = 2 for 4-bit codes (8-bit index).
template <int B>
struct UnitCfg {
  static constexpr int U = (B == 4) ? 2 : 4;
  static constexpr int IBITS = U * B;
  static constexpr int N = 1 << IBITS;
  static constexpr int DW = U / 2;
  static constexpr int WORDS = N * DW;
};
template <int B>
struct alignas(16) LevelTable {
  uint32_t w[UnitCfg<B>::WORDS];
  constexpr LevelTable() : w{} {
    using C = UnitCfg<B>;
    for (int idx = 0; idx < C::N; ++idx)
      for (int p = 0; p < C::DW; ++p) {
        const int c0 = (idx >> (B * (2 * p))) & ((1 << B) - 1);
        const int c1 = (idx >> (B * (2 * p + 1))) & ((1 << B) - 1);
        w[idx * C::DW + p] = (uint32_t)f16_bits_exact(code_value<B>(c0)) |
                             ((uint32_t)f16_bits_exact(code_value<B>(c1)) << 16);
      }
  }
};

// float16 bits of magnitudes 2k and 2k+1 (low, high half).
template <int B>
__host__ __device__ constexpr uint32_t mag_word(int k) {
  return (uint32_t)f16_bits_exact(magnitude<B>(2 * k)) |
         ((2 * k + 1 < (1 << (B - 1))) ? (uint32_t)f16_bits_exact(magnitude<B>(2 * k + 1)) << 16 : 0u);
}

// float16 levels of codes c0 (low half) and c1 (high half): the magnitudes
// are picked by v_perm_b32 from the constant magnitude words (byte selector
// 2q, 2q+1 per half), then the sign bits are applied.
template <int B>
__device__ __forceinline__ uint32_t level_pair(uint32_t c0, uint32_t c1) {
  constexpr uint32_t QM = (1u << (B - 1)) - 1u;
  const uint32_t sgn = ((c0 >> (B - 1)) << 15) | ((c1 >> (B - 1)) << 31);
  const uint32_t q0 = c0 & QM & 3u, q1 = c1 & QM & 3u;
  const uint32_t sel = 0x01000100u + (q0 | (q1 << 16)) * 0x202u;
  if constexpr (B == 2) {
    return __builtin_amdgcn_perm(mag_word<2>(0), mag_word<2>(0), sel) ^ sgn;
  } else if constexpr (B == 3) {
    return __builtin_amdgcn_perm(mag_word<3>(1), mag_word<3>(0), sel) ^ sgn;
  } else {
    const uint32_t lo = __builtin_amdgcn_perm(mag_word<4>(1), mag_word<4>(0), sel);
    const uint32_t hi = __builtin_amdgcn_perm(mag_word<4>(3), mag_word<4>(2), sel);
    const uint32_t m = ((c0 & 4u) ? 0xffffu : 0u) | ((c1 & 4u) ? 0xffff0000u : 0u);
    return ((hi & m) | (lo & ~m)) ^ sgn;
  }
}

// Writes the level table (the layout of LevelTable<B>) to shared memory
// with NT threads; computed from the magnitudes, no global memory read.
template <int B, int NT>
__device__ __forceinline__ void build_level_table(uint32_t *lut, int tid) {
  using C = UnitCfg<B>;
  constexpr uint32_t CM = (1u << B) - 1u;
#pragma unroll
  for (int j = 0; j < (C::N + NT - 1) / NT; ++j) {
    const uint32_t e = (uint32_t)tid + (uint32_t)NT * j;
    if (C::N % NT == 0 || e < (uint32_t)C::N) {
      if constexpr (C::DW == 2) {
        const uint32_t lo = level_pair<B>(e & CM, (e >> B) & CM);
        const uint32_t hi = level_pair<B>((e >> (2 * B)) & CM, (e >> (3 * B)) & CM);
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x2_t *>(lut + 2 * e) = u32x2_t{lo, hi};
      } else {
        lut[e] = level_pair<B>(e & CM, (e >> B) & CM);
      }
    }
  }
}

// Pair table for the decode kernels: entry e (the 2B-bit concatenation of
// two codes, first code in the low bits) holds their two float16 levels
// (first in the low half).  It is stored in 64 copies with copy c of entry e
// at dword 64e + c, and lane l of a wave always reads copy l: whatever the
// indices, the 64 lanes of one lookup touch 64 consecutive banks' worth of
// distinct dwords (no bank conflicts), unlike a single-copy table whose
// random lookups pile onto the same banks.
template <int B>
struct PairCfg {
  static constexpr int BITS = 2 * B;
  static constexpr int N = 1 << BITS;
  static constexpr int WORDS = N * 64;
};

template <int B, int NT>
__device__ __forceinline__ void build_pair_table(uint32_t *tab, int tid) {
  using P = PairCfg<B>;
  constexpr uint32_t CM = (1u << B) - 1u;
  static_assert(P::WORDS % NT == 0 && NT % 64 == 0, "pair table fill");
#pragma unroll
  for (int j = 0; j < P::WORDS / NT; ++j) {
    // entry (tid + NT j) / 64 is the same for a whole wave
    const uint32_t e = (uint32_t)__builtin_amdgcn_readfirstlane((tid >> 6) + (NT / 64) * j);
    tab[tid + NT * j] = level_pair<B>(e & CM, e >> B);
  }
}

// The fixed random sign flip: element d negated iff bit d%64 of word d/64 is
// set (the first two SplitMix64 outputs from state 0).
constexpr uint64_t kSignWord0 = 0xe220a8397b1dcdafull;
constexpr uint64_t kSignWord1 = 0x6e789e6aa1b965f4ull;

__device__ __forceinline__ uint32_t sign_bit_of(int d) {
  return (uint32_t)((d < 64 ? kSignWord0 >> d : kSignWord1 >> (d - 64)) & 1u);
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
