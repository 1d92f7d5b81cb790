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

// The fixed random sign flip: element d negated iff bit d%64 of word d/64 is
// set (the first two SplitMix64 outputs from state 0).
constexpr uint64_t kSignWord0 = 0xe220a8397b1dcdafull;
constexpr uint64_t kSignWord1 = 0x6e789e6aa1b965f4ull;

// ---------------------------------------------------------------- wave helpers

__device__ __forceinline__ float shfl_xor_f(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// In-place unnormalized 128-point Walsh-Hadamard transform of one group held
// by one wave, lane j owning elements j (a) and j + 64 (b).  Stages
// h = 1, 2, .., 64 in ascending order; in each pair the lower element gets
// lower + upper and the upper one lower - upper.  Each stage is a single
// IEEE float32 add or subtract of the same two operands, so the result is
// bit-identical to any other schedule of the same stages.
__device__ __forceinline__ void wht128_wave(float &a, float &b, int lane) {
#pragma clang fp contract(off)
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const float pa = shfl_xor_f(a, h);
    const float pb = shfl_xor_f(b, h);
    const bool upper = (lane & h) != 0;
    a = upper ? (pa - a) : (a + pa);
    b = upper ? (pb - b) : (b + pb);
  }
  const float s = a + b;
  const float d = a - b;
  a = s;
  b = d;
}

__device__ __forceinline__ float flip_sign(float x, uint32_t negate) {
  return __uint_as_float(__float_as_uint(x) ^ (negate << 31));
}

template <typename T>
__host__ __device__ constexpr T ceil_div(T a, T b) {
  return (a + b - 1) / b;
}

}  // namespace tq
