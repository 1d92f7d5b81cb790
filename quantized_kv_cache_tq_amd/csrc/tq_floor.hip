// tq_floor.hip -- launch and streaming floors for the benchmark (not part of
// the attention library; built into libtq_floor.so).
//
// What one kernel launch replayed from a graph costs with no work, and what a
// kernel that only streams a buffer once (the bytes of one decode call, no
// arithmetic) takes: the time below which no decode call of that size can
// go on this device, whatever its arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kThreads) void floor_empty_kernel(float *out) {
  // never true for a launch of kThreads threads; keeps the store in the code
  if (threadIdx.x == kThreads) out[0] = 0.f;
}

// Workgroup b reads vectors [b per, (b + 1) per) of the buffer, 16 bytes per
// lane and load, and writes one folded word per lane of its first wave.
__global__ __launch_bounds__(kThreads) void floor_read_kernel(const uint4 *__restrict__ p, int64_t per,
                                                              float *__restrict__ out) {
  const uint4 *b = p + per * blockIdx.x;
  uint32_t acc = 0;
  for (int64_t i = threadIdx.x; i < per; i += (int64_t)kThreads * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + (int64_t)kThreads * u;
      v[u] = j < per ? b[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t s[kThreads];
  s[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x < 64) {
    uint32_t a = 0;
    for (int k = threadIdx.x; k < kThreads; k += 64) a ^= s[k];
    out[(int64_t)blockIdx.x * 64 + threadIdx.x] = (float)a;
  }
}

}  // namespace

extern "C" {

// One launch of `grid` workgroups that do nothing.  out: device buffer of at
// least one float (never written).  Returns the hipError_t of the launch.
int tqf_empty(int grid, float *out, void *stream) {
  if (grid < 1 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(floor_empty_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream, out);
  return (int)hipGetLastError();
}

// One launch of `grid` workgroups reading the nbytes of buf (device) once.
// nbytes must be a positive multiple of 16 * grid; out: device buffer of
// 64 * grid floats.  Returns the hipError_t of the launch.
int tqf_read(const void *buf, int64_t nbytes, int grid, float *out, void *stream) {
  if (!buf || !out || grid < 1 || nbytes <= 0 || nbytes % (16LL * grid) != 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(floor_read_kernel, dim3(grid), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint4 *)buf, nbytes / 16 / grid, out);
  return (int)hipGetLastError();
}

}  // extern "C"
