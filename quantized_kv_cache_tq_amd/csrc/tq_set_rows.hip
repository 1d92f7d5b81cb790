// tq_set_rows.hip -- the SET_ROWS quantizer: float32 rows -> packed b-bit
// codes + float16 group norms.
//
// [PR36] (a), the llama-cpp-turboquant SET_ROWS butterfly commit, describes
// the kernel as a sign flip and a 128-point butterfly (h = 1..64) per group;
// the CUDA kernel spread a group over several 32-wide warps and kept block
// barriers for h = 32 and 64.  Here a pair of lanes quantizes one group: lane
// half h = lane & 1 holds elements 64h .. 64h + 63 in registers, so the sum of
// squares, the butterfly stages h = 1 .. 32, the codes and the bit packing
// are per-lane arithmetic, and only the last stage (h = 64) and the last step
// of the sum exchange values between the two lanes (one DPP read each).
// Every instruction of a wave thus advances 32 groups.  (With a group spread
// over 32 lanes the per-group work -- the correctly rounded square root and
// division, the gathering of the packed words -- ran on all 32 lanes, and
// every butterfly stage across lanes took an exchange and a select: about
// three times the vector instructions per group.  With one lane per group
// the compiler's schedule of the 128-value transform ran out of registers.)
// A wave takes 32 consecutive rows of one (kv head, group) column: its loads
// read whole 256-byte half groups and its stores write consecutive cells'
// code blocks when the cell indices are consecutive.
//
// Bit-exact contract (float32, no contraction): see tq_set_rows in tq.h.
#include "tq_common.h"

namespace tq {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSrWaves = 4;                 // waves per workgroup
constexpr int kSrHalf = kGroup / 2;         // elements per lane
constexpr int kSrRows = 32;                 // rows (groups) per task
constexpr int kSrTasks = 1;                 // tasks per wave

// v from the partner lane (lane ^ 1, a DPP quad permute).  Every lane's
// source lane is valid, so the bound-control bit never acts; it is set so
// that the exchange needs no register for an unused old value and folds into
// the instruction that consumes it.
__device__ __forceinline__ float from_partner(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// 2 acc + bit as one add with the comparison's lane mask as its carry-in
// (written as plain C the compiler selects the bit into a register first).
__device__ __forceinline__ uint32_t push_bit(uint32_t acc, bool bit) {
  const uint64_t m = __builtin_amdgcn_ballot_w64(bit);
  uint32_t r;
  uint64_t co;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(co) : "v"(acc), "s"(m));
  return r;
}

// Bit b of the code of y.  b = B - 1 is the sign, (y < 0).  Below it is the
// magnitude index qs = #{k : |y| > threshold k}, found by binary search over
// the sorted thresholds: each bit, most significant first, compares |y| with
// the middle threshold of the range the higher bits left (so NaN, failing
// every comparison, takes index 0).
template <int B>
__device__ __forceinline__ bool code_bit(float y, int b) {
  if (b == B - 1) return y < 0.f;
  const float a = __builtin_fabsf(y);
  if constexpr (B == 2) {
    return a > threshold<2>(1);
  } else if constexpr (B == 3) {
    const bool c2 = a > threshold<3>(2);
    if (b == 1) return c2;
    return a > (c2 ? threshold<3>(3) : threshold<3>(1));
  } else {
    const bool c4 = a > threshold<4>(4);
    if (b == 2) return c4;
    const bool c2 = a > (c4 ? threshold<4>(6) : threshold<4>(2));
    if (b == 1) return c2;
    return a > (c4 ? (c2 ? threshold<4>(7) : threshold<4>(5)) : (c2 ? threshold<4>(3) : threshold<4>(1)));
  }
}

template <int B>
__global__ __launch_bounds__(64 * kSrWaves) void set_rows_kernel(
    uint8_t *__restrict__ codes, uint16_t *__restrict__ norms, const float *__restrict__ src,
    const int64_t *__restrict__ cell_idx, int64_t n_rows, int32_t n_kv, int32_t n_groups_per_head,
    int64_t n_cells) {
#pragma clang fp contract(off)
  // sign masks of the random flip (bit 31 set where an element is negated)
  __shared__ __align__(16) uint32_t smask[kGroup];
  if (threadIdx.x < kGroup) smask[threadIdx.x] = sign_bit_of(threadIdx.x) << 31;
  __syncthreads();

  const int lane = threadIdx.x & 63, h = lane & 1;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cols = n_kv * n_groups_per_head;                 // (kv head, group) columns of a row
  const int64_t n_tasks = ceil_div<int64_t>(n_rows, kSrRows) * cols;
  const int64_t task0 = ((int64_t)blockIdx.x * kSrWaves + wave) * kSrTasks;
  if (task0 >= n_tasks) return;                              // uniform: the whole wave

  // (row tile, column) of the wave's tasks: one division, then steps
  int64_t ttile[kSrTasks];
  int tcol[kSrTasks];
  {
    int64_t tile = task0 / cols;
    int col = (int)(task0 - tile * cols);
#pragma unroll
    for (int k = 0; k < kSrTasks; ++k) {
      ttile[k] = tile;
      tcol[k] = col;
      if (++col == cols) {
        col = 0;
        ++tile;
      }
    }
  }

  // loads of task k (kSrRows rows of one column); a task past the end
  // reloads valid rows and stores nothing
  auto load = [&](int k, float (&u)[kSrHalf], int64_t &cell) {
    const int64_t tile = task0 + k < n_tasks ? ttile[k] : ttile[0];
    const int col = task0 + k < n_tasks ? tcol[k] : tcol[0];
    const int64_t row = tile * kSrRows + (lane >> 1);
    const int64_t lrow = row < n_rows ? row : n_rows - 1;    // a dead lane loads a valid row
    const float4 *g = reinterpret_cast<const float4 *>(src + (lrow * cols + col) * kGroup);
#pragma unroll
    for (int v = 0; v < kSrHalf / 4; ++v) {
      const float4 f = g[2 * v + h];
      u[4 * v] = f.x; u[4 * v + 1] = f.y; u[4 * v + 2] = f.z; u[4 * v + 3] = f.w;
    }
    cell = cell_idx[lrow];
  };

  auto quantize = [&](int k, float (&u)[kSrHalf], int64_t cell) {
    const int64_t tile = ttile[k];
    const int col = tcol[k];
    const int head = col / n_groups_per_head, grp = col - head * n_groups_per_head;
    const bool live = task0 + k < n_tasks && tile * kSrRows + (lane >> 1) < n_rows;

    // 1. norm: the sum of squares added in the butterfly's pairing order
    //    (neighbours, then partials at distance 2, 4, .., 64).  Distances 1
    //    and 2 stay inside a lane's chunk, distance 4 adds the two lanes'
    //    chunk partials (both lanes get the same bits: the operands meet
    //    commuted), distances 8 .. 64 pair the lane's chunks in order: pend[l]
    //    holds a finished left partial until its right sibling is done.
    // 2. sign flip, 3. the butterfly stages that stay inside one chunk pair
    //    of lanes: h = 1, 2 inside the chunk, h = 4 between the two lanes.
    //    Both run chunk by chunk in load order, so each chunk's share is
    //    computed while the later chunks are still arriving.  The lane stage
    //    is x + c p with p the partner's value and c = +1 in the lower lane,
    //    -1 in the upper (the product by +-1 is exact, so the fused form
    //    rounds like the plain add or subtract): the upper lane so holds
    //    b - a, the butterfly's a - b negated, and the later stages keep that
    //    sign on all its values (both operands of each carry it); its factor
    //    1/norm is negated to match, so y below is exactly the transform over
    //    norm
    const u32x4_t *sm = reinterpret_cast<const u32x4_t *>(smask);
    const float c4 = h ? -1.f : 1.f;
    float pend[5];
#pragma unroll
    for (int v = 0; v < kSrHalf / 4; ++v) {
      float *x = u + 4 * v;
      const float s01 = x[0] * x[0] + x[1] * x[1];
      const float s23 = x[2] * x[2] + x[3] * x[3];
      const float q = s01 + s23;
      float t = q + from_partner(q);
      int l = 0;
#pragma unroll
      for (; (v >> l) & 1; ++l) t = pend[l] + t;
      pend[l] = t;
      const u32x4_t m = sm[2 * v + h];
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(__float_as_uint(x[k]) ^ m[k]);
      const float a0 = x[0] + x[1], a1 = x[0] - x[1], a2 = x[2] + x[3], a3 = x[2] - x[3];
      x[0] = a0 + a2;
      x[1] = a1 + a3;
      x[2] = a0 - a2;
      x[3] = a1 - a3;
#pragma unroll
      for (int k = 0; k < 4; ++k) x[k] = __builtin_fmaf(from_partner(x[k]), c4, x[k]);
    }
    const float n2 = pend[4];
    const float norm = __builtin_sqrtf(n2);                  // correctly rounded
    const float inv = norm > 0.f ? 1.0f / norm : 0.f;        // correctly rounded

    // 3. (cont.) stages h = 8 .. 64 between the lane's chunks
    auto local_stage = [&](int d) {   // pairs (i, i + d) of the lane's values
#pragma unroll
      for (int i = 0; i < kSrHalf; ++i)
        if (!(i & d)) {
          const float a = u[i], b = u[i + d];
          u[i] = a + b;
          u[i + d] = a - b;
        }
    };
    local_stage(4);
    local_stage(8);
    local_stage(16);
    local_stage(32);
    const float inv_s = flip_sign(inv, (uint32_t)h);

    // 4. unit-variance coordinates, 5. codes, 6. pack: element e's code at
    //    bits B e .. B e + B - 1 of the group's little-endian bit stream.  The
    //    lane places its own elements' codes into an image of the whole
    //    group's 4B dwords (as the lower lane's elements 8v + r, r < 4, i =
    //    4v + r; the upper lane's sit 4B bits higher, applied below), ORs in
    //    the partner's image and stores its half.  Each dword is built from
    //    its top bit down, one bit per instruction: w = 2 w + bit takes the
    //    bit as the carry-in of one add, and a run of the partner's bits is
    //    one shift.  An element's bits are the comparisons of code_bit,
    //    recomputed where each is pushed
    float ys[kSrHalf];
#pragma unroll
    for (int i = 0; i < kSrHalf; ++i) ys[i] = u[i] * inv_s;
    uint32_t word[4 * B];
#pragma unroll
    for (int w = 4 * B - 1; w >= 0; --w) {
      uint32_t acc = 0u;
      int zrun = 0;
#pragma unroll
      for (int p = 32 * w + 31; p >= 32 * w; --p) {
        const int e = p / B, b = p - e * B;
        if ((e & 7) >= 4) {       // the partner's element: a zero bit here
          ++zrun;
          continue;
        }
        if (zrun > 0) acc <<= zrun;
        zrun = 0;
        const bool bit = code_bit<B>(ys[4 * (e >> 3) + (e & 7)], b);
        acc = push_bit(acc, bit);
      }
      if (zrun > 0) acc <<= zrun;
      word[w] = acc;
    }
    // the upper lane's chunk fields sit 4B bits higher: shift its image
    // (a funnel shift across the dwords)
    uint32_t img[4 * B];
#pragma unroll
    for (int w = 4 * B - 1; w >= 0; --w) {
      const uint32_t lo = w > 0 ? word[w - 1] : 0u;
      const uint32_t shifted = (4 * B == 32) ? lo : __builtin_amdgcn_alignbit(word[w], lo, 32 - 4 * B);
      img[w] = h ? shifted : word[w];
    }
#pragma unroll
    for (int w = 0; w < 4 * B; ++w) img[w] |= (uint32_t)__float_as_int(from_partner(__int_as_float((int)img[w])));
    if (live && cell >= 0 && cell < n_cells) {
      const int64_t slot = ((int64_t)head * n_cells + cell) * n_groups_per_head + grp;
      uint8_t *dst = codes + slot * (16 * B) + 8 * B * h;     // this lane's 8B bytes (8-byte aligned)
#pragma unroll
      for (int v = 0; v < B; ++v)
        reinterpret_cast<u32x2_t *>(dst)[v] =
            u32x2_t{h ? img[2 * B + 2 * v] : img[2 * v], h ? img[2 * B + 2 * v + 1] : img[2 * v + 1]};
      if (h == 0) {
        const _Float16 h16 = (_Float16)norm;
        norms[slot] = __builtin_bit_cast(uint16_t, h16);
      }
    }
  };

  // two register sets: the next task's loads are in flight while the current
  // one is computed
  float ua[kSrHalf], ub[kSrHalf];
  int64_t ca, cb;
  load(0, ua, ca);
#pragma unroll
  for (int k = 0; k < kSrTasks; k += 2) {
    if (k + 1 < kSrTasks) load(k + 1, ub, cb);
    quantize(k, ua, ca);
    if (k + 1 < kSrTasks) {
      if (k + 2 < kSrTasks) load(k + 2, ua, ca);
      quantize(k + 1, ub, cb);
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
  const int64_t tasks = ceil_div<int64_t>(n_rows, kSrRows) * (int64_t)c.n_kv_heads * gph;
  const int64_t blocks = ceil_div<int64_t>(tasks, kSrWaves * kSrTasks);
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks), block(64 * kSrWaves);
  switch (c.type) {
    case TQ_TURBO2:
      hipLaunchKernelGGL((set_rows_kernel<2>), grid, block, 0, stream, c.codes, c.norms, src, cell_idx, n_rows,
                         c.n_kv_heads, gph, c.n_cells);
      break;
    case TQ_TURBO3:
      hipLaunchKernelGGL((set_rows_kernel<3>), grid, block, 0, stream, c.codes, c.norms, src, cell_idx, n_rows,
                         c.n_kv_heads, gph, c.n_cells);
      break;
    default:
      hipLaunchKernelGGL((set_rows_kernel<4>), grid, block, 0, stream, c.codes, c.norms, src, cell_idx, n_rows,
                         c.n_kv_heads, gph, c.n_cells);
      break;
  }
  return hipGetLastError();
}

}  // namespace tq
