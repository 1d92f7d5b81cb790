// tq_api.hip -- host side of the C ABI declared in include/tq.h: argument
// validation, workspace sizing and kernel dispatch.  Nothing here allocates
// device memory; every check happens before the first HIP call.
#include <string.h>

#include <mutex>

#include "tq_common.h"
#include "tq_launch.h"

using namespace tq;

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool valid_type(int t) { return t == TQ_TURBO2 || t == TQ_TURBO3 || t == TQ_TURBO4; }
// a cache may also hold the 8-bit block format (an asymmetric cache's K)
bool valid_cache_type(int t) { return valid_type(t) || t == TQ_Q8; }

tq_status check_cache(const tq_cache *c) {
  if (!c) return TQ_ERR_INVALID_ARG;
  if (!valid_cache_type(c->type) || c->head_dim < kGroup || c->head_dim % kGroup != 0 ||
      c->n_kv_heads < 1 || c->n_cells < 1 || c->reserved != 0)
    return TQ_ERR_INVALID_ARG;
  if (!c->codes || !c->norms || !aligned(c->codes, 16) || !aligned(c->norms, 4))
    return TQ_ERR_INVALID_ARG;
  return TQ_OK;
}

// K and V of one attention call: the same kv heads and cells (the kernels
// address both with one cell count) and the same turbo type, unless the call
// takes an 8-bit block K beside a turbo V; the head widths must match unless
// the call allows them to differ.
tq_status check_pair(const tq_cache *k, const tq_cache *v, bool same_width = true,
                     bool q8_k = false) {
  tq_status s = check_cache(k);
  if (s != TQ_OK) return s;
  s = check_cache(v);
  if (s != TQ_OK) return s;
  if (k->n_kv_heads != v->n_kv_heads || k->n_cells != v->n_cells) return TQ_ERR_INVALID_ARG;
  if (v->type == TQ_Q8 || (k->type == TQ_Q8 && !q8_k)) return TQ_ERR_UNSUPPORTED;
  if (k->type != TQ_Q8 && k->type != v->type) return TQ_ERR_INVALID_ARG;
  if (same_width && k->head_dim != v->head_dim) return TQ_ERR_INVALID_ARG;
  return TQ_OK;
}

tq_status from_hip(hipError_t e) {
  return e == hipSuccess ? TQ_OK : e == hipErrorNotSupported ? TQ_ERR_UNSUPPORTED : TQ_ERR_HIP;
}

}  // namespace

extern "C" {

const char *tq_version(void) { return "libtq 0.1.0 (gfx950)"; }

const char *tq_status_str(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case TQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

tq_status tq_cache_plane_bytes(int type, int32_t head_dim, int32_t n_kv_heads, int64_t n_cells,
                               size_t *codes_bytes, size_t *norms_bytes) {
  if (!valid_cache_type(type) || head_dim < kGroup || head_dim % kGroup || n_kv_heads < 1 ||
      n_cells < 1)
    return TQ_ERR_INVALID_ARG;
  const size_t rows = (size_t)n_kv_heads * (size_t)n_cells;
  if (type == TQ_Q8) {   // one byte per element, a float16 scale per 32
    if (codes_bytes) *codes_bytes = rows * (size_t)head_dim;
    if (norms_bytes) *norms_bytes = rows * (size_t)(head_dim / 32) * 2u;
    return TQ_OK;
  }
  const size_t groups = rows * (size_t)(head_dim / kGroup);
  if (codes_bytes) *codes_bytes = groups * 16u * (size_t)type;
  if (norms_bytes) *norms_bytes = groups * 2u;
  return TQ_OK;
}

tq_status tq_codebook(int type, float *code_values, float *mag_thresholds, uint64_t *sign_words) {
  if (!valid_type(type)) return TQ_ERR_INVALID_ARG;
  const int n = 1 << type;
  for (int c = 0; c < n; ++c) {
    if (!code_values) break;
    code_values[c] = type == 2 ? code_value<2>(c) : type == 3 ? code_value<3>(c) : code_value<4>(c);
  }
  for (int k = 1; k < n / 2; ++k) {
    if (!mag_thresholds) break;
    mag_thresholds[k - 1] =
        type == 2 ? threshold<2>(k) : type == 3 ? threshold<3>(k) : threshold<4>(k);
  }
  if (sign_words) {
    sign_words[0] = kSignWord0;
    sign_words[1] = kSignWord1;
  }
  return TQ_OK;
}

tq_status tq_set_rows(const tq_cache *dst, const float *src, const int64_t *cell_idx,
                      int64_t n_rows, tq_stream_t stream) {
  tq_status s = check_cache(dst);
  if (s != TQ_OK) return s;
  if (n_rows < 0) return TQ_ERR_INVALID_ARG;
  if (n_rows == 0) return TQ_OK;
  if (!src || !cell_idx || !aligned(src, 16) || !aligned(cell_idx, 8)) return TQ_ERR_INVALID_ARG;
  return from_hip(launch_set_rows(*dst, src, cell_idx, n_rows, (hipStream_t)stream));
}

// ---------------------------------------------------------------- decode

// The scratch array of tq_attn_decode_static: one copy per GPU (the code
// object's device globals), holding a call's split partials.  Host code
// never passes the array's name to a kernel (on the host it names a stand-in,
// not device memory): each device's address comes from hipGetSymbolAddress,
// taken once per device with that device current.
static __device__ __align__(256) uint8_t scratch[TQ_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// This device's address of the scratch array (looked up on the first call on
// the device, kept afterwards).
hipError_t scratch_address(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

static tq_status decode_check(const tq_cache *k, const tq_cache *v, int64_t kv_len,
                              int32_t n_q_heads) {
  tq_status s = check_pair(k, v, /*same_width=*/false, /*q8_k=*/true);
  if (s != TQ_OK) return s;
  if (kv_len < 1 || kv_len > k->n_cells) return TQ_ERR_INVALID_ARG;
  if (n_q_heads < 1 || n_q_heads % k->n_kv_heads) return TQ_ERR_INVALID_ARG;
  if ((k->head_dim != 128 && k->head_dim != 256) || (v->head_dim != 128 && v->head_dim != 256))
    return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

static tq_status batch_check(int32_t n_seq, int32_t n_rows) {
  if (n_seq < 0 || n_seq > 65535 || n_rows < 1 || n_rows > 16) return TQ_ERR_INVALID_ARG;
  return TQ_OK;
}

static tq_status decode_call(const tq_cache *k, const tq_cache *v, int32_t n_seq, int32_t n_rows,
                             const int64_t *seq_start, const int32_t *seq_len, int64_t kv_len,
                             const void *q, int q_dtype, int32_t n_q_heads, float scale,
                             float sparse_v_tau, float *out, void *workspace,
                             size_t workspace_bytes, tq_stream_t stream, int path = TQ_DECODE_AUTO) {
  if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (!(scale == scale) || !(sparse_v_tau == sparse_v_tau) || sparse_v_tau < 0.f)
    return TQ_ERR_INVALID_ARG;
  DecodePlan p;
  if (tq_status st = from_hip(plan_decode(*k, *v, kv_len, n_q_heads, n_rows, n_seq, &p, path))) return st;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < p.workspace_bytes)
    return TQ_ERR_WORKSPACE;
  return from_hip(launch_decode(*k, *v, seq_start, seq_len, kv_len, q, q_dtype, n_q_heads, scale,
                                sparse_v_tau, out, workspace, p, (hipStream_t)stream));
}

tq_status tq_attn_decode_workspace(const tq_cache *k, const tq_cache *v, int64_t kv_len,
                                   int32_t n_q_heads, size_t *bytes) {
  tq_status s = decode_check(k, v, kv_len, n_q_heads);
  if (s != TQ_OK) return s;
  if (!bytes) return TQ_ERR_INVALID_ARG;
  DecodePlan p;
  if (tq_status st = from_hip(plan_decode(*k, *v, kv_len, n_q_heads, 1, 1, &p))) return st;
  *bytes = p.workspace_bytes;
  return TQ_OK;
}

tq_status tq_attn_decode(const tq_cache *k, const tq_cache *v, int64_t kv_len, const void *q,
                         int q_dtype, int32_t n_q_heads, float scale, float sparse_v_tau,
                         float *out, void *workspace, size_t workspace_bytes,
                         tq_stream_t stream) {
  tq_status s = decode_check(k, v, kv_len, n_q_heads);
  if (s != TQ_OK) return s;
  return decode_call(k, v, 1, 1, nullptr, nullptr, kv_len, q, q_dtype, n_q_heads, scale, sparse_v_tau,
                     out, workspace, workspace_bytes, stream);
}

tq_status tq_attn_decode_path_workspace(const tq_cache *k, const tq_cache *v, int64_t kv_len,
                                        int32_t n_q_heads, int path, size_t *bytes) {
  tq_status s = decode_check(k, v, kv_len, n_q_heads);
  if (s != TQ_OK) return s;
  if (!bytes) return TQ_ERR_INVALID_ARG;
  DecodePlan p;
  if (tq_status st = from_hip(plan_decode(*k, *v, kv_len, n_q_heads, 1, 1, &p, path)))
    return st == TQ_ERR_HIP ? TQ_ERR_INVALID_ARG : st;
  *bytes = p.workspace_bytes;
  return TQ_OK;
}

tq_status tq_attn_decode_path(const tq_cache *k, const tq_cache *v, int64_t kv_len, const void *q,
                              int q_dtype, int32_t n_q_heads, float scale, float sparse_v_tau, int path,
                              float *out, void *workspace, size_t workspace_bytes, tq_stream_t stream) {
  tq_status s = decode_check(k, v, kv_len, n_q_heads);
  if (s != TQ_OK) return s;
  if (path != TQ_DECODE_AUTO && path != TQ_DECODE_MATRIX && path != TQ_DECODE_TABLE) return TQ_ERR_INVALID_ARG;
  return decode_call(k, v, 1, 1, nullptr, nullptr, kv_len, q, q_dtype, n_q_heads, scale, sparse_v_tau,
                     out, workspace, workspace_bytes, stream, path);
}

tq_status tq_attn_decode_static(const tq_cache *k, const tq_cache *v, int64_t kv_len, const void *q,
                                int q_dtype, int32_t n_q_heads, float scale, float sparse_v_tau,
                                float *out, tq_stream_t stream) {
  tq_status s = decode_check(k, v, kv_len, n_q_heads);
  if (s != TQ_OK) return s;
  if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (!(scale == scale) || !(sparse_v_tau == sparse_v_tau) || sparse_v_tau < 0.f)
    return TQ_ERR_INVALID_ARG;
  DecodePlan p;
  if (tq_status st = from_hip(plan_decode(*k, *v, kv_len, n_q_heads, 1, 1, &p))) return st;
  if (p.workspace_bytes > (size_t)TQ_STATIC_SCRATCH_BYTES) return TQ_ERR_WORKSPACE;
  void *ws = nullptr;
  if (tq_status st = from_hip(scratch_address(&ws))) return st;
  // every split the merge reads is written by the split kernel first, so
  // nothing in the array needs clearing
  return from_hip(launch_decode(*k, *v, nullptr, nullptr, kv_len, q, q_dtype, n_q_heads, scale, sparse_v_tau,
                                out, ws, p, (hipStream_t)stream));
}

tq_status tq_attn_decode_batch_workspace(const tq_cache *k, const tq_cache *v, int32_t n_seq,
                                         int32_t n_rows, int64_t max_kv_len, int32_t n_q_heads,
                                         size_t *bytes) {
  tq_status s = decode_check(k, v, max_kv_len, n_q_heads);
  if (s != TQ_OK) return s;
  if ((s = batch_check(n_seq, n_rows)) != TQ_OK) return s;
  if (!bytes) return TQ_ERR_INVALID_ARG;
  if (n_seq == 0) {
    *bytes = 0;
    return TQ_OK;
  }
  DecodePlan p;
  if (tq_status st = from_hip(plan_decode(*k, *v, max_kv_len, n_q_heads, n_rows, n_seq, &p))) return st;
  *bytes = p.workspace_bytes;
  return TQ_OK;
}

tq_status tq_attn_decode_batch(const tq_cache *k, const tq_cache *v, int32_t n_seq, int32_t n_rows,
                               const int64_t *seq_start, const int32_t *seq_len, int64_t max_kv_len,
                               const void *q, int q_dtype, int32_t n_q_heads, float scale,
                               float sparse_v_tau, float *out, void *workspace,
                               size_t workspace_bytes, tq_stream_t stream) {
  tq_status s = decode_check(k, v, max_kv_len, n_q_heads);
  if (s != TQ_OK) return s;
  if ((s = batch_check(n_seq, n_rows)) != TQ_OK) return s;
  if (!seq_start || !seq_len || !aligned(seq_start, 8) || !aligned(seq_len, 4)) return TQ_ERR_INVALID_ARG;
  if (n_seq == 0) return TQ_OK;
  return decode_call(k, v, n_seq, n_rows, seq_start, seq_len, max_kv_len, q, q_dtype, n_q_heads, scale,
                     sparse_v_tau, out, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------- prefill

static tq_status prefill_check(const tq_cache *k, int64_t n_rows, int32_t n_q_heads,
                               int64_t kv_len) {
  tq_status s = check_cache(k);
  if (s != TQ_OK) return s;
  if (n_rows < 0 || kv_len < 1 || kv_len > k->n_cells) return TQ_ERR_INVALID_ARG;
  if (n_q_heads < 1 || n_q_heads % k->n_kv_heads) return TQ_ERR_INVALID_ARG;
  if ((k->head_dim != 128 && k->head_dim != 256) || n_q_heads / k->n_kv_heads > 8)
    return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

// Calls of at most this many query rows take the split-key decode kernels:
// one sequence of q_pos0 + n_rows cells from cell 0 whose row r sees cells
// <= q_pos0 + r (the same layouts for q and out).  The tiled kernel has one
// workgroup per two 32-row tiles and kv head and no key split, so a few rows
// after a long prefix ran on a handful of compute units: measured at 16 q / 8
// kv heads, head_dim 256, 3 rows after 1024 cells 37.3 us tiled against 8.9
// us split, after 16384 cells 447 us against 17 us, and 64 rows after 1024
// cells 75.9 us against 18.4 us.
constexpr int64_t kPrefillSplitRows = 64;
// ... as long as their split partials, sized for kv_len, stay within this
// many bytes (else the tiled kernel, which needs none)
constexpr size_t kPrefillSplitMaxWorkspace = size_t(256) << 20;

// Whether a prefill call takes the split-key kernels; the decision depends
// only on arguments the workspace query also has (kv_len, not q_pos0), so
// the query and the call agree.
static tq_status prefill_split_plan(const tq_cache &k, int64_t n_rows, int32_t n_q_heads, int64_t kv_len,
                                    bool *split, size_t *bytes) {
  *split = false;
  *bytes = 0;
  if (n_rows < 1 || n_rows > kPrefillSplitRows) return TQ_OK;
  DecodePlan dp;
  if (tq_status st = from_hip(plan_decode(k, k, kv_len, n_q_heads, (int)n_rows, 1, &dp))) return st;
  if (dp.workspace_bytes > kPrefillSplitMaxWorkspace) return TQ_OK;
  *split = true;
  *bytes = dp.workspace_bytes;
  return TQ_OK;
}

tq_status tq_attn_prefill_workspace(const tq_cache *k, int64_t n_rows, int32_t n_q_heads,
                                    int64_t kv_len, size_t *bytes) {
  tq_status s = prefill_check(k, n_rows, n_q_heads, kv_len);
  if (s != TQ_OK) return s;
  if (!bytes) return TQ_ERR_INVALID_ARG;
  bool split = false;
  size_t split_bytes = 0;
  if (tq_status st = prefill_split_plan(*k, n_rows, n_q_heads, kv_len, &split, &split_bytes)) return st;
  if (split) {
    // sized for the longest sequence the call may see (q_pos0 + n_rows <= kv_len)
    *bytes = split_bytes;
    return TQ_OK;
  }
  PrefillPlan p;
  if (plan_prefill(*k, n_rows, n_q_heads, kv_len, &p) != hipSuccess) return TQ_ERR_HIP;
  *bytes = p.workspace_bytes;
  return TQ_OK;
}

tq_status tq_attn_prefill(const tq_cache *k, const tq_cache *v, int64_t kv_len, const void *q,
                          int q_dtype, int64_t n_rows, int32_t n_q_heads, int64_t q_pos0,
                          float scale, float *out, void *workspace, size_t workspace_bytes,
                          tq_stream_t stream) {
  tq_status s = check_pair(k, v);
  if (s != TQ_OK) return s;
  s = prefill_check(k, n_rows, n_q_heads, kv_len);
  if (s != TQ_OK) return s;
  if (q_pos0 < 0 || q_pos0 + n_rows > kv_len) return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_F32 && q_dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
  if (!(scale == scale)) return TQ_ERR_INVALID_ARG;
  if (n_rows == 0) return TQ_OK;
  if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return TQ_ERR_INVALID_ARG;
  bool split = false;
  size_t split_bytes = 0;
  if (tq_status st = prefill_split_plan(*k, n_rows, n_q_heads, kv_len, &split, &split_bytes)) return st;
  if (split) {
    // planned for kv_len, as the workspace query sizes it (the tile count of
    // the plan is not monotone in the length, so a plan for the shorter
    // sequence could need more splits than the query provided); its grid
    // covers the sequence and splits past its q_pos0 + n_rows cells exit
    const int64_t len = q_pos0 + n_rows;
    DecodePlan dp;
    if (tq_status st = from_hip(plan_decode(*k, *v, kv_len, n_q_heads, (int)n_rows, 1, &dp))) return st;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < dp.workspace_bytes)
      return TQ_ERR_WORKSPACE;
    return from_hip(launch_decode(*k, *v, nullptr, nullptr, len, q, q_dtype, n_q_heads, scale, 0.f, out,
                                  workspace, dp, (hipStream_t)stream));
  }
  PrefillPlan p;
  if (plan_prefill(*k, n_rows, n_q_heads, kv_len, &p) != hipSuccess) return TQ_ERR_HIP;
  if (p.workspace_bytes && (!workspace || !aligned(workspace, 256) ||
                            workspace_bytes < p.workspace_bytes))
    return TQ_ERR_WORKSPACE;
  return from_hip(launch_prefill(*k, *v, kv_len, q, q_dtype, n_rows, n_q_heads, q_pos0, scale,
                                 out, workspace, p, (hipStream_t)stream));
}

// ---------------------------------------------------------------- int8 prompt

static tq_status int8_check(int64_t n_q, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                            int64_t ctx_len) {
  if (n_q < 0 || ctx_len < 1 || n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads)
    return TQ_ERR_INVALID_ARG;
  if (head_dim < 1) return TQ_ERR_INVALID_ARG;
  if (head_dim != 128 || n_q_heads / n_kv_heads > 16) return TQ_ERR_UNSUPPORTED;
  return TQ_OK;
}

tq_status tq_attn_int8_prompt_workspace(int64_t n_q, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t head_dim, int64_t ctx_len, size_t *bytes) {
  tq_status s = int8_check(n_q, n_q_heads, n_kv_heads, head_dim, ctx_len);
  if (s != TQ_OK) return s;
  if (!bytes) return TQ_ERR_INVALID_ARG;
  Int8Plan p;
  if (plan_int8(n_q, n_q_heads, n_kv_heads, ctx_len, &p) != hipSuccess) return TQ_ERR_HIP;
  *bytes = p.workspace_bytes;
  return TQ_OK;
}

tq_status tq_attn_int8_prompt(const float *q, int64_t n_q, int32_t n_q_heads, const int8_t *k,
                              const int8_t *v, const uint16_t *k_scale, const uint16_t *v_scale,
                              int32_t n_kv_heads, int32_t head_dim, const int32_t *page_table,
                              int64_t n_phys_pages, int64_t ctx_len, int64_t q_pos0, float scale,
                              float *out, void *workspace, size_t workspace_bytes,
                              tq_stream_t stream) {
  tq_status s = int8_check(n_q, n_q_heads, n_kv_heads, head_dim, ctx_len);
  if (s != TQ_OK) return s;
  if (q_pos0 < 0 || q_pos0 + n_q > ctx_len || n_phys_pages < 1) return TQ_ERR_INVALID_ARG;
  if (!(scale == scale)) return TQ_ERR_INVALID_ARG;
  if (n_q == 0) return TQ_OK;
  if (!q || !k || !v || !k_scale || !v_scale || !page_table || !out) return TQ_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(k_scale, 4) ||
      !aligned(v_scale, 4) || !aligned(page_table, 4) || !aligned(out, 16))
    return TQ_ERR_INVALID_ARG;
  Int8Plan p;
  if (plan_int8(n_q, n_q_heads, n_kv_heads, ctx_len, &p) != hipSuccess) return TQ_ERR_HIP;
  if (p.workspace_bytes && (!workspace || !aligned(workspace, 256) ||
                            workspace_bytes < p.workspace_bytes))
    return TQ_ERR_WORKSPACE;
  return from_hip(launch_int8(q, n_q, n_q_heads, k, v, k_scale, v_scale, n_kv_heads, page_table,
                              n_phys_pages, ctx_len, q_pos0, scale, out, workspace, p,
                              (hipStream_t)stream));
}

}  // extern "C"
