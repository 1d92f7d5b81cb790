/*
 * tq.h -- C ABI of libtq.so: attention over a TurboQuant-compressed KV cache
 * on one AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [PR36]    llama-cpp-turboquant pull request 36: (a) SET_ROWS butterfly on
 *             warp shuffles, (b) asymmetric-K head-dim fix, (c) decode
 *             Q x centroid lookup table, (d) four VEC flash-attention changes.
 *   [PR28]    "HIP/turbo3: graph-safe decode + inline-dequant TILE prefill on
 *             gfx1201 (RDNA4)".
 *   [QSA1821] "#1821 qsa_prompt_attn: int8 K/V prefetched in registers and
 *             sharing one buffer (Turing / sm_75)".
 *
 * General rules for every entry point:
 *   - Pointers are DEVICE pointers unless marked [host].  The caller owns every
 *     buffer; the library never allocates, frees or memsets device memory, so
 *     every call may be recorded into a HIP graph (the failure of [PR28]
 *     "Graph-safe decode" was an allocation during stream capture).
 *   - All argument checks run on the host before any HIP call; a rejected
 *     call returns a negative tq_status and enqueues nothing.  TQ_OK means the
 *     work was enqueued on `stream`; faults surface at the caller's
 *     synchronization.  TQ_ERR_HIP reports a failed launch.
 *   - Calls that share an output or workspace buffer on the same device must
 *     be ordered by the caller (same stream or events).
 *   - No call reads or writes memory outside the extents stated here for
 *     valid arguments.  Values in device buffers that the host cannot check
 *     (cell indices, page-table entries) are bounds-checked in the kernels:
 *     an out-of-range cell index drops that row, an out-of-range page entry
 *     masks that page's keys; results are then unspecified but no access
 *     leaves the stated extents.
 */
#ifndef TQ_H
#define TQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A hipStream_t (NULL = the legacy null stream). */
typedef struct ihipStream_t *tq_stream_t;

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1, /* a null/misaligned pointer or an out-of-contract size */
  TQ_ERR_UNSUPPORTED = -2, /* a valid request this build has no kernel for */
  TQ_ERR_WORKSPACE = -3,   /* workspace pointer null/misaligned or too small */
  TQ_ERR_HIP = -4          /* the HIP runtime reported an error */
} tq_status;

/* Cache element types ([PR36] (c)/(d) results table: turbo2, turbo3, turbo4):
 * b = 2, 3, 4 bits per element, 2^b reconstruction levels.  TQ_Q8 is the
 * 8-bit block format of an asymmetric cache's K ([PR36] (b): K kept in
 * 8-bit blocks beside a turbo V); it serves as the K cache of
 * tq_attn_decode / tq_attn_decode_batch only. */
typedef enum { TQ_TURBO2 = 2, TQ_TURBO3 = 3, TQ_TURBO4 = 4, TQ_Q8 = 8 } tq_type;

/* Element type of a query tensor. */
typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

/*
 * One compressed cache (the K cache or the V cache of one layer).
 *
 * Every head_dim-wide row of every kv head is cut into G = head_dim/128
 * groups of 128 elements ([PR36] (a): 7 butterfly stages, h = 1..64; a
 * 192-wide head is padded to 256 in [PR36] (b)).  Each group stores
 *   - 16*b code bytes: one little-endian bit stream in which element e's
 *     b-bit code occupies stream bits b*e .. b*e+b-1, low bit first (stream
 *     bit k is bit k%8 of byte k/8).  A code is a (b-1)-bit magnitude index
 *     ("qs") with the sign bit on top (set = negative); 8 elements take 3
 *     bytes for turbo3, as the "2 qs bytes + 1 signs byte" of [PR36] (c);
 *   - one float16 norm (the group's L2 norm), so a turbo2 group is 34 bytes
 *     against 256 for float16, the 7.5x of [PR36] (d).
 * Planes (head-major, so one kv head's cells are contiguous):
 *   codes : uint8  [n_kv_heads][n_cells][G][16*b]   16-byte aligned
 *   norms : uint16 [n_kv_heads][n_cells][G]         float16 bits, 4-byte aligned
 * A TQ_Q8 cache cuts every row into blocks of 32 elements, each stored as
 * 32 int8 codes and one float16 scale d (element = code * d; not rotated):
 *   codes : int8   [n_kv_heads][n_cells][head_dim/32][32]   16-byte aligned
 *   norms : uint16 [n_kv_heads][n_cells][head_dim/32]       float16 scales, 4-byte aligned
 */
typedef struct {
  int32_t type;       /* tq_type */
  int32_t head_dim;   /* multiple of 128, >= 128 */
  int32_t n_kv_heads; /* >= 1 */
  int32_t reserved;   /* must be 0 */
  int64_t n_cells;    /* capacity in cells (tokens), >= 1 */
  uint8_t *codes;     /* device */
  uint16_t *norms;    /* device */
} tq_cache;

const char *tq_version(void);
const char *tq_status_str(int status);

/* [host] Byte sizes of the two planes of a cache with these dimensions. */
tq_status tq_cache_plane_bytes(int type, int32_t head_dim, int32_t n_kv_heads, int64_t n_cells,
                               size_t *codes_bytes /*[host]*/, size_t *norms_bytes /*[host]*/);

/*
 * [host] The fixed parameters of the code ([PR36] (c) gives only the number of
 * levels; these are chosen values, identical for K, V and Q):
 *   code_values[2^b]       reconstruction level of each code: +-magnitude, the
 *                          magnitudes being the Lloyd-Max levels of N(0,1)
 *                          (computed in double precision) rounded to float32;
 *   mag_thresholds[2^(b-1)-1]  the midpoints of neighbouring double-precision
 *                          levels, rounded to float32;
 *   sign_words[2]          the random sign flip: element d of a group is
 *                          negated iff bit d%64 of sign_words[d/64] is set
 *                          (the first two SplitMix64 outputs from state 0).
 * Any output pointer may be NULL.
 */
tq_status tq_codebook(int type, float *code_values /*[host]*/, float *mag_thresholds /*[host]*/,
                      uint64_t *sign_words /*[host]*/);

/*
 * SET_ROWS ([PR36] (a)): quantize n_rows rows into the cache cells cell_idx[r].
 *   src      float32 [n_rows][n_kv_heads][head_dim], 16-byte aligned
 *   cell_idx int64 [n_rows], each in [0, n_cells); duplicates give an
 *            unspecified one of the rows; out-of-range rows are dropped.
 * Per 128-element group x, in IEEE float32 without fused multiply-add:
 *   n2 = sum of x_d^2 added in the butterfly's pairing order (partials at
 *   distance 1, 2, 4, .., 64); norm = sqrt(n2) correctly rounded, stored as
 *   float16 (nearest-even); u = sign flip of x; seven butterfly stages
 *   h = 1, 2, .., 64 in that order, the lower element of each pair taking
 *   a + b and the upper a - b ([PR36] (a)); y = u * (1/norm) (0 if norm is
 *   not > 0); sign bit = (y < 0); qs = #{k : |y| > mag_thresholds[k]}.
 * For a TQ_Q8 cache, per 32-element block x: d = float16(max|x_i| / 127)
 * (float32 division, nearest-even to float16); code_i = clamp(rint(x_i / d),
 * -127, 127) with x_i / d the correctly rounded float32 quotient by the
 * stored d and ties to even; all codes 0 when d is 0 or not finite.
 * The written bytes and norms are a pure function of the source values.
 * n_rows == 0 is a no-op.
 */
tq_status tq_set_rows(const tq_cache *dst, const float *src, const int64_t *cell_idx,
                      int64_t n_rows, tq_stream_t stream);

/*
 * Decode attention: one query row over cells [0, kv_len) ([PR36] (c),(d):
 * decode over a turbo cache, the single-column flash-attention case;
 * [PR28] "Graph-safe decode").
 *   q    [n_q_heads][k->head_dim], float32 or bfloat16 (q_dtype), 16-byte aligned
 *   out  float32 [n_q_heads][v->head_dim], 16-byte aligned
 * Computes, for q head h and kv head g = h / (n_q_heads / n_kv_heads):
 *   out[h] = sum_j softmax_j(scale * <q[h], k_hat_j>) v_hat_j,
 * with k_hat, v_hat the dequantized rows: x_hat = s (.) H w / sqrt(128) per
 * group, w_d = code_values[code_d] * norm / sqrt(128), H the 128-point
 * Sylvester-Hadamard matrix.  (The kernels work in the rotated domain,
 * rotating q in and the output back out.)
 * k may also be a TQ_Q8 cache beside a turbo v ([PR36] (b): the
 * asymmetric cache): its rows are used as stored (code * scale, no
 * rotation) and only v's rotation is undone on the output.
 * Requires k and v of the same turbo type (or k TQ_Q8), n_kv_heads and n_cells,
 * 1 <= kv_len <= n_cells, n_q_heads a multiple of n_kv_heads (else
 * TQ_ERR_INVALID_ARG); this build takes head widths of 128 or 256 for each
 * of k and v, which may differ ([PR36] (b): a 192-wide K head padded to 256
 * beside 128-wide V heads, decoded natively; else TQ_ERR_UNSUPPORTED).  A
 * workgroup serves P (query row, q head) pairs of one kv head (n_pairs =
 * n_rep here, n_rows * n_rep in the batched call below).  When both caches
 * are turbo with 128-wide heads and either n_pairs <= 8 or there is one
 * sequence (the "fused" case), P = 8 and a kv head's pairs take
 * ceil(n_pairs / 8) pair groups of workgroups over the same cells.
 * Otherwise P = 16 when n_pairs > 8 and both caches are turbo with 128-wide
 * heads (the two sets of eight share one decode of the cells), else P = 8;
 * more pairs take more workgroups over the same cells.
 * sparse_v_tau >= 0 ([PR36] (d) item 3; 0 = off): a key whose weight
 * e^(s - m) is below tau is left out of the value sum and kept in the
 * normalizer, with m a reference no larger than the true maximum.  In the
 * fused case a wave scores aligned blocks of 16 tb keys in turn, tb the
 * largest of 4, 2, 1 with W(tb) = ceil(kv_len / 128 tb) * n_kv_heads *
 * ceil(n_pairs / 8) >= C, C the device's compute units (else 1), and m is
 * the maximum of the keys it has
 * scored up to and including the key's block: that block's own maximum
 * while W(tb) < 2C (one block per wave; for the batched call below, kv_len
 * is max_kv_len and W is multiplied by n_seq).  Otherwise m is the maximum
 * over the
 * aligned block of 16 T keys that one wave scores, T the largest of 8, 4,
 * 2, 1 with T (k->head_dim + v->head_dim) / 128 <= 16 and
 * W(T) = ceil(kv_len / 64T) * n_kv_heads * ceil(n_pairs / P) >= C, else 1;
 * and 4 in place of 8 when W(8) > C (n_rep = n_q_heads / n_kv_heads; for
 * the batched call below, kv_len is max_kv_len and W is multiplied by
 * n_seq).
 * The output then differs from the dense one by at most
 * sum over {j : e^(s_j - m*) < tau} of (e^(s_j - m*) / sum_i e^(s_i - m*)) |v_j|_2
 * (m* the true maximum).  In the first case above, a 16-key tile whose
 * weights are all left out also skips its value products.  A NaN or negative tau
 * is TQ_ERR_INVALID_ARG.
 * The workspace holds per-split partial results; its size comes from
 * tq_attn_decode_workspace for the same caches and arguments on the same
 * device (it grows with v->head_dim).
 */
tq_status tq_attn_decode_workspace(const tq_cache *k, const tq_cache *v, int64_t kv_len,
                                   int32_t n_q_heads, size_t *bytes /*[host]*/);
tq_status tq_attn_decode(const tq_cache *k, const tq_cache *v, int64_t kv_len, const void *q,
                         int q_dtype, int32_t n_q_heads, float scale, float sparse_v_tau,
                         float *out, void *workspace, size_t workspace_bytes, tq_stream_t stream);

/*
 * Decode with an explicit choice of kernel ([PR36] (c): the decode reads a
 * per-query-head table of query x level products in shared memory).  Same
 * arguments, requirements and result as tq_attn_decode, plus path:
 *   TQ_DECODE_AUTO    the route tq_attn_decode takes;
 *   TQ_DECODE_MATRIX  every code decoded once per kv head to its level,
 *                     scores and values on the matrix cores for all the kv
 *                     head's q heads at once;
 *   TQ_DECODE_TABLE   the table of [PR36] (c): per split, lut[h][p][e] =
 *                     q_h[2p] c[e0] + q_h[2p+1] c[e1] in float32 for the
 *                     code pair e = (e0, e1) of elements 2p, 2p+1, a key's
 *                     score 64 table reads per q head; values accumulated
 *                     in float32 per (head, element).  Requires turbo2 or
 *                     turbo3 caches with 128-wide K and V heads and at most 8
 *                     q heads per kv head (else TQ_ERR_UNSUPPORTED).  The
 *                     sparse-V reference of a key is the maximum of its
 *                     256-key split.
 * An unknown path is TQ_ERR_INVALID_ARG.  The workspace size depends on the
 * path: it comes from tq_attn_decode_path_workspace with the same path.
 * TQ_DECODE_AUTO never picks the table: measured on MI355X it is slower at
 * every shape tried (1 to 8 q heads per kv head).
 */
typedef enum { TQ_DECODE_AUTO = 0, TQ_DECODE_MATRIX = 1, TQ_DECODE_TABLE = 2 } tq_decode_path;
tq_status tq_attn_decode_path_workspace(const tq_cache *k, const tq_cache *v, int64_t kv_len,
                                        int32_t n_q_heads, int path, size_t *bytes /*[host]*/);
tq_status tq_attn_decode_path(const tq_cache *k, const tq_cache *v, int64_t kv_len, const void *q,
                              int q_dtype, int32_t n_q_heads, float scale, float sparse_v_tau, int path,
                              float *out, void *workspace, size_t workspace_bytes, tq_stream_t stream);

/*
 * Decode without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments, requirements and
 * result as tq_attn_decode, with the split partials kept in a device array
 * that the library owns, TQ_STATIC_SCRATCH_BYTES on every GPU the library
 * runs on, held until the process ends.  The call allocates nothing.  A
 * call whose partials (the size tq_attn_decode_workspace reports) exceed the
 * array returns TQ_ERR_WORKSPACE and enqueues nothing.  Every call on a GPU
 * shares that GPU's array: calls that may overlap on one GPU (other streams
 * or threads) race and must be ordered by the caller.
 */
#define TQ_STATIC_SCRATCH_BYTES (16u << 20)
tq_status tq_attn_decode_static(const tq_cache *k, const tq_cache *v, int64_t kv_len, const void *q,
                                int q_dtype, int32_t n_q_heads, float scale, float sparse_v_tau,
                                float *out, tq_stream_t stream);

/*
 * Batched decode: n_seq sequences with n_rows (1..16) query rows each, in
 * one call ([PR28] "Graph-safe decode": query batches of at most two rows
 * take the single-row decode kernel, not the tile kernel; here any number
 * of sequences share one launch).
 *   seq_start int64 [n_seq], seq_len int32 [n_seq]: DEVICE arrays, 8- and
 *             4-byte aligned, read by the kernels, so a captured graph
 *             replays with whatever they hold at replay time.  Sequence i
 *             owns cells [seq_start[i], seq_start[i] + seq_len[i]) of every
 *             kv head (sequences may share cells).
 *   q    [n_seq][n_rows][n_q_heads][k->head_dim], float32 or bfloat16, 16-byte aligned
 *   out  float32 [n_seq][n_rows][n_q_heads][v->head_dim], 16-byte aligned
 * Row r of sequence i is the query at position seq_len[i] - n_rows + r of
 * that sequence and sees its cells j <= seq_len[i] - n_rows + r (causal;
 * the same formula as tq_attn_decode over those cells).  max_kv_len (host,
 * 1 <= max_kv_len <= n_cells) sizes the grid and the workspace: every
 * seq_len[i] must be at most max_kv_len.  The kernels clamp the arrays'
 * entries so that no access leaves the cache (seq_start into [0, n_cells],
 * seq_len into [0, min(max_kv_len, n_cells - seq_start)]); a row that sees
 * no cell (seq_len[i] < n_rows - r) is written as zeros.  n_seq == 0 is a
 * no-op.  Same requirements on k, v, n_q_heads and sparse_v_tau as
 * tq_attn_decode; the workspace size comes from
 * tq_attn_decode_batch_workspace for the same caches and arguments.  Calls
 * that share a workspace must not run concurrently.
 */
tq_status tq_attn_decode_batch_workspace(const tq_cache *k, const tq_cache *v, int32_t n_seq,
                                         int32_t n_rows, int64_t max_kv_len, int32_t n_q_heads,
                                         size_t *bytes /*[host]*/);
tq_status tq_attn_decode_batch(const tq_cache *k, const tq_cache *v, int32_t n_seq, int32_t n_rows,
                               const int64_t *seq_start, const int32_t *seq_len, int64_t max_kv_len,
                               const void *q, int q_dtype, int32_t n_q_heads, float scale,
                               float sparse_v_tau, float *out, void *workspace,
                               size_t workspace_bytes, tq_stream_t stream);

/*
 * Prefill / speculative-verify attention: n_rows query rows
 * ([PR28] "Inline-dequant TILE prefill": multi-row batches that read the
 * turbo cache directly, dequantizing as the tiles are loaded).
 *   q    [n_rows][n_q_heads][head_dim], float32 or bfloat16, 16-byte aligned
 *   out  float32 [n_rows][n_q_heads][head_dim], 16-byte aligned
 * Query row r sits at position q_pos0 + r and sees cells j <= q_pos0 + r
 * (causal, aligned so that the last row sees q_pos0 + n_rows - 1 keys + 1).
 * Same formula and head mapping as decode.  Requires k and v of the same
 * type, head_dim, n_kv_heads and n_cells, and
 * 0 <= q_pos0, q_pos0 + n_rows <= kv_len <= n_cells; n_rows == 0 is a no-op.
 * This build supports turbo2, turbo3 and turbo4 with head_dim 128 or 256
 * and at most 8 q heads per kv head (others: TQ_ERR_UNSUPPORTED; [PR28]
 * "Scope / honesty" validates its fast path for turbo3 at head_dim 256 only;
 * the other types use the same kernel with a wider or narrower pair table,
 * head_dim 128 the same kernel with half the products per tile).
 * Calls of at most 64 rows run the split-key decode kernels instead of the
 * tiled ones, as one sequence of q_pos0 + n_rows cells whose row r sees
 * cells <= q_pos0 + r (the tiled kernel has no key split, so a few rows
 * after a long prefix would occupy a handful of compute units), as long as
 * their split partials for kv_len cells fit 256 MiB.  [PR28]
 * "Graph-safe decode" routes only batches of at most two rows to its decode
 * kernel.  A tiled call whose grid would occupy at most half the compute
 * units while kv_len spans at least 16 key tiles of 64 splits the key range
 * too, merging the partials in a second kernel.  Such calls need a
 * workspace; tq_attn_prefill_workspace with the call's k, n_rows, n_q_heads
 * and kv_len gives its size (any q_pos0), at most 256 MiB, and 0 when none
 * is needed.  When n_q_heads / n_kv_heads does not divide 64 (3, 5, 6, 7), a
 * 64-qrow tile of the tiled kernel holds floor(64 / n_rep) rows of each
 * head.  Every path meets the same accuracy bar.
 */
tq_status tq_attn_prefill_workspace(const tq_cache *k, int64_t n_rows, int32_t n_q_heads,
                                    int64_t kv_len, size_t *bytes /*[host]*/);
tq_status tq_attn_prefill(const tq_cache *k, const tq_cache *v, int64_t kv_len, const void *q,
                          int q_dtype, int64_t n_rows, int32_t n_q_heads, int64_t q_pos0,
                          float scale, float *out, void *workspace, size_t workspace_bytes,
                          tq_stream_t stream);

/*
 * Paged int8 prompt attention ([QSA1821] What / Change).
 *   q          float32 [n_q][n_q_heads][head_dim], 16-byte aligned
 *   k, v       int8 [n_phys_pages*32][n_kv_heads][head_dim], 16-byte aligned
 *   k_scale, v_scale  float16 bits [n_phys_pages*32][n_kv_heads], 4-byte aligned
 *   page_table int32 [ceil(ctx_len/32)]: logical 32-cell chunk i is stored at
 *              physical chunk page_table[i] (0 <= entry < n_phys_pages)
 *   out        float32 [n_q][n_q_heads][head_dim], 16-byte aligned
 * Logical cell j is physical row page_table[j/32]*32 + j%32; its key is
 * k[row][g][:] * k_scale[row][g] (symmetric, no zero point), likewise v.
 * Query i sits at position q_pos0 + i and sees logical cells
 * j <= q_pos0 + i; same softmax formula and head mapping as decode.
 * The result depends only on the logical order, never on where the chunks
 * sit physically ([QSA1821] Change: same bytes, same arithmetic, same bits).
 * Requires 0 <= q_pos0, q_pos0 + n_q <= ctx_len, head_dim == 128 and at most
 * 16 q heads per kv head in this build.
 */
tq_status tq_attn_int8_prompt_workspace(int64_t n_q, int32_t n_q_heads, int32_t n_kv_heads,
                                        int32_t head_dim, int64_t ctx_len,
                                        size_t *bytes /*[host]*/);
tq_status tq_attn_int8_prompt(const float *q, int64_t n_q, int32_t n_q_heads, const int8_t *k,
                              const int8_t *v, const uint16_t *k_scale, const uint16_t *v_scale,
                              int32_t n_kv_heads, int32_t head_dim, const int32_t *page_table,
                              int64_t n_phys_pages, int64_t ctx_len, int64_t q_pos0, float scale,
                              float *out, void *workspace, size_t workspace_bytes,
                              tq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */
