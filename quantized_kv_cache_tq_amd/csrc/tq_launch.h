// tq_launch.h -- launch plans and launchers behind the C ABI (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/tq.h"

namespace tq {

// Number of compute units of the current device (cached per device).
hipError_t device_cu_count(int *n_cu);

hipError_t launch_set_rows(const tq_cache &c, const float *src, const int64_t *cell_idx,
                           int64_t n_rows, hipStream_t stream);

struct DecodePlan {
  int tiles_per_wave;    // 16-key tiles per key range (4 ranges per workgroup)
  int keys_per_split;    // 64 * tiles_per_wave
  int n_split;           // splits of the longest sequence
  int n_rows;            // query rows per sequence
  int n_seq;             // sequences per call
  int pairs;             // (row, q head) pairs per workgroup: 8 or 16
  int head_groups;       // workgroups per (split, kv head): `pairs` (row, q head) pairs each
  int fused;             // 1: the fused kernel (tiles_per_wave = tiles per wave block)
  int nb;                // fused kernel: blocks per wave
  int lut;               // 1: the Q x centroid table kernel (256 keys per split)
  size_t workspace_bytes;
};
// max_len: the longest sequence the call may see (sizes the grid).  path: a
// tq_decode_path; TQ_DECODE_TABLE needs one row of one sequence from cell 0
// (no device length arrays), 128-wide turbo2/turbo3 heads and at most 8 q
// heads per kv head, else hipErrorNotSupported.
hipError_t plan_decode(const tq_cache &k, const tq_cache &v, int64_t max_len, int32_t n_q_heads,
                       int n_rows, int n_seq, DecodePlan *p, int path = TQ_DECODE_AUTO);
// seq_start / seq_len: device arrays [n_seq] (null: one sequence of kv_len
// cells from cell 0); kv_len is otherwise the largest length allowed.
hipError_t launch_decode(const tq_cache &k, const tq_cache &v, const int64_t *seq_start,
                         const int32_t *seq_len, int64_t kv_len, const void *q, int q_dtype,
                         int32_t n_q_heads, float scale, float sparse_v_tau, float *out,
                         void *workspace, const DecodePlan &p, hipStream_t stream);

struct PrefillPlan {
  int rows_per_tile;     // query rows per workgroup
  int n_row_tiles;
  int paired;            // 1: tiles p and n_row_tiles - 1 - p share a workgroup
  int keys_per_split;    // key range per workgroup (multiple of the key tile)
  int max_splits;        // splits of the longest row tile
  size_t workspace_bytes;
};
hipError_t plan_prefill(const tq_cache &k, int64_t n_rows, int32_t n_q_heads, int64_t kv_len,
                        PrefillPlan *p);
// Merge n_split partials [rows_out][n_split][dv + 4] (16 x unnormalized
// rotated sums, log2-domain maximum, weight sum; maximum -inf for an empty
// one) into out [rows_out][dv] with the inverse rotation; a split holds
// 2^split_log2 keys.
hipError_t launch_split_merge(const float *ws, int n_split, int split_log2, int dv, int64_t rows_out,
                              float *out, hipStream_t stream);
hipError_t launch_prefill(const tq_cache &k, const tq_cache &v, int64_t kv_len, const void *q,
                          int q_dtype, int64_t n_rows, int32_t n_q_heads, int64_t q_pos0,
                          float scale, float *out, void *workspace, const PrefillPlan &p,
                          hipStream_t stream);

struct Int8Plan {
  int queries_per_tile;
  int n_q_tiles;
  int keys_per_split;
  int n_split;
  size_t workspace_bytes;
};
hipError_t plan_int8(int64_t n_q, int32_t n_q_heads, int32_t n_kv_heads, int64_t ctx_len,
                     Int8Plan *p);
hipError_t launch_int8(const float *q, int64_t n_q, int32_t n_q_heads, const int8_t *k,
                       const int8_t *v, const uint16_t *k_scale, const uint16_t *v_scale,
                       int32_t n_kv_heads, const int32_t *page_table, int64_t n_phys_pages,
                       int64_t ctx_len, int64_t q_pos0, float scale, float *out, void *workspace,
                       const Int8Plan &p, hipStream_t stream);

}  // namespace tq
