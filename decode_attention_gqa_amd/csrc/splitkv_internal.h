// splitkv_internal.h -- declarations shared by the library's own HIP sources
// (kernel launchers and the C-ABI host code). Not installed, not part of the
// ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace splitkv {

// Arguments of the partial kernel, passed by value.
struct PartialArgs {
  const float *q;            // [B][n_q][n_head][HD] fp32
  const uint16_t *k;         // [B][max_ctx][n_kv_head][HD] fp16 bits
  const uint16_t *v;         // same layout
  const int32_t *positions;  // [B]
  // Split records of record head H = t * n_head + h (t the query row):
  float *partials;           // oc sums [B][n_splits][n_q * n_head][HD]
  float *headers;            // {mx, S, lo, hi} [B][n_q * n_head][n_splits][4]
  int n_head;
  int n_kv_head;
  int max_ctx;
  int n_splits;
  int block_len;             // 0: chunk = ceil(nkv / n_splits)
  float scale_log2;          // scale * log2(e): scores are kept in base-2 units
  int kv_group;              // per-query-head form only: n_head / n_kv_head
  int n_q;                   // query rows per sequence (1: one-token decode)
  // Several-row form with more than one block of rows per sequence: 1 when
  // the grid is dim3(8 * row blocks, n_splits / 8, n_kv_head * batch), which
  // puts the row blocks of one (split, KV head, sequence) 8 apart in the
  // dispatch order; 0 for the plain grid dim3(n_splits, n_kv_head, batch *
  // row blocks).
  int pair_rows;
  // A decode step with the KV-cache append folded in (matrix-core kernel,
  // n_q = 1): each sequence's new row (fp32 [B][1][n_kv_head][HD]) is written
  // at position positions[b] into the caches k_app / v_app (the same buffers
  // as k / v) by the workgroup whose split holds that position, which also
  // uses the converted values for that row. All four null otherwise.
  const float *k_new;
  const float *v_new;
  uint16_t *k_app;
  uint16_t *v_app;
};

struct CombineArgs {
  const float *partials;     // oc sums [B][n_splits][n_head][HD]
  const float *headers;      // {mx, S, lo, hi} [B][n_head][n_splits][4]
  float *out;                // [B][n_head][HD]
  int n_head;
  int n_splits;
};

// Arguments of the KV-cache append kernel.
struct AppendArgs {
  const float *k_new;        // [B][n_rows][n_kv_head][head_dim] fp32
  const float *v_new;        // same layout
  uint16_t *k_cache;         // [B][max_ctx][n_kv_head][head_dim] fp16 bits
  uint16_t *v_cache;         // same layout
  const int32_t *positions;  // [B]; the last new row goes to positions[b]
  int n_rows;
  int row_elems;             // n_kv_head * head_dim (a multiple of 8)
  int max_ctx;
};

// Launchers: enqueue one kernel on `stream` and return hipGetLastError().
// The host code validates every argument before calling them.
// Query rows that share one matrix-core partial workgroup for n_q rows per
// sequence (1 for the vector-ALU kernel's head sizes is the caller's rule).
int rows_per_workgroup(int head_dim, int group, int n_q);

hipError_t launch_partial(int head_dim, int group, const PartialArgs &a,
                          int batch, hipStream_t stream);
hipError_t launch_combine(int head_dim, const CombineArgs &a, int batch,
                          hipStream_t stream);
hipError_t launch_partial_per_head(int head_dim, const PartialArgs &a,
                                   int batch, hipStream_t stream);
hipError_t launch_append(const AppendArgs &a, int batch, hipStream_t stream);
hipError_t launch_probe_read(const void *buf, size_t bytes, uint32_t *sink,
                             int grid, hipStream_t stream);
hipError_t launch_probe_copy(const void *src, void *dst, size_t bytes,
                             int grid, hipStream_t stream);

// Compiled shapes.
constexpr bool head_dim_supported(int hd) {
  return hd == 8 || hd == 16 || hd == 32 || hd == 64 || hd == 128 || hd == 256;
}
constexpr int kMaxGroup = 8;

}  // namespace splitkv
