// splitkv_partial_common.h -- device helpers shared by the two partial
// kernels (the VALU kernel for head_dim 8/16/32 and the MFMA kernel for
// head_dim 64/128/256): live length and split bounds, exp2, DPP moves, the
// exact merge of online-softmax states, and the workgroup's final merge that
// writes one record per query head.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitkv_internal.h"

namespace splitkv {
namespace detail {

constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                      0xF, false));
}

// Rows [lo, hi) of split `sp` of sequence `b` ("10 · R4 — decode
// split-attention dim-parallel rewrite", section 2.2; "Red Lite dev35",
// Change, for the fixed block length). The live length is read from device
// memory; every thread of the workgroup computes the same values.
struct SplitRange {
  long long lo;
  long long hi;
};

// Every value fits in 32 bits: nkv <= max_ctx < 2^31; with a fixed block
// length the host checks block_len * n_splits <= INT_MAX, and otherwise
// (sp + 1) * chunk < nkv + n_splits. (This runs between the live-length load
// and the first K/V load of every workgroup, so it avoids 64-bit division.)
// p = positions[b], read by the caller (so that it can issue the read early).
__device__ __forceinline__ SplitRange split_range_at(const PartialArgs &a,
                                                     int sp, int p) {
  const uint32_t mc = (uint32_t)a.max_ctx;
  const uint32_t nkv = p < 0 ? 0u : ((uint32_t)p >= mc ? mc : (uint32_t)p + 1u);
  const uint32_t ns = (uint32_t)a.n_splits;
  const uint32_t chunk =
      a.block_len > 0 ? (uint32_t)a.block_len : (nkv + ns - 1u) / ns;
  const uint32_t lo = (uint32_t)sp * chunk;
  const uint32_t h = lo + chunk;
  SplitRange r;
  r.lo = lo;
  r.hi = h < nkv ? h : nkv;
  return r;
}
__device__ __forceinline__ SplitRange split_range(const PartialArgs &a,
                                                  int sp, int b) {
  return split_range_at(a, sp, a.positions[b]);
}

// The (sequence, query row) a partial workgroup serves: blockIdx.z =
// b * n_q + t. With several query rows ("dotLLM issue #199", comment 1,
// section 2: seqQ > 1 with a causal mask from positionOffset) row t sits at
// position positions[b] - (n_q - 1 - t) and sees the cache rows before and
// at it: its live length is clamp(positions[b] + 1 - (n_q - 1 - t), 0,
// max_ctx). The splits are those of the last row (live length nkv_b), the
// same for every row, and row t stops at min(hi, its live length).
struct RowSel {
  int b;
  int t;
};
__device__ __forceinline__ RowSel row_sel(const PartialArgs &a) {
  RowSel r;
  if (a.n_q == 1) {
    r.b = blockIdx.z;
    r.t = 0;
  } else {
    r.b = blockIdx.z / a.n_q;
    r.t = blockIdx.z - r.b * a.n_q;
  }
  return r;
}

// End of query row t of sequence b within the split [lo, hi); p =
// positions[b].
__device__ __forceinline__ long long row_end_pos(const PartialArgs &a, int p,
                                                 int t, long long hi) {
  long long n = (long long)p + 1 - (a.n_q - 1 - t);
  n = n < 0 ? 0 : (n > a.max_ctx ? a.max_ctx : n);
  return n < hi ? n : hi;
}
__device__ __forceinline__ long long row_end_at(const PartialArgs &a, int b,
                                                int t, long long hi) {
  return row_end_pos(a, a.positions[b], t, hi);
}
__device__ __forceinline__ long long row_end(const PartialArgs &a,
                                             const RowSel &rs, long long hi) {
  if (a.n_q == 1) return hi;  // the one row is the last row: nkv_b >= hi
  return row_end_at(a, rs.b, rs.t, hi);
}

// Offsets for query row t of sequence b: its first q element, and the parts
// of the record of split sp and record head t * n_head + head: the first of
// its HD output sums ([B][S][n_q * n_head][HD]) and its 4-float header
// ([B][n_q * n_head][S][4]).
__device__ __forceinline__ size_t q_offset(const PartialArgs &a,
                                           const RowSel &rs, int head, int hd) {
  return (((size_t)rs.b * a.n_q + rs.t) * a.n_head + head) * (size_t)hd;
}
__device__ __forceinline__ size_t oc_offset(const PartialArgs &a,
                                            const RowSel &rs, int sp,
                                            int head, int hd) {
  return ((((size_t)rs.b * a.n_splits + sp) * a.n_q + rs.t) * a.n_head +
          head) * (size_t)hd;
}
__device__ __forceinline__ size_t hdr_offset(const PartialArgs &a, int b,
                                             int t, int sp, int head) {
  return ((((size_t)b * a.n_q + t) * a.n_head + head) * a.n_splits + sp) * 4;
}

// Merge (m2, s2) into (m, s) and return the weights (c1, c2) applied to the
// two accumulators; base-2 units; a -inf state has weight exactly 0.
struct MergeW {
  float c1;
  float c2;
};
__device__ __forceinline__ MergeW merge_weights(float &m, float &s, float m2,
                                                float s2) {
  const float mn = fmaxf(m, m2);
  MergeW w;
  w.c1 = (m == neg_inf()) ? 0.0f : fast_exp2(m - mn);
  w.c2 = (m2 == neg_inf()) ? 0.0f : fast_exp2(m2 - mn);
  s = s * w.c1 + s2 * w.c2;
  m = mn;
  return w;
}

// Final step of a partial workgroup: the kWaves per-wave states in LDS
// (max and sum per head in base-2 units, unnormalised output per head and
// dim) are merged exactly and written as the records of the G query heads of
// KV head hk: oc[0..HD) and the header { mx (natural-log units), S, lo, hi }.
// Must be called by all threads after a barrier.
template <int HD, int G>
__device__ __forceinline__ void write_records(
    const PartialArgs &a, int sp, int hk, const RowSel &rs,
    const SplitRange &rg, const float (&sm_m)[kWaves][G],
    const float (&sm_s)[kWaves][G], const float (&sm_o)[kWaves][G][HD]) {
  float *oc0 = a.partials + oc_offset(a, rs, sp, hk * G, HD);
  for (int idx = threadIdx.x; idx < G * HD; idx += kThreads) {
    const int g = idx / HD;
    const int d = idx % HD;
    float m = neg_inf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) m = fmaxf(m, sm_m[w][g]);
    float s = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm_m[w][g];
      const float c = (mw == neg_inf()) ? 0.0f : fast_exp2(mw - m);
      s = fmaf(c, sm_s[w][g], s);
      o = fmaf(c, sm_o[w][g][d], o);
    }
    oc0[(size_t)g * HD + d] = o;
    if (d == 0)
      *reinterpret_cast<float4 *>(a.headers +
                                  hdr_offset(a, rs.b, rs.t, sp, hk * G + g)) =
          make_float4(m * kLn2,  // -inf stays -inf
                      s, __builtin_bit_cast(float, (int32_t)rg.lo),
                      __builtin_bit_cast(float, (int32_t)rg.hi));
  }
}

}  // namespace detail

// Launchers of the two kernel families (one per translation unit).
hipError_t launch_partial_valu(int head_dim, int group, const PartialArgs &a,
                               int batch, hipStream_t stream);
hipError_t launch_partial_mfma(int head_dim, int group, const PartialArgs &a,
                               int batch, hipStream_t stream);

}  // namespace splitkv
