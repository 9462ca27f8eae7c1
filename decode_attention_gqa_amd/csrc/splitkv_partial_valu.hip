// splitkv_partial_valu.hip -- partial kernel of split-KV grouped-query
// decode attention for gfx950 (CDNA4, wave64), vector-ALU form, used for the
// small head dims (8, 16, 32) where a 32-deep MFMA step does not fit a row.
//
// One workgroup per (split, KV head, sequence), grid dim3(n_splits,
// n_kv_head, batch), independent of the live length ("10 · R4 — decode
// split-attention dim-parallel rewrite", section 2.2: static grid, nkv read
// from positions[] on the device). The workgroup computes all G query heads of
// its KV head, so each K/V row is read from HBM once per group ("Red Lite dev35
// — long-context decode: grouped split-K attention", Change).
//
// Geometry (the lane<->dim binding of "10 · R4", section 2.4, re-derived for
// 64-lane wavefronts):
//   - a lane owns 8 consecutive head dims of one row: one 16-byte fp16 load
//     per row for K and one for V; L = HD/8 lanes cover a row, so one load
//     instruction of a wave reads R = 64/L whole rows, fully coalesced;
//   - the q·k dot of a row is the lane's 8-dim partial summed over its L lanes
//     with DPP row permutations (quad xor 1 and 2, half-row and row mirrors),
//     after which every lane of the row holds the row's score for every head;
//   - the loaded K and V slice is converted once and reused by all G heads in
//     registers;
//   - each of the R row slots of a wave keeps its own online-softmax state per
//     head (mx, S, oc) over the rows it visits, with oc in VGPRs sized at
//     compile time (8 dims x G heads, no scratch; "10 · R4", section 6);
//   - rows are handled T per slot per step: all 2T loads are issued first,
//     then one max/rescale per step amortises the correction exp over T rows
//     ("10 · R4", section 2.4: batch the loads ahead of the serial chain);
//   - at the end the slot states are merged across lanes, the waves merge
//     through LDS, and the workgroup writes one record per query head.
// Scores are kept in base-2 units (q pre-multiplied by scale*log2(e)) so the
// kernel uses the hardware exp2; the record stores mx in natural-log units.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitkv_internal.h"
#include "splitkv_partial_common.h"

namespace splitkv {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));

using detail::dpp_mov;
using detail::fast_exp2;
using detail::kThreads;
using detail::kWaves;
using detail::neg_inf;

template <int HD>
struct Geometry {
  static constexpr int L = HD / 8;          // lanes per row
  static constexpr int R = 64 / L;          // row slots per wave
  static constexpr int T = 4;               // rows per slot per step
  static constexpr int ROWS_WAVE = R * T;   // rows per wave per step
  static constexpr int ROWS_STEP = kWaves * ROWS_WAVE;
  static_assert(HD % 8 == 0 && L >= 1 && L <= 32, "head_dim");
};


// Sum over the L lanes of a row (lanes [r*L, r*L + L)); every lane of the row
// receives the same value (each step adds a commutative pair).
template <int L>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (L >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (L >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (L >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (L >= 16) x += dpp_mov<0x140>(x); // row_mirror
  if constexpr (L >= 32)                         // lane ^ 16 (swizzle)
    x += __builtin_bit_cast(
        float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
  return x;
}

__device__ __forceinline__ void cvt8(const uint4 &u, float (&f)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float2v p =
        __builtin_convertvector(__builtin_bit_cast(half2v, w[i]), float2v);
    f[2 * i] = p.x;
    f[2 * i + 1] = p.y;
  }
}

// Merge online-softmax state (m2, s2, a2) into (m, s, a); base-2 units.
template <int N>
__device__ __forceinline__ void merge_state(float &m, float &s, float (&a)[N],
                                            float m2, float s2,
                                            const float (&a2)[N]) {
  const float mn = fmaxf(m, m2);
  const float c1 = (m == neg_inf()) ? 0.0f : fast_exp2(m - mn);
  const float c2 = (m2 == neg_inf()) ? 0.0f : fast_exp2(m2 - mn);
  s = s * c1 + s2 * c2;
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = a[i] * c1 + a2[i] * c2;
  m = mn;
}

template <int HD, int G>
__global__ __launch_bounds__(kThreads) void partial_valu_kernel(PartialArgs a) {
  using Geo = Geometry<HD>;
  constexpr int L = Geo::L;
  constexpr int R = Geo::R;
  constexpr int T = Geo::T;

  const int sp = blockIdx.x;
  const int hk = blockIdx.y;
  const detail::RowSel rs = detail::row_sel(a);
  const int b = rs.b;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int slot = lane / L;
  const int li = lane % L;

  // a1 + a2: live length (read on the device) and this split's rows.
  // With several query rows, this row's rows end at min(hi, its length).
  const detail::SplitRange rg = detail::split_range(a, sp, b);
  const long long lo = rg.lo;
  const long long hi = detail::row_end(a, rs, rg.hi);

  // a3: the group's queries, this lane's 8 dims, pre-scaled to base-2 units.
  float qv[G][8];
  {
    const float *qb = a.q + detail::q_offset(a, rs, hk * G, HD) + li * 8;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float4 x0 = *reinterpret_cast<const float4 *>(qb + g * HD);
      const float4 x1 = *reinterpret_cast<const float4 *>(qb + g * HD + 4);
      qv[g][0] = x0.x * a.scale_log2; qv[g][1] = x0.y * a.scale_log2;
      qv[g][2] = x0.z * a.scale_log2; qv[g][3] = x0.w * a.scale_log2;
      qv[g][4] = x1.x * a.scale_log2; qv[g][5] = x1.y * a.scale_log2;
      qv[g][6] = x1.z * a.scale_log2; qv[g][7] = x1.w * a.scale_log2;
    }
  }

  float mx[G], ssum[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mx[g] = neg_inf();
    ssum[g] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[g][i] = 0.0f;
  }

  const size_t row_stride = (size_t)a.n_kv_head * HD;  // elements
  const size_t seq_base =
      ((size_t)b * (size_t)a.max_ctx * a.n_kv_head + hk) * HD + li * 8;
  const uint16_t *kbase = a.k + seq_base;
  const uint16_t *vbase = a.v + seq_base;

  // a4 + a5: stream the split's rows; the loop bound is workgroup-uniform.
  for (long long base = lo; base < hi; base += Geo::ROWS_STEP) {
    const long long row0 = base + (long long)wave * Geo::ROWS_WAVE + slot;
    uint4 kr[T], vr[T];
    bool valid[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const long long row = row0 + t * R;
      valid[t] = row < hi;
      kr[t] = make_uint4(0, 0, 0, 0);
      vr[t] = make_uint4(0, 0, 0, 0);
      if (valid[t]) {
        kr[t] = *reinterpret_cast<const uint4 *>(kbase + (size_t)row * row_stride);
        vr[t] = *reinterpret_cast<const uint4 *>(vbase + (size_t)row * row_stride);
      }
    }
    float s[T][G];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float kf[8];
      cvt8(kr[t], kf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = qv[g][0] * kf[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) d = fmaf(qv[g][i], kf[i], d);
        d = row_sum<L>(d);
        s[t][g] = valid[t] ? d : neg_inf();
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mn = mx[g];
#pragma unroll
      for (int t = 0; t < T; ++t) mn = fmaxf(mn, s[t][g]);
      // mn == -inf only if this slot has seen no row yet: nothing to scale.
      const float corr = (mn == neg_inf()) ? 1.0f : fast_exp2(mx[g] - mn);
      ssum[g] *= corr;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[g][i] *= corr;
      mx[g] = mn;
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float vf[8];
      cvt8(vr[t], vf);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float e = valid[t] ? fast_exp2(s[t][g] - mx[g]) : 0.0f;
        ssum[g] += e;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(e, vf[i], acc[g][i]);
      }
    }
  }

  // a6: merge the R slot states of the wave (lanes with equal li hold the
  // same dims), then the waves through LDS, and write the records.
#pragma unroll
  for (int off = L; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m2 = __shfl_xor(mx[g], off);
      const float s2 = __shfl_xor(ssum[g], off);
      float a2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a2[i] = __shfl_xor(acc[g][i], off);
      merge_state<8>(mx[g], ssum[g], acc[g], m2, s2, a2);
    }
  }

  __shared__ float sm_mx[kWaves][G];
  __shared__ float sm_s[kWaves][G];
  __shared__ float sm_acc[kWaves][G][HD];
  if (slot == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sm_acc[wave][g][li * 8 + i] = acc[g][i];
      if (li == 0) {
        sm_mx[wave][g] = mx[g];
        sm_s[wave][g] = ssum[g];
      }
    }
  }
  __syncthreads();

  detail::write_records<HD, G>(a, sp, hk, rs, rg, sm_mx, sm_s, sm_acc);
}

template <int HD, int G>
hipError_t launch_one(const PartialArgs &a, int batch, hipStream_t stream) {
  hipLaunchKernelGGL((partial_valu_kernel<HD, G>),
                     dim3(a.n_splits, a.n_kv_head, batch * a.n_q),
                     dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_hd(int group, const PartialArgs &a, int batch,
                     hipStream_t stream) {
  switch (group) {
    case 1: return launch_one<HD, 1>(a, batch, stream);
    case 2: return launch_one<HD, 2>(a, batch, stream);
    case 3: return launch_one<HD, 3>(a, batch, stream);
    case 4: return launch_one<HD, 4>(a, batch, stream);
    case 5: return launch_one<HD, 5>(a, batch, stream);
    case 6: return launch_one<HD, 6>(a, batch, stream);
    case 7: return launch_one<HD, 7>(a, batch, stream);
    case 8: return launch_one<HD, 8>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_partial_valu(int head_dim, int group, const PartialArgs &a,
                               int batch, hipStream_t stream) {
  switch (head_dim) {
    case 8: return launch_hd<8>(group, a, batch, stream);
    case 16: return launch_hd<16>(group, a, batch, stream);
    case 32: return launch_hd<32>(group, a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace splitkv
