// splitkv_combine.hip -- combine kernel of split-KV decode attention (gfx950).
//
// Merges the split records exactly as "10 · R4 — decode split-attention
// dim-parallel rewrite", section 2.1 defines the combine:
//   gmx = max over splits of mx,  w = exp(mx - gmx),
//   S = sum w*S_sp,  acc = sum w*oc_sp,  o = acc / S  (0 when S <= 0).
// A record with mx = -inf (an idle split) gets weight exactly 0, also when all
// records are idle and gmx itself is -inf.
//
// Grid dim3(n_head, head_dim / DC, batch): one workgroup per (query head,
// slice of DC head dims, sequence), so the merge reads are spread over many
// compute units. Inside, C = DC/4 threads cover one record's slice with
// 16-byte loads and NG = 256/C record groups run side by side; each thread
// takes every NG-th record, several per pass with all loads issued before the
// arithmetic, and keeps a running (max, sum, acc) with the same exact
// re-weighting; the NG partial states are merged through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitkv_internal.h"

namespace splitkv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// exp(x - m) for x <= m, with exp(-inf - m) = 0 and a zero weight when m is
// itself -inf (then every x is -inf too).
__device__ __forceinline__ float weight(float x, float m) {
  return (x == neg_inf()) ? 0.0f : __builtin_amdgcn_exp2f((x - m) * kLog2e);
}

template <int HD>
struct CombineGeo {
  static constexpr int DC = HD < 32 ? HD : 32;  // dims per workgroup
  static constexpr int C = DC / 4;              // threads per record slice
  static constexpr int NG = kThreads / C;       // record groups
};

template <int HD>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  using Geo = CombineGeo<HD>;
  constexpr int DC = Geo::DC;
  constexpr int C = Geo::C;
  constexpr int NG = Geo::NG;
  constexpr size_t pstr = 4 + HD;

  const int h = blockIdx.x;
  const int d_base = blockIdx.y * DC;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int c = tid % C;
  const int g0 = tid / C;
  const size_t rstride = (size_t)a.n_head * pstr;
  const float *base =
      a.partials + ((size_t)b * a.n_splits * a.n_head + h) * pstr;
  const int dofs = 4 + d_base + 4 * c;

  float m = neg_inf(), s = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int sp0 = g0; sp0 < a.n_splits; sp0 += NG * kUnroll) {
    float2 hdr[kUnroll];
    float4 oc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int sp = sp0 + u * NG;
      hdr[u] = make_float2(neg_inf(), 0.0f);
      oc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (sp < a.n_splits) {
        const float *r = base + (size_t)sp * rstride;
        hdr[u] = *reinterpret_cast<const float2 *>(r);
        oc[u] = *reinterpret_cast<const float4 *>(r + dofs);
      }
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) mn = fmaxf(mn, hdr[u].x);
    const float keep = weight(m, mn);
    s *= keep;
    acc.x *= keep; acc.y *= keep; acc.z *= keep; acc.w *= keep;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float w = weight(hdr[u].x, mn);
      s = fmaf(w, hdr[u].y, s);
      acc.x = fmaf(w, oc[u].x, acc.x);
      acc.y = fmaf(w, oc[u].y, acc.y);
      acc.z = fmaf(w, oc[u].z, acc.z);
      acc.w = fmaf(w, oc[u].w, acc.w);
    }
    m = mn;
  }

  __shared__ float sm_m[NG];
  __shared__ float sm_s[NG];
  __shared__ float4 sm_acc[NG][C];
  sm_acc[g0][c] = acc;
  if (c == 0) {
    sm_m[g0] = m;
    sm_s[g0] = s;
  }
  __syncthreads();

  for (int i = tid; i < DC; i += kThreads) {
    float gm = neg_inf();
    for (int g = 0; g < NG; ++g) gm = fmaxf(gm, sm_m[g]);
    float st = 0.0f, o = 0.0f;
    const int ci = i / 4, lane = i % 4;
    for (int g = 0; g < NG; ++g) {
      const float w = weight(sm_m[g], gm);
      st = fmaf(w, sm_s[g], st);
      const float4 v = sm_acc[g][ci];
      const float x = lane == 0 ? v.x : lane == 1 ? v.y : lane == 2 ? v.z : v.w;
      o = fmaf(w, x, o);
    }
    a.out[((size_t)b * a.n_head + h) * HD + d_base + i] =
        (st > 0.0f) ? o / st : 0.0f;
  }
}

template <int HD>
hipError_t launch_one(const CombineArgs &a, int batch, hipStream_t stream) {
  hipLaunchKernelGGL((combine_kernel<HD>),
                     dim3(a.n_head, HD / CombineGeo<HD>::DC, batch),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(int head_dim, const CombineArgs &a, int batch,
                          hipStream_t stream) {
  switch (head_dim) {
    case 8: return launch_one<8>(a, batch, stream);
    case 16: return launch_one<16>(a, batch, stream);
    case 32: return launch_one<32>(a, batch, stream);
    case 64: return launch_one<64>(a, batch, stream);
    case 128: return launch_one<128>(a, batch, stream);
    case 256: return launch_one<256>(a, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace splitkv
