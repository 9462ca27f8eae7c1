// splitkv_combine.hip -- combine kernel of split-KV decode attention (gfx950).
//
// Merges the split records exactly as "10 · R4 — decode split-attention
// dim-parallel rewrite", section 2.1 defines the combine:
//   gmx = max over splits of mx,  w = exp(mx - gmx),
//   S = sum w*S_sp,  acc = sum w*oc_sp,  o = acc / S  (0 when S <= 0).
// A record with mx = -inf (an idle split) gets weight exactly 0, also when all
// records are idle and gmx itself is -inf.
//
// The records' output sums are [batch][n_splits][n_head][head_dim] and their
// headers {mx, S, lo, hi} [batch][n_head][n_splits][4], so a 32-dim slice of
// a record is one aligned 128-byte line and a head's headers are contiguous:
// each line is fetched by one workgroup only.
//
// Grid dim3(n_head, head_dim / DC, batch): one workgroup per (query head,
// slice of DC head dims, sequence), so the merge reads are spread over many
// compute units. Inside, C = DC/4 threads cover one record's slice with
// 16-byte loads and NG = 256/C record groups run side by side; each thread
// takes every NG-th record, several per pass with all loads issued before the
// arithmetic, and keeps a running (max, sum, acc) with the same exact
// re-weighting. The NG partial states are merged by lane exchanges inside
// each wave (a DPP rotation for lanes 8 apart, v_permlane16/32_swap for 16
// and 32) and through LDS across the four waves.
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

// One lane's running state: max, weight sum, weighted output slice.
struct State {
  float m;
  float s;
  float4 acc;
};

__device__ __forceinline__ float xchg(float x, int off) {
  const int b = __builtin_bit_cast(int, x);
  const bool upper = (threadIdx.x & off) != 0;
  if (off == 32) {
    // v_permlane32_swap(x, x): every lane gets (x of lane & ~32, x of lane | 32)
    const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    return __builtin_bit_cast(float, (int)(upper ? r[0] : r[1]));
  }
  if (off == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(b, b, false, false);
    return __builtin_bit_cast(float, (int)(upper ? r[0] : r[1]));
  }
  if (off == 8)  // rotation by 8 within each row of 16 lanes = lane ^ 8
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, b, 0x128, 0xF, 0xF, true));
  return __shfl_xor(x, off);
}

// The state of the lane `off` places away (lane ^ off).
__device__ __forceinline__ State partner(const State &x, int off) {
  State o;
  o.m = xchg(x.m, off);
  o.s = xchg(x.s, off);
  o.acc.x = xchg(x.acc.x, off);
  o.acc.y = xchg(x.acc.y, off);
  o.acc.z = xchg(x.acc.z, off);
  o.acc.w = xchg(x.acc.w, off);
  return o;
}

// Exact merge of two states (weights exp(m_i - max), 0 for an empty state).
__device__ __forceinline__ void merge(float &m, float &s, float4 &acc,
                                      const State &o) {
  const float mn = fmaxf(m, o.m);
  const float c1 = weight(m, mn);
  const float c2 = weight(o.m, mn);
  s = s * c1 + o.s * c2;
  acc.x = acc.x * c1 + o.acc.x * c2;
  acc.y = acc.y * c1 + o.acc.y * c2;
  acc.z = acc.z * c1 + o.acc.z * c2;
  acc.w = acc.w * c1 + o.acc.w * c2;
  m = mn;
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

  const int h = blockIdx.x;
  const int d_base = blockIdx.y * DC;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int c = tid % C;
  const int g0 = tid / C;
  // The output sums of this (sequence, head), one record every n_head * HD
  // floats, and its headers, 4 floats apart, each through one raw buffer
  // view based at the first record: the per-record offsets are 32-bit (the
  // host keeps a sequence's records below 2 GiB), with no 64-bit address
  // arithmetic per load (28q hd128 at 32K rows, 128 splits: 3.21 against
  // 3.28-3.33 us).
  const float *obase =
      a.partials + ((size_t)b * a.n_splits * a.n_head + h) * HD;
  const float *hbase =
      a.headers + ((size_t)b * a.n_head + h) * a.n_splits * 4;
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(obase), (short)0, 0x7FFFFFFF, 0x00020000);
  const __amdgpu_buffer_rsrc_t hb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(hbase), (short)0, 0x7FFFFFFF, 0x00020000);
  const uint32_t rbytes = (uint32_t)((size_t)a.n_head * HD * sizeof(float));
  const uint32_t dofs = (uint32_t)(d_base + 4 * c) * 4u;

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
        const auto h2 = __builtin_amdgcn_raw_buffer_load_b64(
            hb, (int)(16u * (uint32_t)sp), 0, 0);
        const auto o4 = __builtin_amdgcn_raw_buffer_load_b128(
            rb, (int)((uint32_t)sp * rbytes + dofs), 0, 0);
        hdr[u] = make_float2(__builtin_bit_cast(float, (unsigned)h2[0]),
                             __builtin_bit_cast(float, (unsigned)h2[1]));
        oc[u] = make_float4(__builtin_bit_cast(float, (unsigned)o4[0]),
                            __builtin_bit_cast(float, (unsigned)o4[1]),
                            __builtin_bit_cast(float, (unsigned)o4[2]),
                            __builtin_bit_cast(float, (unsigned)o4[3]));
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

  // Merge the NG record groups: first across the groups of each wave with
  // lane exchanges (groups are C lanes apart), then across the waves through
  // LDS. Every lane of a group holds the same (m, s).
#pragma unroll
  for (int off = C; off < 64; off <<= 1) {
    State o = partner(State{m, s, acc}, off);
    merge(m, s, acc, o);
  }
  constexpr int kW = kThreads / 64;
  __shared__ float sm_m[kW];
  __shared__ float sm_s[kW];
  __shared__ float4 sm_acc[kW][C];
  const int wave = tid >> 6;
  const int lane = tid & 63;
  if (lane < C) {
    sm_acc[wave][lane] = acc;
    if (lane == 0) {
      sm_m[wave] = m;
      sm_s[wave] = s;
    }
  }
  __syncthreads();
  if (tid < C) {
    float gm = neg_inf();
#pragma unroll
    for (int w = 0; w < kW; ++w) gm = fmaxf(gm, sm_m[w]);
    float st = 0.0f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const float wt = weight(sm_m[w], gm);
      st = fmaf(wt, sm_s[w], st);
      const float4 x = sm_acc[w][tid];
      o.x = fmaf(wt, x.x, o.x);
      o.y = fmaf(wt, x.y, o.y);
      o.z = fmaf(wt, x.z, o.z);
      o.w = fmaf(wt, x.w, o.w);
    }
    float4 r;
    r.x = (st > 0.0f) ? o.x / st : 0.0f;
    r.y = (st > 0.0f) ? o.y / st : 0.0f;
    r.z = (st > 0.0f) ? o.z / st : 0.0f;
    r.w = (st > 0.0f) ? o.w / st : 0.0f;
    *reinterpret_cast<float4 *>(
        &a.out[((size_t)b * a.n_head + h) * HD + d_base + 4 * tid]) = r;
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
