// splitkv_combine.hip -- combine kernel of split-KV decode attention (gfx950).
//
// One workgroup (4 waves) per (query head, sequence), grid dim3(n_head,
// batch). It merges the split records exactly as "10 · R4 — decode
// split-attention dim-parallel rewrite", section 2.1 defines the combine:
//   gmx = max over splits of mx,  w = exp(mx - gmx),
//   S = sum w*S_sp,  acc = sum w*oc_sp,  o = acc / S  (0 when S <= 0).
// A record with mx = -inf (an idle split) gets weight exactly 0, also when all
// records are idle and gmx itself is -inf.
// Work split: the records are spread over the workgroup (each lane holds
// max(1, HD/64) dims of a record, so one wave reads 64/lanes-per-record
// records per pass, 16-byte or smaller contiguous reads); the per-lane partial
// sums are merged through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitkv_internal.h"

namespace splitkv {
namespace {

constexpr int kThreads = 256;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

template <int HD>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  constexpr int DPL = HD >= 64 ? HD / 64 : 1;  // dims per lane
  constexpr int LPR = HD / DPL;                // lanes per record
  constexpr int RPB = kThreads / LPR;          // records per pass
  constexpr size_t pstr = 4 + HD;

  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const size_t rstride = (size_t)a.n_head * pstr;
  const float *base =
      a.partials + ((size_t)b * a.n_splits * a.n_head + h) * pstr;

  // Global max over the split records.
  __shared__ float sm_red[kThreads / 64];
  float m = neg_inf();
  for (int sp = tid; sp < a.n_splits; sp += kThreads)
    m = fmaxf(m, base[(size_t)sp * rstride]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) sm_red[tid >> 6] = m;
  __syncthreads();
  float gmx = sm_red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) gmx = fmaxf(gmx, sm_red[w]);

  // Weighted sums.
  const int rsub = tid / LPR;
  const int d0 = (tid % LPR) * DPL;
  float acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) acc[i] = 0.0f;
  float ssum = 0.0f;
  for (int sp = rsub; sp < a.n_splits; sp += RPB) {
    const float *r = base + (size_t)sp * rstride;
    const float mxs = r[0];
    const float w = (mxs == neg_inf())
                        ? 0.0f
                        : __builtin_amdgcn_exp2f((mxs - gmx) * kLog2e);
    ssum = fmaf(w, r[1], ssum);
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = fmaf(w, r[4 + d0 + i], acc[i]);
  }

  __shared__ float sm_acc[RPB][HD];
  __shared__ float sm_s[RPB];
#pragma unroll
  for (int i = 0; i < DPL; ++i) sm_acc[rsub][d0 + i] = acc[i];
  if (tid % LPR == 0) sm_s[rsub] = ssum;
  __syncthreads();

  for (int d = tid; d < HD; d += kThreads) {
    float s = 0.0f, o = 0.0f;
    for (int r = 0; r < RPB; ++r) {
      s += sm_s[r];
      o += sm_acc[r][d];
    }
    a.out[((size_t)b * a.n_head + h) * HD + d] = (s > 0.0f) ? o / s : 0.0f;
  }
}

template <int HD>
hipError_t launch_one(const CombineArgs &a, int batch, hipStream_t stream) {
  hipLaunchKernelGGL((combine_kernel<HD>), dim3(a.n_head, batch),
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
