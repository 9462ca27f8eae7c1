// splitkv_append.hip -- KV-cache append kernel (gfx950).
//
// dotLLM issue #199, comment 1, section 1 (the cache update that comes ahead
// of attention in a decode step): the step's freshly projected key and value
// rows are converted to half precision and stored at their positions, and
// only then do the attention kernels read the cache. Row
// t of the n_rows new rows of sequence b goes to position
//   p = positions[b] - (n_rows - 1) + t,
// so the last new row sits at positions[b] and the live length after the
// append is positions[b] + 1 -- the same positions[] array the attention
// kernels read. Rows with p outside [0, max_ctx) are not written. positions[]
// is read on the device, so a captured graph appends at the current length on
// every replay.
//
// The conversion is the hardware's fp32 -> fp16 (round to nearest even under
// the default rounding mode, fp16 subnormals kept, overflow to infinity).
//
// Grid dim3(ceil(row/(8*64)), n_rows, batch), 64 threads: each thread takes 8
// consecutive elements of one new row (two 16-byte fp32 loads per cache) and
// stores them as one 16-byte fp16 store, for K and for V.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "splitkv_internal.h"

namespace splitkv {
namespace {

constexpr int kAppendThreads = 64;

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 a = (_Float16)lo;
  const _Float16 b = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ uint4 to_f16x8(const float4 x, const float4 y) {
  return make_uint4(pack_f16x2(x.x, x.y), pack_f16x2(x.z, x.w),
                    pack_f16x2(y.x, y.y), pack_f16x2(y.z, y.w));
}

__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const int t = blockIdx.y;
  const int b = blockIdx.z;
  const long long p =
      (long long)a.positions[b] - (long long)(a.n_rows - 1) + t;
  if (p < 0 || p >= a.max_ctx) return;
  const int row = a.row_elems;                     // n_kv_head * head_dim
  const int i = (blockIdx.x * kAppendThreads + threadIdx.x) * 8;
  if (i >= row) return;
  const size_t src = ((size_t)b * a.n_rows + t) * row + i;
  const size_t dst = ((size_t)b * a.max_ctx + (size_t)p) * row + i;
  const float4 *kn = reinterpret_cast<const float4 *>(a.k_new + src);
  const float4 *vn = reinterpret_cast<const float4 *>(a.v_new + src);
  const float4 k0 = kn[0], k1 = kn[1];
  const float4 v0 = vn[0], v1 = vn[1];
  *reinterpret_cast<uint4 *>(a.k_cache + dst) = to_f16x8(k0, k1);
  *reinterpret_cast<uint4 *>(a.v_cache + dst) = to_f16x8(v0, v1);
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, int batch, hipStream_t stream) {
  const int per_block = kAppendThreads * 8;
  const int gx = (a.row_elems + per_block - 1) / per_block;
  hipLaunchKernelGGL(append_kernel, dim3(gx, a.n_rows, batch),
                     dim3(kAppendThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace splitkv
