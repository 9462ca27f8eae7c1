// splitkv_host.hip -- the C ABI of libsplitkv.so (declared in
// include/splitkv.h and include/splitkv_probe.h): argument validation, shape
// dispatch, the split heuristic and the launches. Validation is pure host code
// and runs before any HIP call, so every error path can be exercised on a
// machine without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <climits>
#include <cmath>
#include <mutex>

#include "splitkv.h"
#include "splitkv_internal.h"
#include "splitkv_probe.h"

// Scratch of splitkv_decode_attn_noalloc: the split records of one call live
// here instead of in a caller buffer. Every device that runs the library holds
// its own copy (allocated when the code object is loaded, kept until the
// process ends). In host code `scratch` names a host-side stand-in, not
// device memory: kernels get the address that hipGetSymbolAddress returns for
// the current device, resolved once per device and cached below.
static __device__ __align__(256) float
    scratch[SPLITKV_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr double kLog2e = 1.44269504088896340736;
constexpr int kMaxSplits = 65535;
constexpr int kMaxGridYZ = 65535;

bool aligned(const void *p, uintptr_t n) {
  return (reinterpret_cast<uintptr_t>(p) % n) == 0;
}

int check_shape(int batch, int n_head, int n_kv_head, int head_dim,
                int max_ctx, int n_splits, int block_len) {
  if (batch < 1 || n_head < 1 || n_kv_head < 1 || max_ctx < 1 ||
      n_splits < 1 || block_len < 0)
    return SPLITKV_EINVAL;
  if (n_head % n_kv_head != 0) return SPLITKV_EINVAL;
  if (!splitkv::head_dim_supported(head_dim)) return SPLITKV_EUNSUPPORTED;
  if (n_head / n_kv_head > splitkv::kMaxGroup) return SPLITKV_EUNSUPPORTED;
  if (n_splits > kMaxSplits || n_kv_head > kMaxGridYZ || batch > kMaxGridYZ)
    return SPLITKV_EINVAL;
  if ((long long)max_ctx + n_splits >= (long long)INT_MAX) return SPLITKV_EINVAL;
  // A sequence's K (or V) cache, plus one tile of rows past its end, must
  // stay below 4 GiB: the kernels address it with 32-bit byte offsets.
  if (((long long)max_ctx + 64) * n_kv_head * head_dim * 2 >= (1LL << 32))
    return SPLITKV_EINVAL;
  if (block_len > 0) {
    // The fixed-length rule must reach every position the cache can hold.
    if ((long long)block_len * n_splits < max_ctx) return SPLITKV_EINVAL;
    if ((long long)block_len * n_splits > (long long)INT_MAX)
      return SPLITKV_EINVAL;
  }
  return SPLITKV_OK;
}

int check_combine_shape(int batch, int n_head, int head_dim, int n_splits) {
  if (batch < 1 || n_head < 1 || n_splits < 1) return SPLITKV_EINVAL;
  if (!splitkv::head_dim_supported(head_dim)) return SPLITKV_EUNSUPPORTED;
  if (n_splits > kMaxSplits || n_head > kMaxGridYZ || batch > kMaxGridYZ)
    return SPLITKV_EINVAL;
  // The combine addresses one sequence's records with 32-bit byte offsets.
  if ((long long)n_splits * n_head * (4 + head_dim) * 4 > (long long)INT_MAX)
    return SPLITKV_EINVAL;
  return SPLITKV_OK;
}

int check_partial(const float *q, const uint16_t *k, const uint16_t *v,
                  const int32_t *positions, const float *partials, int batch,
                  int n_head, int n_kv_head, int head_dim, int max_ctx,
                  int n_splits, int block_len, float scale) {
  if (!q || !k || !v || !positions || !partials) return SPLITKV_EINVAL;
  const int st = check_shape(batch, n_head, n_kv_head, head_dim, max_ctx,
                             n_splits, block_len);
  if (st != SPLITKV_OK) return st;
  if (!std::isfinite(scale)) return SPLITKV_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) ||
      !aligned(partials, 16) || !aligned(positions, 4))
    return SPLITKV_EALIGN;
  return SPLITKV_OK;
}

int check_combine(const float *partials, const float *out, int batch,
                  int n_head, int head_dim, int n_splits) {
  if (!partials || !out) return SPLITKV_EINVAL;
  const int st = check_combine_shape(batch, n_head, head_dim, n_splits);
  if (st != SPLITKV_OK) return st;
  if (!aligned(partials, 16) || !aligned(out, 16)) return SPLITKV_EALIGN;
  return SPLITKV_OK;
}

// The records buffer holds the output sums of every record first
// ([batch][n_splits][rec_heads][head_dim]), then their 4-float headers
// ([batch][rec_heads][n_splits][4]); rec_heads = n_q * n_head.
template <typename T>
T *headers_of(T *partials, int batch, int rec_heads, int head_dim,
              int n_splits) {
  return partials +
         (size_t)batch * n_splits * rec_heads * (size_t)head_dim;
}

int do_partial(const float *q, const uint16_t *k, const uint16_t *v,
               const int32_t *positions, float *partials, int batch,
               int n_head, int n_kv_head, int head_dim, int max_ctx,
               int n_splits, int block_len, float scale, void *stream,
               bool per_head = false, int n_q = 1,
               const float *k_new = nullptr, const float *v_new = nullptr,
               uint16_t *k_app = nullptr, uint16_t *v_app = nullptr) {
  splitkv::PartialArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.positions = positions;
  a.partials = partials;
  a.headers = headers_of(partials, batch, n_q * n_head, head_dim, n_splits);
  a.n_head = n_head;
  a.n_kv_head = n_kv_head;
  a.max_ctx = max_ctx;
  a.n_splits = n_splits;
  a.block_len = block_len;
  a.scale_log2 = (float)((double)scale * kLog2e);
  a.kv_group = n_head / n_kv_head;
  a.n_q = n_q;
  a.pair_rows = 0;  // chosen by the several-row launcher
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_app = k_app;
  a.v_app = v_app;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      per_head ? splitkv::launch_partial_per_head(head_dim, a, batch, s)
               : splitkv::launch_partial(head_dim, n_head / n_kv_head, a,
                                         batch, s);
  return e == hipSuccess ? SPLITKV_OK : SPLITKV_ELAUNCH;
}

constexpr size_t kScratchBytes = SPLITKV_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::atomic<float *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (first call on a device: one
// hipGetSymbolAddress with that device current).
int scratch_on_current_device(float **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SPLITKV_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return SPLITKV_EUNSUPPORTED;
  float *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void *addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess ||
          addr == nullptr)
        return SPLITKV_ELAUNCH;
      p = static_cast<float *>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SPLITKV_OK;
}

int do_combine(const float *partials, float *out, int batch, int n_head,
               int head_dim, int n_splits, void *stream) {
  splitkv::CombineArgs a;
  a.partials = partials;
  a.headers = headers_of(partials, batch, n_head, head_dim, n_splits);
  a.out = out;
  a.n_head = n_head;
  a.n_splits = n_splits;
  const hipError_t e = splitkv::launch_combine(
      head_dim, a, batch, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SPLITKV_OK : SPLITKV_ELAUNCH;
}

}  // namespace

extern "C" {

int splitkv_abi_version(void) { return SPLITKV_ABI_VERSION; }

const char *splitkv_strerror(int status) {
  switch (status) {
    case SPLITKV_OK: return "ok";
    case SPLITKV_EINVAL: return "invalid argument";
    case SPLITKV_EUNSUPPORTED: return "unsupported head_dim or group size";
    case SPLITKV_EALIGN: return "misaligned pointer";
    case SPLITKV_ELAUNCH: return "kernel launch failed";
    case SPLITKV_ESCRATCH:
      return "split records exceed the allocation-free entry point's scratch";
    default: return "unknown status";
  }
}

size_t splitkv_partials_bytes(int batch, int n_head, int head_dim,
                              int n_splits) {
  if (batch < 1 || n_head < 1 || head_dim < 1 || n_splits < 1) return 0;
  return (size_t)batch * (size_t)n_splits * (size_t)n_head *
         (size_t)(4 + head_dim) * sizeof(float);
}

int splitkv_workgroups_per_cu(int head_dim, int group) {
  if (!splitkv::head_dim_supported(head_dim) || group < 1 ||
      group > splitkv::kMaxGroup)
    return 0;
  // From the compiler's resource report of each instantiation: waves per
  // SIMD x 4 SIMDs / waves per workgroup, and no more than the LDS of a
  // compute unit holds (160 KiB; the head_dim-256 kernel runs 8-wave
  // workgroups of 143 KB: one per unit); a build check keeps this table
  // equal to the report.
  switch (head_dim) {
    case 8: { static const int t[8] = {4, 4, 3, 3, 2, 2, 2, 2}; return t[group - 1]; }
    case 16: { static const int t[8] = {4, 3, 3, 2, 2, 2, 2, 1}; return t[group - 1]; }
    case 32: { static const int t[8] = {4, 3, 3, 2, 2, 2, 2, 1}; return t[group - 1]; }
    case 64: return 7;
    case 128: return 4;
    case 256: return 1;
    default: return 0;
  }
}

int splitkv_pick_splits(int batch, int n_head, int n_kv_head, int head_dim,
                        int max_ctx, int cu_count, int *n_splits,
                        int *block_len) {
  return splitkv_pick_splits_rows(batch, 1, n_head, n_kv_head, head_dim,
                                  max_ctx, cu_count, n_splits, block_len);
}

int splitkv_pick_splits_rows(int batch, int n_q, int n_head, int n_kv_head,
                             int head_dim, int max_ctx, int cu_count,
                             int *n_splits, int *block_len) {
  if (!n_splits || !block_len || cu_count < 1 || n_q < 1) return SPLITKV_EINVAL;
  const int st =
      check_shape(batch, n_head, n_kv_head, head_dim, max_ctx, 1, 0);
  if (st != SPLITKV_OK) return st;
  const int group = n_head / n_kv_head;
  // Workgroups per split: one per (KV head, sequence, block of rows that
  // share a workgroup's MFMA columns). The rows of one sequence have about
  // the same length, so only several sequences call for the balancing rule.
  const int rows = head_dim >= 64
                       ? splitkv::rows_per_workgroup(head_dim, group, n_q)
                       : 1;
  const long long units =
      (long long)batch * ((n_q + rows - 1) / rows) * n_kv_head;
  long long wpc = splitkv_workgroups_per_cu(head_dim, group);
  // The matrix-core kernel (head_dim >= 64): at most 256 / head_dim resident
  // workgroups per compute unit (2 at hd 128). Each wave keeps one 16-row
  // K/V tile in flight, 16 x 4*head_dim bytes; more resident workgroups
  // measured slower (at 32K rows, 192 splits at the full occupancy took
  // 18.1 us per layer against 17.1 at 128): they only add per-split fixed
  // costs (query load, merge, records) and deeper memory queues.
  if (head_dim >= 64 && wpc > 256 / head_dim) wpc = 256 / head_dim;
  // One full round of resident workgroups. With one sequence every split
  // has the same work, so a single round is best; a few workgroups past it
  // would cost a whole second round, hence the floor.
  long long s = wpc * cu_count / units;
  // With 8-wave workgroups (head_dim 256) a split of up to 8 tiles (128
  // rows) is computed in one round of its waves; more splits than the
  // full-length rows need for that add records (a longer combine) and
  // per-split fixed costs, not parallelism the memory system can use
  // (16q/2kv, max_ctx 8,400: 66 splits 10.77 against 11.08 us per layer at
  // 128 at the full length, 8.12 against 8.70 at 1,024 rows; 0.05-0.12 us
  // slower at 2,048-4,096 rows, 0.05 faster at 6,000).
  if (head_dim >= 256) {
    const long long fit = ((long long)max_ctx + 127) / 128;
    if (s > fit) s = fit;
  }
  // With several sequences the lengths can differ and the host does not see
  // them: about 16 workgroups per compute unit let the dispatcher balance
  // the load, as long as a full-length split still has ~1024 rows to
  // amortise its fixed costs (query load, merge, record store).
  const long long bal = (16LL * cu_count + units - 1) / units;
  const long long bal_cap = max_ctx / 1024;
  const long long s_bal = bal < bal_cap ? bal : bal_cap;
  if (batch > 1 && s_bal > s) s = s_bal;
  if (s < 1) s = 1;
  // A full-length split keeps at least 32 rows (one wave's tile).
  const long long cap = max_ctx / 32 > 1 ? max_ctx / 32 : 1;
  if (s > cap) s = cap;
  if (s > kMaxSplits) s = kMaxSplits;
  *n_splits = (int)s;
  *block_len = 0;
  return SPLITKV_OK;
}

int splitkv_partial(const float *q, const uint16_t *k_cache,
                    const uint16_t *v_cache, const int32_t *positions,
                    float *partials, int batch, int n_head, int n_kv_head,
                    int head_dim, int max_ctx, int n_splits, int block_len,
                    float scale, void *stream) {
  const int st = check_partial(q, k_cache, v_cache, positions, partials, batch,
                               n_head, n_kv_head, head_dim, max_ctx, n_splits,
                               block_len, scale);
  if (st != SPLITKV_OK) return st;
  return do_partial(q, k_cache, v_cache, positions, partials, batch, n_head,
                    n_kv_head, head_dim, max_ctx, n_splits, block_len, scale,
                    stream);
}

int splitkv_combine(const float *partials, float *out, int batch, int n_head,
                    int head_dim, int n_splits, void *stream) {
  const int st =
      check_combine(partials, out, batch, n_head, head_dim, n_splits);
  if (st != SPLITKV_OK) return st;
  return do_combine(partials, out, batch, n_head, head_dim, n_splits, stream);
}

int splitkv_decode_attn(const float *q, const uint16_t *k_cache,
                        const uint16_t *v_cache, const int32_t *positions,
                        float *partials, float *out, int batch, int n_head,
                        int n_kv_head, int head_dim, int max_ctx, int n_splits,
                        int block_len, float scale, void *stream) {
  int st = check_partial(q, k_cache, v_cache, positions, partials, batch,
                         n_head, n_kv_head, head_dim, max_ctx, n_splits,
                         block_len, scale);
  if (st != SPLITKV_OK) return st;
  st = check_combine(partials, out, batch, n_head, head_dim, n_splits);
  if (st != SPLITKV_OK) return st;
  st = do_partial(q, k_cache, v_cache, positions, partials, batch, n_head,
                  n_kv_head, head_dim, max_ctx, n_splits, block_len, scale,
                  stream);
  if (st != SPLITKV_OK) return st;
  return do_combine(partials, out, batch, n_head, head_dim, n_splits, stream);
}

int splitkv_decode_attn_noalloc(const float *q, const uint16_t *k_cache,
                                const uint16_t *v_cache,
                                const int32_t *positions, float *out, int batch,
                                int n_head, int n_kv_head, int head_dim,
                                int max_ctx, int n_splits, int block_len,
                                float scale, void *stream) {
  if (!q || !k_cache || !v_cache || !positions || !out) return SPLITKV_EINVAL;
  int st = check_shape(batch, n_head, n_kv_head, head_dim, max_ctx, n_splits,
                       block_len);
  if (st != SPLITKV_OK) return st;
  st = check_combine_shape(batch, n_head, head_dim, n_splits);
  if (st != SPLITKV_OK) return st;
  if (!std::isfinite(scale)) return SPLITKV_EINVAL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, 16) || !aligned(positions, 4))
    return SPLITKV_EALIGN;
  if (splitkv_partials_bytes(batch, n_head, head_dim, n_splits) > kScratchBytes)
    return SPLITKV_ESCRATCH;
  float *recs = nullptr;
  st = scratch_on_current_device(&recs);
  if (st != SPLITKV_OK) return st;
  // The partial kernel writes every record of the call (idle splits too), so
  // nothing left in the scratch by an earlier call is read.
  st = do_partial(q, k_cache, v_cache, positions, recs, batch, n_head,
                  n_kv_head, head_dim, max_ctx, n_splits, block_len, scale,
                  stream);
  if (st != SPLITKV_OK) return st;
  return do_combine(recs, out, batch, n_head, head_dim, n_splits, stream);
}

int splitkv_partial_rows(const float *q, const uint16_t *k_cache,
                         const uint16_t *v_cache, const int32_t *positions,
                         float *partials, int batch, int n_q, int n_head,
                         int n_kv_head, int head_dim, int max_ctx, int n_splits,
                         int block_len, float scale, void *stream) {
  const int st = check_partial(q, k_cache, v_cache, positions, partials, batch,
                               n_head, n_kv_head, head_dim, max_ctx, n_splits,
                               block_len, scale);
  if (st != SPLITKV_OK) return st;
  if (n_q < 1 || (long long)batch * n_q > kMaxGridYZ ||
      (long long)n_q * n_head > kMaxGridYZ)
    return SPLITKV_EINVAL;
  return do_partial(q, k_cache, v_cache, positions, partials, batch, n_head,
                    n_kv_head, head_dim, max_ctx, n_splits, block_len, scale,
                    stream, false, n_q);
}

int splitkv_decode_attn_rows(const float *q, const uint16_t *k_cache,
                             const uint16_t *v_cache, const int32_t *positions,
                             float *partials, float *out, int batch, int n_q,
                             int n_head, int n_kv_head, int head_dim,
                             int max_ctx, int n_splits, int block_len,
                             float scale, void *stream) {
  int st = check_partial(q, k_cache, v_cache, positions, partials, batch,
                         n_head, n_kv_head, head_dim, max_ctx, n_splits,
                         block_len, scale);
  if (st != SPLITKV_OK) return st;
  if (n_q < 1 || (long long)batch * n_q > kMaxGridYZ ||
      (long long)n_q * n_head > kMaxGridYZ)
    return SPLITKV_EINVAL;
  st = check_combine(partials, out, batch, n_q * n_head, head_dim, n_splits);
  if (st != SPLITKV_OK) return st;
  st = do_partial(q, k_cache, v_cache, positions, partials, batch, n_head,
                  n_kv_head, head_dim, max_ctx, n_splits, block_len, scale,
                  stream, false, n_q);
  if (st != SPLITKV_OK) return st;
  return do_combine(partials, out, batch, n_q * n_head, head_dim, n_splits,
                    stream);
}

int splitkv_partial_per_head(const float *q, const uint16_t *k_cache,
                             const uint16_t *v_cache, const int32_t *positions,
                             float *partials, int batch, int n_head,
                             int n_kv_head, int head_dim, int max_ctx,
                             int n_splits, int block_len, float scale,
                             void *stream) {
  const int st = check_partial(q, k_cache, v_cache, positions, partials, batch,
                               n_head, n_kv_head, head_dim, max_ctx, n_splits,
                               block_len, scale);
  if (st != SPLITKV_OK) return st;
  if (head_dim < 64) return SPLITKV_EUNSUPPORTED;   // matrix-core family only
  if (n_head > kMaxGridYZ) return SPLITKV_EINVAL;
  return do_partial(q, k_cache, v_cache, positions, partials, batch, n_head,
                    n_kv_head, head_dim, max_ctx, n_splits, block_len, scale,
                    stream, true);
}

int splitkv_append_kv(const float *k_new, const float *v_new,
                      uint16_t *k_cache, uint16_t *v_cache,
                      const int32_t *positions, int batch, int n_rows,
                      int n_kv_head, int head_dim, int max_ctx, void *stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !positions)
    return SPLITKV_EINVAL;
  if (batch < 1 || n_rows < 1 || n_kv_head < 1 || max_ctx < 1)
    return SPLITKV_EINVAL;
  if (!splitkv::head_dim_supported(head_dim)) return SPLITKV_EUNSUPPORTED;
  if (batch > kMaxGridYZ || n_rows > kMaxGridYZ || n_kv_head > kMaxGridYZ)
    return SPLITKV_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(positions, 4))
    return SPLITKV_EALIGN;
  splitkv::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.positions = positions;
  a.n_rows = n_rows;
  a.row_elems = n_kv_head * head_dim;
  a.max_ctx = max_ctx;
  return splitkv::launch_append(a, batch, static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? SPLITKV_OK
             : SPLITKV_ELAUNCH;
}

int splitkv_decode_step(const float *q, const float *k_new, const float *v_new,
                        uint16_t *k_cache, uint16_t *v_cache,
                        const int32_t *positions, float *partials, float *out,
                        int batch, int n_head, int n_kv_head, int head_dim,
                        int max_ctx, int n_splits, int block_len, float scale,
                        void *stream) {
  int st = check_partial(q, k_cache, v_cache, positions, partials, batch,
                         n_head, n_kv_head, head_dim, max_ctx, n_splits,
                         block_len, scale);
  if (st != SPLITKV_OK) return st;
  st = check_combine(partials, out, batch, n_head, head_dim, n_splits);
  if (st != SPLITKV_OK) return st;
  if (!k_new || !v_new) return SPLITKV_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return SPLITKV_EALIGN;
  if (head_dim >= 64) {
    // matrix-core kernel: the append is folded into the partial kernel
    st = do_partial(q, k_cache, v_cache, positions, partials, batch, n_head,
                    n_kv_head, head_dim, max_ctx, n_splits, block_len, scale,
                    stream, false, 1, k_new, v_new, k_cache, v_cache);
  } else {
    st = splitkv_append_kv(k_new, v_new, k_cache, v_cache, positions, batch, 1,
                           n_kv_head, head_dim, max_ctx, stream);
    if (st != SPLITKV_OK) return st;
    st = do_partial(q, k_cache, v_cache, positions, partials, batch, n_head,
                    n_kv_head, head_dim, max_ctx, n_splits, block_len, scale,
                    stream);
  }
  if (st != SPLITKV_OK) return st;
  return do_combine(partials, out, batch, n_head, head_dim, n_splits, stream);
}

int splitkv_probe_read(const void *buf, size_t bytes, uint32_t *sink,
                       int grid, void *stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || grid < 1 ||
      grid > (1 << 20))
    return SPLITKV_EINVAL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return SPLITKV_EALIGN;
  return splitkv::launch_probe_read(buf, bytes, sink, grid,
                                    static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? SPLITKV_OK
             : SPLITKV_ELAUNCH;
}

int splitkv_probe_copy(const void *src, void *dst, size_t bytes, int grid,
                       void *stream) {
  if (!src || !dst || bytes == 0 || bytes % 16 != 0 || grid < 1 ||
      grid > (1 << 20))
    return SPLITKV_EINVAL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return SPLITKV_EALIGN;
  const uintptr_t s = reinterpret_cast<uintptr_t>(src);
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst);
  if (s < d + bytes && d < s + bytes) return SPLITKV_EINVAL;  // overlap
  return splitkv::launch_probe_copy(src, dst, bytes, grid,
                                    static_cast<hipStream_t>(stream)) ==
                 hipSuccess
             ? SPLITKV_OK
             : SPLITKV_ELAUNCH;
}

}  // extern "C"
