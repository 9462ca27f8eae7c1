// splitkv_partial.hip -- picks the partial kernel family by head_dim: the
// matrix-core kernel where a row holds whole 32-dim MFMA steps (64, 128, 256),
// the vector-ALU kernel for the small head dims (8, 16, 32).
#include <hip/hip_runtime.h>

#include "splitkv_internal.h"
#include "splitkv_partial_common.h"

namespace splitkv {

hipError_t launch_partial(int head_dim, int group, const PartialArgs &a,
                          int batch, hipStream_t stream) {
  if (head_dim >= 64) return launch_partial_mfma(head_dim, group, a, batch, stream);
  return launch_partial_valu(head_dim, group, a, batch, stream);
}

}  // namespace splitkv
