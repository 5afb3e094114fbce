// attn_bwd -- gradients of exact softmax attention, recomputing P from the saved lse.
#include "common.h"
#include "internal.h"

namespace ra {

size_t bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Sq) {
  const size_t n = (size_t)(B * Hq * Sq) * sizeof(float);
  return (n + 255) / 256 * 256;
}

int launch_attn_bwd(const BwdArgs &, int, int, hipStream_t) { return RA_ERR_UNSUPPORTED; }

}  // namespace ra
