// Backward GroupedGEMM (placeholder until the backward kernels land).
#include "common.h"

namespace moe_launch {
size_t grouped_bwd_ws_bytes(int, int, int, int, int) { return 0; }
int grouped_bwd(const void*, const void*, const void*, const moe_weights*, const int32_t*, int,
                void*, float*, float*, float*, void*, hipStream_t) {
  return MOE_ERR_DTYPE;
}
}  // namespace moe_launch
