// Fused gather -> GEMM-1 -> GEMM-2 -> combine (token-tile pipelined).
#include "moe_internal.h"

namespace moe {

size_t fused_ws_bytes(int T, int H, int E, int k, int I) {
  (void)T; (void)H; (void)E; (void)k; (void)I;
  return 256;
}

int fused_impl(const void*, const int32_t*, const int32_t*, const int32_t*, const float*,
               int, int, int, int, int, int, int, int, int, const void*, const void*,
               void*, void*, void*, void*, size_t, hipStream_t) {
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
