// Entry points whose kernels are not built yet: they reject every call.
#include "tsg_internal.hpp"

tsg_status tsg_op_moe(tsg_ctx* ctx, const void*, const int32_t*, const float*, const void*,
                      const void*, float*, int32_t*, int32_t*, void*, size_t, int, int, int, int,
                      int, const tsg_opts*, int, void*) {
  return tsgh::fail(ctx, TSG_E_UNSUPPORTED, "moe_expert_combine is not available in this build");
}
size_t tsg_moe_workspace(int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }
