// Expert-parallel MoE shard (kernels not built yet: the entry point reports
// MP_ERR_UNSUPPORTED).
#include "common.h"

extern "C" size_t mp_grouped_expert_gemm_workspace(int64_t, int64_t, int64_t, int, int) { return 0; }

extern "C" int mp_grouped_expert_gemm(int64_t, int64_t, int64_t, int, int, int, const void*, const int32_t*,
                                      const float*, const void*, const void*, void*, int32_t*, int32_t*, void*, size_t,
                                      hipStream_t) {
  return mp::fail(MP_ERR_UNSUPPORTED, "mp_grouped_expert_gemm: not implemented");
}
