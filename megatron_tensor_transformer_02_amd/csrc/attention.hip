// Head-partitioned causal attention (kernels not built yet: the entry points
// report MP_ERR_UNSUPPORTED).
#include "common.h"

extern "C" int mp_head_attention(mp_dtype, int, int, int, int, int, int, const void*, const void*, const void*,
                                 void*, void*, float*, hipStream_t) {
  return mp::fail(MP_ERR_UNSUPPORTED, "mp_head_attention: not implemented");
}

extern "C" size_t mp_head_attention_bwd_workspace(mp_dtype, int, int, int, int, int) { return 0; }

extern "C" int mp_head_attention_bwd(mp_dtype, int, int, int, int, int, int, const void*, const void*, const void*,
                                     const void*, const float*, const void*, void*, float*, float*, void*, size_t,
                                     hipStream_t) {
  return mp::fail(MP_ERR_UNSUPPORTED, "mp_head_attention_bwd: not implemented");
}
