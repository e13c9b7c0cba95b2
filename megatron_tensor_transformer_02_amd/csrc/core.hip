// Status reporting, version and device checks of libmp.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "common.h"

namespace mp {

static thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() { return MP_OK; }

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MP_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return MP_OK;
}

static bool debug_checks_on() {
  const char* v = getenv("MP_DEBUG_CHECKS");
  return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
}

int debug_check_range(const char* fn, const char* what, const int32_t* idx, int64_t n, int64_t lo, int64_t hi,
                      hipStream_t s) {
  if (!debug_checks_on() || n <= 0 || idx == nullptr) return MP_OK;
  std::vector<int32_t> host(static_cast<size_t>(n));
  hipError_t e = hipMemcpyAsync(host.data(), idx, static_cast<size_t>(n) * sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return fail(MP_ERR_HIP, "%s: debug check of %s: %s", fn, what, hipGetErrorString(e));
  for (int64_t i = 0; i < n; ++i)
    if (host[i] < lo || host[i] >= hi)
      return fail(MP_ERR_DATA, "%s: %s[%lld] = %d lies outside [%lld, %lld)", fn, what, (long long)i, host[i],
                  (long long)lo, (long long)hi);
  return MP_OK;
}

__global__ void count_zero_kernel(unsigned long long* count) {
  if (threadIdx.x == 0) *count = 0;
}

// Counts idx[i] outside [lo, hi): per-thread counts over a grid-stride loop,
// a block sum in LDS, one integer atomic add per block (exact in any order).
__global__ __launch_bounds__(256) void count_outside_kernel(const int32_t* __restrict__ idx, int64_t n, int64_t lo,
                                                            int64_t hi, unsigned long long* count) {
  __shared__ unsigned int part[256];
  unsigned int c = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t v = idx[i];
    c += (v < lo || v >= hi) ? 1u : 0u;
  }
  part[threadIdx.x] = c;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0 && part[0] != 0) atomicAdd(count, static_cast<unsigned long long>(part[0]));
}

}  // namespace mp

extern "C" int mp_check_indices(const int32_t* idx, int64_t n, int64_t lo, int64_t hi, uint64_t* bad_count,
                                hipStream_t s) {
  static const char* fn = "mp_check_indices";
  MP_REQUIRE(n >= 0 && lo <= hi, MP_ERR_SHAPE, "%s: n=%lld, [lo, hi) = [%lld, %lld)", fn, (long long)n,
             (long long)lo, (long long)hi);
  MP_REQUIRE(n == 0 || idx != nullptr, MP_ERR_NULL, "%s: idx is NULL", fn);
  MP_REQUIRE_PTR(bad_count);
  MP_REQUIRE((reinterpret_cast<uintptr_t>(bad_count) & 7u) == 0, MP_ERR_ALIGN, "%s: bad_count is not 8-byte aligned",
             fn);
  auto* c = reinterpret_cast<unsigned long long*>(bad_count);
  mp::count_zero_kernel<<<1, 64, 0, s>>>(c);
  if (n > 0) {
    const int64_t blocks = mp::ceil_div(n, 256);
    mp::count_outside_kernel<<<static_cast<unsigned>(blocks < 1024 ? blocks : 1024), 256, 0, s>>>(idx, n, lo, hi, c);
  }
  return mp::check_launch(fn);
}

extern "C" int mp_version(void) { return 100; }  // 0.1.0

extern "C" const char* mp_last_error(void) { return mp::g_last_error; }

extern "C" int mp_device_supported(int device) {
  hipDeviceProp_t prop;
  const hipError_t e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return mp::fail(MP_ERR_HIP, "mp_device_supported: %s", hipGetErrorString(e));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return mp::fail(MP_ERR_UNSUPPORTED, "mp_device_supported: device %d is %s, not gfx950", device, prop.gcnArchName);
  return MP_OK;
}
