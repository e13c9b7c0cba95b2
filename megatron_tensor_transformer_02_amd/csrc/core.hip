// Status reporting, version and device checks of libmp.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

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

}  // namespace mp

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
