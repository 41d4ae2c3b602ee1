// Error reporting, version and the device-flag check of the C ABI.
#include "common.h"

#include <stdarg.h>
#include <stdio.h>

namespace nc {

namespace {
thread_local char g_err[512] = "";
}

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(NC_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return NC_OK;
}

}  // namespace nc

extern "C" const char* nc_last_error(void) { return nc::g_err; }

extern "C" const char* nc_version(void) { return "libnc 0.1.0 (gfx950)"; }

extern "C" int nc_sync_status(const int32_t* flag, void* stream) {
  NC_REQUIRE(flag, NC_ERR_INVALID_ARG, "sync_status: null flag");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t h = 0;
  NC_CHECK_HIP(hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, s));
  NC_CHECK_HIP(hipStreamSynchronize(s));
  if (h != 0) return nc::set_error(NC_ERR_DEVICE_FLAG, "device flag raised: a token id was outside [0, V)");
  return NC_OK;
}
