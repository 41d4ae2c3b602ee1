// Error reporting, version and the device-flag check of the C ABI.
#include "common.h"

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

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

bool debug_mode() {
  static const bool on = [] {
    const char* v = getenv("NC_DEBUG");
    return v != nullptr && v[0] == '1' && v[1] == '\0';
  }();
  return on;
}

int api_done(int rc, void* stream, const char* name) {
  if (rc != NC_OK || !debug_mode()) return rc;
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return set_error(NC_ERR_HIP, "%s: %s (found by the NC_DEBUG=1 check)", name, hipGetErrorString(e));
  return NC_OK;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(NC_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return NC_OK;
}

namespace {
struct Probe {
  std::mutex mu;
  std::atomic<int> family{NC_PROBE_OFF};
  std::vector<hipEvent_t> ev;  // 2 per launch
  int used = 0;                // pairs recorded
  int open = -1;               // pair whose end is pending
  int64_t dropped = 0;
  double flops = 0;
} g_probe;

void probe_release() {
  for (hipEvent_t e : g_probe.ev) (void)hipEventDestroy(e);
  g_probe.ev.clear();
  g_probe.used = 0;
  g_probe.open = -1;
  g_probe.dropped = 0;
  g_probe.flops = 0;
}
}  // namespace

// Whether launches of `family` are timed while the timer is armed for `armed`.
bool probe_match(int armed, int family) {
  if (family == NC_PROBE_OFF) return false;
  if (armed == family) return true;
  return armed == NC_PROBE_GEMM && (family == NC_PROBE_GEMM_WGRAD || family == NC_PROBE_GEMM_NT);
}

void probe_begin(int family, hipStream_t s) {
  if (!probe_match(g_probe.family.load(std::memory_order_relaxed), family)) return;
  std::lock_guard<std::mutex> lk(g_probe.mu);
  if (!probe_match(g_probe.family.load(), family)) return;
  if (2 * (g_probe.used + 1) > (int)g_probe.ev.size()) {
    ++g_probe.dropped;
    return;
  }
  g_probe.open = g_probe.used;
  (void)hipEventRecord(g_probe.ev[2 * g_probe.used], s);
}

void probe_end(int family, hipStream_t s, double flops) {
  if (!probe_match(g_probe.family.load(std::memory_order_relaxed), family)) return;
  std::lock_guard<std::mutex> lk(g_probe.mu);
  if (!probe_match(g_probe.family.load(), family) || g_probe.open != g_probe.used) return;
  (void)hipEventRecord(g_probe.ev[2 * g_probe.used + 1], s);
  g_probe.flops += flops;
  ++g_probe.used;
  g_probe.open = -1;
}

}  // namespace nc

extern "C" int nc_probe_start(int family, int max_launches) {
  NC_REQUIRE(family >= NC_PROBE_OFF && family <= NC_PROBE_GEMM, NC_ERR_INVALID_ARG, "probe: unknown family %d",
             family);
  NC_REQUIRE(max_launches >= 0 && max_launches <= (1 << 20), NC_ERR_INVALID_ARG, "probe: max_launches %d",
             max_launches);
  std::lock_guard<std::mutex> lk(nc::g_probe.mu);
  nc::g_probe.family.store(NC_PROBE_OFF);
  nc::probe_release();
  if (family == NC_PROBE_OFF) return NC_OK;
  nc::g_probe.ev.resize(2 * (size_t)max_launches);
  for (size_t i = 0; i < nc::g_probe.ev.size(); ++i) {
    const hipError_t e = hipEventCreate(&nc::g_probe.ev[i]);
    if (e != hipSuccess) {
      nc::g_probe.ev.resize(i);
      nc::probe_release();
      return nc::set_error(NC_ERR_HIP, "probe: hipEventCreate: %s", hipGetErrorString(e));
    }
  }
  nc::g_probe.family.store(family);
  return NC_OK;
}

extern "C" int nc_probe_stop(double* total_ms, int64_t* launches, double* flops) {
  NC_REQUIRE(total_ms && launches && flops, NC_ERR_INVALID_ARG, "probe: null output pointer");
  std::lock_guard<std::mutex> lk(nc::g_probe.mu);
  nc::g_probe.family.store(NC_PROBE_OFF);
  double ms = 0;
  int rc = NC_OK;
  for (int i = 0; i < nc::g_probe.used && rc == NC_OK; ++i) {
    float t = 0;
    hipError_t e = hipEventSynchronize(nc::g_probe.ev[2 * i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, nc::g_probe.ev[2 * i], nc::g_probe.ev[2 * i + 1]);
    if (e != hipSuccess) rc = nc::set_error(NC_ERR_HIP, "probe: event %d: %s", i, hipGetErrorString(e));
    ms += t;
  }
  *total_ms = ms;
  *launches = nc::g_probe.used;
  *flops = nc::g_probe.flops;
  if (rc == NC_OK && nc::g_probe.dropped)
    rc = nc::set_error(NC_ERR_WORKSPACE, "probe: %lld launches beyond max_launches were not timed",
                       (long long)nc::g_probe.dropped);
  nc::probe_release();
  return rc;
}

extern "C" const char* nc_last_error(void) { return nc::g_err; }

extern "C" const char* nc_version(void) { return "libnc 0.1.0 (gfx950)"; }

extern "C" int nc_debug_mode(void) { return nc::debug_mode() ? 1 : 0; }

extern "C" int nc_sync_status(const int32_t* flag, void* stream) {
  NC_REQUIRE(flag, NC_ERR_INVALID_ARG, "sync_status: null flag");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t h = 0;
  NC_CHECK_HIP(hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, s));
  NC_CHECK_HIP(hipStreamSynchronize(s));
  if (h != 0) return nc::set_error(NC_ERR_DEVICE_FLAG, "device flag raised: a token id was outside [0, V)");
  return nc::api_done(NC_OK, stream, "nc_sync_status");
}
