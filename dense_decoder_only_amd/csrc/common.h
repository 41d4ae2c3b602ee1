// Shared device/host helpers for libnc (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <algorithm>
#include <vector>

#include "nc.h"

namespace nc {

// ---------------------------------------------------------------------------
// Element types.  bf16 values travel as raw 16-bit patterns (uint16_t) so that
// host and device agree bit for bit; conversions round to nearest even.
// ---------------------------------------------------------------------------
typedef uint16_t bf16;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(bf16 b) { return __uint_as_float((uint32_t)b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ bf16 f2bf(float f) { return (bf16)(pack_bf16x2(f, 0.f) & 0xffffu); }

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16> {
  __device__ __forceinline__ static float load(const bf16* p) { return bf2f(*p); }
  __device__ __forceinline__ static void store(bf16* p, float v) { *p = f2bf(v); }
};
template <typename T> __device__ __forceinline__ float ld(const T* p) { return Elem<T>::load(p); }
template <typename T> __device__ __forceinline__ void st(T* p, float v) { Elem<T>::store(p, v); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// Host-side error reporting: every entry point returns an nc_status and leaves
// a message for nc_last_error() (thread-local).
// ---------------------------------------------------------------------------
int set_error(int code, const char* fmt, ...);
int check_launch(const char* what);
// Debug mode (environment variable NC_DEBUG=1, read once per process): every
// entry point that takes a stream synchronizes it before returning and
// reports any HIP error it finds, so that a failing kernel is named by the
// call that launched it.  Not for use under stream capture.
bool debug_mode();
int api_done(int rc, void* stream, const char* name);
// Kernel timer hooks (nc_probe_*): cheap no-ops unless `family` is armed.
void probe_begin(int family, hipStream_t s);
void probe_end(int family, hipStream_t s, double flops);

}  // namespace nc

#define NC_REQUIRE(cond, code, ...)                         \
  do {                                                      \
    if (!(cond)) return ::nc::set_error((code), __VA_ARGS__); \
  } while (0)

#define NC_CHECK_HIP(expr)                                                         \
  do {                                                                             \
    hipError_t e_ = (expr);                                                        \
    if (e_ != hipSuccess)                                                          \
      return ::nc::set_error(NC_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

#define NC_TRY(expr)                 \
  do {                               \
    int rc_ = (expr);                \
    if (rc_ != NC_OK) return rc_;    \
  } while (0)
