// Parameter-free RMSNorm (forward and backward) and the token-embedding
// gather fused with the norm that follows it.  Release-news page
// "Karpathy再放大招…", section 技術細節與問答: the token embedding is followed by
// a norm; RMSNorm has no learnable parameters.
//
// One 64-lane wavefront per row, four rows per 256-thread block; each lane
// moves 4 elements per access (16 bytes fp32 / 8 bytes bf16), so a row of
// d = 1280 is read in 5 coalesced passes.  Rows up to 2048 wide stay in
// registers between the reduction and the scaling pass; wider rows are read
// twice.  These kernels are bound by HBM bandwidth.
#include "common.h"
#include "ops.h"

namespace nc {
namespace {

// Rows are read and written once: non-temporal (streaming) accesses keep them
// from displacing what the neighbouring GEMMs hold in L2.
typedef float nf4 __attribute__((ext_vector_type(4)));
typedef unsigned nu2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float4 load4(const float* p) {
  const nf4 t = __builtin_nontemporal_load(reinterpret_cast<const nf4*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ float4 load4(const bf16* p) {
  const nu2 u = __builtin_nontemporal_load(reinterpret_cast<const nu2*>(p));
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ void store4(float* p, float4 v) {
  const nf4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<nf4*>(p));
}
__device__ __forceinline__ void store4(bf16* p, float4 v) {
  const nu2 t = {pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)};
  __builtin_nontemporal_store(t, reinterpret_cast<nu2*>(p));
}
// Cached loads, for the embedding gather: the Zipf head's rows recur.
__device__ __forceinline__ float4 load4_cached(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4_cached(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }
__device__ __forceinline__ float4 scale4(float4 a, float s) { return make_float4(a.x * s, a.y * s, a.z * s, a.w * s); }

// Rows of up to 64 * 4 * CV elements are held in registers between the two
// passes (CV float4 per lane), so each element is read from HBM once.
constexpr int CV = 8;

template <typename TX, typename TY>
__global__ __launch_bounds__(256) void rmsnorm_fwd_reg_kernel(const TX* __restrict__ x, int64_t rows, int d,
                                                              float eps, TY* __restrict__ y,
                                                              float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const TX* xr = x + row * d;
  float4 v[CV];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < CV; ++k) {
    const int c = lane * 4 + k * 256;
    if (c < d) {
      v[k] = load4(xr + c);
      ss += dot4(v[k], v[k]);
    }
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)d + eps);
  TY* yr = y + row * d;
#pragma unroll
  for (int k = 0; k < CV; ++k) {
    const int c = lane * 4 + k * 256;
    if (c < d) store4(yr + c, scale4(v[k], r));
  }
  if (lane == 0 && rstd) rstd[row] = r;
}

template <typename TG, typename TY, bool FIX = false>
__global__ __launch_bounds__(256) void rmsnorm_bwd_reg_kernel(const TG* __restrict__ g, const TY* __restrict__ y,
                                                              const float* __restrict__ rstd, int64_t rows, int d,
                                                              float* __restrict__ dx, int accumulate,
                                                              bf16* __restrict__ dx_bf16, GradRowFix fix = {}) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const TG* gr = g + row * d;
  const TY* yr = y + row * d;
  float* dr = dx + row * d;
  // the accumulated dx is loaded with g and y, ahead of the row reduction,
  // so that its latency is not paid a second time after it
  float4 gv[CV], yv[CV], pv[CV];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < CV; ++k) {
    const int c = lane * 4 + k * 256;
    if (c < d) {
      gv[k] = load4(gr + c);
      yv[k] = load4(yr + c);
      pv[k] = accumulate ? load4(dr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  if constexpr (FIX) {
    const float rs = fix.rs[row], qs = fix.qs[row];
    const int32_t t = fix.tgt[row];
    const bool hit = (uint32_t)t < (uint32_t)fix.V;
    const bf16* ur = fix.U + (int64_t)(hit ? t : 0) * d;
#pragma unroll
    for (int k = 0; k < CV; ++k) {
      const int c = lane * 4 + k * 256;
      if (c < d) {
        const float4 u = hit ? load4_cached(ur + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        gv[k] = make_float4(gv[k].x * rs - qs * u.x, gv[k].y * rs - qs * u.y, gv[k].z * rs - qs * u.z,
                            gv[k].w * rs - qs * u.w);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < CV; ++k)
    if (lane * 4 + k * 256 < d) s += dot4(gv[k], yv[k]);
  const float r = rstd[row];
  const float mean = wave_sum(s) / (float)d;
#pragma unroll
  for (int k = 0; k < CV; ++k) {
    const int c = lane * 4 + k * 256;
    if (c < d) {
      float4 o = make_float4(r * (gv[k].x - yv[k].x * mean), r * (gv[k].y - yv[k].y * mean),
                             r * (gv[k].z - yv[k].z * mean), r * (gv[k].w - yv[k].w * mean));
      if (accumulate) o = make_float4(o.x + pv[k].x, o.y + pv[k].y, o.z + pv[k].z, o.w + pv[k].w);
      store4(dr + c, o);
      if (dx_bf16) store4(dx_bf16 + row * d + c, o);
    }
  }
}

template <typename TX, typename TY>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const TX* __restrict__ x, int64_t rows, int d,
                                                          float eps, TY* __restrict__ y,
                                                          float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const TX* xr = x + row * d;
  float ss = 0.f;
  for (int c = lane * 4; c < d; c += 256) {
    const float4 v = load4(xr + c);
    ss += dot4(v, v);
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)d + eps);
  TY* yr = y + row * d;
  for (int c = lane * 4; c < d; c += 256) store4(yr + c, scale4(load4(xr + c), r));
  if (lane == 0 && rstd) rstd[row] = r;
}

// dx (+)= r * (g - y * mean(g * y)); optional bf16 copy of the result.
template <typename TG, typename TY>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const TG* __restrict__ g, const TY* __restrict__ y,
                                                          const float* __restrict__ rstd, int64_t rows, int d,
                                                          float* __restrict__ dx, int accumulate,
                                                          bf16* __restrict__ dx_bf16) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const TG* gr = g + row * d;
  const TY* yr = y + row * d;
  float s = 0.f;
  for (int c = lane * 4; c < d; c += 256) s += dot4(load4(gr + c), load4(yr + c));
  const float mean = wave_sum(s) / (float)d;
  const float r = rstd[row];
  float* dr = dx + row * d;
  for (int c = lane * 4; c < d; c += 256) {
    const float4 gv = load4(gr + c), yv = load4(yr + c);
    float4 o = make_float4(r * (gv.x - yv.x * mean), r * (gv.y - yv.y * mean), r * (gv.z - yv.z * mean),
                           r * (gv.w - yv.w * mean));
    if (accumulate) {
      const float4 p = load4(dr + c);
      o = make_float4(o.x + p.x, o.y + p.y, o.z + p.z, o.w + p.w);
    }
    store4(dr + c, o);
    if (dx_bf16) store4(dx_bf16 + row * d + c, o);
  }
}

// Gather rows of `table` by token id; optional bit-exact copy and RMSNorm.
template <typename T>
__global__ __launch_bounds__(256) void embed_fwd_kernel(const int32_t* __restrict__ ids, int64_t n,
                                                        const T* __restrict__ table, int64_t V, int d,
                                                        T* __restrict__ rows_out, float* __restrict__ x_out,
                                                        float* __restrict__ x_copy, float* __restrict__ rstd,
                                                        float eps, int32_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const int32_t id = ids[row];
  const bool ok = id >= 0 && id < V;
  if (!ok && lane == 0 && flag) *flag = 1;
  const T* src = table + (int64_t)(ok ? id : 0) * d;
  if (rows_out) {
    // raw copy of the row's bits, 8 bytes per access
    const int per = 8 / sizeof(T);
    for (int c = lane * per; c < d; c += 64 * per) {
      uint2 v = ok ? *reinterpret_cast<const uint2*>(src + c) : make_uint2(0, 0);
      *reinterpret_cast<uint2*>(rows_out + row * d + c) = v;
    }
  }
  if (x_out) {
    float ss = 0.f;
    for (int c = lane * 4; c < d; c += 256) {
      const float4 v = ok ? load4_cached(src + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      ss += dot4(v, v);
    }
    ss = wave_sum(ss);
    const float r = 1.f / sqrtf(ss / (float)d + eps);
    for (int c = lane * 4; c < d; c += 256) {
      const float4 v = ok ? load4_cached(src + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      store4(x_out + row * d + c, scale4(v, r));
      if (x_copy) store4(x_copy + row * d + c, scale4(v, r));
    }
    if (lane == 0 && rstd) rstd[row] = r;
  }
}

template <typename TG, typename TY>
int launch_bwd(const void* g, const void* y, const float* rstd, int64_t rows, int d, float* dx, int acc,
               bf16* dxb, hipStream_t s) {
  const unsigned blocks = (unsigned)cdiv(rows, 4);
  if (d <= 256 * CV) {
    rmsnorm_bwd_reg_kernel<TG, TY><<<blocks, 256, 0, s>>>(static_cast<const TG*>(g), static_cast<const TY*>(y), rstd,
                                                           rows, d, dx, acc, dxb);
    return check_launch("rmsnorm_bwd_reg_kernel");
  }
  rmsnorm_bwd_kernel<TG, TY><<<blocks, 256, 0, s>>>(static_cast<const TG*>(g), static_cast<const TY*>(y), rstd,
                                                     rows, d, dx, acc, dxb);
  return check_launch("rmsnorm_bwd_kernel");
}

template <typename TX, typename TY>
int launch_fwd(const void* x, int64_t rows, int d, float eps, void* y, float* rstd, hipStream_t s) {
  const unsigned blocks = (unsigned)cdiv(rows, 4);
  if (d <= 256 * CV) {
    rmsnorm_fwd_reg_kernel<TX, TY><<<blocks, 256, 0, s>>>(static_cast<const TX*>(x), rows, d, eps,
                                                           static_cast<TY*>(y), rstd);
    return check_launch("rmsnorm_fwd_reg_kernel");
  }
  rmsnorm_fwd_kernel<TX, TY><<<blocks, 256, 0, s>>>(static_cast<const TX*>(x), rows, d, eps, static_cast<TY*>(y),
                                                     rstd);
  return check_launch("rmsnorm_fwd_kernel");
}

}  // namespace

int rmsnorm_fwd(const void* x, int xdt, int64_t rows, int d, float eps, void* y, int ydt, float* rstd,
                hipStream_t s) {
  NC_REQUIRE(x && y, NC_ERR_INVALID_ARG, "rmsnorm_fwd: null pointer");
  NC_REQUIRE(rows >= 0 && d > 0, NC_ERR_INVALID_ARG, "rmsnorm_fwd: bad shape");
  NC_REQUIRE(d % 8 == 0, NC_ERR_UNSUPPORTED, "rmsnorm_fwd: d must be a multiple of 8");
  NC_REQUIRE((xdt == NC_F32 || xdt == NC_BF16) && (ydt == NC_F32 || ydt == NC_BF16), NC_ERR_INVALID_ARG,
             "rmsnorm_fwd: bad dtype");
  if (rows == 0) return NC_OK;
  if (xdt == NC_F32 && ydt == NC_F32) return launch_fwd<float, float>(x, rows, d, eps, y, rstd, s);
  if (xdt == NC_F32 && ydt == NC_BF16) return launch_fwd<float, bf16>(x, rows, d, eps, y, rstd, s);
  if (xdt == NC_BF16 && ydt == NC_F32) return launch_fwd<bf16, float>(x, rows, d, eps, y, rstd, s);
  return launch_fwd<bf16, bf16>(x, rows, d, eps, y, rstd, s);
}

int rmsnorm_bwd(const void* g, int gdt, const void* y, int ydt, const float* rstd, int64_t rows, int d,
                float* dx, int accumulate, void* dx_bf16, hipStream_t s, const GradRowFix* fix) {
  NC_REQUIRE(g && y && rstd && dx, NC_ERR_INVALID_ARG, "rmsnorm_bwd: null pointer");
  NC_REQUIRE(rows >= 0 && d > 0, NC_ERR_INVALID_ARG, "rmsnorm_bwd: bad shape");
  NC_REQUIRE(d % 8 == 0, NC_ERR_UNSUPPORTED, "rmsnorm_bwd: d must be a multiple of 8");
  NC_REQUIRE((gdt == NC_F32 || gdt == NC_BF16) && (ydt == NC_F32 || ydt == NC_BF16), NC_ERR_INVALID_ARG,
             "rmsnorm_bwd: bad dtype");
  if (rows == 0) return NC_OK;
  bf16* dxb = static_cast<bf16*>(dx_bf16);
  if (fix) {
    NC_REQUIRE(gdt == NC_F32 && d <= 256 * CV && fix->rs && fix->qs && fix->tgt && fix->U, NC_ERR_INVALID_ARG,
               "rmsnorm_bwd: the row fix needs an fp32 gradient, d <= 2048 and its arrays");
    const unsigned blocks = (unsigned)cdiv(rows, 4);
    if (ydt == NC_F32)
      rmsnorm_bwd_reg_kernel<float, float, true><<<blocks, 256, 0, s>>>(
          static_cast<const float*>(g), static_cast<const float*>(y), rstd, rows, d, dx, accumulate, dxb, *fix);
    else
      rmsnorm_bwd_reg_kernel<float, bf16, true><<<blocks, 256, 0, s>>>(
          static_cast<const float*>(g), static_cast<const bf16*>(y), rstd, rows, d, dx, accumulate, dxb, *fix);
    return check_launch("rmsnorm_bwd_reg_kernel");
  }
  if (gdt == NC_F32 && ydt == NC_F32) return launch_bwd<float, float>(g, y, rstd, rows, d, dx, accumulate, dxb, s);
  if (gdt == NC_F32 && ydt == NC_BF16) return launch_bwd<float, bf16>(g, y, rstd, rows, d, dx, accumulate, dxb, s);
  if (gdt == NC_BF16 && ydt == NC_F32) return launch_bwd<bf16, float>(g, y, rstd, rows, d, dx, accumulate, dxb, s);
  return launch_bwd<bf16, bf16>(g, y, rstd, rows, d, dx, accumulate, dxb, s);
}

int embed_fwd(const int32_t* ids, int64_t n, const void* table, int dtype, int64_t V, int d, void* rows_out,
              float* x_out, float* rstd, float eps, int32_t* flag, hipStream_t s, float* x_copy) {
  NC_REQUIRE(ids && table, NC_ERR_INVALID_ARG, "embed_fwd: null pointer");
  NC_REQUIRE(n >= 0 && V > 0 && d > 0, NC_ERR_INVALID_ARG, "embed_fwd: bad shape");
  NC_REQUIRE(d % 8 == 0, NC_ERR_UNSUPPORTED, "embed_fwd: d must be a multiple of 8");
  NC_REQUIRE(dtype == NC_F32 || dtype == NC_BF16, NC_ERR_INVALID_ARG, "embed_fwd: bad dtype");
  NC_REQUIRE(!((rstd || x_copy) && !x_out), NC_ERR_INVALID_ARG, "embed_fwd: rstd and x_copy need x_out");
  if (n == 0) return NC_OK;
  const unsigned blocks = (unsigned)cdiv(n, 4);
  if (dtype == NC_F32)
    embed_fwd_kernel<float><<<blocks, 256, 0, s>>>(ids, n, static_cast<const float*>(table), V, d,
                                                   static_cast<float*>(rows_out), x_out, x_copy, rstd, eps, flag);
  else
    embed_fwd_kernel<bf16><<<blocks, 256, 0, s>>>(ids, n, static_cast<const bf16*>(table), V, d,
                                                  static_cast<bf16*>(rows_out), x_out, x_copy, rstd, eps, flag);
  return check_launch("embed_fwd_kernel");
}

}  // namespace nc

extern "C" int nc_rmsnorm_fwd(const void* x, int xdt, int64_t rows, int d, float eps, void* y, int ydt,
                              float* rstd, void* stream) {
  return nc::api_done(nc::rmsnorm_fwd(x, xdt, rows, d, eps, y, ydt, rstd, static_cast<hipStream_t>(stream)),
                      stream, "nc_rmsnorm_fwd");
}

extern "C" int nc_rmsnorm_bwd(const void* dy, int dydt, const void* y, int ydt, const float* rstd, int64_t rows,
                              int d, float* dx, int accumulate, void* dx_bf16, void* stream) {
  return nc::api_done(nc::rmsnorm_bwd(dy, dydt, y, ydt, rstd, rows, d, dx, accumulate, dx_bf16, static_cast<hipStream_t>(stream)),
                      stream, "nc_rmsnorm_bwd");
}

extern "C" int nc_embed_fwd(const int32_t* ids, int64_t n, const void* table, int dtype, int64_t V, int d,
                            void* rows_out, float* x_out, float* rstd, float eps, int32_t* flag, void* stream) {
  return nc::api_done(nc::embed_fwd(ids, n, table, dtype, V, d, rows_out, x_out, rstd, eps, flag,
                       static_cast<hipStream_t>(stream), nullptr), stream, "nc_embed_fwd");
}
