// Causal multi-query attention: H query heads share one key/value head
// (release-news page "Karpathy再放大招…", section 技術細節與問答: multi-query
// attention).  Scores are scale * q.k with scale = 1/sqrt(hd), masked to keys
// u <= t, softmax over u.
//
// Layout: the packed projection output qkv [B*T, (H+2)*hd] holds per token the
// H normalized query heads, the normalized key head and the value head.  With
// one shared K/V head the H query heads of a token are just H more rows
// against the same keys, so the kernels index query rows r = t*H + h of a
// sequence and map each to its position t = r / H.
//
// bf16 with head_dim 128 runs on the matrix-core kernels of attn_mfma.hip.
// This file holds the direct (scalar) kernels used otherwise (the fp32
// configuration, head_dim 64): one wavefront per query row (forward, dQ) or
// per key row (dK, dV), keys or query rows processed in chunks of 64 with the
// probabilities shared through LDS.
#include "common.h"
#include "ops.h"
#include "attn_mfma.h"

namespace nc {
namespace {

template <typename T>
__device__ __forceinline__ float dot_lds_global(const float* __restrict__ a, const T* __restrict__ b, int hd) {
  float s = 0.f;
  for (int c = 0; c < hd; ++c) s = fmaf(a[c], ld(b + c), s);
  return s;
}

template <typename T>
__global__ __launch_bounds__(64) void attn_fwd_simple_kernel(const T* __restrict__ qkv, int Tlen, int H, int hd,
                                                             float scale, T* __restrict__ o,
                                                             float* __restrict__ lse) {
  __shared__ float q[128];
  __shared__ float p[64];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t tok = row / H;
  const int h = (int)(row - tok * H);
  const int t = (int)(tok % Tlen);
  const int64_t tok0 = tok - t;
  const int64_t S = (int64_t)(H + 2) * hd;
  for (int c = lane; c < hd; c += 64) q[c] = ld(qkv + tok * S + (int64_t)h * hd + c);
  __syncthreads();
  const T* kbase = qkv + tok0 * S + (int64_t)H * hd;
  const T* vbase = qkv + tok0 * S + (int64_t)(H + 1) * hd;
  float m = -INFINITY;
  for (int u = lane; u <= t; u += 64) m = fmaxf(m, dot_lds_global(q, kbase + u * S, hd) * scale);
  m = wave_max(m);
  float l = 0.f;
  for (int u = lane; u <= t; u += 64) l += expf(dot_lds_global(q, kbase + u * S, hd) * scale - m);
  l = wave_sum(l);
  const float inv_l = 1.f / l;
  float acc0 = 0.f, acc1 = 0.f;
  for (int u0 = 0; u0 <= t; u0 += 64) {
    const int u = u0 + lane;
    p[lane] = u <= t ? expf(dot_lds_global(q, kbase + u * S, hd) * scale - m) * inv_l : 0.f;
    __syncthreads();
    const int n = min(64, t - u0 + 1);
    for (int uu = 0; uu < n; ++uu) {
      const T* v = vbase + (int64_t)(u0 + uu) * S;
      acc0 = fmaf(p[uu], ld(v + lane), acc0);
      if (lane + 64 < hd) acc1 = fmaf(p[uu], ld(v + lane + 64), acc1);
    }
    __syncthreads();
  }
  T* orow = o + tok * (int64_t)H * hd + (int64_t)h * hd;
  if (lane < hd) st(orow + lane, acc0);
  if (lane + 64 < hd) st(orow + lane + 64, acc1);
  if (lane == 0) lse[row] = m + logf(l);
}

// dQ for one query row; also stores D = do . o for the key-side kernel.
template <typename T>
__global__ __launch_bounds__(64) void attn_bwd_dq_simple_kernel(const T* __restrict__ qkv, const T* __restrict__ o,
                                                                const T* __restrict__ dout,
                                                                const float* __restrict__ lse, int Tlen, int H,
                                                                int hd, float scale, float* __restrict__ dqkv,
                                                                float* __restrict__ Dbuf) {
  __shared__ float q[128];
  __shared__ float dq_[128];
  __shared__ float ds[64];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int64_t tok = row / H;
  const int h = (int)(row - tok * H);
  const int t = (int)(tok % Tlen);
  const int64_t tok0 = tok - t;
  const int64_t S = (int64_t)(H + 2) * hd;
  const T* orow = o + tok * (int64_t)H * hd + (int64_t)h * hd;
  const T* dorow = dout + tok * (int64_t)H * hd + (int64_t)h * hd;
  float dpart = 0.f;
  for (int c = lane; c < hd; c += 64) {
    q[c] = ld(qkv + tok * S + (int64_t)h * hd + c);
    const float g = ld(dorow + c);
    dq_[c] = g;  // holds dO until the loop below
    dpart = fmaf(g, ld(orow + c), dpart);
  }
  const float D = wave_sum(dpart);
  if (lane == 0) Dbuf[row] = D;
  __syncthreads();
  const T* kbase = qkv + tok0 * S + (int64_t)H * hd;
  const T* vbase = qkv + tok0 * S + (int64_t)(H + 1) * hd;
  const float L = lse[row];
  float acc0 = 0.f, acc1 = 0.f;
  for (int u0 = 0; u0 <= t; u0 += 64) {
    const int u = u0 + lane;
    float v = 0.f;
    if (u <= t) {
      const float p = expf(dot_lds_global(q, kbase + u * S, hd) * scale - L);
      const float dp = dot_lds_global(dq_, vbase + u * S, hd);
      v = p * (dp - D) * scale;
    }
    ds[lane] = v;
    __syncthreads();
    const int n = min(64, t - u0 + 1);
    for (int uu = 0; uu < n; ++uu) {
      const T* k = kbase + (int64_t)(u0 + uu) * S;
      acc0 = fmaf(ds[uu], ld(k + lane), acc0);
      if (lane + 64 < hd) acc1 = fmaf(ds[uu], ld(k + lane + 64), acc1);
    }
    __syncthreads();
  }
  float* out = dqkv + tok * S + (int64_t)h * hd;
  if (lane < hd) out[lane] = acc0;
  if (lane + 64 < hd) out[lane + 64] = acc1;
}

// dK and dV of one key row u: sums over every query row (t, h) with t >= u.
template <typename T>
__global__ __launch_bounds__(64) void attn_bwd_dkv_simple_kernel(const T* __restrict__ qkv,
                                                                 const T* __restrict__ dout,
                                                                 const float* __restrict__ lse,
                                                                 const float* __restrict__ Dbuf, int Tlen, int H,
                                                                 int hd, float scale, float* __restrict__ dqkv) {
  __shared__ float k[128];
  __shared__ float v[128];
  __shared__ float pp[64];
  __shared__ float ds[64];
  const int lane = threadIdx.x;
  const int64_t tok = blockIdx.x;
  const int u = (int)(tok % Tlen);
  const int64_t tok0 = tok - u;
  const int64_t S = (int64_t)(H + 2) * hd;
  for (int c = lane; c < hd; c += 64) {
    k[c] = ld(qkv + tok * S + (int64_t)H * hd + c);
    v[c] = ld(qkv + tok * S + (int64_t)(H + 1) * hd + c);
  }
  __syncthreads();
  const int64_t rows = (int64_t)Tlen * H;
  const int64_t rbeg = (int64_t)u * H;
  float dk0 = 0.f, dk1 = 0.f, dv0 = 0.f, dv1 = 0.f;
  for (int64_t r0 = rbeg; r0 < rows; r0 += 64) {
    const int64_t r = r0 + lane;
    float pv = 0.f, dsv = 0.f;
    if (r < rows) {
      const int64_t t = r / H;
      const int h = (int)(r - t * H);
      const T* q = qkv + (tok0 + t) * S + (int64_t)h * hd;
      const T* g = dout + (tok0 + t) * (int64_t)H * hd + (int64_t)h * hd;
      float s = 0.f, dp = 0.f;
      for (int c = 0; c < hd; ++c) {
        s = fmaf(ld(q + c), k[c], s);
        dp = fmaf(ld(g + c), v[c], dp);
      }
      const int64_t grow = tok0 * H + r;
      pv = expf(s * scale - lse[grow]);
      dsv = pv * (dp - Dbuf[grow]) * scale;
    }
    pp[lane] = pv;
    ds[lane] = dsv;
    __syncthreads();
    const int n = (int)min<int64_t>(64, rows - r0);
    for (int rr = 0; rr < n; ++rr) {
      const int64_t t = (r0 + rr) / H;
      const int h = (int)(r0 + rr - t * H);
      const T* q = qkv + (tok0 + t) * S + (int64_t)h * hd;
      const T* g = dout + (tok0 + t) * (int64_t)H * hd + (int64_t)h * hd;
      dk0 = fmaf(ds[rr], ld(q + lane), dk0);
      dv0 = fmaf(pp[rr], ld(g + lane), dv0);
      if (lane + 64 < hd) {
        dk1 = fmaf(ds[rr], ld(q + lane + 64), dk1);
        dv1 = fmaf(pp[rr], ld(g + lane + 64), dv1);
      }
    }
    __syncthreads();
  }
  float* dk_out = dqkv + tok * S + (int64_t)H * hd;
  float* dv_out = dqkv + tok * S + (int64_t)(H + 1) * hd;
  if (lane < hd) {
    dk_out[lane] = dk0;
    dv_out[lane] = dv0;
  }
  if (lane + 64 < hd) {
    dk_out[lane + 64] = dk1;
    dv_out[lane + 64] = dv1;
  }
}

template <typename T>
int fwd_simple(const void* qkv, int B, int T_, int H, int hd, float scale, void* o, float* lse, hipStream_t s) {
  const int64_t rows = (int64_t)B * T_ * H;
  attn_fwd_simple_kernel<T><<<(unsigned)rows, 64, 0, s>>>(static_cast<const T*>(qkv), T_, H, hd, scale,
                                                          static_cast<T*>(o), lse);
  return check_launch("attn_fwd_simple_kernel");
}

template <typename T>
int bwd_simple(const void* qkv, const void* o, const void* dout, const float* lse, int B, int T_, int H, int hd,
               float scale, float* dqkv, float* Dbuf, hipStream_t s) {
  const int64_t rows = (int64_t)B * T_ * H;
  attn_bwd_dq_simple_kernel<T><<<(unsigned)rows, 64, 0, s>>>(static_cast<const T*>(qkv), static_cast<const T*>(o),
                                                             static_cast<const T*>(dout), lse, T_, H, hd, scale,
                                                             dqkv, Dbuf);
  NC_TRY(check_launch("attn_bwd_dq_simple_kernel"));
  attn_bwd_dkv_simple_kernel<T><<<(unsigned)((int64_t)B * T_), 64, 0, s>>>(
      static_cast<const T*>(qkv), static_cast<const T*>(dout), lse, Dbuf, T_, H, hd, scale, dqkv);
  return check_launch("attn_bwd_dkv_simple_kernel");
}

int validate(const void* qkv, int dtype, int B, int T, int H, int hd) {
  NC_REQUIRE(qkv, NC_ERR_INVALID_ARG, "mqa_attn: null qkv");
  NC_REQUIRE(B > 0 && T > 0 && H > 0, NC_ERR_INVALID_ARG, "mqa_attn: bad shape");
  NC_REQUIRE(hd == 64 || hd == 128, NC_ERR_UNSUPPORTED, "mqa_attn: head_dim must be 64 or 128");
  NC_REQUIRE(dtype == NC_F32 || dtype == NC_BF16, NC_ERR_INVALID_ARG, "mqa_attn: bad dtype");
  NC_REQUIRE((int64_t)B * T * H < (1ll << 31), NC_ERR_UNSUPPORTED, "mqa_attn: too many rows");
  return NC_OK;
}

}  // namespace

size_t mqa_attn_bwd_workspace_bytes(int B, int T, int H) {
  return std::max(align_up((size_t)B * T * H * sizeof(float), 256), attn_mfma_bwd_workspace_bytes(B, T, H));
}

int mqa_attn_fwd(const void* qkv, int dtype, int B, int T, int H, int hd, float scale, void* o, float* lse,
                 hipStream_t s) {
  NC_TRY(validate(qkv, dtype, B, T, H, hd));
  NC_REQUIRE(o && lse, NC_ERR_INVALID_ARG, "mqa_attn_fwd: null output");
  if (dtype == NC_F32) return fwd_simple<float>(qkv, B, T, H, hd, scale, o, lse, s);
  if (hd == 128) return attn_mfma_fwd(qkv, B, T, H, scale, o, lse, s);
  return fwd_simple<bf16>(qkv, B, T, H, hd, scale, o, lse, s);
}

bool attn_rope_bwd_fusable(int dtype, int hd) { return dtype == NC_BF16 && hd == 128; }

int mqa_attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse, int dtype, int B, int T, int H,
                 int hd, float scale, float* dqkv, void* ws, size_t ws_bytes, hipStream_t s, const AttnRopeBwd* fuse) {
  NC_TRY(validate(qkv, dtype, B, T, H, hd));
  if (fuse) {
    NC_REQUIRE(attn_rope_bwd_fusable(dtype, hd), NC_ERR_UNSUPPORTED, "mqa_attn_bwd: fused RoPE backward needs bf16, hd 128");
    NC_REQUIRE(fuse->rstd_q && fuse->rstd_k && fuse->table && fuse->dqkv, NC_ERR_INVALID_ARG,
               "mqa_attn_bwd: null fused-output pointer");
  } else {
    NC_REQUIRE(dqkv, NC_ERR_INVALID_ARG, "mqa_attn_bwd: null pointer");
  }
  NC_REQUIRE(o && dout && lse, NC_ERR_INVALID_ARG, "mqa_attn_bwd: null pointer");
  NC_REQUIRE(ws && ws_bytes >= mqa_attn_bwd_workspace_bytes(B, T, H), NC_ERR_WORKSPACE,
             "mqa_attn_bwd: workspace too small (%zu < %zu)", ws_bytes, mqa_attn_bwd_workspace_bytes(B, T, H));
  float* Dbuf = static_cast<float*>(ws);
  if (dtype == NC_F32) return bwd_simple<float>(qkv, o, dout, lse, B, T, H, hd, scale, dqkv, Dbuf, s);
  if (hd == 128) return attn_mfma_bwd(qkv, o, dout, lse, B, T, H, scale, dqkv, ws, s, fuse);
  return bwd_simple<bf16>(qkv, o, dout, lse, B, T, H, hd, scale, dqkv, Dbuf, s);
}

}  // namespace nc

extern "C" int nc_mqa_attn_fwd(const void* qkv, int dtype, int B, int T, int H, int hd, float scale, void* o,
                               float* lse, void* stream) {
  return nc::api_done(nc::mqa_attn_fwd(qkv, dtype, B, T, H, hd, scale, o, lse, static_cast<hipStream_t>(stream)),
                      stream, "nc_mqa_attn_fwd");
}

extern "C" size_t nc_mqa_attn_bwd_workspace_bytes(int B, int T, int H) {
  return nc::mqa_attn_bwd_workspace_bytes(B, T, H);
}

extern "C" int nc_mqa_attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse, int dtype, int B,
                               int T, int H, int hd, float scale, float* dqkv_hat, void* ws, size_t ws_bytes,
                               void* stream) {
  return nc::api_done(nc::mqa_attn_bwd(qkv, o, dout, lse, dtype, B, T, H, hd, scale, dqkv_hat, ws, ws_bytes,
                          static_cast<hipStream_t>(stream)), stream, "nc_mqa_attn_bwd");
}
