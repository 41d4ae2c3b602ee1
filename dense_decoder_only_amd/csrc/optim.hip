// AdamW update with the bf16 weight refresh.  The release-news page
// ("Karpathy再放大招…", section 技術細節與問答) names Muon + AdamW as the
// optimizers; this is the published AdamW (Loshchilov and Hutter, "Decoupled
// Weight Decay Regularization"): bias-corrected Adam moments and a weight
// decay applied to the parameter, not the gradient.
//
// One pass over HBM: 16-byte loads of p, m, v, g, 16-byte stores of p, m, v
// and an 8-byte store of the bf16 copy per four parameters.  The bias corrections are folded into two scalars
// on the host in double precision.  Bound by HBM bandwidth (28-30 bytes per
// parameter).
#include "common.h"

#include <cmath>

namespace nc {
namespace {

struct AdamWArgs {
  float lr, beta1, beta2, eps, decay;  // decay = 1 - lr * weight_decay
  float inv_bc1, inv_bc2;              // 1 / (1 - beta^t)
  float gscale;
};

__device__ __forceinline__ float adamw1(float p, float& m, float& v, float g, const AdamWArgs& a) {
  g *= a.gscale;
  m = a.beta1 * m + (1.f - a.beta1) * g;
  v = a.beta2 * v + (1.f - a.beta2) * g * g;
  const float mh = m * a.inv_bc1, vh = v * a.inv_bc2;
  return p * a.decay - a.lr * mh / (sqrtf(vh) + a.eps);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
constexpr int kAdamWUnroll = 2;  // float4 groups per thread, all loads issued before the math

// Each thread owns kAdamWUnroll float4 groups 256 apart, so every load of a
// wave is a contiguous 1 KiB.  The data is touched once: loads and stores are
// nontemporal, so the stream does not evict what the step keeps in L2/MALL.
__global__ __launch_bounds__(256) void adamw_kernel(float* __restrict__ P, float* __restrict__ Mo,
                                                    float* __restrict__ Vo, const float* __restrict__ G,
                                                    bf16* __restrict__ W, int64_t n, AdamWArgs a) {
  const int64_t n4 = n >> 2;
  f32x4* P4 = reinterpret_cast<f32x4*>(P);
  f32x4* M4 = reinterpret_cast<f32x4*>(Mo);
  f32x4* V4 = reinterpret_cast<f32x4*>(Vo);
  const f32x4* G4 = reinterpret_cast<const f32x4*>(G);
  u32x2* W2 = reinterpret_cast<u32x2*>(W);
  const int64_t stride = (int64_t)gridDim.x * 256 * kAdamWUnroll;
  for (int64_t i0 = (int64_t)blockIdx.x * 256 * kAdamWUnroll + threadIdx.x; i0 < n4; i0 += stride) {
    f32x4 p[kAdamWUnroll], m[kAdamWUnroll], v[kAdamWUnroll], g[kAdamWUnroll];
#pragma unroll
    for (int u = 0; u < kAdamWUnroll; ++u) {
      const int64_t i = i0 + u * 256;
      if (i < n4) {
        p[u] = __builtin_nontemporal_load(P4 + i);
        m[u] = __builtin_nontemporal_load(M4 + i);
        v[u] = __builtin_nontemporal_load(V4 + i);
        g[u] = __builtin_nontemporal_load(G4 + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kAdamWUnroll; ++u) {
      const int64_t i = i0 + u * 256;
      if (i < n4) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float mc = m[u][c], vc = v[u][c];
          p[u][c] = adamw1(p[u][c], mc, vc, g[u][c], a);
          m[u][c] = mc;
          v[u][c] = vc;
        }
        __builtin_nontemporal_store(p[u], P4 + i);
        __builtin_nontemporal_store(m[u], M4 + i);
        __builtin_nontemporal_store(v[u], V4 + i);
        if (W) {
          const u32x2 w = {pack_bf16x2(p[u][0], p[u][1]), pack_bf16x2(p[u][2], p[u][3])};
          __builtin_nontemporal_store(w, W2 + i);
        }
      }
    }
  }
  // tail (n not a multiple of 4)
  for (int64_t i = (n4 << 2) + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float m = Mo[i], v = Vo[i];
    const float p = adamw1(P[i], m, v, G[i], a);
    P[i] = p;
    Mo[i] = m;
    Vo[i] = v;
    if (W) W[i] = f2bf(p);
  }
}

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

int adamw_step(float* P, float* M, float* V, const float* G, void* W, int64_t n, int t, float lr, float beta1,
               float beta2, float eps, float wd, float gscale, hipStream_t s) {
  NC_REQUIRE(n >= 0 && t >= 1, NC_ERR_INVALID_ARG, "adamw: n must be >= 0 and t >= 1");
  if (n == 0) return NC_OK;  // nothing to update; the pointers may be null
  NC_REQUIRE(P && M && V && G, NC_ERR_INVALID_ARG, "adamw: null pointer");
  NC_REQUIRE(al16(P) && al16(M) && al16(V) && al16(G) && (!W || (reinterpret_cast<uintptr_t>(W) & 7u) == 0),
             NC_ERR_INVALID_ARG, "adamw: fp32 arrays must be 16-byte and the bf16 copy 8-byte aligned");
  AdamWArgs a;
  a.lr = lr;
  a.beta1 = beta1;
  a.beta2 = beta2;
  a.eps = eps;
  a.decay = (float)(1.0 - (double)lr * (double)wd);
  a.inv_bc1 = (float)(1.0 / (1.0 - std::pow((double)beta1, (double)t)));
  a.inv_bc2 = (float)(1.0 / (1.0 - std::pow((double)beta2, (double)t)));
  a.gscale = gscale;
  // one pass: a workgroup per 256 * kAdamWUnroll float4 groups (the loop only strides past 2^30 groups)
  const unsigned blocks =
      (unsigned)std::min<int64_t>(cdiv(std::max<int64_t>(n >> 2, 1), 256 * kAdamWUnroll), int64_t(1) << 30);
  adamw_kernel<<<blocks, 256, 0, s>>>(P, M, V, G, static_cast<bf16*>(W), n, a);
  return check_launch("adamw_kernel");
}

}  // namespace nc

extern "C" int nc_adamw_step(float* master, float* m, float* v, const float* grad, void* weights_lp, int64_t n,
                             int t, float lr, float beta1, float beta2, float eps, float weight_decay,
                             float grad_scale, void* stream) {

                       return nc::api_done(nc::adamw_step(master, m, v, grad, weights_lp, n, t, lr, beta1, beta2, eps, weight_decay, grad_scale,
                        static_cast<hipStream_t>(stream)), stream, "nc_adamw_step");
}
