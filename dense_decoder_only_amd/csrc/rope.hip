// Rotary position embedding followed by the per-head RMS norm of queries and
// of the single key head (release-news page "Karpathy再放大招…", section
// 技術細節與問答: RoPE with no positional embedding; QK norm).
//
// Pairing (i, i + hd/2), rotation by +theta(t, i) = t * base^(-2 i / hd), RoPE
// before the norm.  The (cos, sin) table is computed in fp64 and rounded to
// fp32 once.  Generic kernels: one wavefront per (token, head); lane
// i < hd/2 owns the pair (i, i + hd/2), so the rotation and the norm need no
// data exchange beyond one wave-wide sum.  bf16 with head_dim 128 has its own
// kernels with 16 lanes per head (below).  Works in place on the packed
// [tokens, (H+2) hd] QKV projection output; these kernels are bound by HBM
// bandwidth.
#include "common.h"

namespace nc {
namespace {

__global__ void rope_table_kernel(float* table, int T, int hd, double base) {
  const int half = hd / 2;
  const int64_t total = (int64_t)T * half;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(e / half), i = (int)(e % half);
    const double th = (double)t * pow(base, -2.0 * (double)i / (double)hd);
    table[2 * e] = (float)cos(th);
    table[2 * e + 1] = (float)sin(th);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void rope_qknorm_fwd_kernel(T* __restrict__ qkv, int64_t M, int Tlen, int H,
                                                              int hd, const float* __restrict__ table, float eps,
                                                              float* __restrict__ rstd_q,
                                                              float* __restrict__ rstd_k) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int heads = H + 1;
  if (item >= M * heads) return;
  const int64_t tok = item / heads;
  const int head = (int)(item - tok * heads);
  const int t = (int)(tok % Tlen);
  const int half = hd >> 1;
  T* x = qkv + tok * (int64_t)(H + 2) * hd + (int64_t)head * hd;
  float ya = 0.f, yb = 0.f;
  if (lane < half) {
    const float a = ld(x + lane), b = ld(x + lane + half);
    const float c = table[2 * ((int64_t)t * half + lane)], s = table[2 * ((int64_t)t * half + lane) + 1];
    ya = a * c - b * s;
    yb = a * s + b * c;
  }
  const float ss = wave_sum(ya * ya + yb * yb);
  const float r = 1.f / sqrtf(ss / (float)hd + eps);
  if (lane < half) {
    st(x + lane, ya * r);
    st(x + lane + half, yb * r);
  }
  if (lane == 0) {
    if (head < H) rstd_q[tok * H + head] = r;
    else rstd_k[tok] = r;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void rope_qknorm_bwd_kernel(const float* __restrict__ dhat,
                                                              const T* __restrict__ yhat,
                                                              const float* __restrict__ rstd_q,
                                                              const float* __restrict__ rstd_k,
                                                              const float* __restrict__ table, int64_t M, int Tlen,
                                                              int H, int hd, T* __restrict__ dqkv) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int heads = H + 2;
  if (item >= M * heads) return;
  const int64_t tok = item / heads;
  const int head = (int)(item - tok * heads);
  const int64_t base = tok * (int64_t)heads * hd + (int64_t)head * hd;
  if (head == H + 1) {  // value head: gradient passes through
    for (int c = lane; c < hd; c += 64) st(dqkv + base + c, dhat[base + c]);
    return;
  }
  const int t = (int)(tok % Tlen);
  const int half = hd >> 1;
  float ga = 0.f, gb = 0.f, ya = 0.f, yb = 0.f;
  if (lane < half) {
    ga = dhat[base + lane];
    gb = dhat[base + lane + half];
    ya = ld(yhat + base + lane);
    yb = ld(yhat + base + lane + half);
  }
  const float mean = wave_sum(ga * ya + gb * yb) / (float)hd;
  const float r = head < H ? rstd_q[tok * H + head] : rstd_k[tok];
  if (lane < half) {
    const float pa = r * (ga - ya * mean), pb = r * (gb - yb * mean);
    const float c = table[2 * ((int64_t)t * half + lane)], s = table[2 * ((int64_t)t * half + lane) + 1];
    st(dqkv + base + lane, pa * c + pb * s);          // rotate back by -theta
    st(dqkv + base + lane + half, -pa * s + pb * c);
  }
}

// bf16, head_dim 128: a 16-lane group per (token, head); lane j owns the
// pairs (i, i + 64) for i = 4 j .. 4 j + 3, so each lane moves two 8-byte
// pieces of x and one 32-byte piece of the table, and the norm is a 16-lane
// sum.  Four heads per wavefront.
__device__ __forceinline__ float group16_sum(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

__device__ __forceinline__ void unpack4(uint2 u, float (&f)[4]) {
  f[0] = __uint_as_float(u.x << 16);
  f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16);
  f[3] = __uint_as_float(u.y & 0xffff0000u);
}

__global__ __launch_bounds__(256) void rope_qknorm_fwd_bf16_kernel(bf16* __restrict__ qkv, int64_t M, int Tlen, int H,
                                                                   const float* __restrict__ table, float eps,
                                                                   float* __restrict__ rstd_q,
                                                                   float* __restrict__ rstd_k) {
  const int j = threadIdx.x & 15;
  const int64_t item = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int heads = H + 1;
  if (item >= M * heads) return;
  const int64_t tok = item / heads;
  const int head = (int)(item - tok * heads);
  const int t = (int)(tok % Tlen);
  bf16* x = qkv + tok * (int64_t)(H + 2) * 128 + (int64_t)head * 128 + 4 * j;
  float a[4], b[4];
  // read and written once, in place: streaming (non-temporal) accesses
  typedef unsigned nu2 __attribute__((ext_vector_type(2)));
  const nu2 la = __builtin_nontemporal_load(reinterpret_cast<const nu2*>(x));
  const nu2 lb = __builtin_nontemporal_load(reinterpret_cast<const nu2*>(x + 64));
  unpack4(make_uint2(la.x, la.y), a);
  unpack4(make_uint2(lb.x, lb.y), b);
  const float4* tb = reinterpret_cast<const float4*>(table + ((int64_t)t * 64 + 4 * j) * 2);
  const float4 cs0 = tb[0], cs1 = tb[1];  // (cos, sin) of pairs 4j .. 4j+3
  const float c[4] = {cs0.x, cs0.z, cs1.x, cs1.z}, sn[4] = {cs0.y, cs0.w, cs1.y, cs1.w};
  float ya[4], yb[4], ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ya[e] = a[e] * c[e] - b[e] * sn[e];
    yb[e] = a[e] * sn[e] + b[e] * c[e];
    ss += ya[e] * ya[e] + yb[e] * yb[e];
  }
  ss = group16_sum(ss);
  const float r = 1.f / sqrtf(ss / 128.f + eps);
  const nu2 sa = {pack_bf16x2(ya[0] * r, ya[1] * r), pack_bf16x2(ya[2] * r, ya[3] * r)};
  const nu2 sb = {pack_bf16x2(yb[0] * r, yb[1] * r), pack_bf16x2(yb[2] * r, yb[3] * r)};
  __builtin_nontemporal_store(sa, reinterpret_cast<nu2*>(x));
  __builtin_nontemporal_store(sb, reinterpret_cast<nu2*>(x + 64));
  if (j == 0) {
    if (head < H) rstd_q[tok * H + head] = r;
    else rstd_k[tok] = r;
  }
}

__global__ __launch_bounds__(256) void rope_qknorm_bwd_bf16_kernel(const float* __restrict__ dhat,
                                                                   const bf16* __restrict__ yhat,
                                                                   const float* __restrict__ rstd_q,
                                                                   const float* __restrict__ rstd_k,
                                                                   const float* __restrict__ table, int64_t M,
                                                                   int Tlen, int H, bf16* __restrict__ dqkv) {
  const int j = threadIdx.x & 15;
  const int64_t item = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int heads = H + 2;
  if (item >= M * heads) return;
  const int64_t tok = item / heads;
  const int head = (int)(item - tok * heads);
  const int64_t base = tok * (int64_t)heads * 128 + (int64_t)head * 128;
  if (head == H + 1) {  // value head: the gradient passes through, rounded to bf16
    const float4 g0 = *reinterpret_cast<const float4*>(dhat + base + 8 * j);
    const float4 g1 = *reinterpret_cast<const float4*>(dhat + base + 8 * j + 4);
    *reinterpret_cast<uint4*>(dqkv + base + 8 * j) =
        make_uint4(pack_bf16x2(g0.x, g0.y), pack_bf16x2(g0.z, g0.w), pack_bf16x2(g1.x, g1.y), pack_bf16x2(g1.z, g1.w));
    return;
  }
  const int t = (int)(tok % Tlen);
  const float4 ga4 = *reinterpret_cast<const float4*>(dhat + base + 4 * j);
  const float4 gb4 = *reinterpret_cast<const float4*>(dhat + base + 64 + 4 * j);
  const float ga[4] = {ga4.x, ga4.y, ga4.z, ga4.w}, gb[4] = {gb4.x, gb4.y, gb4.z, gb4.w};
  float ya[4], yb[4];
  unpack4(*reinterpret_cast<const uint2*>(yhat + base + 4 * j), ya);
  unpack4(*reinterpret_cast<const uint2*>(yhat + base + 64 + 4 * j), yb);
  float dot = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) dot += ga[e] * ya[e] + gb[e] * yb[e];
  const float mean = group16_sum(dot) / 128.f;
  const float r = head < H ? rstd_q[tok * H + head] : rstd_k[tok];
  const float4* tb = reinterpret_cast<const float4*>(table + ((int64_t)t * 64 + 4 * j) * 2);
  const float4 cs0 = tb[0], cs1 = tb[1];
  const float c[4] = {cs0.x, cs0.z, cs1.x, cs1.z}, sn[4] = {cs0.y, cs0.w, cs1.y, cs1.w};
  float oa[4], ob[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float pa = r * (ga[e] - ya[e] * mean), pb = r * (gb[e] - yb[e] * mean);
    oa[e] = pa * c[e] + pb * sn[e];  // rotate back by -theta
    ob[e] = -pa * sn[e] + pb * c[e];
  }
  *reinterpret_cast<uint2*>(dqkv + base + 4 * j) = make_uint2(pack_bf16x2(oa[0], oa[1]), pack_bf16x2(oa[2], oa[3]));
  *reinterpret_cast<uint2*>(dqkv + base + 64 + 4 * j) = make_uint2(pack_bf16x2(ob[0], ob[1]), pack_bf16x2(ob[2], ob[3]));
}

}  // namespace

int rope_table(float* table, int T, int hd, float base, hipStream_t s) {
  NC_REQUIRE(table, NC_ERR_INVALID_ARG, "rope_table: null pointer");
  NC_REQUIRE(T > 0 && hd > 0 && hd % 2 == 0, NC_ERR_INVALID_ARG, "rope_table: bad shape");
  const int64_t total = (int64_t)T * (hd / 2);
  const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(total, 256), 1024);
  rope_table_kernel<<<blocks, 256, 0, s>>>(table, T, hd, (double)base);
  return check_launch("rope_table_kernel");
}

int rope_qknorm_fwd(void* qkv, int dtype, int B, int T, int H, int hd, const float* table, float eps,
                    float* rstd_q, float* rstd_k, hipStream_t s) {
  NC_REQUIRE(qkv && table && rstd_q && rstd_k, NC_ERR_INVALID_ARG, "rope_qknorm_fwd: null pointer");
  NC_REQUIRE(B > 0 && T > 0 && H > 0, NC_ERR_INVALID_ARG, "rope_qknorm_fwd: bad shape");
  NC_REQUIRE(hd == 64 || hd == 128, NC_ERR_UNSUPPORTED, "rope_qknorm_fwd: head_dim must be 64 or 128");
  NC_REQUIRE(dtype == NC_F32 || dtype == NC_BF16, NC_ERR_INVALID_ARG, "rope_qknorm_fwd: bad dtype");
  const int64_t M = (int64_t)B * T;
  if (dtype == NC_BF16 && hd == 128) {
    rope_qknorm_fwd_bf16_kernel<<<(unsigned)cdiv(M * (H + 1), 16), 256, 0, s>>>(static_cast<bf16*>(qkv), M, T, H,
                                                                                table, eps, rstd_q, rstd_k);
    return check_launch("rope_qknorm_fwd_bf16_kernel");
  }
  const unsigned blocks = (unsigned)cdiv(M * (H + 1), 4);
  if (dtype == NC_F32)
    rope_qknorm_fwd_kernel<float><<<blocks, 256, 0, s>>>(static_cast<float*>(qkv), M, T, H, hd, table, eps, rstd_q,
                                                         rstd_k);
  else
    rope_qknorm_fwd_kernel<bf16><<<blocks, 256, 0, s>>>(static_cast<bf16*>(qkv), M, T, H, hd, table, eps, rstd_q,
                                                        rstd_k);
  return check_launch("rope_qknorm_fwd_kernel");
}

int rope_qknorm_bwd(const float* dhat, const void* yhat, const float* rstd_q, const float* rstd_k,
                    const float* table, int dtype, int B, int T, int H, int hd, void* dqkv, hipStream_t s) {
  NC_REQUIRE(dhat && yhat && rstd_q && rstd_k && table && dqkv, NC_ERR_INVALID_ARG,
             "rope_qknorm_bwd: null pointer");
  NC_REQUIRE(B > 0 && T > 0 && H > 0, NC_ERR_INVALID_ARG, "rope_qknorm_bwd: bad shape");
  NC_REQUIRE(hd == 64 || hd == 128, NC_ERR_UNSUPPORTED, "rope_qknorm_bwd: head_dim must be 64 or 128");
  NC_REQUIRE(dtype == NC_F32 || dtype == NC_BF16, NC_ERR_INVALID_ARG, "rope_qknorm_bwd: bad dtype");
  const int64_t M = (int64_t)B * T;
  if (dtype == NC_BF16 && hd == 128) {
    rope_qknorm_bwd_bf16_kernel<<<(unsigned)cdiv(M * (H + 2), 16), 256, 0, s>>>(
        dhat, static_cast<const bf16*>(yhat), rstd_q, rstd_k, table, M, T, H, static_cast<bf16*>(dqkv));
    return check_launch("rope_qknorm_bwd_bf16_kernel");
  }
  const unsigned blocks = (unsigned)cdiv(M * (H + 2), 4);
  if (dtype == NC_F32)
    rope_qknorm_bwd_kernel<float><<<blocks, 256, 0, s>>>(dhat, static_cast<const float*>(yhat), rstd_q, rstd_k,
                                                         table, M, T, H, hd, static_cast<float*>(dqkv));
  else
    rope_qknorm_bwd_kernel<bf16><<<blocks, 256, 0, s>>>(dhat, static_cast<const bf16*>(yhat), rstd_q, rstd_k,
                                                        table, M, T, H, hd, static_cast<bf16*>(dqkv));
  return check_launch("rope_qknorm_bwd_kernel");
}

}  // namespace nc

extern "C" int nc_rope_table(float* table, int T, int hd, float base, void* stream) {
  return nc::api_done(nc::rope_table(table, T, hd, base, static_cast<hipStream_t>(stream)), stream, "nc_rope_table");
}

extern "C" int nc_rope_qknorm_fwd(void* qkv, int dtype, int B, int T, int H, int hd, const float* table, float eps,
                                  float* rstd_q, float* rstd_k, void* stream) {
  return nc::api_done(nc::rope_qknorm_fwd(qkv, dtype, B, T, H, hd, table, eps, rstd_q, rstd_k, static_cast<hipStream_t>(stream)),
                      stream, "nc_rope_qknorm_fwd");
}

extern "C" int nc_rope_qknorm_bwd(const float* dqkv_hat, const void* qkv_hat, const float* rstd_q,
                                  const float* rstd_k, const float* table, int dtype, int B, int T, int H, int hd,
                                  void* dqkv, void* stream) {
  return nc::api_done(nc::rope_qknorm_bwd(dqkv_hat, qkv_hat, rstd_q, rstd_k, table, dtype, B, T, H, hd, dqkv,
                             static_cast<hipStream_t>(stream)), stream, "nc_rope_qknorm_bwd");
}
