// Untied unembedding, tanh logit softcap and cross entropy, reported as the
// mean loss and as bits per byte.  Release-news page "Karpathy再放大招…",
// section 技術細節與問答: untied embedding/unembedding, logit softcap;
// nano-series page "Karpathy 的 nano 諧系", section nanochat: pretraining loss
// reported in bits per byte.
//
//   z = h U^T, z' = c tanh(z / c), lse_t = log sum_v exp(z'_tv),
//   loss_t = lse_t - z'_{t, y_t}, loss = mean_t loss_t,
//   bpb = sum_t loss_t / (ln 2 * sum_t bytes[y_t]).
//
// Because |z'| < c, exp(z' - c) never overflows, so the softmax needs no
// running maximum: lse = c + log sum exp(z' - c).  The fp32 logits are never
// stored.
//
// bf16 (d a multiple of 64): the logit GEMM's epilogue applies the softcap
// and folds each row's 64-column groups into partial sums of exp(z' - c)
// (and picks z' at the target), so the forward writes only [V/64, M]
// partials.  The backward recomputes the logits with an epilogue that writes
// dz = dloss (softmax(z') - onehot(y)) (1 - (z'/c)^2) in bf16 directly, then
// dh (+)= dz U and dU (+)= dz^T h.  The vocabulary is one chunk unless the
// bf16 dz would exceed 8 GiB.
// The training step instead keeps u = exp(z' - c) (1 - (z'/c)^2) (bf16) from
// the forward's epilogue.  With r_t = dloss exp(c - lse_t) and
// q_t = dloss (1 - (z'_{t,y_t}/c)^2), dz = diag(r) u - q onehot(y), so
//   dh_t = r_t (u U)_t - q_t U[y_t],
//   dU   = u^T (diag(r) h) - sum_t q_t h_t e_{y_t}^T,
// two plain products and row corrections, with no pass over [M, V].
// fp32 (and other shapes): a GEMM writes one [M, Vc] fp32 logit chunk and a
// row kernel folds it (forward) or forms dz from it (backward).
// Partial sums are added in a fixed order and the loss sums in a fixed tree
// order, so results are bitwise reproducible.
#include "common.h"
#include "gemm.h"
#include "ops.h"

namespace nc {
namespace {

constexpr double kLn2 = 0.69314718055994530942;

int chunk_cols(int64_t M, int V) {
  int64_t c = ((int64_t)1 << 28) / std::max<int64_t>(M, 1);  // ~1 GiB of fp32 logits per chunk
  c = c / 256 * 256;
  if (c < 256) c = 256;
  if (c > V) c = V;
  return (int)c;
}

// Fused path: bf16 dz chunk of at most 8 GiB.
int fused_cols(int64_t M, int V) {
  int64_t c = ((int64_t)1 << 32) / std::max<int64_t>(M, 1);
  c = c / 256 * 256;
  if (c < 256) c = 256;
  if (c > V) c = V;
  return (int)c;
}

bool use_fused(int dtype, int d) { return dtype == NC_BF16 && d % 64 == 0; }

struct XentWs {
  int32_t* flag;   // device flag of the public entry points (first int32 of ws)
  float* zbuf;     // [M, Vc] fp32 logit chunk (chunked path)
  void* dz;        // [M, Vc] dtype (backward)
  float* partial;  // [nparts, M]
  float* ztgt;     // [M]
  float* ltok;     // [M]
  float* err;      // [M] u - bf16(u) at the target (stored path)
  float* rs;       // [M] r_t (stored path)
  float* qs;       // [M] q_t, less r_t err_t (stored path)
  void* hs;        // [M, d] bf16 r_t h_t (stored path)
  void* eb_ws;     // target-sorted segmented sums (stored path)
  size_t eb_ws_bytes;
  void* gemm_ws;
  size_t gemm_ws_bytes;
  void* ut;        // U^T [d, V] (bf16 backward)
};

size_t carve(int64_t M, int d, int V, bool fused, XentWs* w, void* base) {
  const int Vc = fused ? fused_cols(M, V) : chunk_cols(M, V);
  const int nparts = fused ? (int)cdiv(V, 64) : (int)cdiv(V, Vc);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes, 256);
    return o;
  };
  const size_t o_f = take(4);
  const size_t o_z = take(fused ? 0 : (size_t)M * Vc * 4);
  const size_t o_dz = take((size_t)M * Vc * (fused ? 2 : 4));
  const size_t o_p = take((size_t)nparts * M * 4);
  const size_t o_t = take((size_t)M * 4);
  const size_t o_l = take((size_t)M * 4);
  const size_t o_e = take((size_t)M * 4);
  const size_t o_rs = take(fused ? (size_t)M * 4 : 0);
  const size_t o_qs = take(fused ? (size_t)M * 4 : 0);
  const size_t o_hs = take(fused ? (size_t)M * d * 2 : 0);
  const size_t ebb = fused ? embed_bwd_workspace_bytes(M, V, d) : 0;
  const size_t o_eb = take(ebb);
  // split-K partials of dU (Vc x d, K = M) and of dh (M x d, K = Vc)
  const size_t gwb = std::max(gemm_workspace_bytes(Vc, d, M), gemm_workspace_bytes(M, d, Vc));
  const size_t o_g = take(gwb);
  const size_t o_ut = take((size_t)V * d * 2);
  if (w) {
    char* b = static_cast<char*>(base);
    w->flag = reinterpret_cast<int32_t*>(b + o_f);
    w->zbuf = reinterpret_cast<float*>(b + o_z);
    w->dz = b + o_dz;
    w->partial = reinterpret_cast<float*>(b + o_p);
    w->ztgt = reinterpret_cast<float*>(b + o_t);
    w->ltok = reinterpret_cast<float*>(b + o_l);
    w->err = reinterpret_cast<float*>(b + o_e);
    w->rs = reinterpret_cast<float*>(b + o_rs);
    w->qs = reinterpret_cast<float*>(b + o_qs);
    w->hs = b + o_hs;
    w->eb_ws = ebb ? b + o_eb : nullptr;
    w->eb_ws_bytes = ebb;
    w->gemm_ws = gwb ? b + o_g : nullptr;
    w->gemm_ws_bytes = gwb;
    w->ut = b + o_ut;
  }
  return off;
}

// Before the logit product: z' at the target starts at 0 for every row, so a
// row whose target lies outside [0, V) (which no column matches) reads a
// defined value; such rows raise the device flag.
__global__ void xent_prep_kernel(const int32_t* __restrict__ tgt, int64_t M, int V, float* __restrict__ ztgt,
                                 float* __restrict__ err, int32_t* __restrict__ flag) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < M; r += (int64_t)gridDim.x * blockDim.x) {
    ztgt[r] = 0.f;
    err[r] = 0.f;
    if ((uint32_t)tgt[r] >= (uint32_t)V) *flag = 1;
  }
}

// One wavefront per row of the chunk: partial sum of exp(z' - c) and, when
// the row's target falls in the chunk, z' at the target.
__global__ __launch_bounds__(256) void xent_fwd_rows_kernel(const float* __restrict__ z, int64_t M, int Vc, int v0,
                                                            float c, const int32_t* __restrict__ tgt,
                                                            float* __restrict__ partial,
                                                            float* __restrict__ ztgt) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* zr = z + row * Vc;
  const int y = tgt[row] - v0;
  const float inv_c = 1.f / c;
  float s = 0.f;
  for (int v = lane * 4; v < Vc; v += 256) {
    const float4 q = *reinterpret_cast<const float4*>(zr + v);
    const float a = c * tanhf(q.x * inv_c), b = c * tanhf(q.y * inv_c);
    const float e = c * tanhf(q.z * inv_c), f = c * tanhf(q.w * inv_c);
    s += expf(a - c) + expf(b - c) + expf(e - c) + expf(f - c);
    if (y >= v && y < v + 4) ztgt[row] = y == v ? a : (y == v + 1 ? b : (y == v + 2 ? e : f));
  }
  s = wave_sum(s);
  if (lane == 0) partial[row] = s;
}

__global__ void xent_finish_kernel(const float* __restrict__ partial, int nch, int64_t M, float c,
                                   const float* __restrict__ ztgt, float* __restrict__ lse,
                                   float* __restrict__ ltok_ws, float* __restrict__ loss_tok) {
  for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < M; r += (int64_t)gridDim.x * blockDim.x) {
    // Sequential sum over the parts; the loads of 16 parts are issued
    // together so one wave per SIMD keeps enough reads in flight.
    float s = 0.f;
    int k = 0;
    for (; k + 16 <= nch; k += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = partial[(int64_t)(k + u) * M + r];
#pragma unroll
      for (int u = 0; u < 16; ++u) s += v[u];
    }
    for (; k < nch; ++k) s += partial[(int64_t)k * M + r];
    const float L = c + logf(s);
    lse[r] = L;
    const float lt = L - ztgt[r];
    ltok_ws[r] = lt;
    if (loss_tok) loss_tok[r] = lt;
  }
}

// Single block: fixed-order sums of the per-token losses and target bytes.
__global__ __launch_bounds__(1024) void xent_reduce_kernel(const float* __restrict__ ltok, int64_t M,
                                                           const int32_t* __restrict__ tgt, int V,
                                                           const float* __restrict__ token_bytes,
                                                           float default_bytes, float* loss, float* bpb) {
  __shared__ double sl[1024];
  __shared__ double sb[1024];
  double a = 0.0, b = 0.0;
  for (int64_t i = threadIdx.x; i < M; i += 1024) {
    a += (double)ltok[i];
    // a target outside [0, V) (flagged by xent_prep_kernel) counts no bytes
    const uint32_t y = (uint32_t)tgt[i];
    b += token_bytes ? (y < (uint32_t)V ? (double)token_bytes[y] : 0.0) : (double)default_bytes;
  }
  sl[threadIdx.x] = a;
  sb[threadIdx.x] = b;
  __syncthreads();
  for (int o = 512; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      sl[threadIdx.x] += sl[threadIdx.x + o];
      sb[threadIdx.x] += sb[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *loss = (float)(sl[0] / (double)M);
    *bpb = (float)(sl[0] / (kLn2 * sb[0]));
  }
}

// dz[t, v] = dloss (exp(z' - lse_t) - [v0 + v == y_t]) (1 - (z'/c)^2).
template <typename T>
__global__ __launch_bounds__(256) void xent_bwd_rows_kernel(const float* __restrict__ z, int64_t M, int Vc, int v0,
                                                            float c, const int32_t* __restrict__ tgt,
                                                            const float* __restrict__ lse, float dloss,
                                                            T* __restrict__ dz) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float* zr = z + row * Vc;
  T* dr = dz + row * Vc;
  const int y = tgt[row] - v0;
  const float L = lse[row];
  const float inv_c = 1.f / c;
  for (int v = lane; v < Vc; v += 64) {
    const float th = tanhf(zr[v] * inv_c);
    const float p = expf(c * th - L);
    const float g = dloss * (p - (v == y ? 1.f : 0.f)) * (1.f - th * th);
    st(dr + v, g);
  }
}

// Stored path, per row t (one wavefront, 4 rows per block):
// r_t = dloss exp(c - lse_t); q_t = dloss (1 - (z'_{t,y}/c)^2) - r_t err_t for
// a target in [0, V), else 0 (such a row has no one-hot term); hs_t = bf16(r_t h_t).
// The err term makes r_t bf16(u_ty) - q_t equal the fp32 r_t u_ty - dloss (1 - th^2).
__global__ __launch_bounds__(256) void xent_rowscale_kernel(const bf16* __restrict__ h, const float* __restrict__ lse,
                                                            const float* __restrict__ ztgt,
                                                            const float* __restrict__ err,
                                                            const int32_t* __restrict__ tgt, int64_t M, int d, int V,
                                                            float c, float dloss, float* __restrict__ rs,
                                                            float* __restrict__ qs, bf16* __restrict__ hs) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const float r = dloss * expf(c - lse[row]);
  if (lane == 0) {
    const float th = ztgt[row] / c;
    rs[row] = r;
    qs[row] = (uint32_t)tgt[row] < (uint32_t)V ? dloss * (1.f - th * th) - r * err[row] : 0.f;
  }
  for (int col = lane * 4; col < d; col += 256) {
    const uint2 u = *reinterpret_cast<const uint2*>(h + row * d + col);
    *reinterpret_cast<uint2*>(hs + row * d + col) =
        make_uint2(pack_bf16x2(r * __uint_as_float(u.x << 16), r * __uint_as_float(u.x & 0xffff0000u)),
                   pack_bf16x2(r * __uint_as_float(u.y << 16), r * __uint_as_float(u.y & 0xffff0000u)));
  }
}

int validate(const void* h, const void* U, int dtype, const int32_t* tgt, int64_t M, int d, int V) {
  NC_REQUIRE(h && U && tgt, NC_ERR_INVALID_ARG, "softcap_xent: null pointer");
  NC_REQUIRE(M > 0 && d > 0 && V > 0, NC_ERR_INVALID_ARG, "softcap_xent: bad shape");
  NC_REQUIRE(d % 8 == 0 && V % 8 == 0 && M % 8 == 0, NC_ERR_UNSUPPORTED,
             "softcap_xent: M, d and V must be multiples of 8");
  NC_REQUIRE(dtype == NC_F32 || dtype == NC_BF16, NC_ERR_INVALID_ARG, "softcap_xent: bad dtype");
  return NC_OK;
}

}  // namespace

size_t xent_workspace_bytes(int64_t M, int d, int V) {
  return std::max(carve(M, d, V, false, nullptr, nullptr), carve(M, d, V, true, nullptr, nullptr));
}

int xent_fwd(const void* h, const void* U, int dtype, const int32_t* tgt, const float* token_bytes, int64_t M, int d,
             int V, float softcap, float* lse, float* loss_tok, float* loss, float* bpb, void* ws, size_t ws_bytes,
             hipStream_t s, bool store_logits, bool* stored, int32_t* flag) {
  if (stored) *stored = false;
  NC_TRY(validate(h, U, dtype, tgt, M, d, V));
  NC_REQUIRE(lse && loss && bpb, NC_ERR_INVALID_ARG, "softcap_xent_fwd: null output");
  NC_REQUIRE(softcap > 0.f, NC_ERR_INVALID_ARG, "softcap_xent_fwd: softcap must be positive");
  NC_REQUIRE(ws && ws_bytes >= xent_workspace_bytes(M, d, V), NC_ERR_WORKSPACE,
             "softcap_xent_fwd: workspace too small");
  const bool fused = use_fused(dtype, d);
  XentWs w;
  carve(M, d, V, fused, &w, ws);
  const int Vc = fused ? fused_cols(M, V) : chunk_cols(M, V);
  const int nch = (int)cdiv(V, Vc);
  const size_t esz = dtype == NC_BF16 ? 2 : 4;
  if (!flag) {  // public entry point: the flag lives in ws and starts clear
    flag = w.flag;
    NC_TRY(fill_zero(flag, 4, s));
  }
  xent_prep_kernel<<<(unsigned)std::min<int64_t>(cdiv(M, 256), 1024), 256, 0, s>>>(tgt, M, V, w.ztgt, w.err, flag);
  NC_TRY(check_launch("xent_prep_kernel"));
  for (int k = 0; k < nch; ++k) {
    const int v0 = k * Vc;
    const int n = std::min(Vc, V - v0);
    GemmDesc g;
    g.transA = 0;
    g.transB = 1;
    g.M = M;
    g.N = n;
    g.K = d;
    g.A = h;
    g.lda = d;
    g.B = static_cast<const char*>(U) + (size_t)v0 * d * esz;
    g.ldb = d;
    g.dtype = dtype;
    if (fused) {
      g.xent = 1;
      g.xc = softcap;
      g.xtgt = tgt;
      g.xpart = w.partial;
      g.xztgt = w.ztgt;
      g.xv0 = v0;
      if (store_logits && nch == 1) {
        g.C = w.dz;
        g.xerr = w.err;
        g.ldc = n;
        if (stored) *stored = true;
      }
      NC_TRY(gemm(g, s));
      continue;
    }
    g.C = w.zbuf;
    g.cdt = NC_F32;
    g.ldc = n;
    NC_TRY(gemm(g, s));
    xent_fwd_rows_kernel<<<(unsigned)cdiv(M, 4), 256, 0, s>>>(w.zbuf, M, n, v0, softcap, tgt,
                                                              w.partial + (int64_t)k * M, w.ztgt);
    NC_TRY(check_launch("xent_fwd_rows_kernel"));
  }
  const int nparts = fused ? (int)cdiv(V, 64) : nch;
  xent_finish_kernel<<<(unsigned)std::min<int64_t>(cdiv(M, 256), 4096), 256, 0, s>>>(w.partial, nparts, M, softcap,
                                                                                       w.ztgt, lse, w.ltok, loss_tok);
  NC_TRY(check_launch("xent_finish_kernel"));
  xent_reduce_kernel<<<1, 1024, 0, s>>>(w.ltok, M, tgt, V, token_bytes, 4.8f, loss, bpb);
  return check_launch("xent_reduce_kernel");
}

int xent_bwd(const void* h, const void* U, int dtype, const int32_t* tgt, const float* lse, int64_t M, int d, int V,
             float softcap, float dloss, float* dh, int dh_acc, float* dU, int dU_acc, void* ws, size_t ws_bytes,
             hipStream_t s, bool from_stored, GradRowFix* defer_fix) {
  NC_TRY(validate(h, U, dtype, tgt, M, d, V));
  NC_REQUIRE(lse && dh && dU, NC_ERR_INVALID_ARG, "softcap_xent_bwd: null pointer");
  NC_REQUIRE(softcap > 0.f, NC_ERR_INVALID_ARG, "softcap_xent_bwd: softcap must be positive");
  NC_REQUIRE(ws && ws_bytes >= xent_workspace_bytes(M, d, V), NC_ERR_WORKSPACE,
             "softcap_xent_bwd: workspace too small");
  const bool fused = use_fused(dtype, d);
  XentWs w;
  carve(M, d, V, fused, &w, ws);
  const int Vc = fused ? fused_cols(M, V) : chunk_cols(M, V);
  const int nch = (int)cdiv(V, Vc);
  const size_t esz = dtype == NC_BF16 ? 2 : 4;
  if (dtype == NC_BF16) NC_TRY(transpose(U, V, d, 2, w.ut, s));
  if (fused && from_stored) {
    NC_REQUIRE(nch == 1 && !dh_acc && defer_fix, NC_ERR_INVALID_ARG,
               "softcap_xent_bwd: the stored path needs a one-chunk vocabulary, a fresh dh and a deferred row fix");
    const unsigned rb = (unsigned)cdiv(M, 4);
    xent_rowscale_kernel<<<rb, 256, 0, s>>>(static_cast<const bf16*>(h), lse, w.ztgt, w.err, tgt, M, d, V, softcap,
                                            dloss, w.rs, w.qs, static_cast<bf16*>(w.hs));
    NC_TRY(check_launch("xent_rowscale_kernel"));
    // dh = r (u U) - q U[y]: the product through U^T (K-contiguous); the row
    // fix goes to the caller, whose norm backward applies it as it reads dh
    GemmDesc gh;
    gh.transA = 0;
    gh.transB = 1;
    gh.M = M;
    gh.N = d;
    gh.K = V;
    gh.A = w.dz;
    gh.lda = V;
    gh.B = w.ut;
    gh.ldb = V;
    gh.C = dh;
    gh.cdt = NC_F32;
    gh.ldc = d;
    gh.dtype = NC_BF16;
    gh.ws = w.gemm_ws;
    gh.ws_bytes = w.gemm_ws_bytes;
    NC_TRY(gemm(gh, s));
    *defer_fix = GradRowFix{w.rs, w.qs, tgt, static_cast<const bf16*>(U), V};
    // dU (+)= u^T (r h), then dU[y_t] -= q_t h_t in target order
    GemmDesc gu;
    gu.transA = 1;
    gu.transB = 0;
    gu.M = V;
    gu.N = d;
    gu.K = M;
    gu.A = w.dz;
    gu.lda = V;
    gu.B = w.hs;
    gu.ldb = d;
    gu.C = dU;
    gu.cdt = NC_F32;
    gu.ldc = d;
    gu.beta = dU_acc ? 1.f : 0.f;
    gu.dtype = NC_BF16;
    gu.ws = w.gemm_ws;
    gu.ws_bytes = w.gemm_ws_bytes;
    NC_TRY(gemm(gu, s));
    return embed_bwd_scaled(tgt, M, static_cast<const bf16*>(h), w.qs, -1.f, d, dU, V, 1, w.eb_ws, w.eb_ws_bytes, s);
  }
  for (int k = 0; k < nch; ++k) {
    const int v0 = k * Vc;
    const int n = std::min(Vc, V - v0);
    const void* Uc = static_cast<const char*>(U) + (size_t)v0 * d * esz;
    GemmDesc g;
    g.transA = 0;
    g.transB = 1;
    g.M = M;
    g.N = n;
    g.K = d;
    g.A = h;
    g.lda = d;
    g.B = Uc;
    g.ldb = d;
    g.dtype = dtype;
    if (fused) {
      g.xent = 2;
      g.xc = softcap;
      g.xdl = dloss;
      g.xtgt = tgt;
      g.xlse = lse;
      g.xv0 = v0;
      g.C = w.dz;
      g.cdt = NC_BF16;
      g.ldc = n;
      NC_TRY(gemm(g, s));
    } else {
      g.C = w.zbuf;
      g.cdt = NC_F32;
      g.ldc = n;
      NC_TRY(gemm(g, s));
      if (dtype == NC_BF16)
        xent_bwd_rows_kernel<bf16><<<(unsigned)cdiv(M, 4), 256, 0, s>>>(w.zbuf, M, n, v0, softcap, tgt, lse, dloss,
                                                                         static_cast<bf16*>(w.dz));
      else
        xent_bwd_rows_kernel<float><<<(unsigned)cdiv(M, 4), 256, 0, s>>>(w.zbuf, M, n, v0, softcap, tgt, lse, dloss,
                                                                          static_cast<float*>(w.dz));
      NC_TRY(check_launch("xent_bwd_rows_kernel"));
    }
    // dh (+)= dz U_c  : [M, n] x [n, d]; in bf16 through U^T (K-contiguous)
    GemmDesc gh;
    gh.transA = 0;
    gh.M = M;
    gh.N = d;
    gh.K = n;
    gh.A = w.dz;
    gh.lda = n;
    if (dtype == NC_BF16) {
      gh.transB = 1;
      gh.B = static_cast<const bf16*>(w.ut) + v0;
      gh.ldb = V;
    } else {
      gh.transB = 0;
      gh.B = Uc;
      gh.ldb = d;
    }
    gh.C = dh;
    gh.cdt = NC_F32;
    gh.ldc = d;
    gh.beta = (k > 0 || dh_acc) ? 1.f : 0.f;
    gh.dtype = dtype;
    gh.ws = w.gemm_ws;
    gh.ws_bytes = w.gemm_ws_bytes;
    NC_TRY(gemm(gh, s));
    // dU_c (+)= dz^T h : [n, M] x [M, d]
    GemmDesc gu;
    gu.transA = 1;
    gu.transB = 0;
    gu.M = n;
    gu.N = d;
    gu.K = M;
    gu.A = w.dz;
    gu.lda = n;
    gu.B = h;
    gu.ldb = d;
    gu.C = dU + (size_t)v0 * d;
    gu.cdt = NC_F32;
    gu.ldc = d;
    gu.beta = dU_acc ? 1.f : 0.f;
    gu.dtype = dtype;
    gu.ws = w.gemm_ws;
    gu.ws_bytes = w.gemm_ws_bytes;
    NC_TRY(gemm(gu, s));
  }
  return NC_OK;
}

}  // namespace nc

extern "C" size_t nc_softcap_xent_workspace_bytes(int64_t M, int d, int V) { return nc::xent_workspace_bytes(M, d, V); }

extern "C" int nc_softcap_xent_fwd(const void* h, const void* U, int dtype, const int32_t* tgt,
                                   const float* token_bytes, int64_t M, int d, int V, float softcap, float* lse,
                                   float* loss_tok, float* loss, float* bpb, void* ws, size_t ws_bytes, void* stream) {

                       return nc::api_done(nc::xent_fwd(h, U, dtype, tgt, token_bytes, M, d, V, softcap, lse, loss_tok, loss, bpb, ws, ws_bytes,
                      static_cast<hipStream_t>(stream)), stream, "nc_softcap_xent_fwd");
}

extern "C" int nc_softcap_xent_bwd(const void* h, const void* U, int dtype, const int32_t* tgt, const float* lse,
                                   int64_t M, int d, int V, float softcap, float dloss, float* dh, int dh_accumulate,
                                   float* dU, int dU_accumulate, void* ws, size_t ws_bytes, void* stream) {

                       return nc::api_done(nc::xent_bwd(h, U, dtype, tgt, lse, M, d, V, softcap, dloss, dh, dh_accumulate, dU, dU_accumulate, ws,
                      ws_bytes, static_cast<hipStream_t>(stream)), stream, "nc_softcap_xent_bwd");
}
