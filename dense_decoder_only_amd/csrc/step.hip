// One training step of the nanochat-style dense decoder: forward and backward
// of the mean next-token loss, with no host sync, on the caller's stream.
// (Built with NC_STEP_SIDE_STREAM=1 the weight-gradient products of the
// backward run on a second, library-owned stream forked from and joined back
// to the caller's stream with events.)
//
// Model (release-news page "Karpathy再放大招…", section 技術細節與問答):
//   x = rms(E[ids])                                  token embedding + norm
//   per layer:  a = rms(x); [q|k|v] = a Wqkv^T; q,k <- rms_hd(rope(q,k))
//               x += mqa(q, k, v) Wo^T               multi-query attention
//               m = rms(x); x += relu(m W1^T)^2 W2^T relu^2 MLP
//   h = rms(x); z' = c tanh(h U^T / c); loss = mean CE(z', y)
// plus bits per byte (nano-series page "Karpathy 的 nano 諧系", section
// nanochat).  Readings where the pages are silent: eps 1e-6 for every norm,
// a final norm before U, RoPE before the QK norm, scale 1/sqrt(hd), c = 15.
//
// Saved for the backward (per layer, in the config dtype): the normalized
// inputs a and m with their rstd, the post-norm qkv, the attention output o
// and its log-sum-exp, and relu(u)^2 of the MLP pre-activation u.  The
// residual stream and all gradients are fp32.
#include "common.h"
#include "gemm.h"
#include "ops.h"

#include <mutex>

namespace nc {
namespace {

// Weight-gradient products on a side stream overlapping the
// activation-gradient chain.  Measured at d20 it gains 1.2% of step time but
// stretches every concurrent kernel (both streams share the CUs), so the
// per-kernel timings stop describing the kernels; off by default.
#ifndef NC_STEP_SIDE_STREAM
#define NC_STEP_SIDE_STREAM 0
#endif

// Versions of a scratch buffer that the side stream may still be reading
// while the main stream writes the next one.
constexpr int kRing = NC_STEP_SIDE_STREAM ? 2 : 1;

struct Layer {
  void *a, *qkv, *o, *m, *a2;  // a2 = relu(u)^2; u itself is not kept
  float *rstd_a, *rstd_q, *rstd_k, *lse, *rstd_m;
};

struct StepWs {
  int32_t* flag;
  float* table;
  float *x, *x0, *rstd0;
  void* h;
  float *rstd_f, *lse_ce;
  void* g_lp[kRing];  // bf16 copies of the residual gradient (read by the side stream)
  float* dm;
  void *du[kRing], *dout, *dqkv[kRing];
  float* dqkv_hat;
  void* wt;  // one layer's transposed weights (bf16 backward): Wqkv^T, Wo^T, W1^T, W2^T
  void *attn_ws, *gemm_ws, *xent_ws, *emb_ws;
  size_t attn_ws_bytes, gemm_ws_bytes, xent_ws_bytes, emb_ws_bytes;
  Layer* layers;  // host array filled by carve
};


// The side stream and a pool of events, one set per device, created on first
// use and kept for the life of the process.  Enqueueing a step holds the
// mutex, so concurrent steps on one device share the side stream in order.
struct SideCtx {
  hipStream_t s2 = nullptr;
  std::vector<hipEvent_t> ev;
  int next = 0;
};
std::mutex g_side_mu;
SideCtx g_side[64];

int side_ctx(SideCtx** out) {
  int dev = 0;
  NC_CHECK_HIP(hipGetDevice(&dev));
  NC_REQUIRE(dev >= 0 && dev < 64, NC_ERR_UNSUPPORTED, "step: device index %d", dev);
  SideCtx& c = g_side[dev];
  if (!c.s2) {
    NC_CHECK_HIP(hipStreamCreateWithFlags(&c.s2, hipStreamNonBlocking));
    c.ev.resize(512);
    for (auto& e : c.ev) NC_CHECK_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  }
  *out = &c;
  return NC_OK;
}

// `to` waits for everything enqueued on `from` so far.
int stream_dep(SideCtx* c, hipStream_t from, hipStream_t to) {
  hipEvent_t e = c->ev[c->next];
  c->next = (c->next + 1) % (int)c->ev.size();
  NC_CHECK_HIP(hipEventRecord(e, from));
  NC_CHECK_HIP(hipStreamWaitEvent(to, e, 0));
  return NC_OK;
}

int validate_cfg(const nc_config* c) {
  NC_REQUIRE(c, NC_ERR_INVALID_ARG, "step: null config");
  NC_REQUIRE(c->n_layer > 0 && c->d_model > 0 && c->n_head > 0 && c->head_dim > 0 && c->d_ff > 0 &&
                 c->vocab > 0 && c->seq_len > 0 && c->batch > 0,
             NC_ERR_INVALID_ARG, "step: every size must be positive");
  NC_REQUIRE(c->n_kv_head == 1, NC_ERR_INVALID_ARG, "step: n_kv_head must be 1 (multi-query attention)");
  NC_REQUIRE(c->n_head * c->head_dim == c->d_model, NC_ERR_INVALID_ARG, "step: n_head * head_dim must equal d_model");
  NC_REQUIRE(c->head_dim == 64 || c->head_dim == 128, NC_ERR_UNSUPPORTED, "step: head_dim must be 64 or 128");
  NC_REQUIRE(c->d_model % 8 == 0 && c->d_ff % 8 == 0 && c->vocab % 8 == 0, NC_ERR_UNSUPPORTED,
             "step: d_model, d_ff and vocab must be multiples of 8");
  NC_REQUIRE(((int64_t)c->batch * c->seq_len) % 8 == 0, NC_ERR_UNSUPPORTED, "step: batch * seq_len must be a multiple of 8");
  NC_REQUIRE(c->dtype == NC_F32 || c->dtype == NC_BF16, NC_ERR_INVALID_ARG, "step: bad dtype");
  NC_REQUIRE(c->softcap > 0.f && c->eps >= 0.f && c->rope_base > 0.f, NC_ERR_INVALID_ARG, "step: bad constants");
  return NC_OK;
}

size_t carve(const nc_config* c, StepWs* w, void* base) {
  const int64_t M = (int64_t)c->batch * c->seq_len;
  const int64_t d = c->d_model, H = c->n_head, hd = c->head_dim, F = c->d_ff, L = c->n_layer;
  const int64_t Q = (H + 2) * hd;
  const size_t e = c->dtype == NC_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes, 256);
    return o;
  };
  char* b = static_cast<char*>(base);
  auto ptr = [&](size_t o) -> void* { return b ? b + o : nullptr; };
  const size_t o_flag = take(4), o_tab = take((size_t)c->seq_len * hd * 4);
  const size_t o_x = take(M * d * 4), o_x0 = take(M * d * 4), o_r0 = take(M * 4);
  const size_t o_h = take(M * d * e), o_rf = take(M * 4), o_lce = take(M * 4);
  size_t o_glp[kRing], o_du[kRing], o_dq[kRing];
  for (int r = 0; r < kRing; ++r) o_glp[r] = take(M * d * e);
  const size_t o_dm = take(M * d * 4);
  for (int r = 0; r < kRing; ++r) o_du[r] = take(M * F * e);
  const size_t o_do = take(M * H * hd * e);
  for (int r = 0; r < kRing; ++r) o_dq[r] = take(M * Q * e);
  const size_t o_dqh = take(M * Q * 4);
  const size_t o_wt = take((size_t)(Q * d + d * H * hd + 2 * F * d) * e);
  const size_t attn_b = mqa_attn_bwd_workspace_bytes(c->batch, c->seq_len, (int)H);
  size_t gemm_b = 0;
  gemm_b = std::max(gemm_b, gemm_workspace_bytes(F, d, M));
  gemm_b = std::max(gemm_b, gemm_workspace_bytes(d, F, M));
  gemm_b = std::max(gemm_b, gemm_workspace_bytes(d, H * hd, M));
  gemm_b = std::max(gemm_b, gemm_workspace_bytes(Q, d, M));
  const size_t xent_b = xent_workspace_bytes(M, (int)d, c->vocab);
  const size_t emb_b = embed_bwd_workspace_bytes(M, c->vocab, (int)d);
  const size_t o_aws = take(attn_b), o_gws = take(gemm_b), o_xws = take(xent_b), o_ews = take(emb_b);
  if (w) {
    w->flag = static_cast<int32_t*>(ptr(o_flag));
    w->table = static_cast<float*>(ptr(o_tab));
    w->x = static_cast<float*>(ptr(o_x));
    w->x0 = static_cast<float*>(ptr(o_x0));
    w->rstd0 = static_cast<float*>(ptr(o_r0));
    w->h = ptr(o_h);
    w->rstd_f = static_cast<float*>(ptr(o_rf));
    w->lse_ce = static_cast<float*>(ptr(o_lce));
    for (int r = 0; r < kRing; ++r) {
      w->g_lp[r] = ptr(o_glp[r]);
      w->du[r] = ptr(o_du[r]);
      w->dqkv[r] = ptr(o_dq[r]);
    }
    w->dm = static_cast<float*>(ptr(o_dm));
    w->dout = ptr(o_do);
    w->dqkv_hat = static_cast<float*>(ptr(o_dqh));
    w->wt = ptr(o_wt);
    w->attn_ws = ptr(o_aws);
    w->attn_ws_bytes = attn_b;
    w->gemm_ws = gemm_b ? ptr(o_gws) : nullptr;
    w->gemm_ws_bytes = gemm_b;
    w->xent_ws = ptr(o_xws);
    w->xent_ws_bytes = xent_b;
    w->emb_ws = ptr(o_ews);
    w->emb_ws_bytes = emb_b;
  }
  for (int64_t l = 0; l < L; ++l) {
    const size_t o_a = take(M * d * e), o_ra = take(M * 4), o_qkv = take(M * Q * e), o_rq = take(M * H * 4),
                 o_rk = take(M * 4), o_o = take(M * H * hd * e), o_lse = take(M * H * 4), o_m = take(M * d * e),
                 o_rm = take(M * 4), o_a2 = take(M * F * e);
    if (w) {
      Layer& ly = w->layers[l];
      ly.a = ptr(o_a);
      ly.rstd_a = static_cast<float*>(ptr(o_ra));
      ly.qkv = ptr(o_qkv);
      ly.rstd_q = static_cast<float*>(ptr(o_rq));
      ly.rstd_k = static_cast<float*>(ptr(o_rk));
      ly.o = ptr(o_o);
      ly.lse = static_cast<float*>(ptr(o_lse));
      ly.m = ptr(o_m);
      ly.rstd_m = static_cast<float*>(ptr(o_rm));
      ly.a2 = ptr(o_a2);
    }
  }
  return off;
}

GemmDesc mk(int ta, int tb, int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
            void* C, int cdt, int64_t ldc, int dtype) {
  GemmDesc g;
  g.transA = ta;
  g.transB = tb;
  g.M = M;
  g.N = N;
  g.K = K;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.ldb = ldb;
  g.C = C;
  g.cdt = cdt;
  g.ldc = ldc;
  g.dtype = dtype;
  return g;
}

}  // namespace

size_t step_workspace_bytes(const nc_config* c) {
  if (validate_cfg(c) != NC_OK) return 0;
  return carve(c, nullptr, nullptr);
}

int step_fwd_bwd(const nc_config* c, const nc_params* p, const nc_grads* gr, const int32_t* ids, const int32_t* tgt,
                 const float* token_bytes, void* ws, size_t ws_bytes, float* loss, float* bpb, float* loss_tok,
                 hipStream_t s) {
  NC_TRY(validate_cfg(c));
  NC_REQUIRE(p && gr && ids && tgt && ws && loss && bpb, NC_ERR_INVALID_ARG, "step: null pointer");
  NC_REQUIRE(p->embed && p->w_qkv && p->w_o && p->w_fc && p->w_proj && p->unembed, NC_ERR_INVALID_ARG,
             "step: null parameter");
  NC_REQUIRE(gr->embed && gr->w_qkv && gr->w_o && gr->w_fc && gr->w_proj && gr->unembed, NC_ERR_INVALID_ARG,
             "step: null gradient");
  NC_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255u) == 0, NC_ERR_INVALID_ARG, "step: ws must be 256-byte aligned");
  const size_t need = carve(c, nullptr, nullptr);
  NC_REQUIRE(ws_bytes >= need, NC_ERR_WORKSPACE, "step: workspace too small (%zu < %zu)", ws_bytes, need);

  const int dt = c->dtype;
  const size_t e = dt == NC_BF16 ? 2 : 4;
  const int B = c->batch, T = c->seq_len, H = c->n_head, hd = c->head_dim, L = c->n_layer, V = c->vocab;
  const int64_t M = (int64_t)B * T, d = c->d_model, F = c->d_ff, Q = (int64_t)(H + 2) * hd, HD = (int64_t)H * hd;
  const float scale = 1.f / sqrtf((float)hd);
  const int acc = gr->accumulate ? 1 : 0;

  std::vector<Layer> layers(L);
  StepWs w;
  w.layers = layers.data();
  carve(c, &w, ws);

  auto wl = [&](const void* base, int64_t l, int64_t per) -> const void* {
    return static_cast<const char*>(base) + (size_t)l * per * e;
  };

  // ---------------------------------------------------------------- forward
  NC_TRY(fill_zero(w.flag, 4, s));
  NC_TRY(rope_table(w.table, T, hd, c->rope_base, s));
  // x0 (kept for the embedding norm's backward) and the residual stream x start equal
  NC_TRY(embed_fwd(ids, M, p->embed, dt, V, (int)d, nullptr, w.x0, w.rstd0, c->eps, w.flag, s, w.x));

  for (int l = 0; l < L; ++l) {
    Layer& ly = layers[l];
    NC_TRY(rmsnorm_fwd(w.x, NC_F32, M, (int)d, c->eps, ly.a, dt, ly.rstd_a, s));
    NC_TRY(gemm(mk(0, 1, M, Q, d, ly.a, d, wl(p->w_qkv, l, Q * d), d, ly.qkv, dt, Q, dt), s));
    NC_TRY(rope_qknorm_fwd(ly.qkv, dt, B, T, H, hd, w.table, c->eps, ly.rstd_q, ly.rstd_k, s));
    NC_TRY(mqa_attn_fwd(ly.qkv, dt, B, T, H, hd, scale, ly.o, ly.lse, s));
    GemmDesc go = mk(0, 1, M, d, HD, ly.o, HD, wl(p->w_o, l, d * HD), HD, w.x, NC_F32, d, dt);
    go.beta = 1.f;
    NC_TRY(gemm(go, s));
    NC_TRY(rmsnorm_fwd(w.x, NC_F32, M, (int)d, c->eps, ly.m, dt, ly.rstd_m, s));
    GemmDesc gf = mk(0, 1, M, F, d, ly.m, d, wl(p->w_fc, l, F * d), d, ly.a2, dt, F, dt);
    gf.epi = NC_EPI_RELU2_SQ;  // only relu(u)^2 is stored; the backward takes relu(u) = sqrt of it
    NC_TRY(gemm(gf, s));
    GemmDesc gp = mk(0, 1, M, d, F, ly.a2, F, wl(p->w_proj, l, d * F), F, w.x, NC_F32, d, dt);
    gp.beta = 1.f;
    NC_TRY(gemm(gp, s));
  }
  NC_TRY(rmsnorm_fwd(w.x, NC_F32, M, (int)d, c->eps, w.h, dt, w.rstd_f, s));
  bool logits_stored = false;
  NC_TRY(xent_fwd(w.h, p->unembed, dt, tgt, token_bytes, M, (int)d, V, c->softcap, w.lse_ce, loss_tok, loss, bpb,
                  w.xent_ws, w.xent_ws_bytes, s, d <= 2048, &logits_stored, w.flag));

  // --------------------------------------------------------------- backward
  // Side stream: the weight-gradient products dW = dY^T X, which nothing in
  // the backward reads.  Each fork makes the side stream wait for the main
  // stream's work so far; before the main stream rewrites a ring buffer it
  // waits for the side stream's work so far (which includes the last reader
  // of that buffer).
  std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
  SideCtx* side = nullptr;
  hipStream_t s2 = s;
  if (NC_STEP_SIDE_STREAM) {
    side_lock.lock();
    NC_TRY(side_ctx(&side));
    s2 = side->s2;
  }
  auto fork = [&]() -> int { return side ? stream_dep(side, s, s2) : NC_OK; };
  auto join = [&]() -> int { return side ? stream_dep(side, s2, s) : NC_OK; };
  int gv = 0, uv = 0, qv = 0;  // ring versions of g_lp, du, dqkv
  // read_done[buffer][slot]: recorded on the side stream after the last side
  // reader of the version in that slot; the main stream waits for it before
  // writing the slot's next version.
  hipEvent_t read_done[3][kRing] = {};
  auto mark_read = [&](int buf, int v) -> int {
    if (!side) return NC_OK;
    hipEvent_t e = side->ev[side->next];
    side->next = (side->next + 1) % (int)side->ev.size();
    NC_CHECK_HIP(hipEventRecord(e, s2));
    read_done[buf][v % kRing] = e;
    return NC_OK;
  };
  auto reuse = [&](int buf, int v) -> int {
    if (side && read_done[buf][v % kRing]) NC_CHECK_HIP(hipStreamWaitEvent(s, read_done[buf][v % kRing], 0));
    return NC_OK;
  };
  enum { B_G = 0, B_DU = 1, B_DQ = 2 };

  float* g = w.x;  // the residual stream is dead: reuse it for its gradient
  auto gop_of = [&](int v) -> void* { return dt == NC_BF16 ? w.g_lp[v % kRing] : static_cast<void*>(g); };
  auto glp_out = [&](int v) -> bf16* { return dt == NC_BF16 ? static_cast<bf16*>(w.g_lp[v % kRing]) : nullptr; };
  // with the stored logits, dh comes as u U plus a row fix that the final
  // norm's backward applies as it reads it
  GradRowFix dh_fix{};
  NC_TRY(xent_bwd(w.h, p->unembed, dt, tgt, w.lse_ce, M, (int)d, V, c->softcap, 1.f / (float)M, w.dm, 0,
                  gr->unembed, acc, w.xent_ws, w.xent_ws_bytes, s, logits_stored, &dh_fix));
  NC_TRY(rmsnorm_bwd(w.dm, NC_F32, w.h, dt, w.rstd_f, M, (int)d, g, 0, glp_out(gv), s,
                     dh_fix.rs ? &dh_fix : nullptr));
  // In fp32 the gradient copy is the residual gradient itself, which the
  // main stream keeps updating: the side stream must then run in line.
  if (dt != NC_BF16 && side) {
    side = nullptr;
    s2 = s;
  }

  // In bf16 the activation gradients dX = dY W use the transposed weights so
  // that every product runs in the K-contiguous (x W^T) form.
  const bool tw = dt == NC_BF16;
  // The gradients w.r.t. the pre-attention and pre-MLP norm outputs (products
  // of bf16 operands) are stored in the config dtype: the norm backward reads
  // them once, and in bf16 that halves their write and read.
  const int dyt = dt == NC_BF16 ? NC_BF16 : NC_F32;
  char* wt = static_cast<char*>(w.wt);
  void* WqkvT = wt;
  void* WoT = wt + (size_t)Q * d * e;
  void* W1T = wt + (size_t)(Q * d + d * HD) * e;
  void* W2T = wt + (size_t)(Q * d + d * HD + F * d) * e;
  auto wgrad = [&](GemmDesc gd) -> int {
    gd.beta = (float)acc;
    gd.ws = w.gemm_ws;
    gd.ws_bytes = w.gemm_ws_bytes;
    return gemm(gd, s2);
  };
  for (int l = L - 1; l >= 0; --l) {
    Layer& ly = layers[l];
    const void* Wqkv = wl(p->w_qkv, l, Q * d);
    const void* Wo = wl(p->w_o, l, d * HD);
    const void* W1 = wl(p->w_fc, l, F * d);
    const void* W2 = wl(p->w_proj, l, d * F);
    if (tw) {
      const void* srcs[4] = {Wqkv, Wo, W1, W2};
      void* dsts[4] = {WqkvT, WoT, W1T, W2T};
      const int64_t rs[4] = {Q, d, F, d}, cs[4] = {d, HD, d, F};
      NC_TRY(transpose4(srcs, rs, cs, dsts, 4, s));
    }
    // MLP: x_out = x_mid + relu(m W1^T)^2 W2^T
    void* gop = gop_of(gv);
    NC_TRY(fork());
    NC_TRY(wgrad(mk(1, 0, d, F, M, gop, d, ly.a2, F, gr->w_proj + (size_t)l * d * F, NC_F32, F, dt)));
    NC_TRY(mark_read(B_G, gv));
    void* du = w.du[uv % kRing];
    NC_TRY(reuse(B_DU, uv));
    GemmDesc g2 = tw ? mk(0, 1, M, F, d, gop, d, W2T, d, du, dt, F, dt) : mk(0, 0, M, F, d, gop, d, W2, F, du, dt, F, dt);
    g2.epi = NC_EPI_RELU2_BWD_SQ;
    g2.aux = ly.a2;
    NC_TRY(gemm(g2, s));
    NC_TRY(fork());
    NC_TRY(wgrad(mk(1, 0, F, d, M, du, F, ly.m, d, gr->w_fc + (size_t)l * F * d, NC_F32, d, dt)));
    NC_TRY(mark_read(B_DU, uv));
    ++uv;
    NC_TRY(gemm(tw ? mk(0, 1, M, d, F, du, F, W1T, F, w.dm, dyt, d, dt) : mk(0, 0, M, d, F, du, F, W1, d, w.dm, dyt, d, dt), s));
    ++gv;
    NC_TRY(reuse(B_G, gv));
    NC_TRY(rmsnorm_bwd(w.dm, dyt, ly.m, dt, ly.rstd_m, M, (int)d, g, 1, glp_out(gv), s));
    // attention: x_mid = x_in + mqa(...) Wo^T
    gop = gop_of(gv);
    NC_TRY(fork());
    NC_TRY(wgrad(mk(1, 0, d, HD, M, gop, d, ly.o, HD, gr->w_o + (size_t)l * d * HD, NC_F32, HD, dt)));
    NC_TRY(mark_read(B_G, gv));
    NC_TRY(gemm(tw ? mk(0, 1, M, HD, d, gop, d, WoT, d, w.dout, dt, HD, dt) : mk(0, 0, M, HD, d, gop, d, Wo, HD, w.dout, dt, HD, dt), s));
    void* dqkv = w.dqkv[qv % kRing];
    NC_TRY(reuse(B_DQ, qv));
    if (attn_rope_bwd_fusable(dt, hd)) {
      // the attention backward also applies the QK-norm and RoPE backward
      const AttnRopeBwd fuse{ly.rstd_q, ly.rstd_k, w.table, dqkv};
      NC_TRY(mqa_attn_bwd(ly.qkv, ly.o, w.dout, ly.lse, dt, B, T, H, hd, scale, nullptr, w.attn_ws, w.attn_ws_bytes, s,
                          &fuse));
    } else {
      NC_TRY(mqa_attn_bwd(ly.qkv, ly.o, w.dout, ly.lse, dt, B, T, H, hd, scale, w.dqkv_hat, w.attn_ws,
                          w.attn_ws_bytes, s));
      NC_TRY(rope_qknorm_bwd(w.dqkv_hat, ly.qkv, ly.rstd_q, ly.rstd_k, w.table, dt, B, T, H, hd, dqkv, s));
    }
    NC_TRY(fork());
    NC_TRY(wgrad(mk(1, 0, Q, d, M, dqkv, Q, ly.a, d, gr->w_qkv + (size_t)l * Q * d, NC_F32, d, dt)));
    NC_TRY(mark_read(B_DQ, qv));
    ++qv;
    NC_TRY(gemm(tw ? mk(0, 1, M, d, Q, dqkv, Q, WqkvT, Q, w.dm, dyt, d, dt) : mk(0, 0, M, d, Q, dqkv, Q, Wqkv, d, w.dm, dyt, d, dt), s));
    ++gv;
    NC_TRY(reuse(B_G, gv));
    NC_TRY(rmsnorm_bwd(w.dm, dyt, ly.a, dt, ly.rstd_a, M, (int)d, g, 1, glp_out(gv), s));
  }
  NC_TRY(join());
  // embedding norm and scatter-add
  NC_TRY(rmsnorm_bwd(g, NC_F32, w.x0, NC_F32, w.rstd0, M, (int)d, w.dm, 0, nullptr, s));
  NC_TRY(embed_bwd(ids, M, w.dm, (int)d, gr->embed, V, acc, w.emb_ws, w.emb_ws_bytes, s));
  return NC_OK;
}

int relu2_mlp(const void* m, const void* w_fc, const void* w_proj, int dtype, int64_t M, int d, int F, float* x,
              void* u_out, void* a2_out, hipStream_t s) {
  NC_REQUIRE(m && w_fc && w_proj && x && u_out && a2_out, NC_ERR_INVALID_ARG, "relu2_mlp: null pointer");
  GemmDesc gf = mk(0, 1, M, F, d, m, d, w_fc, d, u_out, dtype, F, dtype);
  gf.epi = NC_EPI_RELU2;
  gf.aux_out = a2_out;
  NC_TRY(gemm(gf, s));
  GemmDesc gp = mk(0, 1, M, d, F, a2_out, F, w_proj, F, x, NC_F32, d, dtype);
  gp.beta = 1.f;
  return gemm(gp, s);
}

int relu2_mlp_bwd(const void* g_lp, const void* m, const void* u, const void* a2, const void* w_fc, const void* w_proj,
                  int dtype, int64_t M, int d, int F, float* dm, float* dw_fc, float* dw_proj, int accumulate,
                  void* du_buf, void* ws, size_t ws_bytes, hipStream_t s) {
  NC_REQUIRE(g_lp && m && u && a2 && w_fc && w_proj && dm && dw_fc && dw_proj && du_buf, NC_ERR_INVALID_ARG,
             "relu2_mlp_bwd: null pointer");
  GemmDesc g1 = mk(1, 0, d, F, M, g_lp, d, a2, F, dw_proj, NC_F32, F, dtype);
  g1.beta = accumulate ? 1.f : 0.f;
  g1.ws = ws;
  g1.ws_bytes = ws_bytes;
  NC_TRY(gemm(g1, s));
  GemmDesc g2 = mk(0, 0, M, F, d, g_lp, d, w_proj, F, du_buf, dtype, F, dtype);
  g2.epi = NC_EPI_RELU2_BWD;
  g2.aux = u;
  NC_TRY(gemm(g2, s));
  GemmDesc g3 = mk(1, 0, F, d, M, du_buf, F, m, d, dw_fc, NC_F32, d, dtype);
  g3.beta = accumulate ? 1.f : 0.f;
  g3.ws = ws;
  g3.ws_bytes = ws_bytes;
  NC_TRY(gemm(g3, s));
  return gemm(mk(0, 0, M, d, F, du_buf, F, w_fc, d, dm, NC_F32, d, dtype), s);
}

}  // namespace nc

extern "C" size_t nc_step_workspace_bytes(const nc_config* cfg) { return nc::step_workspace_bytes(cfg); }

extern "C" int nc_step_fwd_bwd(const nc_config* cfg, const nc_params* params, const nc_grads* grads,
                               const int32_t* ids, const int32_t* targets, const float* token_bytes, void* ws,
                               size_t ws_bytes, float* loss, float* bpb, float* loss_tok, void* stream) {
  return nc::api_done(nc::step_fwd_bwd(cfg, params, grads, ids, targets, token_bytes, ws, ws_bytes, loss, bpb, loss_tok,
                          static_cast<hipStream_t>(stream)), stream, "nc_step_fwd_bwd");
}

extern "C" int nc_relu2_mlp(const void* m, const void* w_fc, const void* w_proj, int dtype, int64_t M, int d, int F,
                            float* x, void* u_out, void* a2_out, void* stream) {
  return nc::api_done(nc::relu2_mlp(m, w_fc, w_proj, dtype, M, d, F, x, u_out, a2_out, static_cast<hipStream_t>(stream)),
                      stream, "nc_relu2_mlp");
}

extern "C" int nc_relu2_mlp_bwd(const void* g_lp, const void* m, const void* u, const void* a2, const void* w_fc,
                                const void* w_proj, int dtype, int64_t M, int d, int F, float* dm, float* dw_fc,
                                float* dw_proj, int accumulate, void* du_buf, void* ws, size_t ws_bytes,
                                void* stream) {

                       return nc::api_done(nc::relu2_mlp_bwd(g_lp, m, u, a2, w_fc, w_proj, dtype, M, d, F, dm, dw_fc, dw_proj, accumulate, du_buf, ws,
                           ws_bytes, static_cast<hipStream_t>(stream)), stream, "nc_relu2_mlp_bwd");
}
