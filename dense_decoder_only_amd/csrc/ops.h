// Internal launchers behind the C ABI (all enqueue on `s` and return an
// nc_status).  See include/nc.h for argument meaning and layouts.
#pragma once
#include "common.h"

namespace nc {

int rmsnorm_fwd(const void* x, int xdt, int64_t rows, int d, float eps, void* y, int ydt, float* rstd,
                hipStream_t s);
// Row fix of a gradient as rmsnorm_bwd reads it: g_t <- rs[t] g_t - qs[t] U[tgt[t]]
// (U bf16 [V, d]; a target outside [0, V) takes no U row).  The vocabulary
// head's backward hands its dh over in this form.
struct GradRowFix {
  const float* rs;
  const float* qs;
  const int32_t* tgt;
  const bf16* U;
  int V;
};
// fix (optional): fp32 g and d <= 2048 only.
int rmsnorm_bwd(const void* g, int gdt, const void* y, int ydt, const float* rstd, int64_t rows, int d,
                float* dx, int accumulate, void* dx_bf16, hipStream_t s, const GradRowFix* fix = nullptr);
// x_copy (optional): a second copy of x_out.
int embed_fwd(const int32_t* ids, int64_t n, const void* table, int dtype, int64_t V, int d, void* rows_out,
              float* x_out, float* rstd, float eps, int32_t* flag, hipStream_t s,
              float* x_copy = nullptr);
size_t embed_bwd_workspace_bytes(int64_t n, int64_t V, int d);
int embed_bwd(const int32_t* ids, int64_t n, const float* de, int d, float* dtable, int64_t V, int accumulate,
              void* ws, size_t ws_bytes, hipStream_t s);
// dtable[v] (+)= sum over t with ids[t] = v of mul * scale[t] * rows[t] (bf16
// rows), with embed_bwd's workspace, order and accumulate semantics.
int embed_bwd_scaled(const int32_t* ids, int64_t n, const bf16* rows, const float* scale, float mul, int d,
                     float* dtable, int64_t V, int accumulate, void* ws, size_t ws_bytes, hipStream_t s);

int rope_table(float* table, int T, int hd, float base, hipStream_t s);
int rope_qknorm_fwd(void* qkv, int dtype, int B, int T, int H, int hd, const float* table, float eps,
                    float* rstd_q, float* rstd_k, hipStream_t s);
int rope_qknorm_bwd(const float* dhat, const void* yhat, const float* rstd_q, const float* rstd_k,
                    const float* table, int dtype, int B, int T, int H, int hd, void* dqkv, hipStream_t s);

// Optional fusion of the QK-norm + RoPE backward into the attention backward
// (bf16, head_dim 128): the kernels then write dqkv (bf16, the gradient w.r.t.
// the projection output) instead of the fp32 gradients w.r.t. q-hat, k-hat, v.
struct AttnRopeBwd {
  const float* rstd_q;
  const float* rstd_k;
  const float* table;
  void* dqkv;
};
bool attn_rope_bwd_fusable(int dtype, int hd);
size_t mqa_attn_bwd_workspace_bytes(int B, int T, int H);
int mqa_attn_fwd(const void* qkv, int dtype, int B, int T, int H, int hd, float scale, void* o, float* lse,
                 hipStream_t s);
int mqa_attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse, int dtype, int B, int T, int H,
                 int hd, float scale, float* dqkv, void* ws, size_t ws_bytes, hipStream_t s,
                 const AttnRopeBwd* fuse = nullptr);

size_t xent_workspace_bytes(int64_t M, int d, int V);
// store_logits: keep u = exp(z' - c) (1 - (z'/c)^2) in ws (bf16) when the
// fused path covers the vocabulary in one chunk; xent_bwd with from_stored
// then takes the logit gradient from it (a row scale and the target's term)
// instead of recomputing the logit product (same ws, untouched in between;
// dh_acc must be 0).  Returns whether it was stored via *stored.
// Targets outside [0, V) set *flag to 1 (flag = nullptr: the first int32 of
// ws, cleared first); such rows have no target logit and count no bytes.
int xent_fwd(const void* h, const void* U, int dtype, const int32_t* tgt, const float* token_bytes, int64_t M, int d,
             int V, float softcap, float* lse, float* loss_tok, float* loss, float* bpb, void* ws, size_t ws_bytes,
             hipStream_t s, bool store_logits = false, bool* stored = nullptr, int32_t* flag = nullptr);
// defer_fix (required on the stored path): dh is left as u U and *defer_fix
// receives the row fix that makes it dh (valid until ws is next used); the
// caller's rmsnorm_bwd applies it.
int xent_bwd(const void* h, const void* U, int dtype, const int32_t* tgt, const float* lse, int64_t M, int d, int V,
             float softcap, float dloss, float* dh, int dh_acc, float* dU, int dU_acc, void* ws, size_t ws_bytes,
             hipStream_t s, bool from_stored = false, GradRowFix* defer_fix = nullptr);

int fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace nc
