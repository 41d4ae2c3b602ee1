// Internal launchers behind the C ABI (all enqueue on `s` and return an
// nc_status).  See include/nc.h for argument meaning and layouts.
#pragma once
#include "common.h"

namespace nc {

int rmsnorm_fwd(const void* x, int xdt, int64_t rows, int d, float eps, void* y, int ydt, float* rstd,
                hipStream_t s);
int rmsnorm_bwd(const void* g, int gdt, const void* y, int ydt, const float* rstd, int64_t rows, int d,
                float* dx, int accumulate, void* dx_bf16, hipStream_t s);
int embed_fwd(const int32_t* ids, int64_t n, const void* table, int dtype, int64_t V, int d, void* rows_out,
              float* x_out, float* rstd, float eps, int32_t* flag, hipStream_t s);
size_t embed_bwd_workspace_bytes(int64_t n, int64_t V, int d);
int embed_bwd(const int32_t* ids, int64_t n, const float* de, int d, float* dtable, int64_t V, int accumulate,
              void* ws, size_t ws_bytes, hipStream_t s);

int rope_table(float* table, int T, int hd, float base, hipStream_t s);
int rope_qknorm_fwd(void* qkv, int dtype, int B, int T, int H, int hd, const float* table, float eps,
                    float* rstd_q, float* rstd_k, hipStream_t s);
int rope_qknorm_bwd(const float* dhat, const void* yhat, const float* rstd_q, const float* rstd_k,
                    const float* table, int dtype, int B, int T, int H, int hd, void* dqkv, hipStream_t s);

size_t mqa_attn_bwd_workspace_bytes(int B, int T, int H);
int mqa_attn_fwd(const void* qkv, int dtype, int B, int T, int H, int hd, float scale, void* o, float* lse,
                 hipStream_t s);
int mqa_attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse, int dtype, int B, int T, int H,
                 int hd, float scale, float* dqkv, void* ws, size_t ws_bytes, hipStream_t s);

size_t xent_workspace_bytes(int64_t M, int d, int V);
// store_logits: keep the softcapped logits in ws (16-bit fixed point) when the
// fused path covers the vocabulary in one chunk; xent_bwd with from_stored
// then forms dz from them instead of recomputing the logit product (same ws,
// untouched in between).  Returns whether they were stored via *stored.
int xent_fwd(const void* h, const void* U, int dtype, const int32_t* tgt, const float* token_bytes, int64_t M, int d,
             int V, float softcap, float* lse, float* loss_tok, float* loss, float* bpb, void* ws, size_t ws_bytes,
             hipStream_t s, bool store_logits = false, bool* stored = nullptr);
int xent_bwd(const void* h, const void* U, int dtype, const int32_t* tgt, const float* lse, int64_t M, int d, int V,
             float softcap, float dloss, float* dh, int dh_acc, float* dU, int dU_acc, void* ws, size_t ws_bytes,
             hipStream_t s, bool from_stored = false);

int fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace nc
