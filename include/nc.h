/*
 * nc.h — C ABI of libnc: the forward+backward training step of a
 * nanochat-style dense decoder, as hand-written HIP kernels for AMD gfx950.
 *
 * Sources (page title, section):
 *   [NEWS] "Karpathy再放大招：8000行代碼復現ChatGPT全棧，最低成本僅100美元，4小時跑完",
 *          section 技術細節與問答: the architecture list (dense Transformer,
 *          RoPE without positional embedding, QK norm, untied embedding and
 *          unembedding, a norm after the token embedding, relu^2 MLP, RMSNorm
 *          without learnable parameters, bias-free linear layers, multi-query
 *          attention, logit softcap).
 *   [NANO] "Karpathy 的 nano 諧系：nanoGPT、llm.c 到 nanochat", section
 *          nanochat: the loss is reported in bits per byte.
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *     its comment says "host".  The library never allocates, frees or keeps
 *     device memory: scratch space comes from a caller buffer (`ws`) whose
 *     size is queried with the matching *_workspace_bytes call.
 *   - Matrices are row-major.  Token-major activations are [rows, width].
 *     Weight matrices are stored [out, in] (y = x W^T) and stacked per layer
 *     as [L, out, in].
 *   - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *     enqueues work on that stream and returns; nothing synchronizes except
 *     nc_sync_status.
 *   - dtype arguments take nc_dtype values.  bf16 values are raw IEEE bf16
 *     bit patterns; conversions from fp32 round to nearest, ties to even.
 *   - Return value: NC_OK or an nc_status error code.  Arguments are
 *     validated on the host before anything is enqueued; on an error nothing
 *     is enqueued and nc_last_error() returns a message (thread-local).
 *     Nothing aborts, prints or throws across this ABI.
 *   - Calls are thread-safe; the library has no mutable global state other
 *     than the thread-local error message, the kernel timer (nc_probe_*) and
 *     the step's optional side stream, which mutexes guard.
 *   - Out-of-range token ids are caught on the device: the row is treated as
 *     zeros and a device flag (an int32 given by the caller) is set to 1;
 *     nc_sync_status reads it.
 */
#ifndef NC_H_
#define NC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NC_OK = 0,
  NC_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer      */
  NC_ERR_UNSUPPORTED = 2, /* a shape or dtype the library does not implement */
  NC_ERR_WORKSPACE = 3,   /* ws too small for this call                      */
  NC_ERR_HIP = 4,         /* a HIP runtime call failed                       */
  NC_ERR_DEVICE_FLAG = 5  /* a kernel raised the device flag (bad token id)  */
} nc_status;

typedef enum { NC_F32 = 0, NC_BF16 = 1 } nc_dtype;

/* Model shape and constants of one step.  Readings where the pages are
 * silent: eps = 1e-6 inside the square root for every norm; RoPE pairs
 * (i, i + hd/2) rotated by +t * base^(-2i/hd); attention scale 1/sqrt(hd);
 * softcap z' = c tanh(z / c). */
typedef struct {
  int n_layer;    /* L                                                        */
  int d_model;    /* d, a multiple of 8                                       */
  int n_head;     /* H query heads, H * head_dim == d_model                  */
  int head_dim;   /* hd: 64 or 128                                            */
  int n_kv_head;  /* must be 1 (multi-query attention [NEWS])                 */
  int d_ff;       /* F, MLP width, a multiple of 8                           */
  int vocab;      /* V                                                        */
  int seq_len;    /* T                                                        */
  int batch;      /* B sequences; M = B * T tokens                            */
  float softcap;  /* c (15)                                                   */
  float rope_base;/* 10000                                                    */
  float eps;      /* 1e-6                                                     */
  int dtype;      /* NC_F32: everything fp32.  NC_BF16: bf16 weights, GEMM and
                     attention operands and saved activations; fp32
                     accumulation, norms, softmax, loss, residual stream and
                     gradients.                                               */
} nc_config;

/* Weights in cfg.dtype (bf16 bit patterns for NC_BF16). Layouts:
 *   embed [V, d]; w_qkv [L, (H+2) hd, d] = rows of Wq (H hd), Wk (hd), Wv (hd);
 *   w_o [L, d, H hd]; w_fc [L, F, d]; w_proj [L, d, F]; unembed [V, d]. */
typedef struct {
  const void* embed;
  const void* w_qkv;
  const void* w_o;
  const void* w_fc;
  const void* w_proj;
  const void* unembed;
} nc_params;

/* Parameter gradients, always fp32, same layouts as nc_params.  accumulate=0
 * overwrites them, accumulate=1 adds the step's gradient to their contents. */
typedef struct {
  float* embed;
  float* w_qkv;
  float* w_o;
  float* w_fc;
  float* w_proj;
  float* unembed;
  int accumulate;
} nc_grads;

/* Message of the last error on this thread ("" if none). Static storage. */
const char* nc_last_error(void);
/* Library version string. Static storage. */
const char* nc_version(void);

/* 1 if debug mode is on, else 0.  Debug mode is switched on by the
 * environment variable NC_DEBUG=1, read once per process: every entry point
 * that takes a stream then synchronizes that stream before it returns and
 * returns NC_ERR_HIP (with the HIP error in nc_last_error) if a kernel of the
 * call, or anything queued before it, failed.  It must not be used while the
 * stream is being captured into a graph. */
int nc_debug_mode(void);

/* Synchronizes `stream`, then reads the int32 device flag at `flag`.
 * Returns NC_ERR_DEVICE_FLAG if it is nonzero, NC_OK otherwise.  The step's
 * flag is the first int32 of its workspace. */
int nc_sync_status(const int32_t* flag, void* stream);

/* ---------------------------------------------------------------------------
 * Kernel timer, for measurement only.  While armed, every launch of the
 * chosen kernel family -- from any entry point, on any stream -- is bracketed
 * by a pair of HIP events recorded on the stream it is launched on, and the
 * library adds up the algorithmic FLOPs of those launches:
 *   GEMM families: 2 M N K per launch (a split-K launch counts its whole K);
 *   HBM-bound families (small-M GEMM, decode attention): algorithmic bytes
 *   instead of FLOPs (W, A and C once for the GEMM; the cached keys and
 *   values up to each sequence's length, q and o for the attention);
 *   attention (causal, per launch over B sequences of T tokens, H heads of
 *   width hd, counting half of the T x T score square): forward
 *   2 B H hd T^2 (two products), dQ 2 B H hd T^2 (dP and dQ), dK/dV
 *   2 B H hd T^2 (dV and dK); recomputed scores are not counted.
 * The events add a few microseconds per bracketed launch.
 *   nc_probe_start: arms the timer for `family` with room for `max_launches`
 *     launches (events are created here).  Re-arming discards what was
 *     recorded.  Launches beyond the room are not bracketed and are reported
 *     by nc_probe_stop as an error.
 *   nc_probe_stop: waits for the recorded events, writes (host pointers) the
 *     summed elapsed time between each pair, the number of launches and the
 *     summed FLOPs, then disarms and releases the events.
 * ------------------------------------------------------------------------- */
typedef enum {
  NC_PROBE_OFF = 0,
  NC_PROBE_GEMM_WGRAD = 1, /* weight-gradient GEMMs: both operands with K as rows (TN) */
  NC_PROBE_GEMM_NT = 2,    /* K-contiguous GEMMs (forward projections, dX)           */
  NC_PROBE_ATTN_FWD = 3,   /* causal MQA attention forward                           */
  NC_PROBE_ATTN_DQ = 4,    /* attention backward, dQ kernel                          */
  NC_PROBE_ATTN_DKV = 5,   /* attention backward, dK/dV kernel                       */
  NC_PROBE_GEMM_SKINNY = 6, /* small-M GEMMs (M <= 128, decoding): counts bytes       */
  NC_PROBE_DECODE_ATTN = 7, /* decode attention over the key/value cache: bytes       */
  NC_PROBE_GEMM = 8         /* every matrix-core GEMM launch: families 1 and 2 together */
} nc_probe_family;

int nc_probe_start(int family, int max_launches);
int nc_probe_stop(double* total_ms, int64_t* launches, double* flops);

/* ---------------------------------------------------------------------------
 * Whole step: forward and backward of the mean next-token loss [NEWS], with
 * the loss also reported in bits per byte [NANO].
 *   ids, targets : int32 [B, T]; targets are the inputs shifted by one.
 *   token_bytes  : fp32 [V] bytes per token id, or NULL for 4.8 for every id.
 *   ws           : at least nc_step_workspace_bytes(cfg) bytes, 256-aligned.
 *                  Holds the device flag (first int32), saved activations
 *                  and scratch; its contents on entry are ignored.
 *   loss, bpb    : fp32 scalars (device).  loss = mean over the B T tokens of
 *                  the natural-log cross entropy; bpb = sum of losses /
 *                  (ln 2 * sum of token_bytes[target]).
 *   loss_tok     : fp32 [B, T] per-token losses, or NULL.
 *   grads        : fp32 gradients of `loss` w.r.t. every parameter.
 * Errors: NC_ERR_INVALID_ARG (null pointers, n_kv_head != 1, H hd != d),
 *   NC_ERR_UNSUPPORTED (head_dim not 64/128; sizes not multiples of 8),
 *   NC_ERR_WORKSPACE.
 * Streams: everything runs on `stream` (a build with NC_STEP_SIDE_STREAM=1
 *   moves the weight-gradient products to a second stream that the library
 *   creates once per device and orders against `stream` with events; work
 *   enqueued on `stream` afterwards still sees every output).
 */
size_t nc_step_workspace_bytes(const nc_config* cfg);
int nc_step_fwd_bwd(const nc_config* cfg, const nc_params* params, const nc_grads* grads,
                    const int32_t* ids, const int32_t* targets, const float* token_bytes,
                    void* ws, size_t ws_bytes, float* loss, float* bpb, float* loss_tok,
                    void* stream);

/* ---------------------------------------------------------------------------
 * Inference with a key/value cache [NEWS, section 技術細節與問答: the model
 * (multi-query attention, RoPE, QK norm, logit softcap) and its serving
 * engine].  The cache holds each layer's post-RoPE, post-norm key and its
 * value for every position already seen.  By causality the logits at a
 * position depend on tokens up to it only, so prefill and decode return the
 * full forward's softcapped logits row at that position.
 * Supported: dtype NC_BF16, head_dim 128, n_kv_head 1, n_head <= 32,
 * batch <= 128; d_model and d_ff multiples of 64, vocab a multiple of 32.
 *   kv_cache: nc_kv_cache_bytes(cfg, max_len) bytes, 16-byte aligned, bf16
 *             [L][2][B][max_len][128] (keys, then values, of each layer).
 *   ws:       nc_infer_workspace_bytes(cfg, max_len) bytes, 256-byte aligned;
 *             its first int32 is the device flag (nc_sync_status(ws)).
 * Both are caller-owned; the size queries return 0 for an unsupported
 * configuration (or max_len < cfg->seq_len).
 *
 * nc_prefill: ids [B, T] int32 with B = cfg->batch and T = cfg->seq_len, the
 *   prompts.  Runs the forward over all B T tokens, writes positions 0..T-1
 *   of the cache and writes logits [B, V] fp32 = the softcapped logits at
 *   position T-1 of each prompt.  Token ids outside [0, V) raise the flag.
 * nc_decode_step: ids [B] int32, one new token per sequence, at the position
 *   pos[b] (int32, device); positions 0..pos[b]-1 of sequence b must already be
 *   in the cache.  Writes that token's key and value at position pos[b] and
 *   logits [B, V] fp32 = the softcapped logits at pos[b].  The positions may
 *   differ between sequences.  A position outside [0, max_len) or an id
 *   outside [0, V) raises the flag (that sequence's outputs are then
 *   undefined, memory outside the buffers is never touched).
 * Errors: NC_ERR_INVALID_ARG (null or misaligned pointers, n_head hd !=
 *   d_model, max_len < seq_len), NC_ERR_UNSUPPORTED (outside the supported
 *   shapes), NC_ERR_WORKSPACE.
 */
size_t nc_kv_cache_bytes(const nc_config* cfg, int max_len);
size_t nc_infer_workspace_bytes(const nc_config* cfg, int max_len);
int nc_prefill(const nc_config* cfg, const nc_params* params, const int32_t* ids, void* kv_cache,
               int max_len, float* logits, void* ws, size_t ws_bytes, void* stream);
int nc_decode_step(const nc_config* cfg, const nc_params* params, const int32_t* ids, const int32_t* pos,
                   void* kv_cache, int max_len, float* logits, void* ws, size_t ws_bytes, void* stream);

/* Decode attention over a cache [NEWS: multi-query attention]: for every
 * sequence b and query head h,
 *   o[b, h] = sum_{u < lens[b]} softmax_u(q[b, h] . k[b, u] * scale) v[b, u].
 *   q, o: bf16 [B, H, 128]; k_cache, v_cache: bf16 [B, max_len, 128];
 *   lens: int32 [B] (device), clamped to [0, max_len]; a sequence with no
 *   positions gets o = 0.
 *   ws: nc_mqa_decode_workspace_bytes(B, H, max_len) bytes, 256-byte aligned
 *   (fp32 partial results per 64 cached positions).
 * Work is split over 64-position chunks and the chunks are combined in a
 * fixed order (deterministic).  Errors: NC_ERR_INVALID_ARG,
 * NC_ERR_UNSUPPORTED (head_dim != 128, H > 32), NC_ERR_WORKSPACE. */
size_t nc_mqa_decode_workspace_bytes(int B, int H, int max_len);
int nc_mqa_decode_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* lens, int B,
                       int H, int hd, int max_len, float scale, void* o, void* ws, size_t ws_bytes,
                       void* stream);

/* nc_mqa_decode_attn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  Same arguments (minus ws), same kernels,
 * same results.  The chunk partials go to a scratch array of 16 MiB that the
 * library holds in device memory of every GPU it runs on until the process
 * ends; the call allocates nothing.
 *   Limit: nc_mqa_decode_workspace_bytes(B, H, max_len) <= 16 MiB (e.g. 32
 *   sequences x 10 heads x 2048 positions needs 5.3 MB); larger shapes return
 *   NC_ERR_WORKSPACE.  Nothing in the scratch needs clearing between calls.
 *   All calls on one GPU share its scratch: calls that overlap in time on
 *   that GPU (different streams, or threads) race and must be serialized by
 *   the caller; calls on one stream are ordered by it.
 *   The first call on each device looks up the scratch's device address
 *   (hipGetSymbolAddress); make it outside graph capture.
 * Errors: as nc_mqa_decode_attn, with NC_ERR_WORKSPACE for shapes beyond the
 * limit. */
int nc_mqa_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache, const int32_t* lens,
                               int B, int H, int hd, int max_len, float scale, void* o, void* stream);

/* ---------------------------------------------------------------------------
 * Token-embedding gather and the norm that follows it [NEWS: untied
 * embedding; a norm after the token embedding; RMSNorm without parameters].
 *   ids [n] int32; table [V, d] in `dtype`.
 *   rows_out [n, d] (dtype, may be NULL): the gathered rows, bit-exact copies.
 *   x_out [n, d] fp32 (may be NULL): rms(row) = row / sqrt(mean(row^2) + eps).
 *   rstd [n] fp32 (may be NULL, needs x_out): 1 / sqrt(mean(row^2) + eps).
 *   flag: int32 device flag (may be NULL), set to 1 for ids outside [0, V);
 *   such rows are written as zeros. */
int nc_embed_fwd(const int32_t* ids, int64_t n, const void* table, int dtype, int64_t V, int d,
                 void* rows_out, float* x_out, float* rstd, float eps, int32_t* flag, void* stream);

/* Embedding backward: dtable[v] (+)= sum over the positions t with ids[t] = v
 * of de[t], summed in increasing t (deterministic); rows of absent ids are
 * left at 0 (accumulate=0) or untouched (accumulate=1).
 *   ids [n] int32 (must be in [0, V)), de [n, d] fp32, dtable [V, d] fp32.
 *   ws: nc_embed_bwd_workspace_bytes(n, V, d) bytes. */
size_t nc_embed_bwd_workspace_bytes(int64_t n, int64_t V, int d);
int nc_embed_bwd(const int32_t* ids, int64_t n, const float* de, int d, float* dtable, int64_t V,
                 int accumulate, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Parameter-free RMSNorm over rows of length d [NEWS: RMSNorm without
 * learnable parameters]: y = x / sqrt(mean(x^2) + eps).
 *   x [rows, d] in xdt; y [rows, d] in ydt; rstd [rows] fp32 (may be NULL). */
int nc_rmsnorm_fwd(const void* x, int xdt, int64_t rows, int d, float eps, void* y, int ydt,
                   float* rstd, void* stream);

/* RMSNorm backward: dx (+)= rstd * (dy - y * mean(dy * y)), with y the
 * forward output and rstd its scale.
 *   dy [rows, d] in dydt; y [rows, d] in ydt; rstd [rows]; dx [rows, d] fp32.
 *   accumulate=1 adds into dx.  dx_bf16 [rows, d] (may be NULL) receives the
 *   bf16 rounding of the resulting dx. */
int nc_rmsnorm_bwd(const void* dy, int dydt, const void* y, int ydt, const float* rstd,
                   int64_t rows, int d, float* dx, int accumulate, void* dx_bf16, void* stream);

/* ---------------------------------------------------------------------------
 * Rotary embedding followed by per-head RMS norm of queries and the single
 * key head [NEWS: RoPE, no positional embedding; QK norm].
 * nc_rope_table fills table [T, hd/2, 2] fp32 with (cos, sin) of
 * theta(t, i) = t * base^(-2i/hd), computed in fp64 and rounded once. */
int nc_rope_table(float* table, int T, int hd, float base, void* stream);

/* In place on qkv [B T, (H+2) hd] (dtype): for every token t (position
 * t mod T) and every head h < H+1 (H query heads, then the key head):
 * x <- rms_hd(rope(x, t)); rstd_q [B T, H] and rstd_k [B T] receive the norm
 * scales.  The value head (last hd columns) is not touched. */
int nc_rope_qknorm_fwd(void* qkv, int dtype, int B, int T, int H, int hd, const float* table,
                       float eps, float* rstd_q, float* rstd_k, void* stream);

/* Backward of nc_rope_qknorm_fwd.
 *   dqkv_hat [B T, (H+2) hd] fp32: gradients w.r.t. the normalized q, k and
 *     w.r.t. v.
 *   qkv_hat: the forward's in-place output (dtype).
 *   dqkv [B T, (H+2) hd] in dtype: gradients w.r.t. the projection output
 *     (q and k rotated back by -theta after the norm backward; v copied). */
int nc_rope_qknorm_bwd(const float* dqkv_hat, const void* qkv_hat, const float* rstd_q,
                       const float* rstd_k, const float* table, int dtype, int B, int T, int H,
                       int hd, void* dqkv, void* stream);

/* ---------------------------------------------------------------------------
 * Causal multi-query attention [NEWS: multi-query attention]: H query heads
 * share one key/value head.  Inputs are read from the packed buffer
 * qkv [B T, (H+2) hd] (dtype) holding q (heads 0..H-1), k, v per token.
 *   o [B T, H hd] (dtype): o[t, h] = sum_{u <= t} softmax_u(scale q[t,h].k[u]) v[u].
 *   lse [B T H] fp32: natural-log log-sum-exp of the scaled scores per
 *     (token, head) row, kept for the backward. */
int nc_mqa_attn_fwd(const void* qkv, int dtype, int B, int T, int H, int hd, float scale,
                    void* o, float* lse, void* stream);

/* Backward: from dout [B T, H hd] (dtype) writes dqkv_hat [B T, (H+2) hd]
 * fp32 = gradients w.r.t. q (per head), k and v (k and v summed over the H
 * query heads).  ws: nc_mqa_attn_bwd_workspace_bytes(B, T, H) bytes. */
size_t nc_mqa_attn_bwd_workspace_bytes(int B, int T, int H);
int nc_mqa_attn_bwd(const void* qkv, const void* o, const void* dout, const float* lse,
                    int dtype, int B, int T, int H, int hd, float scale, float* dqkv_hat,
                    void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * bf16 GEMM on the matrix cores [NEWS: bias-free linear layers]:
 *   C[M, N] = sum_k A'[m, k] B'[k, n]   (fp32 accumulation)
 *   A' = A [M, K] (lda >= K) if transA == 0, else A^T with A stored [K, M].
 *   B' = B [K, N] (ldb >= N) if transB == 0, else B^T with B stored [N, K].
 * So y = x W^T is (transA=0, transB=1); dx = dy W is (0, 0); dW = dy^T x is
 * (1, 0).  M, N, K and the leading dimensions must be multiples of 8 and the
 * pointers 16-byte aligned.
 * Epilogues (aux / aux_out are bf16 [M, N] with leading dimension ldc):
 *   NC_EPI_STORE     C (cdt) = acc, or C += acc when beta = 1 (cdt = NC_F32).
 *   NC_EPI_RELU2     C (bf16) = acc; aux_out (bf16) = relu(acc)^2 [NEWS: relu^2].
 *   NC_EPI_RELU2_BWD C (bf16) = acc * 2 relu(aux).
 *   NC_EPI_RELU2_SQ  C (bf16) = relu(acc)^2 only (the pre-activation is not
 *                    stored).
 *   NC_EPI_RELU2_BWD_SQ C (bf16) = acc * 2 sqrt(aux) with aux = relu(u)^2,
 *                    i.e. the relu^2 backward from the stored activation.
 * dtype NC_F32 runs the same contraction on fp32 operands (a plain path for
 * small fp32 problems; epilogues as above with fp32 everywhere).
 * Small M (decoding): bf16 (transA=0, transB=1) products with 1 <= M <= 128,
 * N a multiple of 16 and K of 64, with NC_EPI_STORE or NC_EPI_RELU2_SQ, take
 * a kernel that streams B once (M, ldc and C need no alignment there).
 * ws (may be NULL): enables deterministic split-K for tall-K problems; see
 * nc_gemm_workspace_bytes. */
typedef enum {
  NC_EPI_STORE = 0,
  NC_EPI_RELU2 = 1,
  NC_EPI_RELU2_BWD = 2,
  NC_EPI_RELU2_SQ = 3,
  NC_EPI_RELU2_BWD_SQ = 4
} nc_epilogue;
size_t nc_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int nc_gemm_bf16(int transA, int transB, int64_t M, int64_t N, int64_t K, const void* A,
                 int64_t lda, const void* B, int64_t ldb, void* C, int cdt, int64_t ldc, float beta,
                 int epilogue, const void* aux, void* aux_out, int dtype, void* ws, size_t ws_bytes,
                 void* stream);

/* ---------------------------------------------------------------------------
 * relu^2 MLP block with its residual [NEWS: relu^2 activation; bias-free]:
 *   u = m W1^T (bf16 [M, F], saved), a2 = relu(u)^2 (bf16 [M, F], saved),
 *   x += a2 W2^T (x fp32 [M, d], updated in place).
 *   m [M, d], w_fc [F, d], w_proj [d, F] in dtype. */
int nc_relu2_mlp(const void* m, const void* w_fc, const void* w_proj, int dtype, int64_t M, int d,
                 int F, float* x, void* u_out, void* a2_out, void* stream);

/* Backward of nc_relu2_mlp for the gradient g = dL/dx_out (g_lp: g in dtype):
 *   dW2 (+)= g^T a2; du = (g W2) * 2 relu(u); dW1 (+)= du^T m; dm = du W1 (fp32).
 *   du_buf [M, F] (dtype) is scratch for du; ws as for nc_gemm_bf16. */
int nc_relu2_mlp_bwd(const void* g_lp, const void* m, const void* u, const void* a2,
                     const void* w_fc, const void* w_proj, int dtype, int64_t M, int d, int F,
                     float* dm, float* dw_fc, float* dw_proj, int accumulate, void* du_buf,
                     void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Untied unembedding, tanh softcap and cross entropy [NEWS: untied
 * unembedding; logit softcap], reported as loss and bits per byte [NANO].
 * The [M, V] logits are produced in vocabulary chunks inside the kernels and
 * never stored in fp32.
 *   h [M, d], U [V, d] in dtype; tgt [M] int32 in [0, V).
 *   lse [M] fp32: log sum_v exp(z'[t, v]) with z' = c tanh(h U^T / c).
 *   loss_tok [M] fp32 (may be NULL): lse - z'[t, tgt[t]].
 *   loss, bpb: fp32 device scalars (mean loss; sum / (ln 2 * sum bytes)).
 *   token_bytes [V] fp32 or NULL (4.8 per id).
 *   ws: nc_softcap_xent_workspace_bytes(M, d, V) bytes, 256-byte aligned.
 *   Its first int32 is a device flag: nc_softcap_xent_fwd clears it and sets
 *   it to 1 when a target lies outside [0, V) (nc_sync_status(ws) reads it).
 *   Such a row takes z'[t, tgt[t]] = 0 and counts no bytes; no memory outside
 *   the buffers is read.  In the backward such a row has no one-hot term. */
size_t nc_softcap_xent_workspace_bytes(int64_t M, int d, int V);
int nc_softcap_xent_fwd(const void* h, const void* U, int dtype, const int32_t* tgt,
                        const float* token_bytes, int64_t M, int d, int V, float softcap,
                        float* lse, float* loss_tok, float* loss, float* bpb, void* ws,
                        size_t ws_bytes, void* stream);

/* Gradients of dloss * sum_t loss_t (dloss = 1/M for the mean):
 *   dz' = dloss (softmax(z') - onehot(tgt)), dz = dz' (1 - (z'/c)^2),
 *   dh [M, d] fp32 (+)= dz U, dU [V, d] fp32 (+)= dz^T h.
 *   dh_accumulate / dU_accumulate choose += over =. */
int nc_softcap_xent_bwd(const void* h, const void* U, int dtype, const int32_t* tgt,
                        const float* lse, int64_t M, int d, int V, float softcap, float dloss,
                        float* dh, int dh_accumulate, float* dU, int dU_accumulate, void* ws,
                        size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * AdamW parameter update with the bf16 weight refresh, for the training loop
 * that follows the step.  [NEWS] names Muon + AdamW as the optimizers without
 * defining them; this is the published AdamW (decoupled weight decay, bias-
 * corrected moments), with every hyperparameter an argument:
 *   g  = grad_scale * grad
 *   m  = beta1 m + (1 - beta1) g ;  v = beta2 v + (1 - beta2) g^2
 *   p  = p (1 - lr weight_decay) - lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 *   weights_lp (bf16, may be NULL) = p rounded to nearest, ties to even.
 *   master, m, v, grad: fp32 [n] device arrays, 16-byte aligned; master, m
 *   and v are updated in place.  t >= 1 is the step count (1 on the first
 *   update).  One pass over HBM: 28 bytes per parameter (30 with the bf16
 *   copy).
 * n == 0 is a no-op (the pointers may then be NULL).
 * Errors: NC_ERR_INVALID_ARG (null or misaligned pointers, n < 0, t < 1). */
int nc_adamw_step(float* master, float* m, float* v, const float* grad, void* weights_lp, int64_t n, int t,
                  float lr, float beta1, float beta2, float eps, float weight_decay, float grad_scale,
                  void* stream);

#ifdef __cplusplus
}
#endif
#endif /* NC_H_ */
