// Internal GEMM interface shared by the step and the fused entry points.
#pragma once
#include "common.h"

namespace nc {

struct GemmDesc {
  int transA = 0, transB = 1;
  int64_t M = 0, N = 0, K = 0;
  const void* A = nullptr;
  int64_t lda = 0;
  const void* B = nullptr;
  int64_t ldb = 0;
  void* C = nullptr;
  int cdt = NC_F32;
  int64_t ldc = 0;
  float beta = 0.f;
  int epi = NC_EPI_STORE;
  const void* aux = nullptr;
  void* aux_out = nullptr;
  int dtype = NC_BF16;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // Softcap cross-entropy epilogues on the logit product z = h U^T (bf16,
  // K-contiguous operands, K a multiple of 64).  Columns are vocabulary ids
  // xv0 + n.
  //   xent = 1: per row and 64-column group g (vocabulary columns
  //             64 g .. 64 g + 63) xpart[g * M + row] = sum of exp(z' - c),
  //             z' = c tanh(z / c); xztgt[row] = z' at the row's target when
  //             the target is one of these columns.  If C is not null it
  //             receives u = exp(z' - c) (1 - (z'/c)^2) in bf16 (the logit
  //             gradient up to a row scale and the target's one-hot term),
  //             and xerr[row] = u - bf16(u) at the row's target.
  //   xent = 2: C (bf16) = xdl (exp(z' - xlse[row]) - [col == target])
  //             (1 - (z'/c)^2).
  int xent = 0;
  float xc = 0.f, xdl = 0.f;
  const int32_t* xtgt = nullptr;
  const float* xlse = nullptr;
  float* xpart = nullptr;
  float* xztgt = nullptr;
  float* xerr = nullptr;
  int xv0 = 0;
  // capc > 0: C (fp32) = capc tanh(acc / capc), the logit softcap; only for
  // the small-M form (bf16, x W^T, M <= 128), which decoding uses.
  float capc = 0.f;
  // sk_split > 1 (small-M form only, fp32 C, plain store): K is split over
  // sk_split blocks per column slab and C receives sk_split fp32 partial
  // products [sk_split][M][ldc] for the consumer to add in a fixed order.
  int sk_split = 1;
};

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int gemm(const GemmDesc& g, hipStream_t stream);
// Small-M form (gemm_small.hip): bf16 x W^T with M <= 128; gemm() routes
// eligible shapes there.
bool skinny_ok(const GemmDesc& g);
int gemm_skinny(const GemmDesc& g, hipStream_t stream);
// dst [C, R] = src [R, C]^T for 2- or 4-byte elements.
int transpose(const void* src, int64_t R, int64_t C, int elem_bytes, void* dst, hipStream_t s);
// n (1..4) bf16 matrices [R_i, C_i] -> [C_i, R_i] in one launch (sides multiples of 8, 16-byte aligned).
int transpose4(const void* const* src, const int64_t* R, const int64_t* C, void* const* dst, int n, hipStream_t s);

}  // namespace nc
