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
};

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
int gemm(const GemmDesc& g, hipStream_t stream);
// dst [C, R] = src [R, C]^T for 2- or 4-byte elements.
int transpose(const void* src, int64_t R, int64_t C, int elem_bytes, void* dst, hipStream_t s);

}  // namespace nc
