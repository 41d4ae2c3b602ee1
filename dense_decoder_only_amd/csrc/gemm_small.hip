// Small-M products for decoding (one new token per sequence).
#include "common.h"
#include "gemm.h"

namespace nc {
namespace {

enum { E_STORE_F32 = 0, E_ACC_F32 = 1, E_STORE_BF16 = 2, E_RELU2_SQ = 8 };

constexpr float kLog2e = 1.4426950408889634f;

// c tanh(z / c) from one hardware exp2 and reciprocal:
// tanh|x| = (1 - e^{-2|x|}) / (1 + e^{-2|x|}).
__device__ __forceinline__ float softcap_of(float z, float c, float inv_c) {
  const float x = z * inv_c;
  const float t = __builtin_amdgcn_exp2f(-2.f * kLog2e * fabsf(x));
  return copysignf(c * (1.f - t) * __builtin_amdgcn_rcpf(1.f + t), x);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// C[M, N] =
// A[M, K] W[N, K]^T with M <= 128 and both operands K-contiguous.  The work
// is reading W once from HBM (2 N K bytes against 2 M N K FLOPs), so the
// kernel is organised around that stream and its latency, not MFMA reuse:
//  * a block of 16 waves owns 16 rows of W (16 output columns) and every row
//    of A; the 64-wide k-chunks go round-robin over the waves, and each wave
//    issues the loads of up to 4 chunks (W and A) before its first MFMA, so a
//    block has up to 64 chunks (128 KB of W) in flight;
//  * per chunk, lane l reads 32 contiguous bytes of W row n0 + l mod 16 at k
//    offset 16 (l / 16); v_mfma_f32_16x16x32_bf16 takes k-slots 8 (l / 16) ..
//    + 7 from lane l, so MFMA s (0, 1) of a chunk is fed the lane's bytes
//    16 s .. 16 s + 15 of both operands: the k-slot order is permuted the
//    same way for W and A and the two MFMAs sum all 64 k;
//  * the product is issued as C^T (W fragment first): lane l ends with output
//    columns n0 + 4 (l / 16) + q (q = 0..3) of token row l mod 16;
//  * the 16 waves add their sums in LDS in a fixed order (deterministic), one
//    16 x 16 tile at a time, and 256 threads apply the epilogue.
// A (at most 128 x K bf16) stays in L2 across the blocks that re-read it.
// ---------------------------------------------------------------------------
#ifndef NC_SK_CPW
#define NC_SK_CPW 4
#endif
#ifndef NC_SK_WIDE
#define NC_SK_WIDE 256
#endif
constexpr int SK_WAVES = 16, SK_MMAX = 128, SK_CPW = NC_SK_CPW;
enum { E_SOFTCAP_F32 = 10 };  // small-M only: C (fp32) = c tanh(acc / c)
typedef float f32x4_t __attribute__((ext_vector_type(4)));

struct SkinnyParams {
  const bf16* A;
  int64_t lda;
  const bf16* W;
  int64_t ldw;
  void* C;
  int64_t ldc;
  int M, N, K;
  float capc, inv_capc;
  int ksplit;
};

template <int EPI>
__device__ __forceinline__ void skinny_store1(const SkinnyParams& p, int m, int n, float v) {
  const int64_t off = (int64_t)m * p.ldc + n;
  if constexpr (EPI == E_STORE_F32) {
    static_cast<float*>(p.C)[off] = v;
  } else if constexpr (EPI == E_ACC_F32) {
    static_cast<float*>(p.C)[off] += v;
  } else if constexpr (EPI == E_STORE_BF16) {
    static_cast<bf16*>(p.C)[off] = f2bf(v);
  } else if constexpr (EPI == E_RELU2_SQ) {
    const float a = fmaxf(v, 0.f);
    static_cast<bf16*>(p.C)[off] = f2bf(a * a);
  } else {  // E_SOFTCAP_F32
    static_cast<float*>(p.C)[off] = softcap_of(v, p.capc, p.inv_capc);
  }
}

// NMT: 16-row tiles of A held per wave (1, 2, 4 or 8; rows >= M are zero).
// WAVES: 16 (few output columns: more waves share a slab's k-chunks) or 8
// (many columns: two blocks fit a CU).  blockIdx.y = k-split: block (x, y)
// covers k-chunks [y cps, (y + 1) cps) and, with p.ksplit > 1, writes its
// plain fp32 sums to slice y of C ([ksplit][M][ldc]).
template <int EPI, int NMT, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void gemm_skinny_kernel(SkinnyParams p) {
  __shared__ float red[WAVES][4][64];
  // The wave index is made wave-uniform explicitly: the chunk guards below
  // must compile to scalar branches.  Under an EXEC-masked branch an MFMA
  // still runs (it ignores EXEC) and would add whatever the skipped loads
  // left in its registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int nch = p.K >> 6;
  const int cps = (nch + p.ksplit - 1) / p.ksplit;
  const int c_lo = blockIdx.y * cps, c_hi = min(nch, c_lo + cps);
  if (p.ksplit > 1) p.C = static_cast<float*>(p.C) + (int64_t)blockIdx.y * p.M * p.ldc;
  f32x4_t acc[NMT];
#pragma unroll
  for (int i = 0; i < NMT; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16* wrow = p.W + (int64_t)(n0 + r) * p.ldw + 16 * g;
  for (int cb = c_lo + wave; cb < c_hi; cb += SK_CPW * WAVES) {
    bf16x8_t w[SK_CPW][2];
#pragma unroll
    for (int j = 0; j < SK_CPW; ++j) {
      const int c = cb + j * WAVES;
      if (c < c_hi) {
        w[j][0] = *reinterpret_cast<const bf16x8_t*>(wrow + (c << 6));
        w[j][1] = *reinterpret_cast<const bf16x8_t*>(wrow + (c << 6) + 8);
      } else {  // never multiplied (the MFMAs below are skipped), but defined
        w[j][0] = bf16x8_t{};
        w[j][1] = bf16x8_t{};
      }
    }
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int m = mt * 16 + r;
      bf16x8_t x[SK_CPW][2];
#pragma unroll
      for (int j = 0; j < SK_CPW; ++j) {
        const int c = cb + j * WAVES;
        if (c < c_hi && m < p.M) {
          const bf16* xr = p.A + (int64_t)m * p.lda + (c << 6) + 16 * g;
          x[j][0] = *reinterpret_cast<const bf16x8_t*>(xr);
          x[j][1] = *reinterpret_cast<const bf16x8_t*>(xr + 8);
        } else {
          x[j][0] = bf16x8_t{};
          x[j][1] = bf16x8_t{};
        }
      }
#pragma unroll
      for (int j = 0; j < SK_CPW; ++j) {
        if (cb + j * WAVES < c_hi) {
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[j][0], x[j][0], acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[j][1], x[j][1], acc[mt], 0, 0, 0);
        }
      }
    }
  }
  // fixed-order reduction over the waves, one 16 x 16 tile at a time
  const int t = threadIdx.x, pl = t & 63, q = (t >> 6) & 3;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    if (mt * 16 < p.M) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][i][lane] = acc[mt][i];
      __syncthreads();
      if (t < 256) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) v += red[w][q][pl];
        const int m = mt * 16 + (pl & 15);
        if (m < p.M) skinny_store1<EPI>(p, m, n0 + 4 * (pl >> 4) + q, v);
      }
      __syncthreads();
    }
  }
}

template <int EPI, int WAVES>
void launch_skinny_w(const SkinnyParams& p, int nmt, hipStream_t s) {
  const dim3 grid((unsigned)(p.N / 16), (unsigned)p.ksplit);
  if (nmt <= 1) gemm_skinny_kernel<EPI, 1, WAVES><<<grid, WAVES * 64, 0, s>>>(p);
  else if (nmt <= 2) gemm_skinny_kernel<EPI, 2, WAVES><<<grid, WAVES * 64, 0, s>>>(p);
  else if (nmt <= 4) gemm_skinny_kernel<EPI, 4, WAVES><<<grid, WAVES * 64, 0, s>>>(p);
  else gemm_skinny_kernel<EPI, 8, WAVES><<<grid, WAVES * 64, 0, s>>>(p);
}

template <int EPI>
void launch_skinny(const SkinnyParams& p, int nmt, hipStream_t s) {
  // products with blocks to spare (>= 256 slabs x splits): 8-wave blocks, two per CU
  if ((p.N / 16) * p.ksplit >= NC_SK_WIDE) launch_skinny_w<EPI, 8>(p, nmt, s);
  else launch_skinny_w<EPI, 16>(p, nmt, s);
}

// Small-M form if the shapes and epilogue allow it; returns false to let the
// caller take the general path.
}  // namespace

bool skinny_ok(const GemmDesc& g) {
  if (g.dtype != NC_BF16 || g.transA != 0 || g.transB != 1 || g.xent) return false;
  if (g.M < 1 || g.M > SK_MMAX || g.N % 16 != 0 || g.K % 64 != 0) return false;
  if (g.lda % 8 != 0 || g.ldb % 8 != 0) return false;
  if (!aligned16(g.A) || !aligned16(g.B)) return false;
  if (g.sk_split > 1)
    return g.sk_split <= g.K / 64 && g.cdt == NC_F32 && g.beta == 0.f && g.epi == NC_EPI_STORE && g.capc == 0.f;
  if (g.capc > 0.f) return g.cdt == NC_F32 && g.beta == 0.f && g.epi == NC_EPI_STORE;
  if (g.epi == NC_EPI_RELU2_SQ) return g.cdt == NC_BF16;
  return g.epi == NC_EPI_STORE;
}

int gemm_skinny(const GemmDesc& g, hipStream_t s) {
  SkinnyParams p;
  p.A = static_cast<const bf16*>(g.A);
  p.lda = g.lda;
  p.W = static_cast<const bf16*>(g.B);
  p.ldw = g.ldb;
  p.C = g.C;
  p.ldc = g.ldc;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.capc = g.capc;
  p.inv_capc = g.capc > 0.f ? 1.f / g.capc : 0.f;
  p.ksplit = g.sk_split > 1 ? g.sk_split : 1;
  const double bytes = 2.0 * (double)g.N * g.K + 2.0 * (double)g.M * g.K +
                       (double)g.M * g.N * (g.cdt == NC_BF16 ? 2 : (g.beta == 1.f ? 8 : 4)) * p.ksplit;
  const int nmt = (int)cdiv(g.M, 16);
  probe_begin(NC_PROBE_GEMM_SKINNY, s);
  if (g.capc > 0.f) launch_skinny<E_SOFTCAP_F32>(p, nmt, s);
  else if (g.epi == NC_EPI_RELU2_SQ) launch_skinny<E_RELU2_SQ>(p, nmt, s);
  else if (g.cdt == NC_BF16) launch_skinny<E_STORE_BF16>(p, nmt, s);
  else if (g.beta == 1.f) launch_skinny<E_ACC_F32>(p, nmt, s);
  else launch_skinny<E_STORE_F32>(p, nmt, s);
  probe_end(NC_PROBE_GEMM_SKINNY, s, bytes);
  return check_launch("gemm_skinny_kernel");
}

}  // namespace nc
