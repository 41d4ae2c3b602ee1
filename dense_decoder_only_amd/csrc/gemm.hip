// GEMMs of the training step: every bias-free projection, the relu^2 MLP and
// the unembedding's weight/activation gradients (release-news page
// "Karpathy再放大招…", section 技術細節與問答: linear layers carry no bias; the
// MLP uses relu^2).
//
// bf16 path (gfx950 matrix cores): C[M,N] = sum_k A'[m,k] B'[k,n] with fp32
// accumulation in v_mfma_f32_32x32x16_bf16.  Three kernels:
//   * gemm_pipe_kernel: every full-tile product of the step, in two forms
//     (both operands K-contiguous, "NT"; both with K as rows, the weight
//     gradients, "TN").  Block tile 256 x 256 x 64, 512 threads = 8 waves in
//     a 2 x 4 grid of 128 x 64 wave tiles (two waves per SIMD).  Tiles go
//     global -> LDS by buffer_load ... lds in two stages that are separate
//     LDS objects (so the compiler does not make fragment reads wait for the
//     DMA into the other stage), with a rotated k loop that issues the next
//     DMA right after the barrier inside each k-tile's last k-step.  The NT
//     form reads fragments as swizzled 16-byte rows, the TN form with
//     ds_read_b64_tr_b16 straight from the tile as stored.
//   * gemm_mfma8_kernel: the TN form when a k-tile is ragged (register
//     transpose of 8 x 8 blocks instead of transposed LDS reads).
//   * gemm_mfma_kernel: 4 waves of 128 x 128, single-buffered register
//     staging or direct DMA; the remaining layouts (NN, TT, or K not a
//     multiple of 64).
// Epilogues are fused and staged through LDS so that global stores are
// 16-byte and row-contiguous: bf16 or fp32 store, fp32 accumulate (residual
// add / gradient accumulation), relu^2 forward, relu^2 backward from the
// stored relu(u)^2, split-K partial products, and the softcap cross-entropy
// terms of the logit product.  Tall-K problems with few output tiles (the
// weight gradients, K = B*T) split K into fp32 partials reduced in a fixed
// order, so results are bitwise reproducible.
#include "common.h"
#include "gemm.h"
#include "ops.h"

#include <algorithm>

namespace nc {

namespace {

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NT = 256;

#ifndef NC_GEMM_SWZ
#define NC_GEMM_SWZ 1
#endif
// LDS chunk swizzle of a [256][64] bf16 tile: 16-byte chunk c of `row` lives
// at chunk c ^ swz(row).
__host__ __device__ constexpr int swz(int row) { return NC_GEMM_SWZ ? ((row >> 1) & 7) : (row & 7); }

enum { E_STORE_F32 = 0, E_ACC_F32 = 1, E_STORE_BF16 = 2, E_RELU2 = 3, E_RELU2_BWD = 4, E_PARTIAL = 5,
       E_XENT_FWD = 6, E_XENT_BWD = 7, E_RELU2_SQ = 8, E_RELU2_BWD_SQ = 9 };

struct MfmaParams {
  const bf16* A;
  const bf16* B;
  int64_t lda, ldb;
  int M, N, K;
  int k_per_split;
  int tiles_m, tiles_n;
  void* C;
  int64_t ldc;
  const bf16* aux;
  bf16* aux_out;
  // softcap cross-entropy epilogues (see GemmDesc)
  float xc, xinv_c, xdl;
  const int32_t* xtgt;
  const float* xlse;
  float* xpart;
  float* xztgt;
  float* xerr;
  // > 0: split-K launched as one flat grid of tiles x kxcd blocks, split s
  // on XCD s mod 8 (gemm_pipe_kernel only; kxcd a multiple of 8)
  int kxcd = 0;
  int xv0;
  int splits = 1;  // gemm_pipe_kernel: k-splits (work items = tiles x splits)
};

constexpr float kLog2e = 1.4426950408889634f;

// Orders this wave's LDS accesses around a hand-off between its own lanes: all
// of its LDS operations so far have completed (lgkmcnt 0) and the compiler
// moves no memory access across this point.  Global stores stay in flight.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Non-temporal (streaming) global accesses, for the epilogues' outputs and
// their read-once inputs: every CU writes its tile at about the same time, and
// as ordinary stores those tens of MB displaced the operand panels that the
// next tiles read from L2.
typedef float ntf4 __attribute__((ext_vector_type(4)));
typedef unsigned ntu2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st_nt(float* p, float4 v) {
  const ntf4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<ntf4*>(p));
}
__device__ __forceinline__ void st_nt(bf16* p, uint2 v) {
  const ntu2 t = {v.x, v.y};
  __builtin_nontemporal_store(t, reinterpret_cast<ntu2*>(p));
}
__device__ __forceinline__ float4 ld_nt(const float* p) {
  const ntf4 t = __builtin_nontemporal_load(reinterpret_cast<const ntf4*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ uint2 ld_nt(const bf16* p) {
  const ntu2 t = __builtin_nontemporal_load(reinterpret_cast<const ntu2*>(p));
  return make_uint2(t.x, t.y);
}

// c tanh(z / c) from one hardware exp2 and reciprocal:
// tanh|x| = (1 - e^{-2|x|}) / (1 + e^{-2|x|}).
__device__ __forceinline__ float softcap_of(float z, float c, float inv_c) {
  const float x = z * inv_c;
  const float t = __builtin_amdgcn_exp2f(-2.f * kLog2e * fabsf(x));
  return copysignf(c * (1.f - t) * __builtin_amdgcn_rcpf(1.f + t), x);
}

// Logit-gradient epilogue on four consecutive columns of one row; y is the
// row's target column (relative to xv0), L its log-sum-exp times log2(e).
__device__ __forceinline__ void xent_bwd4(const MfmaParams& p, float4 v, int row, int col, int y, float L) {
  const float zz[4] = {v.x, v.y, v.z, v.w};
  float g[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float zc = softcap_of(zz[e], p.xc, p.xinv_c);
    const float th = zc * p.xinv_c;
    const float pr = __builtin_amdgcn_exp2f(zc * kLog2e - L);
    g[e] = p.xdl * (pr - (col + e == y ? 1.f : 0.f)) * (1.f - th * th);
  }
  *reinterpret_cast<uint2*>(static_cast<bf16*>(p.C) + (int64_t)row * p.ldc + col) =
      make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]));
}

// Sum over the 16 lanes of a DPP row (the lanes l with the same l / 16); every
// lane of the row gets the total.  Rotations by 8 and 4 within the row, then
// the two quad exchanges.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_sum(float s) {
  s += dpp_f<0x128>(s);  // row_ror:8
  s += dpp_f<0x124>(s);  // row_ror:4
  s += dpp_f<0x4e>(s);   // quad_perm [2,3,0,1]
  s += dpp_f<0xb1>(s);   // quad_perm [1,0,3,2]
  return s;
}

// Forward cross-entropy epilogue: a 16-lane group (one DPP row) holds one
// row's 64 columns (4 per lane); every lane of the group must call this.  y is
// the row's target column relative to xv0 (-1 for rows past M); ust points at
// the row's stored value for column col (unused when p.C is null: nothing is
// stored).
// With th = tanh(z / c) = sign(z) (1 - t) / (1 + t), t = e^{-2|z|/c}, the
// capped logit is c th and e = exp(c th - c) = 2^{(th - 1) c log2(e)}.  The
// stored value is u = e (1 - th^2) in bf16: the logit gradient is
// dloss (e / S - [col == y]) (1 - th^2) with S the row's sum of e, so the
// backward needs only the row scale dloss / S and the target's term.  The
// target's rounding error u - bf16(u) is kept so that the one-hot term
// cancels against the fp32 value.
__device__ __forceinline__ void xent_fwd4(const MfmaParams& p, float4 v, int row, int col, int gcol64, int y,
                                          bf16* ust) {
  const bool ok = row < p.M;
  const bool in = col < p.N;  // N is a multiple of 8: the 4 columns are all in range or none is
  const float zz[4] = {v.x, v.y, v.z, v.w};
  const float ka = -2.f * kLog2e * p.xinv_c, cl = p.xc * kLog2e;
  float th[4], e[4];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float t = __builtin_amdgcn_exp2f(ka * fabsf(zz[k]));
    th[k] = copysignf((1.f - t) * __builtin_amdgcn_rcpf(1.f + t), zz[k]);
    e[k] = __builtin_amdgcn_exp2f(fmaf(th[k], cl, -cl));
    s += e[k];
  }
  if (!in) s = 0.f;
  const unsigned d = (unsigned)(y - col);
  const bool here = ok && in && d < 4u;
  if (here) p.xztgt[row] = p.xc * (d == 0 ? th[0] : d == 1 ? th[1] : d == 2 ? th[2] : th[3]);
  if (p.C && ok && in) {
    float u[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) u[k] = e[k] * fmaf(-th[k], th[k], 1.f);
    const uint32_t lo = pack_bf16x2(u[0], u[1]), hi = pack_bf16x2(u[2], u[3]);
    const ntu2 w = {lo, hi};
    __builtin_nontemporal_store(w, reinterpret_cast<ntu2*>(ust));
    if (here) {
      const uint32_t pair = d < 2 ? lo : hi;
      const float rounded = __uint_as_float((d & 1) ? (pair & 0xffff0000u) : (pair << 16));
      p.xerr[row] = (d == 0 ? u[0] : d == 1 ? u[1] : d == 2 ? u[2] : u[3]) - rounded;
    }
  }
  s = row16_sum(s);
  if (ok && (threadIdx.x & 15) == 0 && gcol64 < p.N)
    p.xpart[(int64_t)((p.xv0 + gcol64) >> 6) * p.M + row] = s;
}

// Global -> registers: one 256 x 64 tile of an operand.
template <bool KC>
__device__ __forceinline__ void load_tile(const bf16* __restrict__ P, int64_t ld, int r0, int R, int k0,
                                          int kend, int tid, uint4 (&v)[8]) {
  if constexpr (KC) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = tid + NT * i;
      const int row = id >> 3, kc = id & 7;
      int r = r0 + row;
      r = r < R ? r : R - 1;
      const int k = k0 + kc * 8;
      if (k < kend)
        v[i] = *reinterpret_cast<const uint4*>(P + (int64_t)r * ld + k);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  } else {
    const int kb = tid & 7, rb = tid >> 3;
    int r = r0 + rb * 8;
    r = r < R ? r : R - 8;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int k = k0 + kb * 8 + kk;
      if (k < kend)
        v[kk] = *reinterpret_cast<const uint4*>(P + (int64_t)k * ld + r);
      else
        v[kk] = make_uint4(0, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ uint32_t word_of(const uint4& q, int w) {
  return w == 0 ? q.x : (w == 1 ? q.y : (w == 2 ? q.z : q.w));
}

// Registers -> LDS tile [256][64] with the chunk index swizzled by (row & 7).
template <bool KC>
__device__ __forceinline__ void store_tile(bf16* __restrict__ S, int tid, const uint4 (&v)[8]) {
  if constexpr (KC) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = tid + NT * i;
      const int row = id >> 3, kc = id & 7;
      *reinterpret_cast<uint4*>(S + row * BK + ((kc ^ swz(row)) << 3)) = v[i];
    }
  } else {
    // v[kk] holds rows rb*8 + 0..7 at k = kb*8 + kk; write row rb*8 + mm with
    // its eight k values (kk = 0..7) as one 16-byte chunk.
    const int kb = tid & 7, rb = tid >> 3;
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      const int w = mm >> 1;
      uint32_t o[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = word_of(v[2 * p], w), b = word_of(v[2 * p + 1], w);
        o[p] = (mm & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      const int row = rb * 8 + mm;
      *reinterpret_cast<uint4*>(S + row * BK + ((kb ^ swz(row)) << 3)) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

#ifndef NC_GEMM_DIRECT
#define NC_GEMM_DIRECT 1  // K-contiguous tiles go global -> LDS without VGPR staging
#endif
#ifndef NC_GEMM_XCD
#define NC_GEMM_XCD 1     // XCD-aware grouped tile order
#endif
#ifndef NC_GEMM_KXCD
#define NC_GEMM_KXCD 1    // split-K with a multiple of 8 splits: whole k-splits per XCD
#endif
#ifndef NC_GEMM_SPLIT_MODEL
#define NC_GEMM_SPLIT_MODEL 1  // split count from the rounds x k-length model
#endif
#ifndef NC_GEMM_SPLIT_C0
#define NC_GEMM_SPLIT_C0 8     // fixed per-block cost in the model, in k-steps
#endif
#ifndef NC_GEMM_GROUP_M
#define NC_GEMM_GROUP_M 4
#endif

// Direct global -> LDS staging of a K-contiguous 256 x 64 tile with gfx950's
// global_load_lds_dwordx4.  Each wave moves 8 groups of 8 rows (1 KB per
// instruction); lane i of a group lands at byte 16 i of the group, i.e. at
// row i / 8 of the group, physical chunk i % 8, so it fetches the logical
// chunk (i % 8) ^ swz(row) that the swizzle puts there.
__device__ __forceinline__ void stage_direct(const bf16* __restrict__ P, int64_t ld, int r0, int R, int k0, bf16* S,
                                             int wave, int lane) {
  const int rsub = lane >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int grp = wave * 8 + i;
    const int c = (lane & 7) ^ swz(grp * 8 + rsub);
    int r = r0 + grp * 8 + rsub;
    r = r < R ? r : R - 1;
    __builtin_amdgcn_global_load_lds(P + (int64_t)r * ld + k0 + c * 8,
                                     (__attribute__((address_space(3))) void*)(S + grp * 8 * BK), 16, 0, 0);
  }
}

// Applies the epilogue to four consecutive columns (col % 4 == 0) of one row.
template <int EPI>
__device__ __forceinline__ void epilogue4(const MfmaParams& p, float4 v, int row, int col) {
  const int64_t off = (int64_t)row * p.ldc + col;
  if constexpr (EPI == E_STORE_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(p.C) + off) = v;
  } else if constexpr (EPI == E_ACC_F32) {
    float4* c = reinterpret_cast<float4*>(static_cast<float*>(p.C) + off);
    const float4 o = *c;
    *c = make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w);
  } else if constexpr (EPI == E_STORE_BF16) {
    *reinterpret_cast<uint2*>(static_cast<bf16*>(p.C) + off) =
        make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  } else if constexpr (EPI == E_RELU2) {
    *reinterpret_cast<uint2*>(static_cast<bf16*>(p.C) + off) =
        make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    const float a = fmaxf(v.x, 0.f), b = fmaxf(v.y, 0.f), c = fmaxf(v.z, 0.f), d = fmaxf(v.w, 0.f);
    *reinterpret_cast<uint2*>(p.aux_out + off) = make_uint2(pack_bf16x2(a * a, b * b), pack_bf16x2(c * c, d * d));
  } else if constexpr (EPI == E_RELU2_BWD) {
    const uint2 u = *reinterpret_cast<const uint2*>(p.aux + off);
    const float u0 = bf2f((bf16)(u.x & 0xffffu)), u1 = bf2f((bf16)(u.x >> 16));
    const float u2 = bf2f((bf16)(u.y & 0xffffu)), u3 = bf2f((bf16)(u.y >> 16));
    *reinterpret_cast<uint2*>(static_cast<bf16*>(p.C) + off) =
        make_uint2(pack_bf16x2(v.x * 2.f * fmaxf(u0, 0.f), v.y * 2.f * fmaxf(u1, 0.f)),
                   pack_bf16x2(v.z * 2.f * fmaxf(u2, 0.f), v.w * 2.f * fmaxf(u3, 0.f)));
  } else if constexpr (EPI == E_RELU2_SQ) {
    const float a = fmaxf(v.x, 0.f), b = fmaxf(v.y, 0.f), c = fmaxf(v.z, 0.f), d = fmaxf(v.w, 0.f);
    *reinterpret_cast<uint2*>(static_cast<bf16*>(p.C) + off) =
        make_uint2(pack_bf16x2(a * a, b * b), pack_bf16x2(c * c, d * d));
  } else if constexpr (EPI == E_RELU2_BWD_SQ) {
    const uint2 q = *reinterpret_cast<const uint2*>(p.aux + off);
    // hardware square root (about 1 ulp): relu(u) from the stored relu(u)^2
    const float r0 = __builtin_amdgcn_sqrtf(bf2f((bf16)(q.x & 0xffffu)));
    const float r1 = __builtin_amdgcn_sqrtf(bf2f((bf16)(q.x >> 16)));
    const float r2 = __builtin_amdgcn_sqrtf(bf2f((bf16)(q.y & 0xffffu)));
    const float r3 = __builtin_amdgcn_sqrtf(bf2f((bf16)(q.y >> 16)));
    *reinterpret_cast<uint2*>(static_cast<bf16*>(p.C) + off) =
        make_uint2(pack_bf16x2(v.x * 2.f * r0, v.y * 2.f * r1), pack_bf16x2(v.z * 2.f * r2, v.w * 2.f * r3));
  } else {  // E_PARTIAL: [split][M][N] fp32
    static_assert(EPI == E_PARTIAL, "the cross-entropy epilogues are the pipelined kernel's own");
    *reinterpret_cast<float4*>(static_cast<float*>(p.C) + (int64_t)blockIdx.z * p.M * p.N +
                               (int64_t)row * p.N + col) = v;
  }
}

// DIRECT: every k-tile is full (K and the split length are multiples of BK),
// so K-contiguous operands can use the direct global -> LDS path.
template <bool AK, bool BKC, int EPI, bool DIRECT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_mfma_kernel(MfmaParams p) {
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * 2 * BM * BK];
  // LDS: A buffers at [0, 2) * BM*BK, B buffers at [2, 4) * BM*BK.
  bf16* const As = lds;
  bf16* const Bs = lds + 2 * BM * BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Tile order.  Blocks are dealt round-robin to the 8 XCDs (each with its own
  // L2); remap so every XCD gets a contiguous run of the grouped order, in
  // which GROUP_M row tiles sweep the column tiles together, so the A and B
  // k-slices a run needs are shared in that XCD's L2.
  int bid = blockIdx.x;
#if NC_GEMM_XCD
  {
    const int nb = p.tiles_m * p.tiles_n;
    const int per = nb >> 3;
    if (bid < per * 8) bid = (bid & 7) * per + (bid >> 3);
  }
  const int gsize = NC_GEMM_GROUP_M * p.tiles_n;
  const int first_m = (bid / gsize) * NC_GEMM_GROUP_M;
  const int gm = min(p.tiles_m - first_m, NC_GEMM_GROUP_M);
  const int tm = first_m + (bid % gsize) % gm, tn = (bid % gsize) / gm;
#else
  const int tm = bid % p.tiles_m, tn = bid / p.tiles_m;
#endif
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = blockIdx.z * p.k_per_split;
  int kend = kbeg + p.k_per_split;
  kend = kend < p.K ? kend : p.K;
  const int nk = (kend - kbeg + BK - 1) / BK;
  constexpr bool kDirA = AK && DIRECT && NC_GEMM_DIRECT, kDirB = BKC && DIRECT && NC_GEMM_DIRECT;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra[8], rb[8];
  {
    const bool full = DIRECT || kbeg + BK <= kend;
    if (kDirA && full) {
      stage_direct(p.A, p.lda, m0, p.M, kbeg, As, wave, lane);
    } else {
      load_tile<AK>(p.A, p.lda, m0, p.M, kbeg, kend, tid, ra);
      store_tile<AK>(As, tid, ra);
    }
    if (kDirB && full) {
      stage_direct(p.B, p.ldb, n0, p.N, kbeg, Bs, wave, lane);
    } else {
      load_tile<BKC>(p.B, p.ldb, n0, p.N, kbeg, kend, tid, rb);
      store_tile<BKC>(Bs, tid, rb);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  const int frow = lane & 31, fhalf = lane >> 5, fsw = swz(lane & 31);
  // Register-path LDS writes per k-tile (direct staging needs none).
  constexpr int kWrites = (kDirA ? 0 : 8) + (kDirB ? 0 : 8);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1, nxt = cur ^ 1;
    // The loop body has no branches so that it is one scheduling region: the
    // last iteration re-stages the first tile (in bounds) into the idle buffer.
    const int k1 = kt + 1 < nk ? kbeg + (kt + 1) * BK : kbeg;
    if (kDirA) stage_direct(p.A, p.lda, m0, p.M, k1, As + nxt * (BM * BK), wave, lane);
    else load_tile<AK>(p.A, p.lda, m0, p.M, k1, kend, tid, ra);
    if (kDirB) stage_direct(p.B, p.ldb, n0, p.N, k1, Bs + nxt * (BN * BK), wave, lane);
    else load_tile<BKC>(p.B, p.ldb, n0, p.N, k1, kend, tid, rb);

    const bf16* a_s = As + cur * (BM * BK) + (wm * 128 + frow) * BK;
    const bf16* b_s = Bs + cur * (BN * BK) + (wn * 128 + frow) * BK;
    // Fragments for k-step ks + 1 are read from LDS while the 16 MFMAs of
    // step ks issue (two register sets), so LDS latency stays hidden.
    bf16x8_t fa[2][4], fb[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[0][i] = *reinterpret_cast<const bf16x8_t*>(a_s + i * 32 * BK + ((fhalf ^ fsw) << 3));
      fb[0][i] = *reinterpret_cast<const bf16x8_t*>(b_s + i * 32 * BK + ((fhalf ^ fsw) << 3));
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the 8 reads of step 0 first
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks & 1;
      if (ks + 1 < 4) {
        const int ch = (((ks + 1) * 2 + fhalf) ^ fsw) << 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[c ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(a_s + i * 32 * BK + ch);
          fb[c ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(b_s + i * 32 * BK + ch);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][j], fa[c][i], acc[i][j], 0, 0, 0);
      if (ks + 1 < 4) {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // 2 MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read (next step)
        }
      }
    }
    if (!kDirA) store_tile<AK>(As + nxt * (BM * BK), tid, ra);
    if (!kDirB) store_tile<BKC>(Bs + nxt * (BN * BK), tid, rb);
    // last k-step: interleave the staging writes of the next tile
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (g < kWrites) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Epilogue, staged through LDS (free after the last barrier) so global
  // traffic is row-contiguous.  The MFMAs above take B as their first operand,
  // so tile (i, j) is computed transposed: lane l holds output row
  // 32 i + (l & 31) and, in registers 4 q .. 4 q + 3, the four consecutive
  // columns 32 j + 8 q + 4 (l >> 5) + 0..3 -- one 16-byte LDS write each.
  // Per 32-row slab every wave writes its [32][SROW] fp32 region, then reads
  // it back as float4 along rows.
  constexpr int SROW = 132;  // 128 columns + pad: 16 consecutive rows hit distinct banks
  float* stage = reinterpret_cast<float*>(lds) + wave * (32 * SROW);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(stage + (lane & 31) * SROW + j * 32 + 8 * q + 4 * (lane >> 5)) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    __syncthreads();
    for (int it = 0; it < 16; ++it) {
      const int idx = it * 64 + lane;
      const int row = idx >> 5, c4 = (idx & 31) * 4;
      const float4 v = *reinterpret_cast<const float4*>(stage + row * SROW + c4);
      const int grow = m0 + wm * 128 + i * 32 + row, gcol = n0 + wn * 128 + c4;
      if (grow < p.M && gcol < p.N) epilogue4<EPI>(p, v, grow, gcol);
    }
    __syncthreads();
  }
}

// 8-wave form of stage_direct: each of the 8 waves moves 4 groups of 8 rows.
__device__ __forceinline__ void stage_direct8(const bf16* __restrict__ P, int64_t ld, int r0, int R, int k0, bf16* S,
                                              int wave, int lane) {
  const int rsub = lane >> 3;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int grp = wave * 4 + i;
    const int c = (lane & 7) ^ swz(grp * 8 + rsub);
    int r = r0 + grp * 8 + rsub;
    r = r < R ? r : R - 1;
    __builtin_amdgcn_global_load_lds(P + (int64_t)r * ld + k0 + c * 8,
                                     (__attribute__((address_space(3))) void*)(S + grp * 8 * BK), 16, 0, 0);
  }
}

// 8 waves (2 per SIMD) in a 2 x 4 grid of 128 x 64 wave tiles.
//   TN = true:  both operands M/N-contiguous (the weight-gradient form); each
//               half of the block (256 threads) stages one operand through
//               registers with the 8x8 transpose, any K multiple of 8.  Only
//               launched when a k-tile is ragged (full tiles take the
//               pipelined kernel below).
//   TN = false: K-contiguous operands staged by DMA (superseded by the
//               pipelined kernel; kept for the shared code path).
template <int EPI, bool TN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_mfma8_kernel(MfmaParams p) {
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * 2 * BM * BK];
  // LDS: A buffers at [0, 2) * BM*BK, B buffers at [2, 4) * BM*BK.
  bf16* const As = lds;
  bf16* const Bs = lds + 2 * BM * BK;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves of 128 x 64

  // Tile order.  Blocks are dealt round-robin to the 8 XCDs (each with its own
  // L2); remap so every XCD gets a contiguous run of the grouped order, in
  // which GROUP_M row tiles sweep the column tiles together, so the A and B
  // k-slices a run needs are shared in that XCD's L2.
  int bid = blockIdx.x;
#if NC_GEMM_XCD
  {
    const int nb = p.tiles_m * p.tiles_n;
    const int per = nb >> 3;
    if (bid < per * 8) bid = (bid & 7) * per + (bid >> 3);
  }
  const int gsize = NC_GEMM_GROUP_M * p.tiles_n;
  const int first_m = (bid / gsize) * NC_GEMM_GROUP_M;
  const int gm = min(p.tiles_m - first_m, NC_GEMM_GROUP_M);
  const int tm = first_m + (bid % gsize) % gm, tn = (bid % gsize) / gm;
#else
  const int tm = bid % p.tiles_m, tn = bid / p.tiles_m;
#endif
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = blockIdx.z * p.k_per_split;
  int kend = kbeg + p.k_per_split;
  kend = kend < p.K ? kend : p.K;
  const int nk = (kend - kbeg + BK - 1) / BK;

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // TN staging: threads [0, 256) move A, [256, 512) move B.
  const int op = tid >> 8, tl = tid & 255;
  const bf16* const sP = op ? p.B : p.A;
  const int64_t sld = op ? p.ldb : p.lda;
  const int sr0 = op ? n0 : m0, sR = op ? p.N : p.M;
  bf16* const sS = op ? Bs : As;
  uint4 rv[8];
  if constexpr (TN) {
    load_tile<false>(sP, sld, sr0, sR, kbeg, kend, tl, rv);
    store_tile<false>(sS, tl, rv);
  } else {
    stage_direct8(p.A, p.lda, m0, p.M, kbeg, As, wave, lane);
    stage_direct8(p.B, p.ldb, n0, p.N, kbeg, Bs, wave, lane);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int frow = lane & 31, fhalf = lane >> 5, fsw = swz(lane & 31);
  // Register-path LDS writes per k-tile (direct staging needs none).
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1, nxt = cur ^ 1;
    // The loop body has no branches so that it is one scheduling region: the
    // last iteration re-stages the first tile (in bounds) into the idle buffer.
    const int k1 = kt + 1 < nk ? kbeg + (kt + 1) * BK : kbeg;
    if constexpr (TN) {
      load_tile<false>(sP, sld, sr0, sR, k1, kend, tl, rv);
    } else {
      stage_direct8(p.A, p.lda, m0, p.M, k1, As + nxt * (BM * BK), wave, lane);
      stage_direct8(p.B, p.ldb, n0, p.N, k1, Bs + nxt * (BN * BK), wave, lane);
    }

    const bf16* a_s = As + cur * (BM * BK) + (wm * 128 + frow) * BK;
    const bf16* b_s = Bs + cur * (BN * BK) + (wn * 64 + frow) * BK;
    // Fragments for k-step ks + 1 are read from LDS while the 16 MFMAs of
    // step ks issue (two register sets), so LDS latency stays hidden.
    bf16x8_t fa[2][4], fb[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[0][i] = *reinterpret_cast<const bf16x8_t*>(a_s + i * 32 * BK + ((fhalf ^ fsw) << 3));
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[0][j] = *reinterpret_cast<const bf16x8_t*>(b_s + j * 32 * BK + ((fhalf ^ fsw) << 3));
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks & 1;
      if (ks + 1 < 4) {
        const int ch = (((ks + 1) * 2 + fhalf) ^ fsw) << 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[c ^ 1][i] = *reinterpret_cast<const bf16x8_t*>(a_s + i * 32 * BK + ch);
#pragma unroll
        for (int j = 0; j < 2; ++j) fb[c ^ 1][j] = *reinterpret_cast<const bf16x8_t*>(b_s + j * 32 * BK + ch);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][j], fa[c][i], acc[i][j], 0, 0, 0);
      if (ks + 1 < 4) {
#pragma unroll
        for (int g = 0; g < 6; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    }
    if constexpr (TN) {
      store_tile<false>(sS + nxt * (BM * BK), tl, rv);
      // last k-step: interleave the 8 staging writes with its 8 MFMAs
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Epilogue, staged through LDS (free after the last barrier) so global
  // traffic is row-contiguous.  The MFMAs above take B as their first operand,
  // so tile (i, j) is computed transposed: lane l holds output row
  // 32 i + (l & 31) and, in registers 4 q .. 4 q + 3, the four consecutive
  // columns 32 j + 8 q + 4 (l >> 5) + 0..3 -- one 16-byte LDS write each.
  // Per 32-row slab every wave writes its [32][SROW] fp32 region, then reads
  // it back as float4 along rows.
  constexpr int SROW = 68;  // 64 columns + pad
  float* stage = reinterpret_cast<float*>(lds) + wave * (32 * SROW);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(stage + (lane & 31) * SROW + j * 32 + 8 * q + 4 * (lane >> 5)) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    __syncthreads();
    for (int it = 0; it < 8; ++it) {
      const int idx = it * 64 + lane;
      const int row = idx >> 4, c4 = (idx & 15) * 4;
      const float4 v = *reinterpret_cast<const float4*>(stage + row * SROW + c4);
      const int grow = m0 + wm * 128 + i * 32 + row, gcol = n0 + wn * 64 + c4;
      if (grow < p.M && gcol < p.N) epilogue4<EPI>(p, v, grow, gcol);
    }
    __syncthreads();
  }
}

// C[m, n] (+)= sum_z partial[z][m][n], z in increasing order.
__global__ void splitk_reduce_kernel(const float* __restrict__ part, int splits, int M, int N,
                                     float* __restrict__ C, int64_t ldc, int beta) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += part[(int64_t)z * total + i];
    const int64_t m = i / N, n = i - m * N;
    float* c = C + m * ldc + n;
    *c = beta ? *c + s : s;
  }
}

// The same sum four columns at a time (N, ldc and both buffers 16-byte
// aligned), the loads of four splits issued together and added in order.
__global__ void splitk_reduce4_kernel(const float* __restrict__ part, int splits, int M, int N,
                                      float* __restrict__ C, int64_t ldc, int beta) {
  const int64_t total = (int64_t)M * N, total4 = total >> 2;
  for (int64_t i4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i4 < total4;
       i4 += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = i4 * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    int z = 0;
    for (; z + 4 <= splits; z += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = ld_nt(part + (int64_t)(z + u) * total + i);
#pragma unroll
      for (int u = 0; u < 4; ++u) s = make_float4(s.x + v[u].x, s.y + v[u].y, s.z + v[u].z, s.w + v[u].w);
    }
    for (; z < splits; ++z) {
      const float4 v = ld_nt(part + (int64_t)z * total + i);
      s = make_float4(s.x + v.x, s.y + v.y, s.z + v.z, s.w + v.w);
    }
    const int64_t m = i / N, n = i - m * N;
    float4* c = reinterpret_cast<float4*>(C + m * ldc + n);
    if (beta) {
      const float4 o = *c;
      s = make_float4(o.x + s.x, o.y + s.y, o.z + s.z, o.w + s.w);
    }
    *c = s;
  }
}

// ---------------------------------------------------------------------------
// fp32 path: a plain LDS-tiled SIMT kernel over generic strides (the fp32
// configuration is small; this path is about exactness, not speed).
// A'(m, k) = A[m * sam + k * sak], B'(k, n) = B[k * sbk + n * sbn].
// ---------------------------------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int64_t sam,
                                                       int64_t sak, const float* __restrict__ B,
                                                       int64_t sbk, int64_t sbn, int M, int N, int K,
                                                       float* C, int64_t ldc, const float* aux,
                                                       float* aux_out) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = threadIdx.x; e < 16 * 64; e += 256) {
      const int kk = e >> 6, x = e & 63;
      const int k = k0 + kk;
      const int m = m0 + x, n = n0 + x;
      As[kk][x] = (k < K && m < M) ? A[(int64_t)m * sam + (int64_t)k * sak] : 0.f;
      Bs[kk][x] = (k < K && n < N) ? B[(int64_t)k * sbk + (int64_t)n * sbn] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      const int64_t off = (int64_t)m * ldc + n;
      const float v = acc[i][j];
      if constexpr (EPI == E_STORE_F32) {
        C[off] = v;
      } else if constexpr (EPI == E_ACC_F32) {
        C[off] += v;
      } else if constexpr (EPI == E_RELU2) {
        C[off] = v;
        const float rl = fmaxf(v, 0.f);
        aux_out[off] = rl * rl;
      } else if constexpr (EPI == E_RELU2_BWD) {
        C[off] = v * 2.f * fmaxf(aux[off], 0.f);
      } else if constexpr (EPI == E_RELU2_SQ) {
        const float rl = fmaxf(v, 0.f);
        C[off] = rl * rl;
      } else if constexpr (EPI == E_RELU2_BWD_SQ) {
        C[off] = v * 2.f * sqrtf(aux[off]);
      }
    }
  }
}

template <bool AK, bool BKC, bool DIRECT>
hipError_t launch_mfma(int epi, const MfmaParams& p, int splits, hipStream_t s) {
  dim3 grid(p.tiles_m * p.tiles_n, 1, splits);
  dim3 block(NT);
  switch (epi) {
    case E_STORE_F32: gemm_mfma_kernel<AK, BKC, E_STORE_F32, DIRECT><<<grid, block, 0, s>>>(p); break;
    case E_ACC_F32: gemm_mfma_kernel<AK, BKC, E_ACC_F32, DIRECT><<<grid, block, 0, s>>>(p); break;
    case E_STORE_BF16: gemm_mfma_kernel<AK, BKC, E_STORE_BF16, DIRECT><<<grid, block, 0, s>>>(p); break;
    case E_RELU2: gemm_mfma_kernel<AK, BKC, E_RELU2, DIRECT><<<grid, block, 0, s>>>(p); break;
    case E_RELU2_BWD: gemm_mfma_kernel<AK, BKC, E_RELU2_BWD, DIRECT><<<grid, block, 0, s>>>(p); break;
    case E_RELU2_SQ: gemm_mfma_kernel<AK, BKC, E_RELU2_SQ, DIRECT><<<grid, block, 0, s>>>(p); break;
    case E_RELU2_BWD_SQ: gemm_mfma_kernel<AK, BKC, E_RELU2_BWD_SQ, DIRECT><<<grid, block, 0, s>>>(p); break;
    default: gemm_mfma_kernel<AK, BKC, E_PARTIAL, DIRECT><<<grid, block, 0, s>>>(p); break;
  }
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Weight-gradient form (both operands M/N-contiguous, K = tokens) with direct
// staging: tiles are moved exactly as stored, [64 k-rows][256 columns], by
// global_load_lds, and MFMA operands are read transposed from LDS with
// ds_read_b64_tr_b16 (in a 16-lane group lane j receives element j % 4 of the
// 8-byte pieces addressed by lanes j/4, 4 + j/4, 8 + j/4, 12 + j/4; pointing
// lane p at k-row kb + p/4, column c0 + 4 (p % 4) gives lane j the four
// k-rows kb..kb+3 of column c0 + j).  Both operands use the same k-slot order
// (slot e of half h <-> k = 16 ks + 8 (e >> 2) + 4 h + (e & 3)).  16-byte
// chunks are swizzled by c ^ 4 (row & 3), which spreads a 32-lane transposed
// read over all 64 banks.  Used by the pipelined kernel below; every k-tile
// must be full.
// ---------------------------------------------------------------------------
constexpr int TROW = 256;  // columns per staged k-row
__device__ __forceinline__ int tn_off(int row, int c) { return row * TROW + ((c ^ (4 * (row & 3))) << 3); }

__device__ __forceinline__ void stage_tn(const bf16* __restrict__ P, int64_t ld, int c0, int C, int k0, bf16* S,
                                         int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = wave * 4 + i;  // 2 k-rows per 1 KB instruction
    const int row = g * 2 + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (row & 3));
    int col = c0 + c * 8;
    col = col < C ? col : C - 8;
    __builtin_amdgcn_global_load_lds(P + (int64_t)(k0 + row) * ld + col,
                                     (__attribute__((address_space(3))) void*)(S + g * 2 * TROW), 16, 0, 0);
  }
}

typedef __bf16 bf16x4_t __attribute__((__vector_size__(4 * sizeof(__bf16))));

// operand fragment: MFMA rows = columns col0 .. col0 + 31, k-slots from k-rows
// 16 ks + 8 (e >> 2) + 4 h + (e & 3)
__device__ __forceinline__ bf16x8_t frag_tn(const bf16* S, int ks, int col0, int lane) {
  const int g = lane >> 4, p = lane & 15, h = lane >> 5;
  const int col = col0 + 16 * (g & 1) + 4 * (p & 3);
  const int r1 = 16 * ks + 4 * h + (p >> 2);
  const bf16* a1 = S + tn_off(r1, col >> 3) + (col & 7);
  const bf16* a2 = S + tn_off(r1 + 8, col >> 3) + (col & 7);
  const bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)a1);
  const bf16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)a2);
  const uint2 u = __builtin_bit_cast(uint2, x), v = __builtin_bit_cast(uint2, y);
  return __builtin_bit_cast(bf16x8_t, make_uint4(u.x, u.y, v.x, v.y));
}

// ---------------------------------------------------------------------------
// Pipelined 8-wave kernel for both direct-staged forms (TN = false: operands
// K-contiguous, staged with stage_direct8 and read as row fragments;
// TN = true: operands with K as rows, staged with stage_tn and read with
// ds_read_b64_tr_b16).  Same 2 x 4 grid of 128 x 64 wave tiles as above, but
// the k loop is rotated so the MFMA pipe never waits on a barrier-fresh tile:
// the block barrier sits inside the last k-step, after its first MFMAs, and
// right after it the waves issue the A half of tile kt + 2's DMA (into the
// buffer just released) and the first fragment reads of tile kt + 1, while
// the rest of the last k-step's MFMAs run.  The B half follows in the first
// k-step of tile kt + 1.  Each DMA instruction sits behind its own MFMA:
// issued as a burst of eight per wave (64 per CU) they queued in the load
// path and held up the MFMAs behind them (2-3% slower).  Every k-tile must be
// full.
// ---------------------------------------------------------------------------
#ifndef NC_GEMM_PIPE_PRE
#define NC_GEMM_PIPE_PRE 1  // MFMAs of the last k-step issued before the barrier
#endif

// Staging of the pipelined kernel: per stage a scalar buffer resource at the
// tile's first row and column and per-lane loop-invariant 32-bit byte
// offsets, computed once per tile.
struct StageOff {
  uint32_t a[4], b[4];
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const bf16* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), 0, 0x7fffffff, 0x00020000);
}

template <bool TN>
__device__ __forceinline__ void stage_offsets(const MfmaParams& p, int m0, int n0, int wave, int lane, StageOff& o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (TN) {
      const int g = wave * 4 + i;
      const int row = g * 2 + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (row & 3));
      const int ca = min(m0 + c * 8, p.M - 8) - m0, cb = min(n0 + c * 8, p.N - 8) - n0;
      o.a[i] = (uint32_t)(((int64_t)row * p.lda + ca) * 2);
      o.b[i] = (uint32_t)(((int64_t)row * p.ldb + cb) * 2);
    } else {
      const int grp = wave * 4 + i, rsub = lane >> 3;
      const int c = (lane & 7) ^ swz(grp * 8 + rsub);
      const int ra = min(m0 + grp * 8 + rsub, p.M - 1) - m0, rb = min(n0 + grp * 8 + rsub, p.N - 1) - n0;
      o.a[i] = (uint32_t)(((int64_t)ra * p.lda + c * 8) * 2);
      o.b[i] = (uint32_t)(((int64_t)rb * p.ldb + c * 8) * 2);
    }
  }
}

template <bool TN>
__device__ __forceinline__ void pipe_stage_buf(const MfmaParams& p, int m0, int n0, int k0, bf16* a_buf, bf16* b_buf,
                                               int wave, const StageOff& o) {
  const bf16* pa = TN ? p.A + (int64_t)k0 * p.lda + m0 : p.A + (int64_t)m0 * p.lda + k0;
  const bf16* pb = TN ? p.B + (int64_t)k0 * p.ldb + n0 : p.B + (int64_t)n0 * p.ldb + k0;
  const __amdgpu_buffer_rsrc_t ra = tile_rsrc(pa), rb = tile_rsrc(pb);
  // LDS destination of instruction i of this wave (1 KB each)
  const int step = TN ? 2 * TROW : 8 * BK;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = wave * 4 + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(a_buf + g * step), 16,
                                             o.a[i], 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = wave * 4 + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (__attribute__((address_space(3))) void*)(b_buf + g * step), 16,
                                             o.b[i], 0, 0, 0);
  }
}

// One operand's half of a stage from a tile corner already offset to its k-tile.
template <bool TN>
__device__ __forceinline__ void pipe_stage_src(const bf16* src, bf16* buf, int wave, const uint32_t (&o)[4]) {
  const __amdgpu_buffer_rsrc_t ra = tile_rsrc(src);
  const int step = TN ? 2 * TROW : 8 * BK;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(buf + (wave * 4 + i) * step), 16,
                                             o[i], 0, 0, 0);
}

template <bool TN>
__device__ __forceinline__ void pipe_frags(const bf16* a_buf, const bf16* b_buf, int ks, int wm, int wn, int lane,
                                           bf16x8_t (&fa)[4], bf16x8_t (&fb)[2]) {
  if constexpr (TN) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = frag_tn(a_buf, ks, wm * 128 + i * 32, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = frag_tn(b_buf, ks, wn * 64 + j * 32, lane);
  } else {
    const int frow = lane & 31, fhalf = lane >> 5;
    const int ch = ((ks * 2 + fhalf) ^ swz(frow)) << 3;
    const bf16* a_s = a_buf + (wm * 128 + frow) * BK + ch;
    const bf16* b_s = b_buf + (wn * 64 + frow) * BK + ch;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(a_s + i * 32 * BK);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = *reinterpret_cast<const bf16x8_t*>(b_s + j * 32 * BK);
  }
}

// Scheduling pattern: NG groups of one MFMA followed by a share of NRD DS reads.
template <int G, int NG, int NRD>
__device__ __forceinline__ void sched_mfma_ds() {
  if constexpr (G < NG) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NRD / NG + (G < NRD % NG ? 1 : 0), 0);
    sched_mfma_ds<G + 1, NG, NRD>();
  }
}

// DS reads per fragment set: 6 row reads, or 12 transposed half reads.
template <bool TN>
constexpr int pipe_nreads() { return TN ? 12 : 6; }

// s_waitcnt immediate (gfx9 layout: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8) for vmcnt <= 8 with the other two counters left alone: a
// stage is 8 DMA instructions per wave (4 for A, 4 for B) in every staging
// form below (pipe_stage_buf, stage_direct8, stage_tn).
constexpr int kWaitFirstStage = 8 | (7 << 4) | (15 << 8);

#ifndef NC_GEMM_XPF
#define NC_GEMM_XPF 1  // persistent blocks DMA the next work item's first k-tiles under the current one's last
#endif


// Work item -> (tile row, tile column, k-split) of the persistent kernel.
__device__ __forceinline__ void pipe_item(const MfmaParams& p, int item, int nb, int& tm, int& tn, int& split) {
  int bid = item;
#if NC_GEMM_XCD
  if (p.kxcd) {
    // Split-K with a multiple of 8 splits: give every XCD whole k-splits
    // (split s on XCD s mod 8): an XCD then reads only its own k-ranges of
    // the panels, and its tiles (in the grouped order below) share those
    // ranges in its L2.
    const int j = bid >> 3;
    split = (bid & 7) + 8 * (j / nb);
    bid = j % nb;
  } else {
    split = bid / nb;
    bid -= split * nb;
    const int per = nb >> 3;
    if (bid < per * 8) bid = (bid & 7) * per + (bid >> 3);
  }
  const int gsize = NC_GEMM_GROUP_M * p.tiles_n;
  const int first_m = (bid / gsize) * NC_GEMM_GROUP_M;
  const int gm = min(p.tiles_m - first_m, NC_GEMM_GROUP_M);
  tm = first_m + (bid % gsize) % gm;
  tn = (bid % gsize) / gm;
#else
  split = bid / nb;
  bid -= split * nb;
  tm = bid % p.tiles_m;
  tn = bid / p.tiles_m;
#endif
}

template <int EPI, bool TN>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_pipe_kernel(MfmaParams p) {
  // The two stages of each operand are separate LDS objects and the k loop
  // below is unrolled by two, so every DMA and fragment read names its stage
  // at compile time.  The compiler then knows that the reads of one stage do
  // not alias the DMA in flight into the other; with a single array indexed
  // at run time it has to assume they may, and makes the transposed reads
  // (ds_read_b64_tr_b16) wait for that DMA to land.
  __shared__ __attribute__((aligned(16))) bf16 sA0[BM * BK];
  __shared__ __attribute__((aligned(16))) bf16 sA1[BM * BK];
  __shared__ __attribute__((aligned(16))) bf16 sB0[BN * BK];
  __shared__ __attribute__((aligned(16))) bf16 sB1[BN * BK];
  // cross-entropy epilogues: the block's row targets (and log-sum-exps),
  // fetched before the k loop so that their latency is hidden by it
  constexpr bool XENT = EPI == E_XENT_FWD || EPI == E_XENT_BWD;
  __shared__ int32_t s_xt[XENT ? BM : 1];
  __shared__ float s_xl[EPI == E_XENT_BWD ? BM : 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  // Persistent blocks: work item f (a tile, or a tile and k-split) runs on
  // block f mod gridDim.x, items in increasing order, so that a CU goes from
  // one tile to the next without a new block being dispatched.  Blocks are
  // dealt round-robin to the 8 XCDs and gridDim.x is a multiple of 8, so
  // item f still runs on XCD f mod 8.
  const int nb = p.tiles_m * p.tiles_n;
  const int nitems = nb * p.splits;
  // pf_in: this item's first k-tile (stage 0) was DMA'd under the previous
  // item's last k-tile.
  bool pf_in = false;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
  int tm, tn, split;
  pipe_item(p, item, nb, tm, tn, split);
  float* cpart = static_cast<float*>(p.C);  // E_PARTIAL: this split's [M][N] slice
  if constexpr (EPI == E_PARTIAL) cpart += (int64_t)split * p.M * p.N;
  const int m0 = tm * BM, n0 = tn * BN;
  const int kbeg = split * p.k_per_split;
  int kend = kbeg + p.k_per_split;
  kend = kend < p.K ? kend : p.K;
  const int nk = (kend - kbeg) / BK;
  const int klast = kbeg + (nk - 1) * BK;
  // The k loop DMAs two k-tiles past its last one (into the stages the loop
  // order gives them).  With an even k-tile count those are stage 0 (both
  // operands) and stage 1 (A), where the next item's loop expects its first
  // tile and its second tile's A: they then carry that item's data instead of
  // repeating this item's last tile, and the next item starts its products
  // without a prologue.  Both tiles must be whole, so that they share this
  // item's per-lane offsets (the row clamps at the matrix edge are the only
  // difference between tiles).
  // Tile corners (at this item's first k-tile) and the step from one k-tile
  // to the next, per operand.  The k loop DMAs two k-tiles past the last
  // one: "nxt" is where the first of them reads (stage 0, which the next
  // item's loop starts from: its first k-tile, or this item's last one again
  // when there is no prefetch), and the second repeats this item's last
  // k-tile (an L2 hit that the end of the loop waits for).
  const int64_t ksa = TN ? (int64_t)BK * p.lda : BK, ksb = TN ? (int64_t)BK * p.ldb : BK;
  const bf16* const a_cur = TN ? p.A + (int64_t)kbeg * p.lda + m0 : p.A + (int64_t)m0 * p.lda + kbeg;
  const bf16* const b_cur = TN ? p.B + (int64_t)kbeg * p.ldb + n0 : p.B + (int64_t)n0 * p.ldb + kbeg;
  const bf16* const a_last = a_cur + (nk - 1) * ksa;
  const bf16* a_nxt = a_last;
  const bf16* b_nxt = b_cur + (nk - 1) * ksb;
  bool pf_out = false;
#if NC_GEMM_XPF
  if (item + (int)gridDim.x < nitems) {
    int tmn, tnn, spn;
    pipe_item(p, item + gridDim.x, nb, tmn, tnn, spn);
    const int m0n = tmn * BM, n0n = tnn * BN, kbegn = spn * p.k_per_split;
    // even k-tile count: the first DMA past the end lands in stage 0.  Whole
    // tiles: the next item's per-lane offsets equal this item's (the row
    // clamps at the matrix edge are the only difference between tiles).
    pf_out = (nk & 1) == 0 && kbegn < p.K && m0 + BM <= p.M && n0 + BN <= p.N && m0n + BM <= p.M &&
             n0n + BN <= p.N;
    if (pf_out) {
      a_nxt = TN ? p.A + (int64_t)kbegn * p.lda + m0n : p.A + (int64_t)m0n * p.lda + kbegn;
      b_nxt = TN ? p.B + (int64_t)kbegn * p.ldb + n0n : p.B + (int64_t)n0n * p.ldb + kbegn;
    }
  }
#endif
  // corner of virtual k-tile v of this item (v >= nk: past its end)
  auto src_a = [&](int v) { return v < nk ? a_cur + v * ksa : (v == nk ? a_nxt : a_last); };
  auto src_b = [&](int v) { return v < nk ? b_cur + v * ksb : b_nxt; };
  if constexpr (XENT) {
    if (tid < BM) {
      const int r = m0 + tid;
      s_xt[tid] = r < p.M ? p.xtgt[r] - p.xv0 : -1;
      if constexpr (EPI == E_XENT_BWD) s_xl[tid] = r < p.M ? p.xlse[r] * kLog2e : 0.f;
    }
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  StageOff so;
  stage_offsets<TN>(p, m0, n0, wave, lane, so);
  if (!pf_in) {
    pipe_stage_buf<TN>(p, m0, n0, kbeg, sA0, sB0, wave, so);
    pipe_stage_buf<TN>(p, m0, n0, nk > 1 ? kbeg + BK : kbeg, sA1, sB1, wave, so);
    // Only the first stage has to have landed here (vmcnt <= the 8 DMAs of
    // the second stage per wave, expcnt and lgkmcnt not waited on): the
    // second one is waited for at the barrier inside the first k-tile.
    __builtin_amdgcn_s_waitcnt(kWaitFirstStage);
  } else {
    // the first stage arrived under the previous item's last k-tile
    pipe_stage_buf<TN>(p, m0, n0, nk > 1 ? kbeg + BK : kbeg, sA1, sB1, wave, so);
  }
  // A plain s_barrier, not __syncthreads: the latter's release fence would
  // wait for every outstanding load, the second stage's DMA included.  The
  // empty asm keeps the compiler from moving the first fragment reads above
  // it.
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  constexpr int NR = pipe_nreads<TN>();
  bf16x8_t fa[2][4], fb[2][2];
  pipe_frags<TN>(sA0, sB0, 0, wm, wn, lane, fa[0], fb[0]);

  // k-tile kt: its operands are in stage (a_c, b_c); tile kt + 1 is in the
  // other stage (a_o, b_o), and tile kt + 2 is DMA'd into (a_c, b_c) once
  // the block is past its last reads: A right after the barrier in tile kt's
  // last k-step, B in tile kt + 1's first k-step (where this lambda issues B
  // of tile kt + 1 into b_o, released at the previous tile's barrier).
  auto k_tile = [&](const int kt, bf16* a_c, bf16* b_c, bf16* a_o, bf16* b_o, const bf16* src_b1,
                    const bf16* src_a2) {
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const int c = ks & 1;
      if (ks == 0)  // (tile 1's B repeats the prologue's DMA: same data)
        pipe_stage_src<TN>(src_b1, b_o, wave, so.b);
      pipe_frags<TN>(a_c, b_c, ks + 1, wm, wn, lane, fa[c ^ 1], fb[c ^ 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[c][j], fa[c][i], acc[i][j], 0, 0, 0);
      // all of the next k-step's reads go out under the first MFMAs
      if (ks == 0) {
#pragma unroll
        for (int g = 0; g < 3; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, NR / 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      } else {
#pragma unroll
        for (int g = 0; g < 3; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, NR / 3, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 5, 0);
      }
    }
    // last k-step (fragments in set 1): PRE MFMAs, barrier, then the A DMA
    // of tile kt + 2 into the released buffer and tile kt + 1's first
    // fragments under the remaining MFMAs.
#pragma unroll
    for (int q = 0; q < NC_GEMM_PIPE_PRE; ++q)
      acc[q >> 1][q & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1][q & 1], fa[1][q >> 1], acc[q >> 1][q & 1], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // tile kt + 1 has landed (this wave's DMA) and this wave's reads of tile
    // kt are done; the barrier extends both to the whole block
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    pipe_stage_src<TN>(src_a2, a_c, wave, so.a);
    pipe_frags<TN>(a_o, b_o, 0, wm, wn, lane, fa[0], fb[0]);
#pragma unroll
    for (int q = NC_GEMM_PIPE_PRE; q < 8; ++q)
      acc[q >> 1][q & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[1][q & 1], fa[1][q >> 1], acc[q >> 1][q & 1], 0, 0, 0);
    constexpr int POST = 8 - NC_GEMM_PIPE_PRE;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
    sched_mfma_ds<0, POST - 4, NR>();
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    k_tile(kt, sA0, sB0, sA1, sB1, src_b(kt + 1), src_a(kt + 2));
    k_tile(kt + 1, sA1, sB1, sA0, sB0, src_b(kt + 2), src_a(kt + 3));
  }
  if (kt < nk) k_tile(kt, sA0, sB0, sA1, sB1, src_b(kt + 1), src_a(kt + 2));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Epilogue staging: each 32-row block of a wave's accumulators goes through
  // LDS.  With the cross-item prefetch, stage 0 holds the next item's first
  // k-tile while this epilogue runs, so the staging is stage 1 (waves 0-3 in
  // its A, 4-7 in its B): 32 rows x 64 floats per wave, the 16-byte chunks of
  // row r XOR-swizzled by r mod 16.  Otherwise 32 rows of 68 floats, three
  // waves per stage.
#if NC_GEMM_XPF
  constexpr int SROW = 64;
  static_assert(4 * 32 * SROW * 4 <= BM * BK * 2, "epilogue staging does not fit stage 1");
  float* stage = reinterpret_cast<float*>(wave < 4 ? sA1 : sB1) + (wave & 3) * (32 * SROW);
  auto sidx = [](int row, int c4) { return row * SROW + (((c4 >> 2) ^ (row & 15)) << 2); };
#else
  constexpr int SROW = 68;
  static_assert(3 * 32 * SROW * 4 <= BM * BK * 2, "epilogue staging does not fit a stage");
  float* stage = reinterpret_cast<float*>(wave < 3 ? sA0 : (wave < 6 ? sA1 : sB0)) + (wave % 3) * (32 * SROW);
  auto sidx = [](int row, int c4) { return row * SROW + c4; };
#endif
  // Epilogue inputs read from memory are loaded one 32-row slab ahead of
  // their use, so that their latency overlaps the LDS staging: the relu^2
  // backward's stored activation and the accumulated fp32 C.  Element (i, it) of this lane is row
  // m0 + wm 128 + 32 i + (64 it + lane) / 16, columns n0 + wn 64 + 4 (lane % 16) + 0..3.
  constexpr bool PF_AUX = EPI == E_RELU2_BWD || EPI == E_RELU2_BWD_SQ;
  constexpr bool PF_C = EPI == E_ACC_F32;
  const int er0 = m0 + wm * 128 + (lane >> 4), ec = n0 + wn * 64 + (lane & 15) * 4;
  uint2 pa[2][8];
  float4 pc[2][8];
  auto load_aux = [&](int i, uint2 (&dst)[8]) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int grow = er0 + i * 32 + 4 * it;
      dst[it] = grow < p.M && ec < p.N ? ld_nt(p.aux + (int64_t)grow * p.ldc + ec) : make_uint2(0, 0);
    }
  };
  if constexpr (PF_AUX) load_aux(0, pa[0]);
  if constexpr (PF_C) {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int grow = er0 + 4 * it;
      pc[0][it] = grow < p.M && ec < p.N ? ld_nt(static_cast<const float*>(p.C) + (int64_t)grow * p.ldc + ec)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (PF_AUX) {
      if (i + 1 < 4) load_aux(i + 1, pa[(i + 1) & 1]);
    }
    if constexpr (PF_C) {
      if (i + 1 < 4) {
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int grow = er0 + (i + 1) * 32 + 4 * it;
          pc[(i + 1) & 1][it] =
              grow < p.M && ec < p.N ? ld_nt(static_cast<const float*>(p.C) + (int64_t)grow * p.ldc + ec)
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(stage + sidx(lane & 31, j * 32 + 8 * q + 4 * (lane >> 5))) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
    // the staging area is this wave's own: only its lanes' LDS writes have to
    // land before the reads (no block barrier, whose fence would also wait for
    // the previous slab's global stores)
    wave_lds_sync();
    // stored values of the cross-entropy epilogue: this lane's element of
    // iteration it is 4 rows further than that of it - 1
    bf16* code = nullptr;
    if constexpr (EPI == E_XENT_FWD)
      code = static_cast<bf16*>(p.C) + (int64_t)(m0 + wm * 128 + i * 32 + (lane >> 4)) * p.ldc + n0 + wn * 64 +
             (lane & 15) * 4;
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int idx = it * 64 + lane;
      const int row = idx >> 4, c4 = (idx & 15) * 4;
      const float4 v = *reinterpret_cast<const float4*>(stage + sidx(row, c4));
      const int grow = m0 + wm * 128 + i * 32 + row, gcol = n0 + wn * 64 + c4;
      if constexpr (EPI == E_XENT_FWD) {
        xent_fwd4(p, v, grow, gcol, n0 + wn * 64, s_xt[grow - m0], code);
        code += 4 * p.ldc;
      } else if (grow < p.M && gcol < p.N) {
        const int64_t off = (int64_t)grow * p.ldc + gcol;
        if constexpr (EPI == E_XENT_BWD) {
          xent_bwd4(p, v, grow, gcol, s_xt[grow - m0], s_xl[grow - m0]);
        } else if constexpr (EPI == E_RELU2_BWD_SQ) {
          const uint2 q = pa[i & 1][it];
          const float r0 = __builtin_amdgcn_sqrtf(bf2f((bf16)(q.x & 0xffffu)));
          const float r1 = __builtin_amdgcn_sqrtf(bf2f((bf16)(q.x >> 16)));
          const float r2 = __builtin_amdgcn_sqrtf(bf2f((bf16)(q.y & 0xffffu)));
          const float r3 = __builtin_amdgcn_sqrtf(bf2f((bf16)(q.y >> 16)));
          st_nt(static_cast<bf16*>(p.C) + off,
              make_uint2(pack_bf16x2(v.x * 2.f * r0, v.y * 2.f * r1), pack_bf16x2(v.z * 2.f * r2, v.w * 2.f * r3)));
        } else if constexpr (EPI == E_RELU2_BWD) {
          const uint2 u = pa[i & 1][it];
          const float u0 = bf2f((bf16)(u.x & 0xffffu)), u1 = bf2f((bf16)(u.x >> 16));
          const float u2 = bf2f((bf16)(u.y & 0xffffu)), u3 = bf2f((bf16)(u.y >> 16));
          *reinterpret_cast<uint2*>(static_cast<bf16*>(p.C) + off) =
              make_uint2(pack_bf16x2(v.x * 2.f * fmaxf(u0, 0.f), v.y * 2.f * fmaxf(u1, 0.f)),
                         pack_bf16x2(v.z * 2.f * fmaxf(u2, 0.f), v.w * 2.f * fmaxf(u3, 0.f)));
        } else if constexpr (EPI == E_ACC_F32) {
          const float4 o = pc[i & 1][it];
          st_nt(static_cast<float*>(p.C) + off, make_float4(o.x + v.x, o.y + v.y, o.z + v.z, o.w + v.w));
        } else if constexpr (EPI == E_PARTIAL) {
          st_nt(cpart + (int64_t)grow * p.N + gcol, v);
        } else if constexpr (EPI == E_STORE_F32) {
          st_nt(static_cast<float*>(p.C) + off, v);
        } else if constexpr (EPI == E_STORE_BF16) {
          st_nt(static_cast<bf16*>(p.C) + off, make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w)));
        } else if constexpr (EPI == E_RELU2_SQ) {
          const float a = fmaxf(v.x, 0.f), b = fmaxf(v.y, 0.f), c = fmaxf(v.z, 0.f), d = fmaxf(v.w, 0.f);
          st_nt(static_cast<bf16*>(p.C) + off, make_uint2(pack_bf16x2(a * a, b * b), pack_bf16x2(c * c, d * d)));
        } else {
          epilogue4<EPI>(p, v, grow, gcol);
        }
      }
    }
    wave_lds_sync();  // this slab's reads of the staging area precede the next slab's writes
  }
  // The next item's DMA and target fetch reuse the LDS this epilogue read:
  // a block barrier after this wave's LDS reads (its global stores may stay
  // in flight).
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  pf_in = pf_out;
  }
}

// Blocks of the persistent GEMM grid: one per CU (a block's 128 KB of LDS
// leaves room for no second one), a multiple of 8 so that every XCD gets the
// same number.
int persistent_blocks() {
  static int blocks[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!blocks[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) cus = 256;
    blocks[dev] = cus / 8 * 8;
  }
  return blocks[dev];
}

template <bool TN>
hipError_t launch_pipe(int epi, const MfmaParams& p0, int splits, hipStream_t s) {
  MfmaParams p = p0;
  p.splits = splits;
  p.kxcd = NC_GEMM_KXCD && NC_GEMM_XCD && epi == E_PARTIAL && splits > 1 && splits % 8 == 0 ? splits : 0;
  const int items = p.tiles_m * p.tiles_n * splits;
  dim3 grid(std::min(items, persistent_blocks()), 1, 1);
  switch (epi) {
    case E_STORE_F32: gemm_pipe_kernel<E_STORE_F32, TN><<<grid, 512, 0, s>>>(p); break;
    case E_ACC_F32: gemm_pipe_kernel<E_ACC_F32, TN><<<grid, 512, 0, s>>>(p); break;
    case E_STORE_BF16: gemm_pipe_kernel<E_STORE_BF16, TN><<<grid, 512, 0, s>>>(p); break;
    case E_RELU2: gemm_pipe_kernel<E_RELU2, TN><<<grid, 512, 0, s>>>(p); break;
    case E_RELU2_BWD: gemm_pipe_kernel<E_RELU2_BWD, TN><<<grid, 512, 0, s>>>(p); break;
    case E_RELU2_SQ: gemm_pipe_kernel<E_RELU2_SQ, TN><<<grid, 512, 0, s>>>(p); break;
    case E_RELU2_BWD_SQ: gemm_pipe_kernel<E_RELU2_BWD_SQ, TN><<<grid, 512, 0, s>>>(p); break;
    case E_XENT_FWD: gemm_pipe_kernel<E_XENT_FWD, false><<<grid, 512, 0, s>>>(p); break;
    case E_XENT_BWD: gemm_pipe_kernel<E_XENT_BWD, false><<<grid, 512, 0, s>>>(p); break;
    default: gemm_pipe_kernel<E_PARTIAL, TN><<<grid, 512, 0, s>>>(p); break;
  }
  return hipGetLastError();
}

template <bool TN>
hipError_t launch_mfma8(int epi, const MfmaParams& p, int splits, hipStream_t s) {
  dim3 grid(p.tiles_m * p.tiles_n, 1, splits);
  dim3 block(512);
  switch (epi) {
    case E_STORE_F32: gemm_mfma8_kernel<E_STORE_F32, TN><<<grid, block, 0, s>>>(p); break;
    case E_ACC_F32: gemm_mfma8_kernel<E_ACC_F32, TN><<<grid, block, 0, s>>>(p); break;
    case E_STORE_BF16: gemm_mfma8_kernel<E_STORE_BF16, TN><<<grid, block, 0, s>>>(p); break;
    case E_RELU2: gemm_mfma8_kernel<E_RELU2, TN><<<grid, block, 0, s>>>(p); break;
    case E_RELU2_BWD: gemm_mfma8_kernel<E_RELU2_BWD, TN><<<grid, block, 0, s>>>(p); break;
    case E_RELU2_SQ: gemm_mfma8_kernel<E_RELU2_SQ, TN><<<grid, block, 0, s>>>(p); break;
    case E_RELU2_BWD_SQ: gemm_mfma8_kernel<E_RELU2_BWD_SQ, TN><<<grid, block, 0, s>>>(p); break;
    default: gemm_mfma8_kernel<E_PARTIAL, TN><<<grid, block, 0, s>>>(p); break;
  }
  return hipGetLastError();
}

template <bool AK, bool BKC>
hipError_t launch_mfma(int epi, const MfmaParams& p, int splits, bool direct, hipStream_t s) {
  const double flops = 2.0 * p.M * p.N * p.K;
  if (AK && BKC && direct) {
    probe_begin(NC_PROBE_GEMM_NT, s);
    const hipError_t e = launch_pipe<false>(epi, p, splits, s);
    probe_end(NC_PROBE_GEMM_NT, s, flops);
    return e;
  }
  if (!AK && !BKC && direct) {
    probe_begin(NC_PROBE_GEMM_WGRAD, s);
    const hipError_t e = launch_pipe<true>(epi, p, splits, s);
    probe_end(NC_PROBE_GEMM_WGRAD, s, flops);
    return e;
  }
  if (!AK && !BKC) {  // weight-gradient form with a ragged k-tile
    probe_begin(NC_PROBE_GEMM_WGRAD, s);
    const hipError_t e = launch_mfma8<true>(epi, p, splits, s);
    probe_end(NC_PROBE_GEMM_WGRAD, s, flops);
    return e;
  }
  if (direct && (AK || BKC)) return launch_mfma<AK, BKC, true>(epi, p, splits, s);
  return launch_mfma<AK, BKC, false>(epi, p, splits, s);
}

// Split-K count for few-tile, long-K products.  One 512-thread block fits a
// CU (128 KB of LDS), so blocks run in rounds of 256; the estimated time is
// rounds x (k per split + a fixed per-block cost of ~8 k-steps: prologue,
// drain and the fp32 partial store), minimised over the split count.
int choose_splits(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = cdiv(M, BM) * cdiv(N, BN);
  if (tiles >= 512 || K < 4096) return 1;
  const int64_t max_s = K / 1024;
#if NC_GEMM_SPLIT_MODEL
  int64_t best = 1, best_cost = -1;
  for (int64_t s = 1; s <= max_s; ++s) {
    const int64_t kps = cdiv(cdiv(K, s), BK) * BK;
    const int64_t cost = cdiv(tiles * s, 256) * (kps + NC_GEMM_SPLIT_C0 * BK);
    if (best_cost < 0 || cost < best_cost) best = s, best_cost = cost;
  }
  return (int)best;
#else
  int64_t s = cdiv(640, tiles);
  if (s > max_s) s = max_s;
  return s < 1 ? 1 : (int)s;
#endif
}

int split_k_per(int64_t K, int splits) { return (int)(cdiv(cdiv(K, splits), BK) * BK); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }


}  // namespace

// fp32 partial products of the general path's split-K.
size_t split_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  const int s = choose_splits(M, N, K);
  if (s <= 1) return 0;
  return (size_t)s * (size_t)M * (size_t)N * sizeof(float);
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) { return split_workspace_bytes(M, N, K); }

// Logit product with a softcap cross-entropy epilogue (internal; the
// pipelined kernel's K-contiguous form only).
int gemm_xent(const GemmDesc& g, hipStream_t stream) {
  NC_REQUIRE(g.xent == 1 || g.xent == 2, NC_ERR_INVALID_ARG, "gemm: bad cross-entropy mode");
  NC_REQUIRE(g.A && g.B && g.xtgt, NC_ERR_INVALID_ARG, "gemm: null operand");
  NC_REQUIRE(g.dtype == NC_BF16 && g.transA == 0 && g.transB == 1, NC_ERR_UNSUPPORTED,
             "gemm: the cross-entropy epilogues need bf16 K-contiguous operands");
  NC_REQUIRE(g.M > 0 && g.N > 0 && g.K > 0 && g.M < (1ll << 31) && g.N < (1ll << 31), NC_ERR_INVALID_ARG,
             "gemm: bad shape");
  NC_REQUIRE(g.K % BK == 0 && g.N % 8 == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0 && g.lda >= g.K && g.ldb >= g.K,
             NC_ERR_UNSUPPORTED, "gemm: the cross-entropy epilogues need K a multiple of 64");
  NC_REQUIRE(aligned16(g.A) && aligned16(g.B), NC_ERR_INVALID_ARG, "gemm: A and B must be 16-byte aligned");
  NC_REQUIRE(g.xv0 % 64 == 0, NC_ERR_INVALID_ARG, "gemm: vocabulary offset must be a multiple of 64");
  if (g.xent == 1) {
    NC_REQUIRE(g.xpart && g.xztgt, NC_ERR_INVALID_ARG, "gemm: null cross-entropy output");
    if (g.C) NC_REQUIRE(g.xerr && g.ldc >= g.N && g.ldc % 4 == 0, NC_ERR_INVALID_ARG, "gemm: bad stored-logit layout");
  }
  else NC_REQUIRE(g.C && g.xlse && g.cdt == NC_BF16 && g.ldc >= g.N, NC_ERR_INVALID_ARG, "gemm: bad dz output");
  MfmaParams p{};
  p.A = static_cast<const bf16*>(g.A);
  p.B = static_cast<const bf16*>(g.B);
  p.lda = g.lda;
  p.ldb = g.ldb;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.k_per_split = (int)g.K;
  p.tiles_m = (int)cdiv(g.M, BM);
  p.tiles_n = (int)cdiv(g.N, BN);
  p.C = g.C;
  p.ldc = g.ldc;
  p.xc = g.xc;
  p.xinv_c = 1.f / g.xc;
  p.xdl = g.xdl;
  p.xtgt = g.xtgt;
  p.xlse = g.xlse;
  p.xpart = g.xpart;
  p.xztgt = g.xztgt;
  p.xerr = g.xerr;
  p.xv0 = g.xv0;
  const double flops = 2.0 * p.M * p.N * p.K;
  probe_begin(NC_PROBE_GEMM_NT, stream);
  const hipError_t e = launch_pipe<false>(g.xent == 1 ? E_XENT_FWD : E_XENT_BWD, p, 1, stream);
  probe_end(NC_PROBE_GEMM_NT, stream, flops);
  if (e != hipSuccess) return set_error(NC_ERR_HIP, "gemm launch failed: %s", hipGetErrorString(e));
  return NC_OK;
}

int gemm(const GemmDesc& g, hipStream_t stream) {
  if (g.xent) return gemm_xent(g, stream);
  NC_REQUIRE(g.A && g.B && g.C, NC_ERR_INVALID_ARG, "gemm: null operand");
  NC_REQUIRE(g.M > 0 && g.N > 0 && g.K > 0, NC_ERR_INVALID_ARG, "gemm: M, N, K must be positive");
  NC_REQUIRE(g.M < (1ll << 31) && g.N < (1ll << 31) && g.K < (1ll << 31), NC_ERR_UNSUPPORTED,
             "gemm: dimensions must be below 2^31");
  NC_REQUIRE(g.transA == 0 || g.transA == 1, NC_ERR_INVALID_ARG, "gemm: transA must be 0 or 1");
  NC_REQUIRE(g.transB == 0 || g.transB == 1, NC_ERR_INVALID_ARG, "gemm: transB must be 0 or 1");
  NC_REQUIRE(g.dtype == NC_F32 || g.dtype == NC_BF16, NC_ERR_INVALID_ARG, "gemm: bad dtype");
  NC_REQUIRE(g.epi >= NC_EPI_STORE && g.epi <= NC_EPI_RELU2_BWD_SQ, NC_ERR_INVALID_ARG, "gemm: bad epilogue");
  NC_REQUIRE(g.beta == 0.f || g.beta == 1.f, NC_ERR_INVALID_ARG, "gemm: beta must be 0 or 1");
  const int64_t a_rows = g.transA ? g.K : g.M, a_cols = g.transA ? g.M : g.K;
  const int64_t b_rows = g.transB ? g.N : g.K, b_cols = g.transB ? g.K : g.N;
  (void)a_rows; (void)b_rows;
  NC_REQUIRE(g.lda >= a_cols && g.ldb >= b_cols && g.ldc >= g.N, NC_ERR_INVALID_ARG,
             "gemm: leading dimension too small");
  if (g.epi == NC_EPI_RELU2) NC_REQUIRE(g.aux_out, NC_ERR_INVALID_ARG, "gemm: relu2 needs aux_out");
  if (g.epi == NC_EPI_RELU2_BWD || g.epi == NC_EPI_RELU2_BWD_SQ)
    NC_REQUIRE(g.aux, NC_ERR_INVALID_ARG, "gemm: relu2_bwd needs aux");
  if (g.beta == 1.f)
    NC_REQUIRE(g.cdt == NC_F32 && g.epi == NC_EPI_STORE, NC_ERR_INVALID_ARG,
               "gemm: beta = 1 needs an fp32 C and the plain store epilogue");
  if (g.capc > 0.f)
    NC_REQUIRE(skinny_ok(g), NC_ERR_UNSUPPORTED, "gemm: the softcap epilogue is for bf16 products with M <= 128");
  if (g.sk_split > 1)
    NC_REQUIRE(skinny_ok(g), NC_ERR_UNSUPPORTED, "gemm: split partial products are for bf16 products with M <= 128");
  if (skinny_ok(g)) return gemm_skinny(g, stream);

  if (g.dtype == NC_F32) {
    NC_REQUIRE(g.cdt == NC_F32, NC_ERR_INVALID_ARG, "gemm: fp32 operands need an fp32 C");
    const float* A = static_cast<const float*>(g.A);
    const float* B = static_cast<const float*>(g.B);
    const int64_t sam = g.transA ? 1 : g.lda, sak = g.transA ? g.lda : 1;
    const int64_t sbk = g.transB ? 1 : g.ldb, sbn = g.transB ? g.ldb : 1;
    dim3 grid((unsigned)cdiv(g.N, 64), (unsigned)cdiv(g.M, 64));
    float* C = static_cast<float*>(g.C);
    const float* aux = static_cast<const float*>(g.aux);
    float* aux_out = static_cast<float*>(g.aux_out);
    const int M = (int)g.M, N = (int)g.N, K = (int)g.K;
    if (g.epi == NC_EPI_RELU2)
      gemm_f32_kernel<E_RELU2><<<grid, 256, 0, stream>>>(A, sam, sak, B, sbk, sbn, M, N, K, C, g.ldc, aux, aux_out);
    else if (g.epi == NC_EPI_RELU2_BWD)
      gemm_f32_kernel<E_RELU2_BWD><<<grid, 256, 0, stream>>>(A, sam, sak, B, sbk, sbn, M, N, K, C, g.ldc, aux, aux_out);
    else if (g.epi == NC_EPI_RELU2_SQ)
      gemm_f32_kernel<E_RELU2_SQ><<<grid, 256, 0, stream>>>(A, sam, sak, B, sbk, sbn, M, N, K, C, g.ldc, aux, aux_out);
    else if (g.epi == NC_EPI_RELU2_BWD_SQ)
      gemm_f32_kernel<E_RELU2_BWD_SQ><<<grid, 256, 0, stream>>>(A, sam, sak, B, sbk, sbn, M, N, K, C, g.ldc, aux,
                                                              aux_out);
    else if (g.beta == 1.f)
      gemm_f32_kernel<E_ACC_F32><<<grid, 256, 0, stream>>>(A, sam, sak, B, sbk, sbn, M, N, K, C, g.ldc, aux, aux_out);
    else
      gemm_f32_kernel<E_STORE_F32><<<grid, 256, 0, stream>>>(A, sam, sak, B, sbk, sbn, M, N, K, C, g.ldc, aux, aux_out);
    return check_launch("gemm_f32_kernel");
  }

  // bf16 matrix-core path
  NC_REQUIRE(g.M % 8 == 0 && g.N % 8 == 0 && g.K % 8 == 0, NC_ERR_UNSUPPORTED,
             "gemm: bf16 path needs M, N, K multiples of 8 (got %lld %lld %lld)", (long long)g.M,
             (long long)g.N, (long long)g.K);
  NC_REQUIRE(g.lda % 8 == 0 && g.ldb % 8 == 0, NC_ERR_UNSUPPORTED,
             "gemm: bf16 path needs lda, ldb multiples of 8");
  NC_REQUIRE(aligned16(g.A) && aligned16(g.B), NC_ERR_INVALID_ARG, "gemm: A and B must be 16-byte aligned");
  if (g.epi != NC_EPI_STORE) NC_REQUIRE(g.cdt == NC_BF16, NC_ERR_INVALID_ARG, "gemm: relu2 epilogues write bf16");

  MfmaParams p;
  p.A = static_cast<const bf16*>(g.A);
  p.B = static_cast<const bf16*>(g.B);
  p.lda = g.lda;
  p.ldb = g.ldb;
  p.M = (int)g.M;
  p.N = (int)g.N;
  p.K = (int)g.K;
  p.tiles_m = (int)cdiv(g.M, BM);
  p.tiles_n = (int)cdiv(g.N, BN);
  p.C = g.C;
  p.ldc = g.ldc;
  p.aux = static_cast<const bf16*>(g.aux);
  p.aux_out = static_cast<bf16*>(g.aux_out);

  int epi;
  if (g.epi == NC_EPI_RELU2) epi = E_RELU2;
  else if (g.epi == NC_EPI_RELU2_BWD) epi = E_RELU2_BWD;
  else if (g.epi == NC_EPI_RELU2_SQ) epi = E_RELU2_SQ;
  else if (g.epi == NC_EPI_RELU2_BWD_SQ) epi = E_RELU2_BWD_SQ;
  else if (g.cdt == NC_BF16) epi = E_STORE_BF16;
  else epi = g.beta == 1.f ? E_ACC_F32 : E_STORE_F32;

  int splits = 1;
  if (epi == E_STORE_F32 || epi == E_ACC_F32) {
    splits = choose_splits(g.M, g.N, g.K);
    if (splits > 1 && (g.ws == nullptr || g.ws_bytes < split_workspace_bytes(g.M, g.N, g.K))) splits = 1;
  }
  p.k_per_split = splits > 1 ? split_k_per(g.K, splits) : (int)g.K;
  if (splits > 1) splits = (int)cdiv(g.K, p.k_per_split);
  float* final_c = static_cast<float*>(g.C);
  const int final_beta = epi == E_ACC_F32;
  if (splits > 1) {
    p.C = g.ws;
    epi = E_PARTIAL;
  }

  const bool ak = g.transA == 0, bk = g.transB == 1;
  const bool direct = g.K % BK == 0 && p.k_per_split % BK == 0;
  hipError_t e;
  if (ak && bk) e = launch_mfma<true, true>(epi, p, splits, direct, stream);
  else if (ak && !bk) e = launch_mfma<true, false>(epi, p, splits, direct, stream);
  else if (!ak && bk) e = launch_mfma<false, true>(epi, p, splits, direct, stream);
  else e = launch_mfma<false, false>(epi, p, splits, direct, stream);
  if (e != hipSuccess) return set_error(NC_ERR_HIP, "gemm launch failed: %s", hipGetErrorString(e));

  if (splits > 1) {
    const int64_t total = g.M * g.N;
    const uintptr_t align = reinterpret_cast<uintptr_t>(g.ws) | reinterpret_cast<uintptr_t>(final_c);
    if (g.N % 4 == 0 && g.ldc % 4 == 0 && align % 16 == 0) {
      const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(total / 4, 256), 4096);
      splitk_reduce4_kernel<<<blocks, 256, 0, stream>>>(static_cast<const float*>(g.ws), splits, p.M, p.N,
                                                        final_c, g.ldc, final_beta);
      return check_launch("splitk_reduce4_kernel");
    }
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(total, 256), 4096);
    splitk_reduce_kernel<<<blocks, 256, 0, stream>>>(static_cast<const float*>(g.ws), splits, p.M, p.N,
                                                     final_c, g.ldc, final_beta);
    return check_launch("splitk_reduce_kernel");
  }
  return NC_OK;
}

}  // namespace nc

extern "C" size_t nc_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  return nc::gemm_workspace_bytes(M, N, K);
}

extern "C" int nc_gemm_bf16(int transA, int transB, int64_t M, int64_t N, int64_t K, const void* A,
                            int64_t lda, const void* B, int64_t ldb, void* C, int cdt, int64_t ldc,
                            float beta, int epilogue, const void* aux, void* aux_out, int dtype,
                            void* ws, size_t ws_bytes, void* stream) {
  nc::GemmDesc g;
  g.transA = transA;
  g.transB = transB;
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
  g.beta = beta;
  g.epi = epilogue;
  g.aux = aux;
  g.aux_out = aux_out;
  g.dtype = dtype;
  g.ws = ws;
  g.ws_bytes = ws_bytes;
  return nc::api_done(nc::gemm(g, static_cast<hipStream_t>(stream)), stream, "nc_gemm_bf16");
}

// ---------------------------------------------------------------------------
// Transpose of a row-major [R, C] matrix of 2- or 4-byte elements into
// [C, R] (leading dimension R).  64 x 64 tiles through padded LDS; the
// backward turns every x W product into the K-contiguous form with it.
// ---------------------------------------------------------------------------
namespace nc {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int64_t R, int64_t C,
                                                        T* __restrict__ dst) {
  __shared__ T tile[64][65];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int rr = ty + 4 * i;
    if (r0 + rr < R && c0 + tx < C) tile[rr][tx] = src[(r0 + rr) * C + c0 + tx];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int cc = ty + 4 * i;
    if (c0 + cc < C && r0 + tx < R) dst[(c0 + cc) * R + r0 + tx] = tile[tx][cc];
  }
}

// 2-byte elements with R and C multiples of 8 and 16-byte aligned matrices:
// every global access moves 8 elements (16 bytes).  Thread t handles the
// 8-element pieces t and t + 256 of the tile: on the way in, piece id is
// row id / 8 of the tile, columns 8 (id % 8) ..; on the way out, output row
// id / 8 (a tile column), output columns 8 (id % 8) .. (eight tile rows).
// Up to four 2-byte matrices transposed by one launch (a layer's weights):
// block b takes 64 x 64 tile b - first[i] of the job i whose range holds b.
struct TransposeJobs {
  const uint16_t* src[4];
  uint16_t* dst[4];
  int64_t R[4], C[4];
  int first[5];  // first block of each job; first[n] = blocks in all
  int tiles_c[4];
};

__device__ __forceinline__ void transpose_b16x8_tile(const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                                     uint16_t* __restrict__ dst, int64_t r0, int64_t c0,
                                                     uint16_t (&tile)[64][72]);

__global__ __launch_bounds__(256) void transpose_b16x8_batch_kernel(TransposeJobs jb) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];
  const int b = blockIdx.x;
  const int i = b < jb.first[1] ? 0 : (b < jb.first[2] ? 1 : (b < jb.first[3] ? 2 : 3));
  const int k = b - jb.first[i];
  const int64_t r0 = (int64_t)(k / jb.tiles_c[i]) * 64, c0 = (int64_t)(k % jb.tiles_c[i]) * 64;
  transpose_b16x8_tile(jb.src[i], jb.R[i], jb.C[i], jb.dst[i], r0, c0, tile);
}

__global__ __launch_bounds__(256) void transpose_b16x8_kernel(const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                                              uint16_t* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64][72];  // rows 144 bytes apart
  transpose_b16x8_tile(src, R, C, dst, (int64_t)blockIdx.y * 64, (int64_t)blockIdx.x * 64, tile);
}

__device__ __forceinline__ void transpose_b16x8_tile(const uint16_t* __restrict__ src, int64_t R, int64_t C,
                                                     uint16_t* __restrict__ dst, int64_t r0, int64_t c0,
                                                     uint16_t (&tile)[64][72]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int id = t + 256 * k, rr = id >> 3, ch = (id & 7) * 8;
    if (r0 + rr < R && c0 + ch < C)  // C % 8 == 0: the piece is whole
      *reinterpret_cast<uint4*>(&tile[rr][ch]) = *reinterpret_cast<const uint4*>(src + (r0 + rr) * C + c0 + ch);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int id = t + 256 * k, cc = id >> 3, ch = (id & 7) * 8;
    if (c0 + cc < C && r0 + ch < R) {  // R % 8 == 0: the piece is whole
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (uint32_t)tile[ch + 2 * e][cc] | ((uint32_t)tile[ch + 2 * e + 1][cc] << 16);
      *reinterpret_cast<uint4*>(dst + (c0 + cc) * R + r0 + ch) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace

int transpose4(const void* const* src, const int64_t* R, const int64_t* C, void* const* dst, int n, hipStream_t s) {
  NC_REQUIRE(n >= 1 && n <= 4, NC_ERR_INVALID_ARG, "transpose4: 1 to 4 matrices");
  bool whole = true;  // every matrix fits the 16-byte form
  for (int i = 0; i < n; ++i) {
    NC_REQUIRE(src[i] && dst[i] && R[i] > 0 && C[i] > 0, NC_ERR_INVALID_ARG, "transpose4: bad arguments");
    whole = whole && R[i] % 8 == 0 && C[i] % 8 == 0 && aligned16(src[i]) && aligned16(dst[i]) &&
            cdiv(R[i], 64) * cdiv(C[i], 64) < ((int64_t)1 << 28);
  }
  if (!whole) {
    for (int i = 0; i < n; ++i) NC_TRY(transpose(src[i], R[i], C[i], 2, dst[i], s));
    return NC_OK;
  }
  TransposeJobs jb{};
  int blocks = 0;
  for (int i = 0; i < n; ++i) {
    jb.src[i] = static_cast<const uint16_t*>(src[i]);
    jb.dst[i] = static_cast<uint16_t*>(dst[i]);
    jb.R[i] = R[i];
    jb.C[i] = C[i];
    jb.tiles_c[i] = (int)cdiv(C[i], 64);
    jb.first[i] = blocks;
    blocks += (int)(cdiv(R[i], 64) * jb.tiles_c[i]);
  }
  for (int i = n; i <= 4; ++i) jb.first[i] = blocks;
  transpose_b16x8_batch_kernel<<<blocks, 256, 0, s>>>(jb);
  return check_launch("transpose_b16x8_batch_kernel");
}

int transpose(const void* src, int64_t R, int64_t C, int elem_bytes, void* dst, hipStream_t s) {
  NC_REQUIRE(src && dst && R > 0 && C > 0, NC_ERR_INVALID_ARG, "transpose: bad arguments");
  dim3 grid((unsigned)cdiv(C, 64), (unsigned)cdiv(R, 64));
  if (elem_bytes == 2 && R % 8 == 0 && C % 8 == 0 && aligned16(src) && aligned16(dst))
    transpose_b16x8_kernel<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(src), R, C, static_cast<uint16_t*>(dst));
  else if (elem_bytes == 2)
    transpose_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(src), R, C, static_cast<uint16_t*>(dst));
  else
    transpose_kernel<uint32_t><<<grid, 256, 0, s>>>(static_cast<const uint32_t*>(src), R, C, static_cast<uint32_t*>(dst));
  return check_launch("transpose_kernel");
}

}  // namespace nc
