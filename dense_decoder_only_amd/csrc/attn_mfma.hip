// Matrix-core (v_mfma_f32_32x32x16_bf16) kernels for causal multi-query
// attention with head_dim 128 in bf16 (release-news page "Karpathy再放大招…",
// section 技術細節與問答: multi-query attention).
//
// Folding heads into rows.  With one shared K/V head, the H query heads of a
// sequence form one [T*H, 128] matrix of query rows r = t*H + h (position
// t = r / H) against a single [T, 128] key/value pair.  A block therefore
// stages each K/V tile in LDS once and reuses it for all the heads its rows
// cover -- the multi-query saving on K/V traffic is structural.
//
// Register layouts.  Every product is issued so that the softmax direction
// (keys) lies along the MFMA rows and the query rows along the lanes: S^T =
// K Q^T puts one query row per lane column, so row maxima and sums are
// in-lane (plus one exchange with the partner half-wave), and the
// probabilities can feed the next product O^T = V^T P^T straight from
// registers.  A 32x32 output tile gives lane l the column (l & 31) and rows
// 8 (r >> 2) + 4 (l >> 5) + (r & 3), r = 0..15; the k-slots of the next
// product are renumbered to match, which a contraction allows.
//
// LDS tiles.  Row-major [rows][128] tiles swizzle 16-byte chunks by
// (row & 7); transposed [128][64] tiles swizzle 8-byte units by (row & 15).
//
// Kernels: forward (online softmax, writes O and the log-sum-exp), dQ (also
// writes D = rowsum(dO * O)), dK/dV (key blocks of 128 positions, the query
// range split into chunks so that early key blocks do not serialize, partials
// summed in a fixed order by a reduce kernel).  Nothing uses atomics; results
// are bitwise reproducible.
#include "common.h"
#include "attn_mfma.h"

namespace nc {
namespace {

constexpr int HD = 128;
constexpr int QB = 128;   // query rows per forward / dQ block (4 waves x 32)
constexpr int KT = 64;    // keys per tile
constexpr int KB = 128;   // keys per dK/dV block (4 waves x 32)
constexpr int QT = 64;    // query rows per dK/dV tile
constexpr int QCH = 5120; // query rows per dK/dV split
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ int kidx(int row, int chunk) { return row * HD + ((chunk ^ (row & 7)) << 3); }
__device__ __forceinline__ int tidx(int row, int unit) { return row * 64 + ((unit ^ (row & 15)) << 2); }

__device__ __forceinline__ uint32_t wd(const uint4& q, int w) {
  return w == 0 ? q.x : (w == 1 ? q.y : (w == 2 ? q.z : q.w));
}

// 8x8 bf16 transpose: v[kk] holds 8 consecutive columns (hd) of row kk;
// returns in o[mm] the 8 rows (kk = 0..7) of column mm as 4 words.
__device__ __forceinline__ void transpose8(const uint4 (&v)[8], uint32_t (&o)[8][4]) {
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
    const int w = mm >> 1;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t a = wd(v[2 * p], w), b = wd(v[2 * p + 1], w);
      o[mm][p] = (mm & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}

// Write a transposed 8x8 block: LDS rows hd0 + mm, columns col0 .. col0 + 7.
__device__ __forceinline__ void store_t8(bf16* T, int hd0, int col0, const uint32_t (&o)[8][4]) {
  const int u0 = col0 >> 2;
#pragma unroll
  for (int mm = 0; mm < 8; ++mm) {
    const int row = hd0 + mm;
    *reinterpret_cast<uint2*>(T + tidx(row, u0)) = make_uint2(o[mm][0], o[mm][1]);
    *reinterpret_cast<uint2*>(T + tidx(row, u0 + 1)) = make_uint2(o[mm][2], o[mm][3]);
  }
}

__device__ __forceinline__ bf16x8_t frag_k(const bf16* S, int row, int chunk) {
  return *reinterpret_cast<const bf16x8_t*>(S + kidx(row, chunk));
}

// A-operand from a transposed tile: 8 values at columns c0 .. c0+3 and
// c0+8 .. c0+11 of `row` (c0 = 4 * unit index).
__device__ __forceinline__ bf16x8_t frag_t(const bf16* T, int row, int unit) {
  const uint2 a = *reinterpret_cast<const uint2*>(T + tidx(row, unit));
  const uint2 b = *reinterpret_cast<const uint2*>(T + tidx(row, unit + 2));
  return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}

// Registers r = 8 jp .. 8 jp + 7 of a score tile, rounded to bf16, as the
// B operand of the next product.
__device__ __forceinline__ bf16x8_t pack_p(const f32x16& p, int jp) {
  const int b = jp * 8;
  return __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2(p[b + 0], p[b + 1]), pack_bf16x2(p[b + 2], p[b + 3]),
                                                 pack_bf16x2(p[b + 4], p[b + 5]), pack_bf16x2(p[b + 6], p[b + 7])));
}

__device__ __forceinline__ f32x16 mfma(bf16x8_t a, bf16x8_t b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// ------------------------------------------------------------------ forward --
// grid (B, ceil(R / QB)); heavy (late) row blocks first.
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnMfmaArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[KT * HD];
  __shared__ __attribute__((aligned(16))) bf16 Vt[HD * KT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, lc = lane & 31;
  const int H = a.H, T = a.T;
  const int R = T * H;
  const int nrb = (R + QB - 1) / QB;
  const int rb = nrb - 1 - (int)blockIdx.y;
  const int b = blockIdx.x;
  const int r0 = rb * QB;
  const bf16* base = a.qkv + (int64_t)b * T * a.S;

  const int myr = r0 + w * 32 + lc;
  const bool valid = myr < R;
  const int rr = valid ? myr : R - 1;
  const int tq = rr / H;
  const int hq = rr - tq * H;
  bf16x8_t qreg[8];
  {
    const bf16* qp = base + (int64_t)tq * a.S + hq * HD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 16);
  }
  const int tmin = r0 / H;
  const int tmax = min(T - 1, (min(r0 + QB, R) - 1) / H);
  const int ntiles = tmax / KT + 1;

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * KT;
    __syncthreads();  // previous tile fully consumed
    if (tid < 128) {  // V^T: one 8x8 block per thread
      const int kvb = tid & 7, hdb = tid >> 3;
      uint4 v[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int u = min(kv0 + kvb * 8 + kk, T - 1);
        v[kk] = *reinterpret_cast<const uint4*>(base + (int64_t)u * a.S + (H + 1) * HD + hdb * 8);
      }
      uint32_t t8[8][4];
      transpose8(v, t8);
      store_t8(Vt, hdb * 8, kvb * 8, t8);
    } else {  // K row-major: 1024 chunks over 128 threads
      const int t2 = tid - 128;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int id = t2 + 128 * i;
        const int row = id >> 4, c = id & 15;
        const int u = min(kv0 + row, T - 1);
        *reinterpret_cast<uint4*>(Ks + kidx(row, c)) =
            *reinterpret_cast<const uint4*>(base + (int64_t)u * a.S + H * HD + c * 8);
      }
    }
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s[st] = mfma(frag_k(Ks, st * 32 + lc, 2 * ks + h), qreg[ks], s[st]);
    }
    const bool need_mask = kv0 + KT - 1 > tmin;
    float mt = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[st][r] * a.scale_log2;
        if (need_mask) {
          const int kv = kv0 + st * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (kv > tq) x = -INFINITY;
        }
        s[st][r] = x;
        mt = fmaxf(mt, x);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    float ls = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(s[st][r] - m_new);
        s[st][r] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[ht][r] *= alpha;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        const bf16x8_t pb = pack_p(s[st], jp);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) o[ht] = mfma(frag_t(Vt, ht * 32 + lc, 8 * st + 4 * jp + h), pb, o[ht]);
      }
  }

  if (valid) {
    const float inv = 1.f / l_run;
    bf16* op = a.o_out + ((int64_t)b * R + myr) * HD;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int hd = ht * 32 + 8 * q4 + 4 * h;
        *reinterpret_cast<uint2*>(op + hd) =
            make_uint2(pack_bf16x2(o[ht][4 * q4] * inv, o[ht][4 * q4 + 1] * inv),
                       pack_bf16x2(o[ht][4 * q4 + 2] * inv, o[ht][4 * q4 + 3] * inv));
      }
    if (h == 0) a.lse_out[(int64_t)b * R + myr] = (m_run + log2f(l_run)) * (1.f / LOG2E);
  }
}

// ----------------------------------------------------------------------- dQ --
// Also writes D = rowsum(dO * O) for the key-side kernel.
__global__ __launch_bounds__(256) void attn_dq_kernel(AttnMfmaArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[KT * HD];
  __shared__ __attribute__((aligned(16))) bf16 Vs[KT * HD];
  __shared__ __attribute__((aligned(16))) bf16 Kt[HD * KT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, lc = lane & 31;
  const int H = a.H, T = a.T;
  const int R = T * H;
  const int nrb = (R + QB - 1) / QB;
  const int rb = nrb - 1 - (int)blockIdx.y;
  const int b = blockIdx.x;
  const int r0 = rb * QB;
  const bf16* base = a.qkv + (int64_t)b * T * a.S;

  const int myr = r0 + w * 32 + lc;
  const bool valid = myr < R;
  const int rr = valid ? myr : R - 1;
  const int tq = rr / H;
  const int hq = rr - tq * H;
  bf16x8_t qreg[8], dreg[8];
  float dpart = 0.f;
  {
    const bf16* qp = base + (int64_t)tq * a.S + hq * HD + 8 * h;
    const bf16* dp = a.dout + ((int64_t)b * R + rr) * HD + 8 * h;
    const bf16* op = a.o + ((int64_t)b * R + rr) * HD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qreg[ks] = *reinterpret_cast<const bf16x8_t*>(qp + ks * 16);
      const uint4 dv = *reinterpret_cast<const uint4*>(dp + ks * 16);
      const uint4 ov = *reinterpret_cast<const uint4*>(op + ks * 16);
      dreg[ks] = __builtin_bit_cast(bf16x8_t, dv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = wd(dv, e), y = wd(ov, e);
        dpart += __uint_as_float(x << 16) * __uint_as_float(y << 16) +
                 __uint_as_float(x & 0xffff0000u) * __uint_as_float(y & 0xffff0000u);
      }
    }
  }
  const float D = dpart + __shfl_xor(dpart, 32, 64);
  const float lse2 = a.lse[(int64_t)b * R + rr] * LOG2E;
  if (valid && h == 0) a.Dbuf[(int64_t)b * R + myr] = D;

  const int tmin = r0 / H;
  const int tmax = min(T - 1, (min(r0 + QB, R) - 1) / H);
  const int ntiles = tmax / KT + 1;
  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = zero16();

  for (int j = 0; j < ntiles; ++j) {
    const int kv0 = j * KT;
    __syncthreads();
    // K and V row-major: 2 x 1024 chunks, 8 per thread.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 4, c = id & 15;
      const int u = min(kv0 + row, T - 1);
      const bf16* rp = base + (int64_t)u * a.S + H * HD + c * 8;
      *reinterpret_cast<uint4*>(Ks + kidx(row, c)) = *reinterpret_cast<const uint4*>(rp);
      *reinterpret_cast<uint4*>(Vs + kidx(row, c)) = *reinterpret_cast<const uint4*>(rp + HD);
    }
    if (tid < 128) {  // K^T
      const int kvb = tid & 7, hdb = tid >> 3;
      uint4 v[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int u = min(kv0 + kvb * 8 + kk, T - 1);
        v[kk] = *reinterpret_cast<const uint4*>(base + (int64_t)u * a.S + H * HD + hdb * 8);
      }
      uint32_t t8[8][4];
      transpose8(v, t8);
      store_t8(Kt, hdb * 8, kvb * 8, t8);
    }
    __syncthreads();

    f32x16 s[2], dp[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = zero16();
      dp[st] = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s[st] = mfma(frag_k(Ks, st * 32 + lc, 2 * ks + h), qreg[ks], s[st]);
        dp[st] = mfma(frag_k(Vs, st * 32 + lc, 2 * ks + h), dreg[ks], dp[st]);
      }
    }
    const bool need_mask = kv0 + KT - 1 > tmin;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = exp2f(s[st][r] * a.scale_log2 - lse2);
        if (need_mask) {
          const int kv = kv0 + st * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (kv > tq) p = 0.f;
        }
        s[st][r] = p * (dp[st][r] - D);
      }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        const bf16x8_t pb = pack_p(s[st], jp);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) dq[ht] = mfma(frag_t(Kt, ht * 32 + lc, 8 * st + 4 * jp + h), pb, dq[ht]);
      }
  }

  if (valid) {
    float* out = a.dqkv + ((int64_t)b * T + tq) * (int64_t)(H + 2) * HD + hq * HD;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int hd = ht * 32 + 8 * q4 + 4 * h;
        *reinterpret_cast<float4*>(out + hd) =
            make_float4(dq[ht][4 * q4] * a.scale, dq[ht][4 * q4 + 1] * a.scale, dq[ht][4 * q4 + 2] * a.scale,
                        dq[ht][4 * q4 + 3] * a.scale);
      }
  }
}

// -------------------------------------------------------------------- dK/dV --
__device__ __forceinline__ int qbeg_of(int kb, int H) { return ((kb * KB * H) / QT) * QT; }
__device__ __forceinline__ int nsplit_of(int kb, int H, int R) { return (R - qbeg_of(kb, H) + QCH - 1) / QCH; }

// grid (B, nkb * SMAX): block (kb, s) handles key rows kb*128 .. +127 against
// query rows [qbeg + s*QCH, min(R, qbeg + (s+1)*QCH)).  Writes partial dK^T,
// dV^T sums (unscaled) to part[(b * nkb + kb) * SMAX + s].
__global__ __launch_bounds__(256) void attn_dkv_kernel(AttnMfmaArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 Qs[QT * HD];
  __shared__ __attribute__((aligned(16))) bf16 Ds[QT * HD];
  __shared__ __attribute__((aligned(16))) bf16 Qt[HD * QT];
  __shared__ __attribute__((aligned(16))) bf16 Dt[HD * QT];
  __shared__ float lse_s[QT], D_s[QT];
  __shared__ int tpos_s[QT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = lane >> 5, lc = lane & 31;
  const int H = a.H, T = a.T;
  const int R = T * H;
  const int smax = a.smax;
  const int kb = blockIdx.y / smax, sp = blockIdx.y - (blockIdx.y / smax) * smax;
  const int b = blockIdx.x;
  if (sp >= nsplit_of(kb, H, R)) return;
  const bf16* base = a.qkv + (int64_t)b * T * a.S;
  const int u0 = kb * KB;
  const int myu = u0 + w * 32 + lc;  // this lane's key position (column)
  const int uu = min(myu, T - 1);
  bf16x8_t kreg[8], vreg[8];
  {
    const bf16* kp = base + (int64_t)uu * a.S + H * HD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kreg[ks] = *reinterpret_cast<const bf16x8_t*>(kp + ks * 16);
      vreg[ks] = *reinterpret_cast<const bf16x8_t*>(kp + HD + ks * 16);
    }
  }
  const int qs0 = qbeg_of(kb, H) + sp * QCH;
  const int qs1 = min(R, qs0 + QCH);
  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dk[i] = zero16();
    dv[i] = zero16();
  }

  for (int q0 = qs0; q0 < qs1; q0 += QT) {
    __syncthreads();
    // Q and dO row-major: 2 x 1024 chunks.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + 256 * i;
      const int row = id >> 4, c = id & 15;
      const int r = min(q0 + row, R - 1);
      const int t = r / H, hh = r - t * H;
      *reinterpret_cast<uint4*>(Qs + kidx(row, c)) =
          *reinterpret_cast<const uint4*>(base + (int64_t)t * a.S + hh * HD + c * 8);
      *reinterpret_cast<uint4*>(Ds + kidx(row, c)) =
          *reinterpret_cast<const uint4*>(a.dout + ((int64_t)b * R + r) * HD + c * 8);
    }
    {  // Q^T (threads 0..127) and dO^T (threads 128..255), one 8x8 block each
      const int t2 = tid & 127;
      const int qb = t2 & 7, hdb = t2 >> 3;
      uint4 v[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int r = min(q0 + qb * 8 + kk, R - 1);
        if (tid < 128) {
          const int t = r / H, hh = r - t * H;
          v[kk] = *reinterpret_cast<const uint4*>(base + (int64_t)t * a.S + hh * HD + hdb * 8);
        } else {
          v[kk] = *reinterpret_cast<const uint4*>(a.dout + ((int64_t)b * R + r) * HD + hdb * 8);
        }
      }
      uint32_t t8[8][4];
      transpose8(v, t8);
      store_t8(tid < 128 ? Qt : Dt, hdb * 8, qb * 8, t8);
    }
    if (tid < QT) {
      const int r = q0 + tid;
      if (r < R) {
        lse_s[tid] = a.lse[(int64_t)b * R + r] * LOG2E;
        D_s[tid] = a.Dbuf[(int64_t)b * R + r];
        tpos_s[tid] = r / H;
      } else {
        lse_s[tid] = INFINITY;  // p = 0 for rows past the end
        D_s[tid] = 0.f;
        tpos_s[tid] = -1;
      }
    }
    __syncthreads();

    // S = Q K^T and dP = dO V^T: rows q (two 32-row halves), column = key.
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      s[qt] = zero16();
      dp[qt] = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s[qt] = mfma(frag_k(Qs, qt * 32 + lc, 2 * ks + h), kreg[ks], s[qt]);
        dp[qt] = mfma(frag_k(Ds, qt * 32 + lc, 2 * ks + h), vreg[ks], dp[qt]);
      }
    }
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = qt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        float p = exp2f(s[qt][r] * a.scale_log2 - lse_s[qi]);
        if (myu > tpos_s[qi]) p = 0.f;
        s[qt][r] = p;
        dp[qt][r] = p * (dp[qt][r] - D_s[qi]);
      }
    // dV^T += dO^T P ; dK^T += Q^T dS
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        const bf16x8_t pb = pack_p(s[qt], jp);
        const bf16x8_t db = pack_p(dp[qt], jp);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          dv[ht] = mfma(frag_t(Dt, ht * 32 + lc, 8 * qt + 4 * jp + h), pb, dv[ht]);
          dk[ht] = mfma(frag_t(Qt, ht * 32 + lc, 8 * qt + 4 * jp + h), db, dk[ht]);
        }
      }
  }

  // partial [slot][2][KB keys][HD]: lane holds hd = ht*32 + 8 q4 + 4 h + e for key (w*32 + lc)
  float* pk = a.part + ((((int64_t)b * a.nkb + kb) * smax + sp) * 2) * (KB * HD) + (w * 32 + lc) * HD;
  float* pv = pk + KB * HD;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int hd = ht * 32 + 8 * q4 + 4 * h;
      *reinterpret_cast<float4*>(pk + hd) =
          make_float4(dk[ht][4 * q4], dk[ht][4 * q4 + 1], dk[ht][4 * q4 + 2], dk[ht][4 * q4 + 3]);
      *reinterpret_cast<float4*>(pv + hd) =
          make_float4(dv[ht][4 * q4], dv[ht][4 * q4 + 1], dv[ht][4 * q4 + 2], dv[ht][4 * q4 + 3]);
    }
}

// dK = scale * sum_s partial_k[s], dV = sum_s partial_v[s], splits in order.
__global__ __launch_bounds__(256) void attn_dkv_reduce_kernel(AttnMfmaArgs a) {
  const int H = a.H, T = a.T, R = T * H;
  const int kb = blockIdx.x, b = blockIdx.y;
  const int ns = nsplit_of(kb, H, R);
  const float* p0 = a.part + (((int64_t)b * a.nkb + kb) * a.smax * 2) * (KB * HD);
  for (int e = threadIdx.x * 4; e < KB * HD; e += 256 * 4) {
    const int key = e / HD, hd = e - key * HD;
    const int u = kb * KB + key;
    if (u >= T) continue;
    float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
    for (int s = 0; s < ns; ++s) {
      const float4 x = *reinterpret_cast<const float4*>(p0 + (int64_t)s * 2 * KB * HD + e);
      const float4 y = *reinterpret_cast<const float4*>(p0 + (int64_t)s * 2 * KB * HD + KB * HD + e);
      sk.x += x.x; sk.y += x.y; sk.z += x.z; sk.w += x.w;
      sv.x += y.x; sv.y += y.y; sv.z += y.z; sv.w += y.w;
    }
    float* row = a.dqkv + ((int64_t)b * T + u) * (int64_t)(H + 2) * HD;
    *reinterpret_cast<float4*>(row + H * HD + hd) = make_float4(sk.x * a.scale, sk.y * a.scale, sk.z * a.scale, sk.w * a.scale);
    *reinterpret_cast<float4*>(row + (H + 1) * HD + hd) = sv;
  }
}

}  // namespace

int attn_mfma_smax(int T, int H) { return (T * H + QCH - 1) / QCH; }

size_t attn_mfma_bwd_workspace_bytes(int B, int T, int H) {
  const int nkb = (T + KB - 1) / KB;
  const size_t dbuf = align_up((size_t)B * T * H * sizeof(float), 256);
  const size_t part = (size_t)B * nkb * attn_mfma_smax(T, H) * 2 * KB * HD * sizeof(float);
  return dbuf + align_up(part, 256);
}

int attn_mfma_fwd(const void* qkv, int B, int T, int H, float scale, void* o, float* lse, hipStream_t s) {
  AttnMfmaArgs a{};
  a.qkv = static_cast<const bf16*>(qkv);
  a.o_out = static_cast<bf16*>(o);
  a.lse_out = lse;
  a.B = B;
  a.T = T;
  a.H = H;
  a.S = (int64_t)(H + 2) * HD;
  a.scale = scale;
  a.scale_log2 = scale * LOG2E;
  const int nrb = (T * H + QB - 1) / QB;
  attn_fwd_kernel<<<dim3(B, nrb), 256, 0, s>>>(a);
  return check_launch("attn_fwd_kernel");
}

int attn_mfma_bwd(const void* qkv, const void* o, const void* dout, const float* lse, int B, int T, int H, float scale,
                  float* dqkv, void* ws, hipStream_t s) {
  AttnMfmaArgs a{};
  a.qkv = static_cast<const bf16*>(qkv);
  a.o = static_cast<const bf16*>(o);
  a.dout = static_cast<const bf16*>(dout);
  a.lse = lse;
  a.dqkv = dqkv;
  a.B = B;
  a.T = T;
  a.H = H;
  a.S = (int64_t)(H + 2) * HD;
  a.scale = scale;
  a.scale_log2 = scale * LOG2E;
  a.Dbuf = static_cast<float*>(ws);
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up((size_t)B * T * H * sizeof(float), 256));
  a.nkb = (T + KB - 1) / KB;
  a.smax = attn_mfma_smax(T, H);
  const int nrb = (T * H + QB - 1) / QB;
  attn_dq_kernel<<<dim3(B, nrb), 256, 0, s>>>(a);
  NC_TRY(check_launch("attn_dq_kernel"));
  attn_dkv_kernel<<<dim3(B, a.nkb * a.smax), 256, 0, s>>>(a);
  NC_TRY(check_launch("attn_dkv_kernel"));
  attn_dkv_reduce_kernel<<<dim3(a.nkb, B), 256, 0, s>>>(a);
  return check_launch("attn_dkv_reduce_kernel");
}

}  // namespace nc
