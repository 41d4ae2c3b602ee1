// Matrix-core (v_mfma_f32_32x32x16_bf16) kernels for causal multi-query
// attention with head_dim 128 in bf16 (release-news page "Karpathy再放大招…",
// section 技術細節與問答: multi-query attention).
//
// Folding heads into rows.  With one shared K/V head, the H query heads of a
// sequence form one [T*H, 128] matrix of query rows r = t*H + h (position
// t = r / H) against a single [T, 128] key/value pair.  A block therefore
// stages each K/V tile in LDS once for all the heads its rows cover.
//
// Register layouts.  Every product is issued so that the softmax direction
// (keys) lies along the MFMA rows and the query rows along the lanes: S^T =
// K Q^T puts one query row per lane column, so row maxima and sums are
// in-lane (plus one exchange with the partner half-wave), and the
// probabilities feed the next product O^T = V^T P^T straight from
// registers.  A 32x32 output tile gives lane l the column (l & 31) and rows
// 8 (r >> 2) + 4 (l >> 5) + (r & 3), r = 0..15; the k-slots of the next
// product are renumbered to match (slot e of half h <-> key
// 16 jp + 8 (e >> 2) + 4 h + (e & 3)), which a contraction allows.
//
// LDS.  Every operand tile is stored row-major [64 rows][128] exactly as it
// sits in HBM and arrives by direct global -> LDS loads (gfx950
// global_load_lds_dwordx4), double-buffered so the next tile is in flight
// while the current one is consumed.  Operands needed transposed (V^T, K^T,
// Q^T, dO^T) are read with ds_read_b64_tr_b16: in a 16-lane group, lane j
// receives element j % 4 of the 8-byte pieces addressed by lanes j/4,
// 4 + j/4, 8 + j/4 and 12 + j/4, so pointing lane p at row kb + p/4, columns
// c0 + 4 (p % 4) hands lane j the four consecutive rows kb..kb+3 of column
// c0 + j -- exactly four consecutive k-slots of an MFMA A operand.  16-byte
// chunks are XOR-swizzled by ((r & 3) << 2) | ((r >> 2) & 3) so that both the
// row reads and the transposed reads spread over the banks.
//
// Static stages.  The two stages of each staged operand are separate LDS
// objects and the tile loops are unrolled by two, so that every DMA and every
// read names its stage at compile time.  The compiler then knows that the
// reads of the current stage do not alias the DMA in flight into the other;
// with one array indexed at run time it must assume they may, and makes the
// reads wait for that DMA to land, which serialises the prefetch with the
// products.
//
// Kernels: forward (online softmax, writes O and the log-sum-exp), dQ (also
// writes D = rowsum(dO * O)), dK/dV (key blocks of 128 positions, the query
// range split into chunks so that early key blocks do not serialize, partials
// summed in a fixed order by a reduce kernel).  No atomics; results are
// bitwise reproducible.

#include "attn_mfma_dev.h"

namespace nc {
namespace {

// ------------------------------------------------------------------ forward --
// grid (B, ceil(R / QB)); heavy (late) row blocks first.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(AttnMfmaArgs a) {
  // one LDS object per stage; see the note on static stages above
  __shared__ __attribute__((aligned(16))) bf16 Ks0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 Ks1[TILE];
  __shared__ __attribute__((aligned(16))) bf16 Vs0[TILE];
  __shared__ __attribute__((aligned(16))) bf16 Vs1[TILE];
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
  // K/V rows are S apart: buffer resources at the sequence's K and V columns
  // and 32-bit byte offsets (rows past the end read row T - 1)
  const __amdgpu_buffer_rsrc_t krs = row_rsrc(base + H * HD), vrs = row_rsrc(base + (H + 1) * HD);
  auto stage = [&](int j, bf16* Kd, bf16* Vd) {
    const int kv0 = j * KT;
#pragma unroll
    for (int k = 0; k < KT / 16; ++k) {
      const int g = w * (KT / 16) + k;
      const int row = g * 4 + (lane >> 4);
      const uint32_t off = (uint32_t)(min(kv0 + row, T - 1) * (int)a.S + (((lane & 15) ^ tswz(row)) << 3)) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(Kd + g * 4 * HD), 16, off,
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)(Vd + g * 4 * HD), 16, off,
                                               0, 0, 0);
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;

  stage(0, Ks0, Vs0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  uint32_t rof[8], tof[8];
  frag_offsets(lane, rof, tof);
  // key tile j in (K, V); tile j + 1 is DMA'd into (Kn, Vn)
  auto kv_tile = [&](const int j, const bf16* K, const bf16* V, bf16* Kn, bf16* Vn) {
    const int kv0 = j * KT;
    if (j + 1 < ntiles) stage(j + 1, Kn, Vn);
    // The lane offsets pass through an empty asm once per tile, so that the
    // compiler does not hoist a register per (array, offset) pair out of the
    // tile loop; every fragment read is one of them plus an immediate.
    asm volatile("" : "+v"(rof[0]), "+v"(rof[1]), "+v"(rof[2]), "+v"(rof[3]), "+v"(rof[4]), "+v"(rof[5]),
                 "+v"(rof[6]), "+v"(rof[7]));
    asm volatile("" : "+v"(tof[0]), "+v"(tof[1]), "+v"(tof[2]), "+v"(tof[3]), "+v"(tof[4]), "+v"(tof[5]),
                 "+v"(tof[6]), "+v"(tof[7]));

    f32x16 s[2];
    s[0] = zero16();
    s[1] = zero16();
    {
      // K fragments of step j = 8 st + ks read PF - 1 steps ahead (a ring);
      // the two 32-key halves alternate so that back-to-back MFMAs are independent
      constexpr int PF = NC_FWD_PF;
      bf16x8_t fk[PF];
#pragma unroll
      for (int j = 0; j < PF - 1; ++j) fk[j] = frag_at(K + (j & 1) * 32 * HD, rof[j >> 1]);
      __builtin_amdgcn_sched_group_barrier(0x100, PF - 1, 0);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j + PF - 1 < 16) {
          const int jn = j + PF - 1;
          fk[jn % PF] = frag_at(K + (jn & 1) * 32 * HD, rof[jn >> 1]);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        s[j & 1] = mfma(fk[j % PF], qreg[j >> 1], s[j & 1]);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    // Row maxima of the raw scores (the scale is positive, so it commutes
    // with the maximum); the scale is applied inside the exponent below.
    float mt = -INFINITY;
    if (kv0 + KT - 1 > tmin) {  // the tile crosses some row's diagonal
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = kv0 + st * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const float x = kv > tq ? -INFINITY : s[st][r];
          s[st][r] = x;
          mt = fmaxf(mt, x);
        }
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[st][r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * a.scale_log2;
    // Lazy rescaling: the reference maximum only moves when the tile maximum
    // exceeds it by more than 8 (log2 units), so probabilities stay <= 2^8
    // and the rescale of the running sums is skipped (wave-uniformly) on most
    // tiles.  The result does not depend on the reference.
    const bool bump = mt > m_run + 8.f;
    if (__builtin_amdgcn_ballot_w64(bump)) {
      const float m_new = bump ? mt : m_run;
      const float alpha = fexp2(m_run - m_new);
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ht][r] *= alpha;
    }
    float ls = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fexp2(fmaf(s[st][r], a.scale_log2, -m_run));
        s[st][r] = p;
        ls += p;
      }
    ls += __shfl_xor(ls, 32, 64);
    l_run += ls;
    {
      // O^T += V^T P^T, step j = 4 (2 st + jp) + ht, the V^T fragments read
      // PF - 1 steps ahead (a ring)
      constexpr int PF = NC_FWD_PF;
      bf16x8_t fv[PF];
      auto v_read = [&](int j) {
        fv[j % PF] = frag_tr_at(V + ((j >> 3) * 32 + 16 * ((j >> 2) & 1)) * HD, tof[2 * (j & 3)], tof[2 * (j & 3) + 1]);
      };
#pragma unroll
      for (int j = 0; j < PF - 1; ++j) v_read(j);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * (PF - 1), 0);
      bf16x8_t pb = {};
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j + PF - 1 < 16) {
          v_read(j + PF - 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        if ((j & 3) == 0) pb = pack_p(s[j >> 3], (j >> 2) & 1);
        o[j & 3] = mfma(fv[j % PF], pb, o[j & 3]);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < ntiles; j += 2) {
    kv_tile(j, Ks0, Vs0, Ks1, Vs1);
    kv_tile(j + 1, Ks1, Vs1, Ks0, Vs0);
  }
  if (j < ntiles) kv_tile(j, Ks0, Vs0, Ks1, Vs1);

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

// -------------------------------------------------------------------- dK/dV --
__device__ __forceinline__ int qbeg_of(int kb, int H) { return ((kb * KB * H) / QT) * QT; }
__device__ __forceinline__ int nsplit_of(int kb, int H, int R, int qch) { return (R - qbeg_of(kb, H) + qch - 1) / qch; }

// grid (B, nkb * SMAX): block (kb, s) handles key rows kb*128 .. +127 against
// query rows [qbeg + s*qch, min(R, qbeg + (s+1)*qch)).  Writes partial dK^T,
// dV^T sums (unscaled) to part[(b * nkb + kb) * SMAX + s].
//
// Two roles per 32 keys, one wave each, the pair sharing a SIMD (waves w and
// w + 4 of a block run on SIMD w):
//   role P (waves 0-3): S = Q K^T, P = exp(S scale - lse) with the causal
//     mask, P handed to the partner through LDS in fp32, dV^T += dO^T P;
//   role G (waves 4-7): dP = dO V^T, then dS = P (dP - D) with the
//     partner's P, dK^T += Q^T dS.
// A query tile runs in two halves separated by a block barrier:
//   [P: S products, softmax, P to LDS | G: dP products]
//   [P: dV products                   | G: P from LDS, dS, dK products].
// Each wave holds one key-side operand (K or V of its 32 keys, 32 VGPRs) and
// one accumulator set (64), so two waves fit per SIMD, and the softmax VALU
// work of one overlaps the other's matrix-core products.
#ifndef NC_DKV_PRIO
#define NC_DKV_PRIO 1  // wave priorities that order the two roles' work on a SIMD
#endif
__device__ __forceinline__ void lds_barrier() {
  // this wave's LDS writes have landed; outstanding DMA (vmcnt) is not waited for
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_dkv_kernel(AttnMfmaArgs a) {
  // one LDS object per stage; see the note on static stages above
  __shared__ __attribute__((aligned(16))) bf16 Qs0[QTILE];
  __shared__ __attribute__((aligned(16))) bf16 Qs1[QTILE];
  __shared__ __attribute__((aligned(16))) bf16 Ds0[QTILE];
  __shared__ __attribute__((aligned(16))) bf16 Ds1[QTILE];
  // P of the current tile: [key wave][8 float4 of a lane][64 lanes]
  __shared__ __attribute__((aligned(16))) float4 Pex[4 * (QT / 8) * 64];
  __shared__ __attribute__((aligned(16))) float lse_s[2][QT];
  __shared__ __attribute__((aligned(16))) float D_s[2][QT];
  __shared__ __attribute__((aligned(16))) int tpos_s[2][QT];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, h = lane >> 5, lc = lane & 31;
  const bool role_p = wv < 4;  // wave-uniform
  const int w = wv & 3;
  const int H = a.H, T = a.T;
  const int R = T * H;
  const int smax = a.smax;
  const int kb = blockIdx.y / smax, sp = blockIdx.y - (blockIdx.y / smax) * smax;
  const int b = blockIdx.x;
  if (sp >= nsplit_of(kb, H, R, a.qch)) return;
  const bf16* base = a.qkv + (int64_t)b * T * a.S;
  const bf16* dbase = a.dout + (int64_t)b * R * HD;
  const int u0 = kb * KB;
  const int myu = u0 + w * 32 + lc;  // this lane's key position (column)
  const int uu = min(myu, T - 1);
  // role P: the lane's key row; role G: its value row
  bf16x8_t kv[8];
  {
    const bf16* kp = base + (int64_t)uu * a.S + (role_p ? H : H + 1) * HD + 8 * h;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kv[ks] = *reinterpret_cast<const bf16x8_t*>(kp + ks * 16);
  }

  const int qs0 = qbeg_of(kb, H) + sp * a.qch;
  const int qs1 = min(R, qs0 + a.qch);
  const int nq = (qs1 - qs0 + QT - 1) / QT;
  // Staging of the query tiles, through buffer resources, NST instructions
  // (4 rows each) per wave and operand.  Row r = t H + h of the folded query
  // view sits at element t S + h HD of the sequence: not a fixed stride
  // apart, so each lane keeps, for each of its DMA rows, that row's offset
  // and head and advances both by one tile (QT rows: QT / H positions and
  // QT % H heads, with a carry) per staged tile, in place of a division by H
  // per row.  Rows past the end (offsets at or past T S) read row R - 1.  dO
  // rows are HD apart.
  constexpr int NST = QT / 32;
  const int S = (int)a.S;
  const int dtq = QT / H, dhq = QT - dtq * H;
  const int qinc = dtq * S + dhq * HD, qend = T * S, qlast = (T - 1) * S + (H - 1) * HD;
  int qoff[NST], qhd[NST], dchk[NST];
#pragma unroll
  for (int k = 0; k < NST; ++k) {
    const int row = (wv * NST + k) * 4 + (lane >> 4);
    const int c8 = ((lane & 15) ^ tswz(row)) << 3;
    const int r = qs0 + row, t = div_h(r, a.hmagic);
    qhd[k] = r - t * H;
    qoff[k] = t * S + qhd[k] * HD + c8;
    dchk[k] = c8;
  }
  const __amdgpu_buffer_rsrc_t qrs = row_rsrc(base);
  auto stage = [&](int i, bf16* Qd, bf16* Gd) {
    const int q0 = qs0 + i * QT;
    const __amdgpu_buffer_rsrc_t drs = row_rsrc(dbase + (int64_t)q0 * HD);
#pragma unroll
    for (int k = 0; k < NST; ++k) {
      const int g = wv * NST + k;
      const int row = g * 4 + (lane >> 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (__attribute__((address_space(3))) void*)(Qd + g * 4 * HD), 16,
                                               (uint32_t)(qoff[k] < qend ? qoff[k] : qlast + dchk[k]) * 2, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (__attribute__((address_space(3))) void*)(Gd + g * 4 * HD), 16,
                                               (uint32_t)(min(row, R - 1 - q0) * HD + dchk[k]) * 2, 0, 0, 0);
      // advance this row to the next tile
      qhd[k] += dhq;
      qoff[k] += qinc;
      if (qhd[k] >= H) {
        qhd[k] -= H;
        qoff[k] += S - H * HD;
      }
    }
  };
  // per-row statistics of a query tile, loaded by threads 0..63 into registers
  float n_lse = 0.f, n_D = 0.f;
  int n_t = -1;
  auto fetch_stats = [&](int i) {
    const int r = qs0 + i * QT + tid;
    if (tid < QT) {
      if (r < R) {
        n_lse = a.lse[(int64_t)b * R + r];  // scaled by log2(e) in put_stats
        n_D = a.Dbuf[(int64_t)b * R + r];
        n_t = div_h(r, a.hmagic);
      } else {
        n_lse = INFINITY;  // p = 0 for rows past the end
        n_D = 0.f;
        n_t = -1;
      }
    }
  };
  auto put_stats = [&](int buf) {
    if (tid < QT) {
      // scaled here, at the end of the tile's work, so that the wait for the
      // load is not placed ahead of the tile's products
      lse_s[buf][tid] = n_lse * LOG2E;
      D_s[buf][tid] = n_D;
      tpos_s[buf][tid] = n_t;
    }
  };
  f32x16 acc[4];  // role P: dV^T, role G: dK^T (rows hd, column = this lane's key)
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = zero16();

  stage(0, Qs0, Ds0);
  fetch_stats(0);
  put_stats(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  constexpr int NQT = QT / 32;
  // x[qt] (+)= X K^T (role P, X = Q) or X V^T (role G, X = dO): rows are the
  // tile's queries, the column is this lane's key.  The X fragments of step
  // j = 8 qt + ks are read PF - 1 steps ahead of their products (a ring).
  uint32_t rof[8], tof[8];
  frag_offsets(lane, rof, tof);
  auto key_products = [&](const bf16* X, f32x16 (&x)[NQT]) {
    constexpr int NSTEP = NQT * 8, PF = NC_DKV_PF;
    bf16x8_t fx[PF];
#pragma unroll
    for (int j = 0; j < PF - 1; ++j) fx[j] = frag_at(X + (j >> 3) * 32 * HD, rof[j & 7]);
    __builtin_amdgcn_sched_group_barrier(0x100, PF - 1, 0);
#pragma unroll
    for (int j = 0; j < NSTEP; ++j) {
      if (j + PF - 1 < NSTEP) {
        const int jn = j + PF - 1;
        fx[jn % PF] = frag_at(X + (jn >> 3) * 32 * HD, rof[jn & 7]);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      x[j >> 3] = mfma(fx[j % PF], kv[j & 7], x[j >> 3]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  // acc^T += Y^T x: A = Y^T read transposed from the tile, B = x in bf16.
  // Step j = 8 qt + 4 jp + ht; its A fragment is read PF - 1 steps ahead (a
  // ring), which also bounds how many reads the compiler hoists.
  auto hd_products = [&](const bf16* Y, const f32x16 (&x)[NQT]) {
    constexpr int NSTEP = NQT * 8, PF = NC_DKV_PF;
    bf16x8_t fy[PF];
    auto y_read = [&](int j) {
      const bf16* Yr = Y + ((j >> 3) * 32 + 16 * ((j >> 2) & 1)) * HD;
      fy[j % PF] = frag_tr_at(Yr, tof[2 * (j & 3)], tof[2 * (j & 3) + 1]);
    };
#pragma unroll
    for (int j = 0; j < PF - 1; ++j) y_read(j);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (PF - 1), 0);
    bf16x8_t xb = {};
#pragma unroll
    for (int j = 0; j < NSTEP; ++j) {
      if (j + PF - 1 < NSTEP) {
        y_read(j + PF - 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      if ((j & 3) == 0) xb = pack_p(x[j >> 3], (j >> 2) & 1);
      acc[j & 3] = mfma(fy[j % PF], xb, acc[j & 3]);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  // query tile i in (Q, G) with statistics in slot cur; tile i + 1 is DMA'd
  // into (Qn, Gn)
  auto q_tile = [&](const int i, const int cur, const bf16* Q, const bf16* G, bf16* Qn, bf16* Gn) {
    if (i + 1 < nq) {
      stage(i + 1, Qn, Gn);
      fetch_stats(i + 1);
    }
    f32x16 x[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) x[qt] = zero16();
    // The lane offsets pass through an empty asm once per tile, so that the
    // compiler does not hoist a register per (array, offset) pair out of the
    // tile loop (dozens of live registers); every read is then one of these
    // registers plus an immediate.
    asm volatile("" : "+v"(rof[0]), "+v"(rof[1]), "+v"(rof[2]), "+v"(rof[3]), "+v"(rof[4]), "+v"(rof[5]),
                 "+v"(rof[6]), "+v"(rof[7]));
    asm volatile("" : "+v"(tof[0]), "+v"(tof[1]), "+v"(tof[2]), "+v"(tof[3]), "+v"(tof[4]), "+v"(tof[5]),
                 "+v"(tof[6]), "+v"(tof[7]));
    if (role_p) {
      // the partner's dP products queue behind these on the SIMD, so that
      // the softmax below starts early and runs beside them
      if (NC_DKV_PRIO) __builtin_amdgcn_s_setprio(2);
      key_products(Q, x);
      if (NC_DKV_PRIO) __builtin_amdgcn_s_setprio(0);
      // P = 2^(S scale log2(e) - lse log2(e)); keys after a row's position
      // get 2^-inf = 0.  Keys of this block after the earliest query position
      // of the tile need the mask; other tiles skip it (a uniform branch).
      if (u0 + KB - 1 > div_h(qs0 + i * QT, a.hmagic)) {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int q0 = qt * 32 + 8 * g4 + 4 * h;
            const float4 L = *reinterpret_cast<const float4*>(&lse_s[cur][q0]);
            const int4 tp = *reinterpret_cast<const int4*>(&tpos_s[cur][q0]);
            const float Lv[4] = {L.x, L.y, L.z, L.w};
            const int tv[4] = {tp.x, tp.y, tp.z, tp.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float y = fmaf(x[qt][4 * g4 + e], a.scale_log2, -Lv[e]);
              x[qt][4 * g4 + e] = fexp2(myu > tv[e] ? -INFINITY : y);
            }
            Pex[(w * (4 * NQT) + qt * 4 + g4) * 64 + lane] =
                make_float4(x[qt][4 * g4], x[qt][4 * g4 + 1], x[qt][4 * g4 + 2], x[qt][4 * g4 + 3]);
          }
      } else {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int q0 = qt * 32 + 8 * g4 + 4 * h;
            const float4 L = *reinterpret_cast<const float4*>(&lse_s[cur][q0]);
            const float Lv[4] = {L.x, L.y, L.z, L.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) x[qt][4 * g4 + e] = fexp2(fmaf(x[qt][4 * g4 + e], a.scale_log2, -Lv[e]));
            Pex[(w * (4 * NQT) + qt * 4 + g4) * 64 + lane] =
                make_float4(x[qt][4 * g4], x[qt][4 * g4 + 1], x[qt][4 * g4 + 2], x[qt][4 * g4 + 3]);
          }
      }
    } else {
      key_products(G, x);
    }
    lds_barrier();  // P of this tile is in Pex
    if (role_p) {
      hd_products(G, x);  // dV^T += dO^T P
    } else {
      // dS = P (dP - D); this VALU work goes ahead of the partner's dV
      // products, which fill the matrix core meanwhile
      if (NC_DKV_PRIO) __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 P4 = Pex[(w * (4 * NQT) + qt * 4 + g4) * 64 + lane];
          const float4 D4 = *reinterpret_cast<const float4*>(&D_s[cur][qt * 32 + 8 * g4 + 4 * h]);
          x[qt][4 * g4] = P4.x * (x[qt][4 * g4] - D4.x);
          x[qt][4 * g4 + 1] = P4.y * (x[qt][4 * g4 + 1] - D4.y);
          x[qt][4 * g4 + 2] = P4.z * (x[qt][4 * g4 + 2] - D4.z);
          x[qt][4 * g4 + 3] = P4.w * (x[qt][4 * g4 + 3] - D4.w);
        }
      if (NC_DKV_PRIO) __builtin_amdgcn_s_setprio(0);
      hd_products(Q, x);  // dK^T += Q^T dS
    }
    if (i + 1 < nq) put_stats(cur ^ 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  int i = 0;
  for (; i + 1 < nq; i += 2) {
    q_tile(i, 0, Qs0, Ds0, Qs1, Ds1);
    q_tile(i + 1, 1, Qs1, Ds1, Qs0, Ds0);
  }
  if (i < nq) q_tile(i, 0, Qs0, Ds0, Qs1, Ds1);

  // partial [slot][2][KB keys][HD] (dK, then dV): lane holds hd = ht*32 + 8 q4 + 4 h + e for key (w*32 + lc)
  float* pk = a.part + ((((int64_t)b * a.nkb + kb) * smax + sp) * 2 + (role_p ? 1 : 0)) * (KB * HD) + (w * 32 + lc) * HD;
#pragma unroll
  for (int ht = 0; ht < 4; ++ht)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int hd = ht * 32 + 8 * q4 + 4 * h;
      *reinterpret_cast<float4*>(pk + hd) =
          make_float4(acc[ht][4 * q4], acc[ht][4 * q4 + 1], acc[ht][4 * q4 + 2], acc[ht][4 * q4 + 3]);
    }
}

// dK = scale * sum_s partial_k[s], dV = sum_s partial_v[s], splits in order.
__global__ __launch_bounds__(256) void attn_dkv_reduce_kernel(AttnMfmaArgs a) {
  const int H = a.H, T = a.T, R = T * H;
  const int kb = blockIdx.x, b = blockIdx.y;
  const int ns = nsplit_of(kb, H, R, a.qch);
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
    const int64_t tok = (int64_t)b * T + u;
    if (a.dqkv_lp) {
      // QK-norm and RoPE backward of the key row: the 32 threads of a key row
      // are 32 consecutive lanes (4 dims each), and the partner of dim hd in
      // its RoPE pair (hd + 64 or hd - 64) sits 16 lanes away.
      const float g[4] = {sk.x * a.scale, sk.y * a.scale, sk.z * a.scale, sk.w * a.scale};
      const uint2 yu = *reinterpret_cast<const uint2*>(a.qkv + tok * a.S + H * HD + hd);
      const float y[4] = {__uint_as_float(yu.x << 16), __uint_as_float(yu.x & 0xffff0000u),
                          __uint_as_float(yu.y << 16), __uint_as_float(yu.y & 0xffff0000u)};
      float dot = g[0] * y[0] + g[1] * y[1] + g[2] * y[2] + g[3] * y[3];
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 32);
      const float mean = dot * (1.f / 128.f);
      const float r = a.rstd_k[tok];
      float pv[4], qv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = r * (g[e] - y[e] * mean);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[e] = __shfl_xor(pv[e], 16, 32);  // the pair partner's value
      const bool lo = hd < 64;
      const int i = lo ? hd : hd - 64;
      const float4 cs0 = *reinterpret_cast<const float4*>(a.rope_tab + (int64_t)u * 128 + 2 * i);
      const float4 cs1 = *reinterpret_cast<const float4*>(a.rope_tab + (int64_t)u * 128 + 2 * i + 4);
      const float c[4] = {cs0.x, cs0.z, cs1.x, cs1.z}, sn[4] = {cs0.y, cs0.w, cs1.y, cs1.w};
      float o4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)  // rotate back by -theta: (a, b) -> (a c + b s, -a s + b c)
        o4[e] = lo ? pv[e] * c[e] + qv[e] * sn[e] : -qv[e] * sn[e] + pv[e] * c[e];
      bf16* row = a.dqkv_lp + tok * (int64_t)(H + 2) * HD;
      *reinterpret_cast<uint2*>(row + H * HD + hd) = make_uint2(pack_bf16x2(o4[0], o4[1]), pack_bf16x2(o4[2], o4[3]));
      *reinterpret_cast<uint2*>(row + (H + 1) * HD + hd) = make_uint2(pack_bf16x2(sv.x, sv.y), pack_bf16x2(sv.z, sv.w));
    } else {
      float* row = a.dqkv + tok * (int64_t)(H + 2) * HD;
      *reinterpret_cast<float4*>(row + H * HD + hd) =
          make_float4(sk.x * a.scale, sk.y * a.scale, sk.z * a.scale, sk.w * a.scale);
      *reinterpret_cast<float4*>(row + (H + 1) * HD + hd) = sv;
    }
  }
}

}  // namespace

// Query rows per dK/dV split.  Splitting adds partial sums to write and
// reduce and re-stages K and V, so a key block keeps its whole query range
// when the B x nkb key blocks alone make DKV_BLOCKS; otherwise the range is
// cut into chunks of QCH_MIN rows.
int attn_mfma_qch(int B, int T, int H) {
  const int R = T * H, nkb = (T + KB - 1) / KB;
  if ((int64_t)B * nkb < DKV_BLOCKS) return QCH_MIN;
  return std::max((R + QT - 1) / QT * QT, QCH_MIN);
}

int attn_mfma_smax(int B, int T, int H) {
  const int q = attn_mfma_qch(B, T, H);
  return (T * H + q - 1) / q;
}

size_t attn_mfma_bwd_workspace_bytes(int B, int T, int H) {
  const int nkb = (T + KB - 1) / KB;
  const size_t dbuf = align_up((size_t)B * T * H * sizeof(float), 256);
  const size_t part = (size_t)B * nkb * attn_mfma_smax(B, T, H) * 2 * KB * HD * sizeof(float);
  return dbuf + align_up(part, 256);
}

int attn_mfma_fwd(const void* qkv, int B, int T, int H, float scale, void* o, float* lse, hipStream_t s) {
  NC_REQUIRE((uint64_t)T * H * H < ((uint64_t)1 << 32), NC_ERR_UNSUPPORTED, "attention: T * H^2 must be < 2^32");
  // the K/V staging addresses a sequence's rows with 32-bit byte offsets
  NC_REQUIRE((int64_t)T * (H + 2) * HD * 2 < ((int64_t)1 << 31), NC_ERR_UNSUPPORTED,
             "attention: a sequence of T rows of (H + 2) * 128 bf16 must be < 2 GiB");
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
  a.hmagic = (uint32_t)((((uint64_t)1 << 32) + H - 1) / H);
  const int nrb = (T * H + QB - 1) / QB;
  const double fl = 2.0 * B * H * (double)HD * T * T;
  probe_begin(NC_PROBE_ATTN_FWD, s);
  attn_fwd_kernel<<<dim3(B, nrb), 256, 0, s>>>(a);
  probe_end(NC_PROBE_ATTN_FWD, s, fl);
  return check_launch("attn_fwd_kernel");
}

int attn_mfma_bwd(const void* qkv, const void* o, const void* dout, const float* lse, int B, int T, int H, float scale,
                  float* dqkv, void* ws, hipStream_t s, const AttnRopeBwd* fuse) {
  NC_REQUIRE((uint64_t)T * H * H < ((uint64_t)1 << 32), NC_ERR_UNSUPPORTED, "attention: T * H^2 must be < 2^32");
  // the dK/dV staging addresses a sequence's q/k/v rows with 32-bit byte offsets
  NC_REQUIRE((int64_t)T * (H + 2) * HD * 2 < ((int64_t)1 << 31), NC_ERR_UNSUPPORTED,
             "attention: a sequence of T rows of (H + 2) * 128 bf16 must be < 2 GiB");
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
  a.qch = attn_mfma_qch(B, T, H);
  a.smax = attn_mfma_smax(B, T, H);
  a.hmagic = (uint32_t)((((uint64_t)1 << 32) + H - 1) / H);
  if (fuse) {
    a.dqkv_lp = static_cast<bf16*>(fuse->dqkv);
    a.rstd_q = fuse->rstd_q;
    a.rstd_k = fuse->rstd_k;
    a.rope_tab = fuse->table;
  }
  const double fl = 2.0 * B * H * (double)HD * T * T;
  NC_TRY(attn_mfma_dq(a, s));
  probe_begin(NC_PROBE_ATTN_DKV, s);
  attn_dkv_kernel<<<dim3(B, a.nkb * a.smax), 512, 0, s>>>(a);
  probe_end(NC_PROBE_ATTN_DKV, s, fl);
  NC_TRY(check_launch("attn_dkv_kernel"));
  attn_dkv_reduce_kernel<<<dim3(a.nkb, B), 256, 0, s>>>(a);
  return check_launch("attn_dkv_reduce_kernel");
}

}  // namespace nc
