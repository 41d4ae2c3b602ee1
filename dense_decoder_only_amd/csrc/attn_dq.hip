// dQ kernel of the matrix-core attention backward (head_dim 128, bf16); the
// register and LDS layouts are those described at the top of attn_mfma.hip.
// It sits in a file of its own: at 256 VGPRs and two waves per SIMD it is
// at the edge of spilling, and its register allocation then does not move
// with edits to the other attention kernels.
#include "attn_mfma_dev.h"

namespace nc {
namespace {

// ----------------------------------------------------------------------- dQ --
// Also writes D = rowsum(dO * O) for the key-side kernel.
#ifndef NC_ATTN_DQ_WAVES
#define NC_ATTN_DQ_WAVES 2  // waves per SIMD the dQ kernel is compiled for
#endif
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(NC_ATTN_DQ_WAVES, NC_ATTN_DQ_WAVES))) void attn_dq_kernel(AttnMfmaArgs a) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[2 * TILE];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2 * TILE];
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
  // K/V rows are S apart: buffer resources at the sequence's K and V columns
  // and 32-bit byte offsets (rows past the end read row T - 1)
  const __amdgpu_buffer_rsrc_t krs = row_rsrc(base + H * HD), vrs = row_rsrc(base + (H + 1) * HD);
  auto stage = [&](int j, int buf) {
    const int kv0 = j * KT;
#pragma unroll
    for (int k = 0; k < KT / 16; ++k) {
      const int g = w * (KT / 16) + k;
      const int row = g * 4 + (lane >> 4);
      const uint32_t off = (uint32_t)(min(kv0 + row, T - 1) * (int)a.S + (((lane & 15) ^ tswz(row)) << 3)) * 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (__attribute__((address_space(3))) void*)(Ks + buf * TILE + g * 4 * HD),
                                               16, off, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (__attribute__((address_space(3))) void*)(Vs + buf * TILE + g * 4 * HD),
                                               16, off, 0, 0, 0);
    }
  };
  f32x16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = zero16();

  stage(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int j = 0; j < ntiles; ++j) {
    const int cur = j & 1;
    const int kv0 = j * KT;
    if (j + 1 < ntiles) stage(j + 1, cur ^ 1);
    const bf16* K = Ks + cur * TILE;
    const bf16* V = Vs + cur * TILE;

    f32x16 s[2], dp[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = zero16();
      dp[st] = zero16();
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        s[st] = mfma(frag_row(K, st * 32 + lc, 2 * ks + h), qreg[ks], s[st]);
        dp[st] = mfma(frag_row(V, st * 32 + lc, 2 * ks + h), dreg[ks], dp[st]);
      }
    }
    if (kv0 + KT - 1 > tmin) {  // the tile crosses some row's diagonal
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = kv0 + st * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          const float p = kv > tq ? 0.f : fexp2(s[st][r] * a.scale_log2 - lse2);
          s[st][r] = p * (dp[st][r] - D);
        }
    } else {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fexp2(s[st][r] * a.scale_log2 - lse2);
          s[st][r] = p * (dp[st][r] - D);
        }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int jp = 0; jp < 2; ++jp) {
        const bf16x8_t pb = pack_p(s[st], jp);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) dq[ht] = mfma(frag_tr(K, st * 32 + 16 * jp, ht * 32, lane), pb, dq[ht]);
      }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if (a.dqkv_lp) {
    // QK-norm and RoPE backward of the block's 128 query rows, giving the
    // bf16 gradient w.r.t. the projection output:
    //   g' = rstd (g - yhat mean(g yhat)), rotated back by -theta over the
    //   dim pairs (i, i + 64).
    // The fp32 dQ tile goes through LDS (free after the last tile's barrier)
    // so that the row-wise pass holds no MFMA accumulators: waves 0-1 use Ks,
    // 2-3 Vs, 16 KB per wave, 16-byte chunk c of row lc at c ^ lc.
    float* G = reinterpret_cast<float*>(w < 2 ? Ks : Vs) + (w & 1) * 32 * HD;
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = ht * 8 + 2 * q4 + h;
        *reinterpret_cast<float4*>(G + lc * HD + ((c ^ lc) << 2)) =
            make_float4(dq[ht][4 * q4], dq[ht][4 * q4 + 1], dq[ht][4 * q4 + 2], dq[ht][4 * q4 + 3]);
      }
    __syncthreads();
    const int j = tid & 15;  // dims 4 j .. 4 j + 3 and their pair partners + 64
#pragma unroll 1
    for (int row = tid >> 4; row < QB; row += 16) {
      const int qr = r0 + row;
      if (qr >= R) break;
      const int tqr = div_h(qr, a.hmagic), hqr = qr - tqr * H;
      const float* Gr = reinterpret_cast<const float*>((row >> 6) == 0 ? Ks : Vs) + (row & 63) * HD;
      const int sw = row & 31;
      const float4 ga4 = *reinterpret_cast<const float4*>(Gr + ((j ^ sw) << 2));
      const float4 gb4 = *reinterpret_cast<const float4*>(Gr + (((j + 16) ^ sw) << 2));
      const float ga[4] = {ga4.x * a.scale, ga4.y * a.scale, ga4.z * a.scale, ga4.w * a.scale};
      const float gb[4] = {gb4.x * a.scale, gb4.y * a.scale, gb4.z * a.scale, gb4.w * a.scale};
      const int64_t tok = (int64_t)b * T + tqr;
      const bf16* yr = a.qkv + tok * a.S + hqr * HD + 4 * j;
      const uint2 ua = *reinterpret_cast<const uint2*>(yr), ub = *reinterpret_cast<const uint2*>(yr + 64);
      const float ya[4] = {__uint_as_float(ua.x << 16), __uint_as_float(ua.x & 0xffff0000u),
                           __uint_as_float(ua.y << 16), __uint_as_float(ua.y & 0xffff0000u)};
      const float yb[4] = {__uint_as_float(ub.x << 16), __uint_as_float(ub.x & 0xffff0000u),
                           __uint_as_float(ub.y << 16), __uint_as_float(ub.y & 0xffff0000u)};
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) dot += ga[e] * ya[e] + gb[e] * yb[e];
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 16);
      const float mean = dot * (1.f / 128.f);
      const float r = a.rstd_q[(int64_t)b * R + qr];
      const float4* tb = reinterpret_cast<const float4*>(a.rope_tab + ((int64_t)tqr * 64 + 4 * j) * 2);
      const float4 cs0 = tb[0], cs1 = tb[1];  // (cos, sin) of pairs 4 j .. 4 j + 3
      const float cc[4] = {cs0.x, cs0.z, cs1.x, cs1.z}, sn[4] = {cs0.y, cs0.w, cs1.y, cs1.w};
      float oa[4], ob[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pa = r * (ga[e] - ya[e] * mean), pb = r * (gb[e] - yb[e] * mean);
        oa[e] = pa * cc[e] + pb * sn[e];  // rotate back by -theta
        ob[e] = -pa * sn[e] + pb * cc[e];
      }
      bf16* out = a.dqkv_lp + tok * (int64_t)(H + 2) * HD + hqr * HD + 4 * j;
      *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(oa[0], oa[1]), pack_bf16x2(oa[2], oa[3]));
      *reinterpret_cast<uint2*>(out + 64) = make_uint2(pack_bf16x2(ob[0], ob[1]), pack_bf16x2(ob[2], ob[3]));
    }
  } else if (valid) {
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

}  // namespace

int attn_mfma_dq(const AttnMfmaArgs& a, hipStream_t s) {
  const int nrb = (a.T * a.H + QB - 1) / QB;
  const double fl = 2.0 * a.B * a.H * (double)HD * a.T * a.T;
  probe_begin(NC_PROBE_ATTN_DQ, s);
  attn_dq_kernel<<<dim3(a.B, nrb), 256, 0, s>>>(a);
  probe_end(NC_PROBE_ATTN_DQ, s, fl);
  return check_launch("attn_dq_kernel");
}

}  // namespace nc
