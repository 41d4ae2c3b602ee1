// Inference with a key/value cache: prefill of a prompt and one-token decode
// steps of the same model as the training step (release-news page
// "Karpathy再放大招…", section 技術細節與問答: multi-query attention, rotary
// embeddings, QK norm, logit softcap; the page's serving engine keeps such a
// cache).  By causality, the logits at a position depend only on the tokens
// up to it.  Keeping each layer's post-RoPE, post-norm key and its value for
// every earlier position therefore lets a new position be computed without
// recomputing the prefix.
//
// Supported: bf16 weights, head_dim 128, one K/V head, at most 32 query heads
// and 128 sequences.
//
// Cache layout (bf16, caller-owned): [L][2][B][max_len][128], keys then values
// per layer, position-major within a sequence, so one position's key is one
// contiguous 256-byte row.
//
// Decode is bound by HBM: every step reads all projection weights once
// (small-M GEMMs, gemm.hip) and each sequence's cached keys and values once
// (the attention below).
#include "common.h"
#include "gemm.h"
#include "ops.h"

#include <cmath>
#include <mutex>

namespace nc {
namespace {

constexpr int kHd = 128;    // head_dim of the inference path
constexpr int kChunk = 64;  // cached positions per decode-attention wave
constexpr int kMaxHeads = 32;  // query heads: the 32 columns of the attention MFMAs
constexpr int kMaxSeqs = 128;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float sum16(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v += __shfl_xor(v, o, 16);
  return v;
}

__device__ __forceinline__ void unpack4(uint2 u, float (&f)[4]) {
  f[0] = __uint_as_float(u.x << 16);
  f[1] = __uint_as_float(u.x & 0xffff0000u);
  f[2] = __uint_as_float(u.y << 16);
  f[3] = __uint_as_float(u.y & 0xffff0000u);
}

__device__ __forceinline__ int seq_len_of(const int32_t* lens, int b, int len_add, int max_len) {
  const int n = lens[b] + len_add;
  return n < 0 ? 0 : (n > max_len ? max_len : n);
}

// Decode attention, split over the cache: block (chunk, b) is one wave over
// positions 64 chunk .. 64 chunk + 63 of sequence b, for all H query heads
// at once (they share the one K/V head, so each cached row is read once).
// Both products run on the matrix cores (v_mfma_f32_32x32x16_bf16), with
// the heads as the 32 columns (heads >= H have a zero query):
//  * the chunk's key and value rows are loaded 4 rows (1 KB) per instruction
//    and written to LDS in [64][128] tiles whose 16-byte pieces are
//    XOR-swizzled by row; rows at or past the sequence's length are written
//    as zeros (so stale cache contents never reach a product);
//  * S^T = K Q^T: A = key rows (8 consecutive dims per lane from LDS),
//    B = the query (registers, loaded once); lane l ends with head l mod 32
//    and 32 of the 64 positions;
//  * softmax per head in base 2 (scores pre-multiplied by scale log2 e): the
//    lane's 32 values, then one shuffle with the other half-wave;
//  * O^T = V^T P: A = V^T read transposed from the row-major value tile
//    (ds_read_b64_tr_b16), B = the probabilities, rounded to bf16, taken
//    straight from the score registers (the k-slot order of both operands is
//    the same permutation of the 64 positions).
// Writes the unnormalised partial output and (max, sum) per head; chunks at or
// beyond the sequence's length do nothing.
typedef __bf16 bf16x4_t __attribute__((__vector_size__(4 * sizeof(__bf16))));

__device__ __forceinline__ int tswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// element offset of (row, 8-dim piece c) in a swizzled [rows][128] tile
__device__ __forceinline__ int toff(int row, int c) { return row * kHd + ((c ^ tswz(row)) << 3); }

// A operand of X^T from the row-major tile X: output rows are the columns
// col0 .. col0 + 31 of X; the k-slots of lane l are rows
// rbase + 8 (e / 4) + 4 (l / 32) + e mod 4, e = 0..7.
__device__ __forceinline__ bf16x8_t frag_tr(const bf16* S, int rbase, int col0, int lane) {
  const int g = lane >> 4, p = lane & 15, h = lane >> 5;
  const int col = col0 + 16 * (g & 1) + 4 * (p & 3);
  const int r1 = rbase + 4 * h + (p >> 2);
  const bf16* a1 = S + toff(r1, col >> 3) + (col & 7);
  const bf16* a2 = S + toff(r1 + 8, col >> 3) + (col & 7);
  const bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)a1);
  const bf16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)a2);
  const uint2 u = __builtin_bit_cast(uint2, x), v = __builtin_bit_cast(uint2, y);
  return __builtin_bit_cast(bf16x8_t, make_uint4(u.x, u.y, v.x, v.y));
}

__device__ __forceinline__ f32x16 mfma32(bf16x8_t a, bf16x8_t b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// With ROPE the kernel also does the new token's RoPE + QK norm and cache
// append (one launch less per layer): `lens` are then the positions (len_add
// = 1), the projection arrives as fp32 partial sums [parts][B][(H+2) 128],
// every block rotates and normalises the query heads itself (each lane holds
// both members of its RoPE pairs: dims 16 ks + 8 h + e and that + 64), and the
// block whose chunk holds the position computes the key and value, writes them
// to the cache and into its LDS tiles.
struct RopeIn {
  const float* qkv;
  int parts, B;
  double base;
  float eps;
  int32_t* flag;
};

template <bool ROPE>
__global__ __launch_bounds__(64) void decode_attn_split_kernel(const bf16* __restrict__ q, bf16* __restrict__ kc,
                                                               bf16* __restrict__ vc,
                                                               const int32_t* __restrict__ lens, int len_add, int H,
                                                               int max_len, float scale_log2,
                                                               float* __restrict__ part_o,
                                                               float* __restrict__ part_ml, RopeIn ri) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[kChunk * kHd];
  __shared__ __attribute__((aligned(16))) bf16 Vs[kChunk * kHd];
  __shared__ float2 cs_sn[kHd / 2];
  const int chunk = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const int nch = gridDim.x;
  int pnew = 0;
  if constexpr (ROPE) {
    pnew = lens[b];
    if (pnew < 0 || pnew >= max_len) {  // outputs of this sequence stay undefined
      if (chunk == 0 && lane == 0 && ri.flag) *ri.flag = 1;
      return;
    }
  }
  const int len = seq_len_of(lens, b, len_add, max_len);
  const int t0 = chunk * kChunk;
  if (t0 >= len) return;
  const int nvalid = min(kChunk, len - t0);
  const int64_t seq = (int64_t)b * max_len * kHd;
  // stage the chunk: every load of the wave is 4 whole rows
  const int rsub = lane >> 4, cp = lane & 15;
  uint4 kl[kChunk / 4], vl[kChunk / 4];
#pragma unroll
  for (int g = 0; g < kChunk / 4; ++g) {
    const int row = 4 * g + rsub;
    const int64_t off = seq + (int64_t)(t0 + row) * kHd + 8 * cp;
    const bool ok = row < nvalid;
    kl[g] = ok ? *reinterpret_cast<const uint4*>(kc + off) : make_uint4(0, 0, 0, 0);
    vl[g] = ok ? *reinterpret_cast<const uint4*>(vc + off) : make_uint4(0, 0, 0, 0);
  }
  // the query of head lane mod 32, dims 16 ks + 8 h .. + 7 (zero past H)
  const int hcol = lane & 31, h = lane >> 5;
  bf16x8_t qreg[kHd / 16];
  if constexpr (!ROPE) {
#pragma unroll
    for (int ks = 0; ks < kHd / 16; ++ks)
      qreg[ks] = hcol < H ? *reinterpret_cast<const bf16x8_t*>(q + ((int64_t)b * H + hcol) * kHd + 16 * ks + 8 * h)
                          : bf16x8_t{};
  }
  float cs = 0.f, sn = 0.f;
  if constexpr (ROPE) {  // angle of pair `lane` at this position (fp64, rounded to fp32)
    const double th = (double)pnew * pow(ri.base, -2.0 * (double)lane / (double)kHd);
    cs = (float)cos(th);
    sn = (float)sin(th);
    cs_sn[lane] = make_float2(cs, sn);
  }
#pragma unroll
  for (int g = 0; g < kChunk / 4; ++g) {
    const int row = 4 * g + rsub;
    *reinterpret_cast<uint4*>(Ks + toff(row, cp)) = kl[g];
    *reinterpret_cast<uint4*>(Vs + toff(row, cp)) = vl[g];
  }
  if constexpr (ROPE) {
    const int64_t stride = (int64_t)ri.B * (H + 2) * kHd;
    const float* qkvrow = ri.qkv + (int64_t)b * (H + 2) * kHd;
    if (pnew >= t0 && pnew < t0 + kChunk) {
      // the new position's key (rotated, normalised) and value: lane owns dims lane, lane + 64
      const float* kr = qkvrow + H * kHd;
      float ka = 0.f, kb = 0.f, va = 0.f, vb = 0.f;
      for (int k = 0; k < ri.parts; ++k) {
        ka += kr[k * stride + lane];
        kb += kr[k * stride + lane + 64];
        va += kr[k * stride + kHd + lane];
        vb += kr[k * stride + kHd + lane + 64];
      }
      const float ya = ka * cs - kb * sn, yb = ka * sn + kb * cs;
      const float r = 1.f / sqrtf(wave_sum(ya * ya + yb * yb) / (float)kHd + ri.eps);
      const bf16 k0 = f2bf(ya * r), k1 = f2bf(yb * r), v0 = f2bf(va), v1 = f2bf(vb);
      const int row = pnew - t0;
      Ks[toff(row, lane >> 3) + (lane & 7)] = k0;
      Ks[toff(row, (lane + 64) >> 3) + (lane & 7)] = k1;
      Vs[toff(row, lane >> 3) + (lane & 7)] = v0;
      Vs[toff(row, (lane + 64) >> 3) + (lane & 7)] = v1;
      const int64_t crow = seq + (int64_t)pnew * kHd;
      kc[crow + lane] = k0;
      kc[crow + lane + 64] = k1;
      vc[crow + lane] = v0;
      vc[crow + lane + 64] = v1;
    }
    __syncthreads();  // the angle table
    if (hcol < H) {
      const float* qr = qkvrow + hcol * kHd + 8 * h;
      float qv[kHd / 16][8];
#pragma unroll
      for (int ks = 0; ks < kHd / 16; ++ks) {
        const float4 a0 = *reinterpret_cast<const float4*>(qr + 16 * ks);
        const float4 a1 = *reinterpret_cast<const float4*>(qr + 16 * ks + 4);
        qv[ks][0] = a0.x; qv[ks][1] = a0.y; qv[ks][2] = a0.z; qv[ks][3] = a0.w;
        qv[ks][4] = a1.x; qv[ks][5] = a1.y; qv[ks][6] = a1.z; qv[ks][7] = a1.w;
      }
      for (int k = 1; k < ri.parts; ++k) {
#pragma unroll
        for (int ks = 0; ks < kHd / 16; ++ks) {
          const float4 a0 = *reinterpret_cast<const float4*>(qr + k * stride + 16 * ks);
          const float4 a1 = *reinterpret_cast<const float4*>(qr + k * stride + 16 * ks + 4);
          qv[ks][0] += a0.x; qv[ks][1] += a0.y; qv[ks][2] += a0.z; qv[ks][3] += a0.w;
          qv[ks][4] += a1.x; qv[ks][5] += a1.y; qv[ks][6] += a1.z; qv[ks][7] += a1.w;
        }
      }
      float ss = 0.f;
#pragma unroll
      for (int ks = 0; ks < kHd / 32; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 t = cs_sn[16 * ks + 8 * h + e];
          const float a = qv[ks][e], c = qv[ks + 4][e];
          const float ya = a * t.x - c * t.y, yb = a * t.y + c * t.x;
          qv[ks][e] = ya;
          qv[ks + 4][e] = yb;
          ss += ya * ya + yb * yb;
        }
      ss += __shfl_xor(ss, 32, 64);  // the other half of the head's dims
      const float r = 1.f / sqrtf(ss / (float)kHd + ri.eps);
#pragma unroll
      for (int ks = 0; ks < kHd / 16; ++ks)
        qreg[ks] = __builtin_bit_cast(
            bf16x8_t, make_uint4(pack_bf16x2(qv[ks][0] * r, qv[ks][1] * r), pack_bf16x2(qv[ks][2] * r, qv[ks][3] * r),
                                 pack_bf16x2(qv[ks][4] * r, qv[ks][5] * r), pack_bf16x2(qv[ks][6] * r, qv[ks][7] * r)));
    } else {  // lanes l and l ^ 32 share a head, so the shuffle above stays within active lanes
#pragma unroll
      for (int ks = 0; ks < kHd / 16; ++ks) qreg[ks] = bf16x8_t{};
    }
  }
  __syncthreads();
  f32x16 s[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
#pragma unroll
    for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kHd / 16; ++ks)
      s[st] = mfma32(*reinterpret_cast<const bf16x8_t*>(Ks + toff(st * 32 + hcol, 2 * ks + h)), qreg[ks], s[st]);
  }
  float m = -INFINITY;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int pos = st * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      const float x = pos < nvalid ? s[st][r] * scale_log2 : -INFINITY;
      s[st][r] = x;
      m = fmaxf(m, x);
    }
  m = fmaxf(m, __shfl_xor(m, 32, 64));  // finite: position 0 of the chunk is valid
  float l = 0.f;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = __builtin_amdgcn_exp2f(s[st][r] - m);
      s[st][r] = pr;
      l += pr;
    }
  l += __shfl_xor(l, 32, 64);
  f32x16 o[kHd / 32];
#pragma unroll
  for (int ht = 0; ht < kHd / 32; ++ht)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[ht][i] = 0.f;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      const int bb = 8 * jp;
      const bf16x8_t pb = __builtin_bit_cast(
          bf16x8_t, make_uint4(pack_bf16x2(s[st][bb], s[st][bb + 1]), pack_bf16x2(s[st][bb + 2], s[st][bb + 3]),
                               pack_bf16x2(s[st][bb + 4], s[st][bb + 5]), pack_bf16x2(s[st][bb + 6], s[st][bb + 7])));
#pragma unroll
      for (int ht = 0; ht < kHd / 32; ++ht) o[ht] = mfma32(frag_tr(Vs, st * 32 + 16 * jp, ht * 32, lane), pb, o[ht]);
    }
  if (hcol < H) {
    const int64_t pi = ((int64_t)b * nch + chunk) * H + hcol;
    float* dst = part_o + pi * kHd;
#pragma unroll
    for (int ht = 0; ht < kHd / 32; ++ht)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *reinterpret_cast<float4*>(dst + ht * 32 + 8 * rq + 4 * h) =
            make_float4(o[ht][4 * rq], o[ht][4 * rq + 1], o[ht][4 * rq + 2], o[ht][4 * rq + 3]);
    if (h == 0) {
      part_ml[2 * pi] = m;
      part_ml[2 * pi + 1] = l;
    }
  }
}

// Combine the chunks of each (sequence, head): o = sum_c 2^(m_c - M) o_c /
// sum_c 2^(m_c - M) l_c, M = max_c m_c.  One block per (head, sequence),
// one thread per output dimension; the chunk statistics are reduced across
// the block in a fixed tree order, the outputs summed in chunk order
// (deterministic), with the independent chunk loads unrolled so that their
// latencies overlap.  A sequence of length 0 gets zeros.
__global__ __launch_bounds__(kHd) void decode_attn_combine_kernel(const float* __restrict__ part_o,
                                                                  const float* __restrict__ part_ml,
                                                                  const int32_t* __restrict__ lens, int len_add,
                                                                  int H, int max_len, int nch,
                                                                  bf16* __restrict__ out) {
  __shared__ float red[kHd];
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int len = seq_len_of(lens, b, len_add, max_len);
  const int used = (int)cdiv(len, kChunk);
  bf16* dst = out + ((int64_t)b * H + h) * kHd + tid;
  if (used == 0) {
    *dst = 0;
    return;
  }
  const int64_t base = (int64_t)b * nch * H + h;
  float mx = -INFINITY;
  for (int c = tid; c < used; c += kHd) mx = fmaxf(mx, part_ml[2 * (base + (int64_t)c * H)]);
  red[tid] = mx;
  __syncthreads();
#pragma unroll
  for (int w = kHd / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float ls = 0.f;
  for (int c = tid; c < used; c += kHd) {
    const int64_t i = base + (int64_t)c * H;
    ls += __builtin_amdgcn_exp2f(part_ml[2 * i] - M) * part_ml[2 * i + 1];
  }
  red[tid] = ls;
  __syncthreads();
#pragma unroll
  for (int w = kHd / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  const float L = red[0];
  float O = 0.f;
#pragma unroll 8
  for (int c = 0; c < used; ++c) {
    const int64_t i = base + (int64_t)c * H;
    O += __builtin_amdgcn_exp2f(part_ml[2 * i] - M) * part_o[i * kHd + tid];
  }
  *dst = f2bf(O / L);
}

// Prefill: copy each token's post-norm key and its value (columns H 128 and
// (H + 1) 128 of the packed qkv rows) into the cache; 16 bytes per thread.
__global__ __launch_bounds__(256) void cache_fill_kernel(const bf16* __restrict__ qkv, int64_t M, int T, int H,
                                                         bf16* __restrict__ kc, bf16* __restrict__ vc, int max_len) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t tok = i >> 5;
  if (tok >= M) return;
  const int c = (int)(i & 31);
  const int64_t b = tok / T, t = tok - b * T;
  const uint4 v = *reinterpret_cast<const uint4*>(qkv + tok * (H + 2) * kHd + (int64_t)(H + (c >> 4)) * kHd +
                                                  8 * (c & 15));
  bf16* dst = (c < 16 ? kc : vc) + (b * max_len + t) * kHd + 8 * (c & 15);
  *reinterpret_cast<uint4*>(dst) = v;
}

// Decode residual update and norm, one block per token row (d / 4 threads,
// one float4 each, d <= 2048): x += sum over k of part[k] (k in order: the
// k-split partial products of the projection that feeds the residual), then
// y = x / sqrt(mean(x^2) + eps) in bf16.  All loads of a thread are issued
// before the first add.
constexpr int kMaxParts = 8;

__global__ __launch_bounds__(512) void residual_rmsnorm_kernel(float* __restrict__ x, const float* __restrict__ part,
                                                               int parts, int rows, int d, float eps,
                                                               bf16* __restrict__ y) {
  __shared__ float red[8];
  const int row = blockIdx.x, t = threadIdx.x, c = 4 * t;
  const int64_t off = (int64_t)row * d + c, stride = (int64_t)rows * d;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < d) {
    float4 pv[kMaxParts];
#pragma unroll
    for (int q = 0; q < kMaxParts; ++q)
      if (q < parts) pv[q] = *reinterpret_cast<const float4*>(part + q * stride + off);
    a = *reinterpret_cast<const float4*>(x + off);
#pragma unroll
    for (int q = 0; q < kMaxParts; ++q)
      if (q < parts) {
        a.x += pv[q].x;
        a.y += pv[q].y;
        a.z += pv[q].z;
        a.w += pv[q].w;
      }
    *reinterpret_cast<float4*>(x + off) = a;
  }
  float ss = wave_sum(a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w);
  if ((t & 63) == 0) red[t >> 6] = ss;
  __syncthreads();
  ss = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) ss += red[w];
  const float r = 1.f / sqrtf(ss / (float)d + eps);
  if (c < d)
    *reinterpret_cast<uint2*>(y + off) = make_uint2(pack_bf16x2(a.x * r, a.y * r), pack_bf16x2(a.z * r, a.w * r));
}

// rows_out[b] = x[b T + T - 1] (fp32 rows of width d): the last position of
// every prompt.
__global__ __launch_bounds__(256) void last_rows_kernel(const float* __restrict__ x, int B, int T, int d,
                                                        float* __restrict__ rows_out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)B * d) return;
  const int64_t b = i / d, c = i - b * d;
  rows_out[i] = x[(b * T + T - 1) * d + c];
}

int validate_infer(const nc_config* c, int max_len) {
  NC_REQUIRE(c, NC_ERR_INVALID_ARG, "infer: null config");
  NC_REQUIRE(c->dtype == NC_BF16 && c->head_dim == kHd, NC_ERR_UNSUPPORTED,
             "infer: the cache path needs bf16 and head_dim 128");
  NC_REQUIRE(c->n_kv_head == 1, NC_ERR_INVALID_ARG, "infer: n_kv_head must be 1");
  NC_REQUIRE(c->n_layer > 0 && c->n_head > 0 && c->batch > 0 && c->seq_len > 0 && c->vocab > 0, NC_ERR_INVALID_ARG,
             "infer: bad shape");
  NC_REQUIRE((int64_t)c->n_head * kHd == c->d_model, NC_ERR_INVALID_ARG, "infer: n_head * head_dim != d_model");
  NC_REQUIRE(c->n_head <= kMaxHeads, NC_ERR_UNSUPPORTED, "infer: at most %d query heads", kMaxHeads);
  NC_REQUIRE(c->batch <= kMaxSeqs, NC_ERR_UNSUPPORTED, "infer: at most %d sequences", kMaxSeqs);
  NC_REQUIRE(c->d_model <= 2048, NC_ERR_UNSUPPORTED, "infer: d_model must be at most 2048");
  NC_REQUIRE(c->d_model % 64 == 0 && c->d_ff % 64 == 0 && c->vocab % 32 == 0, NC_ERR_UNSUPPORTED,
             "infer: d_model and d_ff must be multiples of 64, vocab of 32");
  NC_REQUIRE(max_len >= c->seq_len, NC_ERR_INVALID_ARG, "infer: max_len %d is below the prompt length %d", max_len,
             c->seq_len);
  return NC_OK;
}

struct InferWs {
  int32_t* flag;
  // decode (one token per sequence)
  float *dx, *drstd;
  void *da, *dout, *dm, *da2, *dh;
  float *part_o, *part_ml;
  float *part_qkv, *part_x;  // k-split partial products of QKV, and of the O / MLP projections
  int ks_qkv, ks_o, ks_p;
  // prefill (B T tokens)
  float *x, *rstd, *rstd_q, *rstd_k, *lse, *table, *xl;
  void *a, *qkv, *o, *a2, *hl;
  void* gemm_ws;
  size_t gemm_ws_bytes;
};

// K-split of a decode projection (N outputs, K inputs) over blocks: about
// 320 blocks of 16 columns, at least 8 k-chunks of 64 per block.
int decode_split(int64_t N, int64_t K) {
  const int64_t slabs = N / 16, nch = K / 64;
  return (int)std::max<int64_t>(1, std::min<int64_t>({cdiv(320, slabs), nch / 8, (int64_t)kMaxParts}));
}

size_t decode_part_floats(int B, int H, int max_len) { return (size_t)B * cdiv(max_len, kChunk) * H; }

size_t carve_infer(const nc_config* c, int max_len, InferWs* w, void* base) {
  const int64_t B = c->batch, T = c->seq_len, M = B * T;
  const int64_t d = c->d_model, H = c->n_head, F = c->d_ff, Q = (H + 2) * kHd, HD = H * kHd;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes, 256);
    return o;
  };
  char* p = static_cast<char*>(base);
  auto at = [&](size_t o) -> void* { return p ? p + o : nullptr; };
  const size_t o_flag = take(4);
  const int ks_qkv = decode_split(Q, d), ks_o = decode_split(d, HD), ks_p = decode_split(d, F);
  const size_t o_dx = take(B * d * 4), o_dr = take(B * 4), o_da = take(B * d * 2),
               o_do = take(B * HD * 2), o_dm = take(B * d * 2), o_da2 = take(B * F * 2),
               o_dh = take(B * d * 2), o_pq = take((size_t)ks_qkv * B * Q * 4),
               o_px = take((size_t)std::max(ks_o, ks_p) * B * d * 4);
  const size_t parts = decode_part_floats((int)B, (int)H, max_len);
  const size_t o_po = take(parts * kHd * 4), o_pml = take(parts * 2 * 4);
  const size_t o_x = take(M * d * 4), o_r = take(M * 4), o_rq = take(M * H * 4), o_rk = take(M * 4),
               o_lse = take(M * H * 4), o_tab = take((size_t)T * kHd * 4), o_xl = take(B * d * 4),
               o_a = take(M * d * 2), o_qkv = take(M * Q * 2), o_o = take(M * HD * 2), o_a2 = take(M * F * 2),
               o_hl = take(B * d * 2);
  const size_t gb = std::max(gemm_workspace_bytes(M, d, HD), gemm_workspace_bytes(M, d, F));
  const size_t o_g = take(gb);
  if (w) {
    w->flag = static_cast<int32_t*>(at(o_flag));
    w->dx = static_cast<float*>(at(o_dx));
    w->drstd = static_cast<float*>(at(o_dr));
    w->da = at(o_da);
    w->part_qkv = static_cast<float*>(at(o_pq));
    w->part_x = static_cast<float*>(at(o_px));
    w->ks_qkv = ks_qkv;
    w->ks_o = ks_o;
    w->ks_p = ks_p;
    w->dout = at(o_do);
    w->dm = at(o_dm);
    w->da2 = at(o_da2);
    w->dh = at(o_dh);
    w->part_o = static_cast<float*>(at(o_po));
    w->part_ml = static_cast<float*>(at(o_pml));
    w->x = static_cast<float*>(at(o_x));
    w->rstd = static_cast<float*>(at(o_r));
    w->rstd_q = static_cast<float*>(at(o_rq));
    w->rstd_k = static_cast<float*>(at(o_rk));
    w->lse = static_cast<float*>(at(o_lse));
    w->table = static_cast<float*>(at(o_tab));
    w->xl = static_cast<float*>(at(o_xl));
    w->a = at(o_a);
    w->qkv = at(o_qkv);
    w->o = at(o_o);
    w->a2 = at(o_a2);
    w->hl = at(o_hl);
    w->gemm_ws = gb ? at(o_g) : nullptr;
    w->gemm_ws_bytes = gb;
  }
  return off;
}

GemmDesc nt(int64_t M, int64_t N, int64_t K, const void* A, const void* W, void* C, int cdt) {
  GemmDesc g;
  g.transA = 0;
  g.transB = 1;
  g.M = M;
  g.N = N;
  g.K = K;
  g.A = A;
  g.lda = K;
  g.B = W;
  g.ldb = K;
  g.C = C;
  g.cdt = cdt;
  g.ldc = N;
  g.dtype = NC_BF16;
  return g;
}

struct CacheView {
  bf16* base;
  int64_t per;  // elements of one [B][max_len][128] block
  bf16* k(int l) const { return base + (int64_t)(2 * l) * per; }
  bf16* v(int l) const { return base + (int64_t)(2 * l + 1) * per; }
};

int check_params(const nc_params* p) {
  NC_REQUIRE(p && p->embed && p->w_qkv && p->w_o && p->w_fc && p->w_proj && p->unembed, NC_ERR_INVALID_ARG,
             "infer: null parameter");
  return NC_OK;
}

}  // namespace

size_t mqa_decode_workspace_bytes(int B, int H, int max_len) {
  if (B <= 0 || H <= 0 || max_len <= 0) return 0;
  const size_t parts = decode_part_floats(B, H, max_len);
  return align_up(parts * kHd * 4, 256) + parts * 2 * 4;
}

// rope == nullptr: q holds the queries, `lens` + len_add the lengths.
// rope != nullptr: the queries, keys and values come as projection partial
// sums (RopeIn) and are rotated and normalised here; `lens` are the new
// positions, each of whose key and value is written to the cache.
int mqa_decode_attn(const void* q, const void* kc, const void* vc, const int32_t* lens, int len_add, int B, int H,
                    int hd, int max_len, float scale, void* o, float* part_o, float* part_ml, hipStream_t s,
                    const RopeIn* rope = nullptr) {
  NC_REQUIRE((q || rope) && kc && vc && lens && o && part_o && part_ml, NC_ERR_INVALID_ARG,
             "decode_attn: null pointer");
  NC_REQUIRE(B > 0 && H > 0 && max_len > 0, NC_ERR_INVALID_ARG, "decode_attn: bad shape");
  NC_REQUIRE(hd == kHd, NC_ERR_UNSUPPORTED, "decode_attn: head_dim must be 128");
  NC_REQUIRE(H <= kMaxHeads, NC_ERR_UNSUPPORTED, "decode_attn: at most %d query heads", kMaxHeads);
  NC_REQUIRE((int64_t)B * max_len <= (int64_t)1 << 31, NC_ERR_UNSUPPORTED, "decode_attn: cache too large");
  const int nch = (int)cdiv(max_len, kChunk);
  NC_REQUIRE(nch < 65536 && B < 65536, NC_ERR_UNSUPPORTED, "decode_attn: grid too large");
  const double bytes = (double)B * max_len * kHd * 2 * 2 + 2.0 * 2 * B * H * kHd;  // cache capacity, q and o
  probe_begin(NC_PROBE_DECODE_ATTN, s);
  if (rope)  // lens are the new positions; the cache receives their keys and values
    decode_attn_split_kernel<true><<<dim3(nch, B), 64, 0, s>>>(
        nullptr, static_cast<bf16*>(const_cast<void*>(kc)), static_cast<bf16*>(const_cast<void*>(vc)), lens, 1, H,
        max_len, scale * kLog2e, part_o, part_ml, *rope);
  else
    decode_attn_split_kernel<false><<<dim3(nch, B), 64, 0, s>>>(
        static_cast<const bf16*>(q), static_cast<bf16*>(const_cast<void*>(kc)),
        static_cast<bf16*>(const_cast<void*>(vc)), lens, len_add, H, max_len, scale * kLog2e, part_o, part_ml,
        RopeIn{});
  decode_attn_combine_kernel<<<dim3(H, B), kHd, 0, s>>>(part_o, part_ml, lens, rope ? 1 : len_add, H, max_len, nch,
                                                        static_cast<bf16*>(o));
  probe_end(NC_PROBE_DECODE_ATTN, s, bytes);
  return check_launch("decode_attn kernels");
}

size_t kv_cache_bytes(const nc_config* c, int max_len) {
  if (validate_infer(c, max_len) != NC_OK) return 0;
  return (size_t)c->n_layer * 2 * c->batch * max_len * kHd * 2;
}

size_t infer_workspace_bytes(const nc_config* c, int max_len) {
  if (validate_infer(c, max_len) != NC_OK) return 0;
  return carve_infer(c, max_len, nullptr, nullptr);
}

int prefill(const nc_config* c, const nc_params* p, const int32_t* ids, void* kv, int max_len, float* logits,
            void* ws, size_t ws_bytes, hipStream_t s) {
  NC_TRY(validate_infer(c, max_len));
  NC_TRY(check_params(p));
  NC_REQUIRE(ids && kv && logits && ws, NC_ERR_INVALID_ARG, "prefill: null pointer");
  NC_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255u) == 0 && (reinterpret_cast<uintptr_t>(kv) & 15u) == 0,
             NC_ERR_INVALID_ARG, "prefill: ws must be 256-byte and the cache 16-byte aligned");
  const size_t need = carve_infer(c, max_len, nullptr, nullptr);
  NC_REQUIRE(ws_bytes >= need, NC_ERR_WORKSPACE, "prefill: workspace too small (%zu < %zu)", ws_bytes, need);
  InferWs w;
  carve_infer(c, max_len, &w, ws);
  const int B = c->batch, T = c->seq_len, H = c->n_head, L = c->n_layer, V = c->vocab;
  const int64_t M = (int64_t)B * T, d = c->d_model, F = c->d_ff, Q = (int64_t)(H + 2) * kHd, HD = (int64_t)H * kHd;
  const float scale = 1.f / sqrtf((float)kHd);
  const CacheView cv{static_cast<bf16*>(kv), (int64_t)B * max_len * kHd};
  auto W = [&](const void* base, int l, int64_t per) { return static_cast<const bf16*>(base) + (int64_t)l * per; };

  NC_TRY(fill_zero(w.flag, 4, s));
  NC_TRY(embed_fwd(ids, M, p->embed, NC_BF16, V, (int)d, nullptr, w.x, w.rstd, c->eps, w.flag, s));
  NC_TRY(rope_table(w.table, T, kHd, c->rope_base, s));
  for (int l = 0; l < L; ++l) {
    NC_TRY(rmsnorm_fwd(w.x, NC_F32, M, (int)d, c->eps, w.a, NC_BF16, w.rstd, s));
    NC_TRY(gemm(nt(M, Q, d, w.a, W(p->w_qkv, l, Q * d), w.qkv, NC_BF16), s));
    NC_TRY(rope_qknorm_fwd(w.qkv, NC_BF16, B, T, H, kHd, w.table, c->eps, w.rstd_q, w.rstd_k, s));
    NC_TRY(mqa_attn_fwd(w.qkv, NC_BF16, B, T, H, kHd, scale, w.o, w.lse, s));
    cache_fill_kernel<<<(unsigned)cdiv(M * 32, 256), 256, 0, s>>>(static_cast<const bf16*>(w.qkv), M, T, H,
                                                                 cv.k(l), cv.v(l), max_len);
    NC_TRY(check_launch("cache_fill_kernel"));
    GemmDesc go = nt(M, d, HD, w.o, W(p->w_o, l, d * HD), w.x, NC_F32);
    go.beta = 1.f;
    go.ws = w.gemm_ws;
    go.ws_bytes = w.gemm_ws_bytes;
    NC_TRY(gemm(go, s));
    NC_TRY(rmsnorm_fwd(w.x, NC_F32, M, (int)d, c->eps, w.a, NC_BF16, w.rstd, s));
    GemmDesc gf = nt(M, F, d, w.a, W(p->w_fc, l, F * d), w.a2, NC_BF16);
    gf.epi = NC_EPI_RELU2_SQ;
    NC_TRY(gemm(gf, s));
    GemmDesc gp = nt(M, d, F, w.a2, W(p->w_proj, l, d * F), w.x, NC_F32);
    gp.beta = 1.f;
    gp.ws = w.gemm_ws;
    gp.ws_bytes = w.gemm_ws_bytes;
    NC_TRY(gemm(gp, s));
  }
  last_rows_kernel<<<(unsigned)cdiv((int64_t)B * d, 256), 256, 0, s>>>(w.x, B, T, (int)d, w.xl);
  NC_TRY(check_launch("last_rows_kernel"));
  NC_TRY(rmsnorm_fwd(w.xl, NC_F32, B, (int)d, c->eps, w.hl, NC_BF16, w.drstd, s));
  GemmDesc gu = nt(B, V, d, w.hl, p->unembed, logits, NC_F32);
  gu.capc = c->softcap;
  return gemm(gu, s);
}

int decode_step(const nc_config* c, const nc_params* p, const int32_t* ids, const int32_t* pos, void* kv,
                int max_len, float* logits, void* ws, size_t ws_bytes, hipStream_t s) {
  NC_TRY(validate_infer(c, max_len));
  NC_TRY(check_params(p));
  NC_REQUIRE(ids && pos && kv && logits && ws, NC_ERR_INVALID_ARG, "decode: null pointer");
  NC_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255u) == 0 && (reinterpret_cast<uintptr_t>(kv) & 15u) == 0,
             NC_ERR_INVALID_ARG, "decode: ws must be 256-byte and the cache 16-byte aligned");
  const size_t need = carve_infer(c, max_len, nullptr, nullptr);
  NC_REQUIRE(ws_bytes >= need, NC_ERR_WORKSPACE, "decode: workspace too small (%zu < %zu)", ws_bytes, need);
  InferWs w;
  carve_infer(c, max_len, &w, ws);
  const int B = c->batch, H = c->n_head, L = c->n_layer, V = c->vocab;
  const int64_t d = c->d_model, F = c->d_ff, Q = (int64_t)(H + 2) * kHd, HD = (int64_t)H * kHd;
  const float scale = 1.f / sqrtf((float)kHd);
  const CacheView cv{static_cast<bf16*>(kv), (int64_t)B * max_len * kHd};
  auto W = [&](const void* base, int l, int64_t per) { return static_cast<const bf16*>(base) + (int64_t)l * per; };

  NC_TRY(fill_zero(w.flag, 4, s));
  NC_TRY(embed_fwd(ids, B, p->embed, NC_BF16, V, (int)d, nullptr, w.dx, w.drstd, c->eps, w.flag, s));
  // Residual norm: x += the partial products of the projection that feeds it,
  // then the norm (the first layer's input is the embedding output itself).
  auto residual_norm = [&](int parts, void* out) -> int {
    residual_rmsnorm_kernel<<<B, (unsigned)align_up((size_t)d / 4, 64), 0, s>>>(w.dx, w.part_x, parts, B, (int)d,
                                                                               c->eps, static_cast<bf16*>(out));
    return check_launch("residual_rmsnorm_kernel");
  };
  for (int l = 0; l < L; ++l) {
    if (l == 0) NC_TRY(rmsnorm_fwd(w.dx, NC_F32, B, (int)d, c->eps, w.da, NC_BF16, w.drstd, s));
    else NC_TRY(residual_norm(w.ks_p, w.da));
    GemmDesc gq = nt(B, Q, d, w.da, W(p->w_qkv, l, Q * d), w.part_qkv, NC_F32);
    gq.sk_split = w.ks_qkv;
    NC_TRY(gemm(gq, s));
    const RopeIn ri{w.part_qkv, w.ks_qkv, B, (double)c->rope_base, c->eps, w.flag};
    NC_TRY(mqa_decode_attn(nullptr, cv.k(l), cv.v(l), pos, 1, B, H, kHd, max_len, scale, w.dout, w.part_o,
                           w.part_ml, s, &ri));
    GemmDesc go = nt(B, d, HD, w.dout, W(p->w_o, l, d * HD), w.part_x, NC_F32);
    go.sk_split = w.ks_o;
    NC_TRY(gemm(go, s));
    NC_TRY(residual_norm(w.ks_o, w.dm));
    GemmDesc gf = nt(B, F, d, w.dm, W(p->w_fc, l, F * d), w.da2, NC_BF16);
    gf.epi = NC_EPI_RELU2_SQ;
    NC_TRY(gemm(gf, s));
    GemmDesc gp = nt(B, d, F, w.da2, W(p->w_proj, l, d * F), w.part_x, NC_F32);
    gp.sk_split = w.ks_p;
    NC_TRY(gemm(gp, s));
  }
  NC_TRY(residual_norm(w.ks_p, w.dh));
  GemmDesc gu = nt(B, V, d, w.dh, p->unembed, logits, NC_F32);
  gu.capc = c->softcap;
  return gemm(gu, s);
}

}  // namespace nc

extern "C" size_t nc_kv_cache_bytes(const nc_config* cfg, int max_len) { return nc::kv_cache_bytes(cfg, max_len); }

extern "C" size_t nc_infer_workspace_bytes(const nc_config* cfg, int max_len) {
  return nc::infer_workspace_bytes(cfg, max_len);
}

extern "C" int nc_prefill(const nc_config* cfg, const nc_params* params, const int32_t* ids, void* kv_cache,
                          int max_len, float* logits, void* ws, size_t ws_bytes, void* stream) {
  return nc::api_done(nc::prefill(cfg, params, ids, kv_cache, max_len, logits, ws, ws_bytes, static_cast<hipStream_t>(stream)),
                      stream, "nc_prefill");
}

extern "C" int nc_decode_step(const nc_config* cfg, const nc_params* params, const int32_t* ids,
                              const int32_t* pos, void* kv_cache, int max_len, float* logits, void* ws,
                              size_t ws_bytes, void* stream) {
  return nc::api_done(nc::decode_step(cfg, params, ids, pos, kv_cache, max_len, logits, ws, ws_bytes,
                         static_cast<hipStream_t>(stream)), stream, "nc_decode_step");
}

// Scratch of nc_mqa_decode_attn_noalloc: the chunk partials (fp32 outputs,
// then (max, sum) pairs) of one decode-attention call, in the layout of the
// workspace nc_mqa_decode_attn takes.  Every GPU the library runs on holds its
// own copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never device memory: the device address is looked up once per
// device with hipGetSymbolAddress and only that address reaches a kernel.
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {};  // per device: the address of that device's `scratch`

// The current device's scratch address (looked up on its first use there).
int decode_scratch(void** out) {
  int dev = 0;
  NC_CHECK_HIP(hipGetDevice(&dev));
  NC_REQUIRE(dev >= 0 && dev < 64, NC_ERR_UNSUPPORTED, "decode_attn_noalloc: device index %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    NC_CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    NC_REQUIRE(p != nullptr, NC_ERR_HIP, "decode_attn_noalloc: no device address for the scratch array");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return NC_OK;
}
}  // namespace

extern "C" size_t nc_mqa_decode_workspace_bytes(int B, int H, int max_len) {
  return nc::mqa_decode_workspace_bytes(B, H, max_len);
}

extern "C" int nc_mqa_decode_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* lens,
                                  int B, int H, int hd, int max_len, float scale, void* o, void* ws, size_t ws_bytes,
                                  void* stream) {
  const size_t need = nc::mqa_decode_workspace_bytes(B, H, max_len);
  NC_REQUIRE(ws && need > 0, NC_ERR_INVALID_ARG, "decode_attn: null workspace or bad shape");
  NC_REQUIRE(ws_bytes >= need, NC_ERR_WORKSPACE, "decode_attn: workspace too small (%zu < %zu)", ws_bytes, need);
  NC_REQUIRE((reinterpret_cast<uintptr_t>(ws) & 255u) == 0, NC_ERR_INVALID_ARG, "decode_attn: ws must be 256-byte aligned");
  const size_t parts = (size_t)B * nc::cdiv(max_len, 64) * H;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + nc::align_up(parts * 128 * 4, 256));
  return nc::api_done(nc::mqa_decode_attn(q, k_cache, v_cache, lens, 0, B, H, hd, max_len, scale, o, part_o, part_ml,
                             static_cast<hipStream_t>(stream)), stream, "nc_mqa_decode_attn");
}

extern "C" int nc_mqa_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* lens, int B, int H, int hd, int max_len, float scale,
                                          void* o, void* stream) {
  const size_t need = nc::mqa_decode_workspace_bytes(B, H, max_len);
  NC_REQUIRE(need > 0, NC_ERR_INVALID_ARG, "decode_attn_noalloc: bad shape");
  NC_REQUIRE(need <= kDecodeScratchBytes, NC_ERR_WORKSPACE,
             "decode_attn_noalloc: B=%d, H=%d, max_len=%d needs %zu bytes of scratch, more than its %zu", B, H,
             max_len, need, kDecodeScratchBytes);
  void* ws = nullptr;
  NC_TRY(decode_scratch(&ws));
  const size_t parts = (size_t)B * nc::cdiv(max_len, 64) * H;
  float* part_o = static_cast<float*>(ws);
  float* part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + nc::align_up(parts * 128 * 4, 256));
  return nc::api_done(nc::mqa_decode_attn(q, k_cache, v_cache, lens, 0, B, H, hd, max_len, scale, o, part_o, part_ml,
                             static_cast<hipStream_t>(stream)), stream, "nc_mqa_decode_attn_noalloc");
}
