// Matrix-core attention kernels (bf16, head_dim 128); see attn_mfma.hip.
#pragma once
#include "common.h"
#include "ops.h"

namespace nc {

struct AttnMfmaArgs {
  const bf16* qkv;     // [B*T, (H+2)*128]: q heads, k, v
  const bf16* o;       // [B*T*H, 128]
  const bf16* dout;    // [B*T*H, 128]
  const float* lse;    // [B*T*H] natural log
  float* lse_out;
  bf16* o_out;
  float* dqkv;         // [B*T, (H+2)*128] fp32
  float* Dbuf;         // [B*T*H]
  float* part;         // dK/dV partials
  int B, T, H;
  int64_t S;           // qkv row stride in elements
  float scale, scale_log2;
  int nkb, smax;
  int qch;             // query rows per dK/dV split (a multiple of 64)
  uint32_t hmagic;     // ceil(2^32 / H): r / H == umulhi(r, hmagic) for r < 2^32 / H^2
  // Backward with the QK-norm and RoPE backward folded in (dqkv_lp != null):
  // the dQ and dK/dV-reduce kernels write the gradient w.r.t. the projection
  // output, bf16 [B*T, (H+2)*128], instead of fp32 dqkv.
  bf16* dqkv_lp;
  const float* rstd_q;    // [B*T, H]
  const float* rstd_k;    // [B*T]
  const float* rope_tab;  // [T, 64, 2] (cos, sin)
};

size_t attn_mfma_bwd_workspace_bytes(int B, int T, int H);
int attn_mfma_fwd(const void* qkv, int B, int T, int H, float scale, void* o, float* lse, hipStream_t s);
int attn_mfma_bwd(const void* qkv, const void* o, const void* dout, const float* lse, int B, int T, int H, float scale,
                  float* dqkv, void* ws, hipStream_t s, const AttnRopeBwd* fuse = nullptr);
// The dQ launch of attn_mfma_bwd (also writes D = rowsum(dO * O) to a.Dbuf).
int attn_mfma_dq(const AttnMfmaArgs& a, hipStream_t s);

}  // namespace nc
