// Device-side pieces shared by the matrix-core attention kernels (attn_mfma.hip
// and attn_dq.hip): tile sizes, the swizzled LDS tile layout, direct
// global -> LDS staging and the MFMA operand reads.  The layouts are described
// at the top of attn_mfma.hip.  Everything here is internal to each file.
#pragma once
#include "common.h"
#include "attn_mfma.h"

namespace nc {
namespace {

constexpr int HD = 128;
constexpr int QB = 128;   // query rows per forward / dQ block (4 waves x 32)
constexpr int KT = 64;    // keys per tile
constexpr int KB = 128;   // keys per dK/dV block (4 waves x 32)
constexpr int QT = 96;    // query rows per dK/dV tile (3 x 32)
// query rows per dK/dV split when the key blocks alone are too few; a multiple
// of QT, so that the splits of a key block cover its rows in whole tiles
constexpr int QCH_MIN = 5184;
static_assert(QCH_MIN % QT == 0, "dK/dV splits must be whole query tiles");
constexpr int DKV_BLOCKS = 512; // dK/dV blocks aimed at: two rounds of one block per CU
#ifndef NC_FWD_PF
#define NC_FWD_PF 3       // forward: K fragments in the score read ring
#endif
#ifndef NC_DKV_PF
#define NC_DKV_PF 4       // dK/dV: fragment pairs in the S / dP read ring
#endif
constexpr int TILE = 64 * HD;  // elements of one [64][128] tile
constexpr int QTILE = QT * HD; // elements of one dK/dV query tile
constexpr float LOG2E = 1.4426950408889634f;

typedef __bf16 bf16x4_t __attribute__((__vector_size__(4 * sizeof(__bf16))));

__device__ __forceinline__ int tswz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// element offset of (row, 8-column chunk c) in a swizzled [rows][128] tile
__device__ __forceinline__ int toff(int row, int c) { return row * HD + ((c ^ tswz(row)) << 3); }

// Direct global -> LDS staging of a [ROWS][128] tile: ROWS / 4 instructions
// of 1 KB (4 rows each), ROWS / 16 per wave.  rowp(row) gives the global
// address of a row.
template <int ROWS = 64, typename RowPtr>
__device__ __forceinline__ void dma_tile(bf16* S, int wave, int lane, RowPtr rowp) {
  const int rsub = lane >> 4, cp = lane & 15;
#pragma unroll
  for (int i = 0; i < ROWS / 16; ++i) {
    const int g = wave * (ROWS / 16) + i;
    const int row = g * 4 + rsub;
    const int c = cp ^ tswz(row);
    __builtin_amdgcn_global_load_lds(rowp(row) + c * 8, (__attribute__((address_space(3))) void*)(S + g * 4 * HD),
                                     16, 0, 0);
  }
}

// Buffer resource whose base is `base` (no range limit below 2^31 bytes):
// the staging loops give per-lane 32-bit byte offsets from it.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const bf16* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(base), 0, 0x7fffffff, 0x00020000);
}

// MFMA operand: 8 consecutive columns (chunk c) of `row`.
__device__ __forceinline__ bf16x8_t frag_row(const bf16* S, int row, int c) {
  return *reinterpret_cast<const bf16x8_t*>(S + toff(row, c));
}

// MFMA A operand of X^T from a row-major tile X: output rows are the columns
// col0 .. col0 + 31 of X, k-slots are rows rbase + 8 (e >> 2) + 4 h + (e & 3).
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

// The same two reads from precomputed per-lane byte offsets (the address of
// every fragment of a tile is then a register plus an immediate).
__device__ __forceinline__ bf16x8_t frag_at(const bf16* S, uint32_t off) {
  return *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const char*>(S) + off);
}
__device__ __forceinline__ bf16x8_t frag_tr_at(const bf16* S, uint32_t o1, uint32_t o2) {
  const char* b = reinterpret_cast<const char*>(S);
  const bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(b + o1));
  const bf16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4_t*)(b + o2));
  const uint2 u = __builtin_bit_cast(uint2, x), v = __builtin_bit_cast(uint2, y);
  return __builtin_bit_cast(bf16x8_t, make_uint4(u.x, u.y, v.x, v.y));
}
// Per-lane byte offsets inside a swizzled [rows][128] tile:
//   row fragment (row 32 q + lc, chunk 2 ks + h):  rof[ks] + 8192 q;
//   transposed fragment (output rows = columns 32 ht .. 32 ht + 31, k-slots
//   from rows 16 m + 4 h + ...): tof[2 ht], tof[2 ht + 1], plus 4096 m.
// Adding a multiple of 16 rows leaves the swizzle unchanged.
__device__ __forceinline__ void frag_offsets(int lane, uint32_t (&rof)[8], uint32_t (&tof)[8]) {
  const int lc = lane & 31, h = lane >> 5, g = lane >> 4, p = lane & 15;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) rof[ks] = (uint32_t)(toff(lc, 2 * ks + h) * 2);
  const int r1 = 4 * h + (p >> 2);
#pragma unroll
  for (int ht = 0; ht < 4; ++ht) {
    const int col = ht * 32 + 16 * (g & 1) + 4 * (p & 3);
    tof[2 * ht] = (uint32_t)((toff(r1, col >> 3) + (col & 7)) * 2);
    tof[2 * ht + 1] = (uint32_t)((toff(r1 + 8, col >> 3) + (col & 7)) * 2);
  }
}

// Registers r = 8 jp .. 8 jp + 7 of a score tile, rounded to bf16, as the
// B operand of the next product.
__device__ __forceinline__ bf16x8_t pack_p(const f32x16& p, int jp) {
  const int b = jp * 8;
  return __builtin_bit_cast(bf16x8_t, make_uint4(pack_bf16x2(p[b + 0], p[b + 1]), pack_bf16x2(p[b + 2], p[b + 3]),
                                                 pack_bf16x2(p[b + 4], p[b + 5]), pack_bf16x2(p[b + 6], p[b + 7])));
}

// 2^x by the hardware v_exp_f32 (results below 2^-126 flush to zero, which
// is immaterial for probabilities that are summed with ones of order 1).
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int div_h(int r, uint32_t hmagic) { return (int)__umulhi((uint32_t)r, hmagic); }

__device__ __forceinline__ f32x16 mfma(bf16x8_t a, bf16x8_t b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ uint32_t wd(const uint4& q, int w) {
  return w == 0 ? q.x : (w == 1 ? q.y : (w == 2 ? q.z : q.w));
}

}  // namespace
}  // namespace nc
