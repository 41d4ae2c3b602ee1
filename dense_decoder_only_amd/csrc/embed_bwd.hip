// Embedding backward (release-news page "Karpathy再放大招…", section
// 技術細節與問答: the token embedding is its own table, untied from the
// unembedding): dE[v] = sum over the positions t with ids[t] = v of de[t].
//
// Deterministic sorted segmented reduction, no floating-point atomics:
//   1. rank: for positions in chunks of 1024, the rank of each position among
//      equal ids earlier in its chunk, and per-chunk id counts;
//   2. column scan over chunks -> per-(chunk, id) base, and per-id counts;
//   3. exclusive scans over ids -> segment offsets and piece offsets;
//   4. place: a stable counting sort of positions by id;
//   5. pieces: every segment is cut into pieces of 64 positions (the Zipf
//      head id holds ~14% of all tokens, so segments are very unequal); each
//      piece sums its rows in position order with one 256-thread block,
//      float4 per thread;
//   6. finish: segments of several pieces add their piece sums in piece order;
//      absent ids get zero rows (or stay untouched when accumulating).
// The summation order depends only on the ids, so results are bitwise
// reproducible run to run.
#include "common.h"
#include "ops.h"

namespace nc {
namespace {

constexpr int CH = 1024;  // positions per rank chunk
constexpr int P = 64;     // positions per piece

struct EbWs {
  int32_t* rank;     // [n]
  int32_t* hist;     // [C, V]
  int32_t* count;    // [V]
  int32_t* npieces;  // [V]
  int32_t* nmulti;   // [V]  npieces if > 1 else 0
  int32_t* offset;   // [V + 1]
  int32_t* poff;     // [V + 1]
  int32_t* ppoff;    // [V + 1]
  int32_t* sorted;   // [n]
  int32_t* piece_v;  // [max_pieces]
  float* partial;    // [max_partial, d]
  int64_t max_pieces, max_partial;
};

int64_t max_pieces_of(int64_t n, int64_t V) { return n / P + std::min(n, V) + 1; }
int64_t max_partial_of(int64_t n) { return n / (P / 2) + 1; }

size_t carve(int64_t n, int64_t V, int d, EbWs* w, void* base) {
  const int64_t C = cdiv(n, CH);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes, 256);
    return o;
  };
  const size_t o_rank = take(n * 4), o_hist = take(C * V * 4), o_cnt = take(V * 4), o_np = take(V * 4),
               o_nm = take(V * 4), o_off = take((V + 1) * 4), o_poff = take((V + 1) * 4),
               o_ppoff = take((V + 1) * 4), o_sorted = take(n * 4), o_pv = take(max_pieces_of(n, V) * 4),
               o_part = take((size_t)max_partial_of(n) * d * 4);
  if (w) {
    char* b = static_cast<char*>(base);
    w->rank = reinterpret_cast<int32_t*>(b + o_rank);
    w->hist = reinterpret_cast<int32_t*>(b + o_hist);
    w->count = reinterpret_cast<int32_t*>(b + o_cnt);
    w->npieces = reinterpret_cast<int32_t*>(b + o_np);
    w->nmulti = reinterpret_cast<int32_t*>(b + o_nm);
    w->offset = reinterpret_cast<int32_t*>(b + o_off);
    w->poff = reinterpret_cast<int32_t*>(b + o_poff);
    w->ppoff = reinterpret_cast<int32_t*>(b + o_ppoff);
    w->sorted = reinterpret_cast<int32_t*>(b + o_sorted);
    w->piece_v = reinterpret_cast<int32_t*>(b + o_pv);
    w->partial = reinterpret_cast<float*>(b + o_part);
    w->max_pieces = max_pieces_of(n, V);
    w->max_partial = max_partial_of(n);
  }
  return off;
}

__global__ void zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ __launch_bounds__(CH) void rank_kernel(const int32_t* __restrict__ ids, int64_t n, int64_t V,
                                                  int32_t* __restrict__ rank, int32_t* __restrict__ hist) {
  __shared__ int32_t sid[CH];
  const int tid = threadIdx.x;
  const int64_t i = (int64_t)blockIdx.x * CH + tid;
  int32_t id = -1;
  if (i < n) {
    id = ids[i];
    if (id < 0 || id >= V) id = -1;
  }
  sid[tid] = id;
  __syncthreads();
  const int cnt = (int)std::min<int64_t>(CH, n - (int64_t)blockIdx.x * CH);
  if (id < 0) return;
  int r = 0;
  bool last = true;
  for (int j = 0; j < cnt; ++j) {
    if (sid[j] == id) {
      if (j < tid) ++r;
      else if (j > tid) last = false;
    }
  }
  rank[i] = r;
  if (last) hist[(int64_t)blockIdx.x * V + id] = r + 1;
}

__global__ void colscan_kernel(int32_t* __restrict__ hist, int64_t C, int64_t V, int32_t* __restrict__ count,
                               int32_t* __restrict__ npieces, int32_t* __restrict__ nmulti) {
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < V; v += (int64_t)gridDim.x * blockDim.x) {
    int32_t run = 0;
    for (int64_t c = 0; c < C; ++c) {
      const int32_t h = hist[c * V + v];
      hist[c * V + v] = run;
      run += h;
    }
    count[v] = run;
    const int32_t np = (run + P - 1) / P;
    npieces[v] = np;
    nmulti[v] = np > 1 ? np : 0;
  }
}

// Exclusive scans of in[k][0, n) into out[k][0, n], out[k][n] = total, one
// 1024-thread block per array k.  The input is taken in spans of 64 Ki
// elements: every thread first issues all 64 of its loads of a span (tile j,
// elements j*4096 + 4*tid .. +3), then the 16 tiles are scanned in order with
// a wavefront shuffle scan and one barrier per tile.
struct Scan3 {
  const int32_t* in[3];
  int32_t* out[3];
};

__global__ __launch_bounds__(1024) void scan_kernel(Scan3 a, int64_t n) {
  constexpr int TILE = 4096, NT = 16;
  __shared__ int32_t wsum[2][16];
  const int32_t* __restrict__ in = a.in[blockIdx.x];
  int32_t* __restrict__ out = a.out[blockIdx.x];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int32_t carry = 0;
  int buf = 0;
  for (int64_t base = 0; base < n; base += (int64_t)TILE * NT) {
    int32_t v[NT][4];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t i = base + (int64_t)j * TILE + tid * 4 + q;
        v[j][q] = i < n ? in[i] : 0;
      }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int32_t t = v[j][0] + v[j][1] + v[j][2] + v[j][3];
      int32_t x = t;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      if (lane == 63) wsum[buf][wid] = x;
      __syncthreads();
      int32_t pre = 0, tot = 0;
#pragma unroll
      for (int w = 0; w < 16; ++w) {
        const int32_t ws = wsum[buf][w];
        pre += w < wid ? ws : 0;
        tot += ws;
      }
      int32_t run = carry + pre + x - t;
      const int64_t i0 = base + (int64_t)j * TILE + tid * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (i0 + q < n) out[i0 + q] = run;
        run += v[j][q];
      }
      carry += tot;
      buf ^= 1;  // the next tile writes the other buffer, so one barrier per tile suffices
    }
  }
  if (tid == 0) out[n] = carry;
}

__global__ void place_kernel(const int32_t* __restrict__ ids, int64_t n, int64_t V, const int32_t* __restrict__ rank,
                             const int32_t* __restrict__ hist, const int32_t* __restrict__ offset,
                             int32_t* __restrict__ sorted) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int32_t id = ids[i];
    if (id < 0 || id >= V) continue;
    const int64_t c = i / CH;
    sorted[offset[id] + hist[c * V + id] + rank[i]] = (int32_t)i;
  }
}

__global__ void piece_table_kernel(const int32_t* __restrict__ npieces, const int32_t* __restrict__ poff, int64_t V,
                                   int32_t* __restrict__ piece_v) {
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < V; v += (int64_t)gridDim.x * blockDim.x) {
    const int32_t np = npieces[v], o = poff[v];
    for (int32_t p = 0; p < np; ++p) piece_v[o + p] = (int32_t)v;
  }
}

// Row sources of the segmented sums: fp32 rows, or bf16 rows times a
// per-position factor (mul * scale[t]).
struct F32Rows {
  const float* p;
  __device__ float4 at(int32_t t, int d, int c) const {
    return *reinterpret_cast<const float4*>(p + (int64_t)t * d + c);
  }
};
struct ScaledBf16Rows {
  const bf16* p;
  const float* scale;
  float mul;
  __device__ float4 at(int32_t t, int d, int c) const {
    const uint2 u = *reinterpret_cast<const uint2*>(p + (int64_t)t * d + c);
    const float f = mul * scale[t];
    return make_float4(f * __uint_as_float(u.x << 16), f * __uint_as_float(u.x & 0xffff0000u),
                       f * __uint_as_float(u.y << 16), f * __uint_as_float(u.y & 0xffff0000u));
  }
};

template <class Src>
__global__ __launch_bounds__(256) void piece_sum_kernel(Src de, int d, const int32_t* __restrict__ sorted,
                                                        const int32_t* __restrict__ offset,
                                                        const int32_t* __restrict__ count,
                                                        const int32_t* __restrict__ npieces,
                                                        const int32_t* __restrict__ poff,
                                                        const int32_t* __restrict__ ppoff,
                                                        const int32_t* __restrict__ piece_v, int64_t V,
                                                        float* __restrict__ partial, float* __restrict__ dtable,
                                                        int accumulate) {
  const int64_t b = blockIdx.x;
  if (b >= poff[V]) return;
  const int32_t v = piece_v[b];
  const int32_t p = (int32_t)(b - poff[v]);
  const int32_t beg = offset[v] + p * P;
  const int32_t end = offset[v] + std::min(count[v], (p + 1) * P);
  const bool single = npieces[v] == 1;
  for (int c = threadIdx.x * 4; c < d; c += 1024) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int32_t k = beg; k < end; ++k) {
      const float4 x = de.at(sorted[k], d, c);
      s.x += x.x;
      s.y += x.y;
      s.z += x.z;
      s.w += x.w;
    }
    if (single) {
      float4* dst = reinterpret_cast<float4*>(dtable + (int64_t)v * d + c);
      if (accumulate) {
        const float4 o = *dst;
        s = make_float4(o.x + s.x, o.y + s.y, o.z + s.z, o.w + s.w);
      }
      *dst = s;
    } else {
      *reinterpret_cast<float4*>(partial + ((int64_t)ppoff[v] + p) * d + c) = s;
    }
  }
}

// One wavefront per (id, 256-column chunk): the head ids have over a hundred
// pieces, so the chunks of one row go to separate waves, and the loads of 8
// pieces are issued together before they are added in piece order.
__global__ __launch_bounds__(256) void finish_kernel(const int32_t* __restrict__ count,
                                                     const int32_t* __restrict__ npieces,
                                                     const int32_t* __restrict__ ppoff,
                                                     const float* __restrict__ partial, int64_t V, int d,
                                                     float* __restrict__ dtable, int accumulate) {
  const int lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int c = (int)blockIdx.y * 256 + lane * 4;
  if (v >= V || c >= d) return;
  const int32_t np = npieces[v];
  if (np == 1) return;  // written by piece_sum_kernel
  float4* dst = reinterpret_cast<float4*>(dtable + v * d + c);
  if (count[v] == 0) {
    if (!accumulate) *dst = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const float* src = partial + (int64_t)ppoff[v] * d + c;
  float4 s = accumulate ? *dst : make_float4(0.f, 0.f, 0.f, 0.f);
  int32_t p = 0;
  for (; p + 8 <= np; p += 8) {
    float4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = *reinterpret_cast<const float4*>(src + (int64_t)(p + u) * d);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s.x += x[u].x;
      s.y += x[u].y;
      s.z += x[u].z;
      s.w += x[u].w;
    }
  }
  for (; p < np; ++p) {
    const float4 x = *reinterpret_cast<const float4*>(src + (int64_t)p * d);
    s.x += x.x;
    s.y += x.y;
    s.z += x.z;
    s.w += x.w;
  }
  *dst = s;
}

}  // namespace

int fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return NC_OK;
  NC_REQUIRE(p && bytes % 4 == 0, NC_ERR_INVALID_ARG, "fill_zero: bad buffer");
  const int64_t words = (int64_t)(bytes / 4);
  zero_kernel<<<(unsigned)std::min<int64_t>(cdiv(words, 256), 8192), 256, 0, s>>>(static_cast<uint32_t*>(p), words);
  return check_launch("zero_kernel");
}

size_t embed_bwd_workspace_bytes(int64_t n, int64_t V, int d) { return carve(n, V, d, nullptr, nullptr); }

namespace {

template <class Src>
int embed_bwd_impl(const int32_t* ids, int64_t n, Src de, int d, float* dtable, int64_t V, int accumulate, void* ws,
                   size_t ws_bytes, hipStream_t s) {
  NC_REQUIRE(n >= 0 && V > 0 && d > 0, NC_ERR_INVALID_ARG, "embed_bwd: bad shape");
  NC_REQUIRE(d % 8 == 0, NC_ERR_UNSUPPORTED, "embed_bwd: d must be a multiple of 8");
  NC_REQUIRE(n < (1ll << 31) && V < (1ll << 31), NC_ERR_UNSUPPORTED, "embed_bwd: sizes must be below 2^31");
  const size_t need = embed_bwd_workspace_bytes(n, V, d);
  NC_REQUIRE(ws && ws_bytes >= need, NC_ERR_WORKSPACE, "embed_bwd: workspace too small (%zu < %zu)", ws_bytes, need);
  EbWs w;
  carve(n, V, d, &w, ws);
  const int64_t C = cdiv(n, CH);
  NC_TRY(fill_zero(w.hist, (size_t)C * V * 4, s));
  if (n > 0) {
    rank_kernel<<<(unsigned)C, CH, 0, s>>>(ids, n, V, w.rank, w.hist);
    NC_TRY(check_launch("rank_kernel"));
  }
  const unsigned vb = (unsigned)std::min<int64_t>(cdiv(V, 256), 4096);
  colscan_kernel<<<vb, 256, 0, s>>>(w.hist, C, V, w.count, w.npieces, w.nmulti);
  NC_TRY(check_launch("colscan_kernel"));
  Scan3 sc{{w.count, w.npieces, w.nmulti}, {w.offset, w.poff, w.ppoff}};
  scan_kernel<<<3, 1024, 0, s>>>(sc, V);
  NC_TRY(check_launch("scan_kernel"));
  if (n > 0) {
    place_kernel<<<(unsigned)std::min<int64_t>(cdiv(n, 256), 4096), 256, 0, s>>>(ids, n, V, w.rank, w.hist, w.offset,
                                                                                  w.sorted);
    NC_TRY(check_launch("place_kernel"));
  }
  piece_table_kernel<<<vb, 256, 0, s>>>(w.npieces, w.poff, V, w.piece_v);
  NC_TRY(check_launch("piece_table_kernel"));
  if (n > 0) {
    piece_sum_kernel<Src><<<(unsigned)w.max_pieces, 256, 0, s>>>(de, d, w.sorted, w.offset, w.count, w.npieces, w.poff,
                                                            w.ppoff, w.piece_v, V, w.partial, dtable, accumulate);
    NC_TRY(check_launch("piece_sum_kernel"));
  }
  finish_kernel<<<dim3((unsigned)cdiv(V, 4), (unsigned)cdiv(d, 256)), 256, 0, s>>>(w.count, w.npieces, w.ppoff, w.partial, V, d, dtable, accumulate);
  return check_launch("finish_kernel");
}

}  // namespace

int embed_bwd(const int32_t* ids, int64_t n, const float* de, int d, float* dtable, int64_t V, int accumulate,
              void* ws, size_t ws_bytes, hipStream_t s) {
  NC_REQUIRE(ids && de && dtable, NC_ERR_INVALID_ARG, "embed_bwd: null pointer");
  return embed_bwd_impl(ids, n, F32Rows{de}, d, dtable, V, accumulate, ws, ws_bytes, s);
}

int embed_bwd_scaled(const int32_t* ids, int64_t n, const bf16* rows, const float* scale, float mul, int d,
                     float* dtable, int64_t V, int accumulate, void* ws, size_t ws_bytes, hipStream_t s) {
  NC_REQUIRE(ids && rows && scale && dtable, NC_ERR_INVALID_ARG, "embed_bwd: null pointer");
  return embed_bwd_impl(ids, n, ScaledBf16Rows{rows, scale, mul}, d, dtable, V, accumulate, ws, ws_bytes, s);
}

}  // namespace nc

extern "C" size_t nc_embed_bwd_workspace_bytes(int64_t n, int64_t V, int d) {
  return nc::embed_bwd_workspace_bytes(n, V, d);
}

extern "C" int nc_embed_bwd(const int32_t* ids, int64_t n, const float* de, int d, float* dtable, int64_t V,
                            int accumulate, void* ws, size_t ws_bytes, void* stream) {
  return nc::api_done(nc::embed_bwd(ids, n, de, d, dtable, V, accumulate, ws, ws_bytes, static_cast<hipStream_t>(stream)),
                      stream, "nc_embed_bwd");
}
