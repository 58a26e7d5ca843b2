// HIP backend for gfx950 (CDNA4): the device side of the shared-prefix
// multi-LoRA attention library.
//
// Kernels
//   append_kernel       K/V row copy into pages (V stored transposed), page
//                       table update, and low-rank rows bf16(X A): MFMA for
//                       bulk row tiles, a block-wide dot product for a few rows.
//   decode_split_kernel one workgroup per (KV head, key range). The range's
//                       K/V tiles are read from HBM once and used by every
//                       listed agent's query rows (all G heads of the group).
//                       Scores, P V_base and P V_lr run on bf16 MFMA with fp32
//                       accumulation; the online-softmax max and sum use
//                       wavefront shuffles. Writes partial (m, l, o, o_lr).
//   decode_merge_kernel merges the partials of one (agent, KV head), then
//                       applies B_i once: o += (P V_lr) B_i[:, g*d:(g+1)*d].
//   prefill_kernel      one workgroup per (KV head, agent, 128 query rows):
//                       the same MFMA tile scheme over the agent's whole view
//                       with a causal mask, B_i applied once per query block.
//
// The method (LRAgent review, "What carries the argument"): V_i = V_base +
// (X A_i) B_i is never formed; attention computes O = P V_base + (P V_lr) B_i.
//
// MFMA tile scheme (v_mfma_f32_16x16x32_bf16, wave64). For a 32-key chunk:
//   S^T[key][row] = K[key][:] . Q[row][:]   A operand = K rows, B operand = Q
//   O^T[d][row]  += V^T[d][keys] . P^T[keys][row]
//   L^T[k][row]  += LR^T[k][keys] . P^T[keys][row]
// A 16x16 C tile puts query row n = lane % 16 in every lane's column, so each
// lane's accumulators belong to one query row and the softmax rescale is one
// scalar per lane. The K rows of the two 16-key score tiles are permuted so
// that lane (n, q) ends up holding the scores of keys 8q..8q+7 of the chunk,
// which is exactly the B-operand slice P^T needs: P never leaves registers.
// V and the low-rank rows are stored transposed in their pages ([d][slot] and
// [rank][slot]) so their A-operand slices are 16 contiguous bytes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <vector>

#include "backend.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr int kPage = 64;           // rows per page in the GPU build
constexpr int kMaxDecodeRows = 64;  // query rows (agents x G) per decode launch
constexpr int kMaxItems = 2048;     // decode work items per launch (partials capacity)
constexpr int kMaxMergeSlots = 1024;
constexpr int kMaxViewPages = 4096;  // prefill view length cap: 262144 tokens
constexpr int kMaxItemPages = 256;

char g_err[256] = "";
void set_err(const char* what, hipError_t e) {
  snprintf(g_err, sizeof g_err, "%s: %s", what, hipGetErrorString(e));
}

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }

__device__ __forceinline__ bf16x8 ld8(const u16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0}); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)p[i];
  return r;
}

__device__ __forceinline__ float xmax16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float xsum16_32(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Row of the permuted 16-key score tile t (0/1) that lane row m loads:
// keys 8*(m/4) + m%4 for tile 0 and 8*(m/4) + 4 + m%4 for tile 1, so the C
// tile entry j of lane group q is key 8q + j (tile 0) or 8q + 4 + j (tile 1).
__device__ __forceinline__ int perm_key(int m, int t) { return 8 * (m >> 2) + 4 * t + (m & 3); }

// ---------------------------------------------------------------------------
// Append: K/V pages + page tables + low-rank rows
// ---------------------------------------------------------------------------

struct AppendParams {
  u16* K;          // layer base [page][Hkv][ps][D]
  u16* VT;         // layer base [page][Hkv][D][ps]
  u16* LRT;        // layer base of plane 0 [page][r][ps]
  uint64_t lr_plane;
  int32_t* tbl;    // layer base [1+N][max_pages]
  int tbl_seq;
  const u16* k;
  const u16* v;
  const u16* x;
  int Hkv, D, r, hidden;
  int do_kv, do_lr, update_tables;
  int n_spans;
  skv::Span spans[skv::kMaxJobSpans];
  int32_t ids[skv::kMaxJobPages];
  int kv_block0[skv::kMaxJobSpans + 1];  // prefix sums of K/V blocks per span
  int lr_block0[skv::kMaxJobSpans + 1];  // prefix sums of low-rank blocks per span
  int lr_kind[skv::kMaxJobSpans];        // 0 zero rows, 1 dot product per row, 2 MFMA tiles
};

constexpr int kLrTile = 64;   // rows per MFMA low-rank block
constexpr int kLrChunk = 256; // hidden columns of A staged in LDS per step

__device__ void append_kv_block(const AppendParams& p, int s, int blk, char* smem) {
  const skv::Span& sp = p.spans[s];
  const int D = p.D;
  const int pi = blk / p.Hkv, h = blk % p.Hkv;
  const int page_idx = sp.first_page + pi;
  const int page = p.ids[sp.ids_off + pi];
  const int lo = (pi == 0) ? sp.pos0 % kPage : 0;
  const int end = sp.pos0 + sp.n;
  const int hi = (page_idx == (end - 1) / kPage) ? (end - 1) % kPage + 1 : kPage;
  const int rows = hi - lo;
  const int src0 = sp.src_row + (page_idx * kPage + lo - sp.pos0);
  // K: rows [lo, hi) of the page, 16-byte vectors
  u16* kdst = p.K + ((uint64_t)page * p.Hkv + h) * kPage * D;
  const int vec_per_row = D / 8;
  for (int i = threadIdx.x; i < rows * vec_per_row; i += blockDim.x) {
    int rr = i / vec_per_row, c = i % vec_per_row;
    const u16* src = p.k + ((uint64_t)(src0 + rr) * p.Hkv + h) * D + c * 8;
    *reinterpret_cast<u32x4*>(kdst + (uint64_t)(lo + rr) * D + c * 8) =
        *reinterpret_cast<const u32x4*>(src);
  }
  // V: stage the rows in LDS, then write the transposed tile [D][slot]
  u16* vs = reinterpret_cast<u16*>(smem);  // [64][D + 8]
  const int ld = D + 8;
  for (int i = threadIdx.x; i < rows * vec_per_row; i += blockDim.x) {
    int rr = i / vec_per_row, c = i % vec_per_row;
    const u16* src = p.v + ((uint64_t)(src0 + rr) * p.Hkv + h) * D + c * 8;
    u32x4 val = *reinterpret_cast<const u32x4*>(src);
    u16* dst = vs + rr * ld + c * 8;
    *reinterpret_cast<u32x2*>(dst) = u32x2{val[0], val[1]};
    *reinterpret_cast<u32x2*>(dst + 4) = u32x2{val[2], val[3]};
  }
  __syncthreads();
  u16* vdst = p.VT + ((uint64_t)page * p.Hkv + h) * D * kPage;
  for (int i = threadIdx.x; i < D * rows; i += blockDim.x) {
    int dd = i / rows, rr = i % rows;
    vdst[(uint64_t)dd * kPage + lo + rr] = vs[rr * ld + dd];
  }
}

__device__ void append_lr_zero_block(const AppendParams& p, int s, int pi) {
  const skv::Span& sp = p.spans[s];
  const int page_idx = sp.first_page + pi;
  const int page = p.ids[sp.ids_off + pi];
  const int lo = (pi == 0) ? sp.pos0 % kPage : 0;
  const int end = sp.pos0 + sp.n;
  const int hi = (page_idx == (end - 1) / kPage) ? (end - 1) % kPage + 1 : kPage;
  u16* dst = p.LRT + sp.plane * p.lr_plane + (uint64_t)page * p.r * kPage;
  const int rows = hi - lo;
  for (int i = threadIdx.x; i < p.r * rows; i += blockDim.x) {
    int k = i / rows, rr = i % rows;
    dst[k * kPage + lo + rr] = 0;
  }
}

// One low-rank row as a block-wide dot product: used when a span has few rows.
__device__ void append_lr_dot_block(const AppendParams& p, int s, int row, char* smem) {
  const skv::Span& sp = p.spans[s];
  const int r = p.r, H = p.hidden;
  const u16* x = p.x + (uint64_t)(sp.src_row + row) * H;
  float acc[32];
#pragma unroll
  for (int k = 0; k < 32; ++k) acc[k] = 0.f;
  for (int u = threadIdx.x; u < H; u += blockDim.x) {
    float xv = bf2f(x[u]);
    const u16* arow = sp.a + (uint64_t)u * r;
#pragma unroll
    for (int k = 0; k < 32; ++k)
      if (k < r) acc[k] += xv * bf2f(arow[k]);
  }
  float* red = reinterpret_cast<float*>(smem);  // [4 waves][32]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    if (k < r) {
      float v = acc[k];
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0) red[w * 32 + k] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < r) {
    const int k = threadIdx.x;
    float v = 0.f;
    for (int ww = 0; ww < (int)(blockDim.x >> 6); ++ww) v += red[ww * 32 + k];
    const int pos = sp.pos0 + row;
    const int page = p.ids[sp.ids_off + pos / kPage - sp.first_page];
    p.LRT[sp.plane * p.lr_plane + (uint64_t)page * r * kPage + k * kPage + pos % kPage] = f2bf(v);
  }
}

// Up to 64 low-rank rows with MFMA: C[row][rank] = X[row][:] . A[:][rank].
// Wave w owns rows 16w..16w+15 of the tile; A is staged transposed in LDS,
// kLrChunk hidden columns at a time, ranks padded to a multiple of 16.
__device__ void append_lr_mfma_block(const AppendParams& p, int s, int tile, char* smem) {
  const skv::Span& sp = p.spans[s];
  const int r = p.r, H = p.hidden;
  const int NB = (r + 15) / 16;
  u16* at = reinterpret_cast<u16*>(smem);  // [NB*16][kLrChunk + 8]
  const int ldA = kLrChunk + 8;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int row = tile * kLrTile + w * 16 + n;  // A-operand row of this lane
  const bool row_ok = row < sp.n;
  const u16* xrow = p.x + (uint64_t)(sp.src_row + (row_ok ? row : 0)) * H;
  f32x4 acc[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
  for (int u0 = 0; u0 < H; u0 += kLrChunk) {
    const int cols = min(kLrChunk, H - u0);
    __syncthreads();
    for (int i = threadIdx.x; i < NB * 16 * cols; i += blockDim.x) {
      int k = i / cols, u = i % cols;
      at[k * ldA + u] = (k < r) ? sp.a[(uint64_t)(u0 + u) * r + k] : (u16)0;
    }
    __syncthreads();
    for (int s32 = 0; s32 < cols; s32 += 32) {
      bf16x8 xa = row_ok ? ld8(xrow + u0 + s32 + 8 * q) : zero8();
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if (nb < NB) {
          bf16x8 ab = *reinterpret_cast<const bf16x8*>(at + (nb * 16 + n) * ldA + s32 + 8 * q);
          acc[nb] = mfma(xa, ab, acc[nb]);
        }
      }
    }
  }
  // C tile: lane holds rank 16nb + n, rows 16w + 4q + j of the tile
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int k = nb * 16 + n;
    if (nb < NB && k < r) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = tile * kLrTile + w * 16 + 4 * q + j;
        if (rr < sp.n) {
          const int pos = sp.pos0 + rr;
          const int page = p.ids[sp.ids_off + pos / kPage - sp.first_page];
          p.LRT[sp.plane * p.lr_plane + (uint64_t)page * r * kPage + k * kPage + pos % kPage] =
              f2bf(acc[nb][j]);
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  __shared__ __attribute__((aligned(16))) char smem[64 * (128 + 8) * 2];
  int b = blockIdx.x;
  if (b == 0 && p.update_tables) {
    for (int s = 0; s < p.n_spans; ++s) {
      const skv::Span& sp = p.spans[s];
      int32_t* t = p.tbl + sp.seq_slot * p.tbl_seq + sp.first_page;
      for (int i = threadIdx.x; i < sp.n_pages; i += blockDim.x) t[i] = p.ids[sp.ids_off + i];
    }
  }
  const int n_kv = p.kv_block0[p.n_spans];
  if (b >= n_kv + p.lr_block0[p.n_spans]) return;
  if (b < n_kv) {
    int s = 0;
    while (b >= p.kv_block0[s + 1]) ++s;
    append_kv_block(p, s, b - p.kv_block0[s], smem);
    return;
  }
  b -= n_kv;
  int s = 0;
  while (b >= p.lr_block0[s + 1]) ++s;
  const int sub = b - p.lr_block0[s];
  if (p.lr_kind[s] == 0)
    append_lr_zero_block(p, s, sub);
  else if (p.lr_kind[s] == 1)
    append_lr_dot_block(p, s, sub, smem);
  else
    append_lr_mfma_block(p, s, sub, smem);
}

// ---------------------------------------------------------------------------
// Decode: split pass
// ---------------------------------------------------------------------------

struct DecodeParams {
  const u16* K;    // layer base [page][Hkv][ps][D]
  const u16* VT;   // layer base [page][Hkv][D][ps]
  const u16* LRT;  // layer base, plane 0
  uint64_t lr_plane;
  const int32_t* tbl;  // layer base [1+N][max_pages]
  int tbl_seq;
  const u16* q;        // [n][Hq][D] (rows of this group start at q)
  float* part;         // [items][R][W]
  int Hkv, Hq, G, r, R, W;
  int n;                          // agents in this group
  int ag_id[SKV_MAX_AGENTS];
  int ag_b[SKV_MAX_AGENTS];
  int ag_S[SKV_MAX_AGENTS];
  int ag_pidx[SKV_MAX_AGENTS];    // index of the agent's plane in planes[]
  int n_planes;
  int planes[SKV_MAX_AGENTS];     // stacked low-rank planes of this group
  int own0[SKV_MAX_AGENTS + 1];   // prefix sums of own items per agent
  int max_b, split, n_shared, items_per_head;
  float scale_log2;
};

template <int D, int RB, int MB>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  constexpr int KS = D / 32, DB = D / 16;
  __shared__ int32_t s_pages[kMaxItemPages];
  extern __shared__ __attribute__((aligned(16))) float s_buf[];  // [RB*16][W]

  const int item = blockIdx.x;
  const int g = item / p.items_per_head;
  const int j = item % p.items_per_head;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, q = lane >> 4;

  // which key range
  bool shared = j < p.n_shared;
  int own_agent = -1, k0, k1;
  const int32_t* table;
  if (shared) {
    k0 = j * p.split;
    k1 = min(k0 + p.split, p.max_b);
    table = p.tbl;
  } else {
    int jj = j - p.n_shared;
    int a = 0;
    while (jj >= p.own0[a + 1]) ++a;
    own_agent = a;
    k0 = (jj - p.own0[a]) * p.split;
    k1 = min(k0 + p.split, p.ag_S[a]);
    table = p.tbl + (1 + p.ag_id[a]) * p.tbl_seq;
  }
  const int pg0 = k0 / kPage;
  const int npg = (k1 - 1) / kPage - pg0 + 1;
  for (int i = threadIdx.x; i < npg; i += blockDim.x) s_pages[i] = table[pg0 + i];

  // per-lane query rows: Q^T B-operand slices and the row's key limit
  bf16x8 qf[RB][KS];
  int lim[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rho = rb * 16 + n;
    const int a = rho / p.G;
    bool ok = rho < p.R && (shared || a == own_agent);
    lim[rb] = ok ? min(k1, shared ? p.ag_b[a] : p.ag_S[a]) : 0;
    const u16* qp = p.q + ((uint64_t)a * p.Hq + g * p.G + rho % p.G) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[rb][s] = ok ? ld8(qp + 32 * s + 8 * q) : zero8();
  }
  // Low-rank A-operand row of this lane in block mb: stacked row sr = 16mb + n.
  // A shared range stacks every plane of the group (plane sr / r, rank sr % r);
  // an agent's own range holds only its own plane (rank sr).
  bool lr_ok[MB];
  const u16* lr_row[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int sr = mb * 16 + n;
    const int pi = shared ? sr / p.r : p.ag_pidx[own_agent];
    const int k = shared ? sr % p.r : sr;
    lr_ok[mb] = shared ? pi < p.n_planes : sr < p.r;
    lr_row[mb] = p.LRT + (uint64_t)p.planes[lr_ok[mb] ? pi : 0] * p.lr_plane + k * kPage;
  }

  float m_run[RB], l_run[RB];
  f32x4 oacc[RB][DB], lacc[RB][MB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -1e30f;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[rb][db] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) lacc[rb][mb] = f32x4{0, 0, 0, 0};
  }
  __syncthreads();

  const int c_begin = k0 / 32 + w, c_end = (k1 + 31) / 32;
  const uint64_t head_off = (uint64_t)g * kPage * D;  // offset of head g inside a page
  const uint64_t page_elems = (uint64_t)p.Hkv * kPage * D;

  bf16x8 kf[2][KS], vf[DB], lf[MB];
  auto load = [&](int c, bf16x8 (&kk)[2][KS], bf16x8 (&vv)[DB], bf16x8 (&ll)[MB]) {
    const int key0 = c * 32;
    const int page = s_pages[key0 / kPage - pg0];
    const int half = (key0 % kPage) / 32;
    const u16* kp = p.K + (uint64_t)page * page_elems + head_off + (uint64_t)(half * 32) * D;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < KS; ++s) kk[t][s] = ld8(kp + perm_key(n, t) * D + 32 * s + 8 * q);
    const u16* vp = p.VT + (uint64_t)page * page_elems + head_off + half * 32 + 8 * q;
#pragma unroll
    for (int db = 0; db < DB; ++db) vv[db] = ld8(vp + (db * 16 + n) * kPage);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      ll[mb] = lr_ok[mb] ? ld8(lr_row[mb] + (uint64_t)page * p.r * kPage + half * 32 + 8 * q)
                         : zero8();
  };

  if (c_begin < c_end) load(c_begin, kf, vf, lf);
  for (int c = c_begin; c < c_end; c += 4) {
    bf16x8 kn[2][KS], vn[DB], ln[MB];
    const bool more = c + 4 < c_end;
    if (more) load(c + 4, kn, vn, ln);
    const int key0 = c * 32;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 s0 = {0, 0, 0, 0}, s1 = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        s0 = mfma(kf[0][s], qf[rb][s], s0);
        s1 = mfma(kf[1][s], qf[rb][s], s1);
      }
      float sc[8];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int kA = key0 + 8 * q + jj, kB = kA + 4;
        sc[jj] = kA < lim[rb] ? s0[jj] * p.scale_log2 : -INFINITY;
        sc[jj + 4] = kB < lim[rb] ? s1[jj] * p.scale_log2 : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
      mx = xmax16_32(mx);
      const float m_new = fmaxf(m_run[rb], mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
      float pv[8], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
        ps += pv[i];
      }
      l_run[rb] = l_run[rb] * alpha + ps;
      m_run[rb] = m_new;
      const bf16x8 pt = pack8(pv);
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[rb][db] = mfma(vf[db], pt, oacc[rb][db] * alpha);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) lacc[rb][mb] = mfma(lf[mb], pt, lacc[rb][mb] * alpha);
    }
    if (more) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[t][s] = kn[t][s];
#pragma unroll
      for (int db = 0; db < DB; ++db) vf[db] = vn[db];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) lf[mb] = ln[mb];
    }
  }

  // Combine the four waves' states in LDS, one wave at a time (deterministic).
  const int W = p.W;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) l_run[rb] = xsum16_32(l_run[rb]);
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int rho = rb * 16 + n;
        float* row = s_buf + rho * W;
        const int a = min(rho / p.G, p.n - 1);
        const int pidx = p.ag_pidx[a];
        float a_old = 0.f, a_new = 1.f, m_c = m_run[rb];
        if (ww > 0) {
          const float m_old = row[D + p.r];
          m_c = fmaxf(m_old, m_run[rb]);
          a_old = __builtin_amdgcn_exp2f(m_old - m_c);
          a_new = __builtin_amdgcn_exp2f(m_run[rb] - m_c);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float* dst = row + db * 16 + 4 * q + jj;
            *dst = (ww > 0 ? a_old * *dst : 0.f) + a_new * oacc[rb][db][jj];
          }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int sr = mb * 16 + 4 * q + jj;
            const int want = shared ? pidx : 0;
            if (sr / p.r == want && sr < p.n_planes * p.r) {
              float* dst = row + D + sr % p.r;
              *dst = (ww > 0 ? a_old * *dst : 0.f) + a_new * lacc[rb][mb][jj];
            }
          }
        if (q == 0) {
          const float l_old = ww > 0 ? row[D + p.r + 1] : 0.f;
          row[D + p.r + 1] = a_old * l_old + a_new * l_run[rb];
          row[D + p.r] = m_c;
        }
      }
    }
    __syncthreads();
  }
  // write the partial rows
  float* dst = p.part + (uint64_t)item * p.R * W;
  for (int i = threadIdx.x; i < p.R * W; i += blockDim.x) dst[i] = s_buf[i];
}

// ---------------------------------------------------------------------------
// Decode: merge partials and apply B_i
// ---------------------------------------------------------------------------

struct MergeParams {
  const float* part;
  const u16* B;   // [N][r][Hkv*D]
  u16* o;         // [n][Hq][D] of this group
  int Hkv, Hq, G, D, r, R, W;
  int n;
  int ag_id[SKV_MAX_AGENTS];
  int own0[SKV_MAX_AGENTS + 1];
  int n_shared, items_per_head;
};

__global__ __launch_bounds__(256) void decode_merge_kernel(MergeParams p) {
  __shared__ float s_w[8][kMaxMergeSlots];
  __shared__ float s_lr[8][32];
  __shared__ float s_o[8][128];
  const int a = blockIdx.x / p.Hkv, g = blockIdx.x % p.Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n_own = p.own0[a + 1] - p.own0[a];
  const int n_slots = p.n_shared + n_own;
  auto slot_item = [&](int s) {
    return g * p.items_per_head + (s < p.n_shared ? s : p.n_shared + p.own0[a] + (s - p.n_shared));
  };
  const int HD = p.Hkv * p.D;
  for (int h0 = 0; h0 < p.G; h0 += 8) {
    const int nr = min(8, p.G - h0);
    // weights per (row, slot): exp2(m_s - M) / L
    for (int rr = w; rr < nr; rr += 4) {
      const int rho = a * p.G + h0 + rr;
      float M = -1e30f;
      for (int s = lane; s < n_slots; s += 64)
        M = fmaxf(M, p.part[((uint64_t)slot_item(s) * p.R + rho) * p.W + p.D + p.r]);
      for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
      float L = 0.f;
      for (int s = lane; s < n_slots; s += 64) {
        const float* row = p.part + ((uint64_t)slot_item(s) * p.R + rho) * p.W;
        float e = __builtin_amdgcn_exp2f(row[p.D + p.r] - M);
        s_w[rr][s] = e;
        L += e * row[p.D + p.r + 1];
      }
      for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
      const float inv = 1.f / L;
      for (int s = lane; s < n_slots; s += 64) s_w[rr][s] *= inv;
    }
    __syncthreads();
    const int E = p.D + p.r;
    for (int i = threadIdx.x; i < nr * E; i += blockDim.x) {
      const int rr = i / E, e = i % E;
      const int rho = a * p.G + h0 + rr;
      float acc = 0.f;
      for (int s = 0; s < n_slots; ++s)
        acc += s_w[rr][s] * p.part[((uint64_t)slot_item(s) * p.R + rho) * p.W + e];
      if (e < p.D)
        s_o[rr][e] = acc;
      else
        s_lr[rr][e - p.D] = acc;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nr * p.D; i += blockDim.x) {
      const int rr = i / p.D, d = i % p.D;
      float acc = s_o[rr][d];
      const u16* bcol = p.B + (uint64_t)p.ag_id[a] * p.r * HD + g * p.D + d;
      for (int k = 0; k < p.r; ++k) acc += s_lr[rr][k] * bf2f(bcol[(uint64_t)k * HD]);
      p.o[((uint64_t)a * p.Hq + g * p.G + h0 + rr) * p.D + d] = f2bf(acc);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Prefill
// ---------------------------------------------------------------------------

constexpr int kPrefRBW = 2;                    // 16-row blocks per wave
constexpr int kPrefRows = 4 * 16 * kPrefRBW;   // query rows per workgroup

struct PrefillParams {
  const u16* K;
  const u16* VT;
  const u16* LRT;
  uint64_t lr_plane;
  const int32_t* tbl;
  int tbl_seq;
  const u16* q;
  const u16* B;
  u16* o;
  int Hkv, Hq, G, r;
  int n;
  int ag_id[SKV_MAX_AGENTS], ag_b[SKV_MAX_AGENTS], ag_S[SKV_MAX_AGENTS];
  int ag_plane[SKV_MAX_AGENTS], ag_nq[SKV_MAX_AGENTS], ag_row0[SKV_MAX_AGENTS];
  int blk0[SKV_MAX_AGENTS + 1];  // prefix sums of query blocks per agent
  float scale_log2;
};

template <int D, int MB>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillParams p) {
  constexpr int KS = D / 32, DB = D / 16, RB = kPrefRBW;
  __shared__ int32_t s_pages[kMaxViewPages];
  __shared__ float s_lr[4][16][33];
  const int g = blockIdx.x % p.Hkv;
  int qb = blockIdx.x / p.Hkv;
  int ai = 0;
  while (qb >= p.blk0[ai + 1]) ++ai;
  qb -= p.blk0[ai];
  const int b = p.ag_b[ai], S = p.ag_S[ai], nq = p.ag_nq[ai];
  const int Lv = b + S;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int rows_total = nq * p.G;
  const int row_blk0 = qb * kPrefRows;
  // highest view position among this block's rows
  const int last_row = min(row_blk0 + kPrefRows, rows_total) - 1;
  const int t_max = Lv - nq + last_row / p.G;

  const int np_sh = (min(b, t_max + 1) + kPage - 1) / kPage;
  const int own_keys = max(0, min(S, t_max + 1 - b));
  const int np_own = (own_keys + kPage - 1) / kPage;
  const int32_t* tsh = p.tbl;
  const int32_t* tow = p.tbl + (1 + p.ag_id[ai]) * p.tbl_seq;
  for (int i = threadIdx.x; i < np_sh + np_own; i += blockDim.x)
    s_pages[i] = i < np_sh ? tsh[i] : tow[i - np_sh];

  bf16x8 qf[RB][KS];
  int tpos[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rho = row_blk0 + w * 16 * RB + rb * 16 + n;
    const bool ok = rho < rows_total;
    const int ti = ok ? rho / p.G : 0;
    tpos[rb] = ok ? Lv - nq + ti : -1;
    const u16* qp = p.q + ((uint64_t)(p.ag_row0[ai] + ti) * p.Hq + g * p.G + rho % p.G) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[rb][s] = ok ? ld8(qp + 32 * s + 8 * q) : zero8();
  }
  const int plane = p.ag_plane[ai];
  const u16* lrb = p.LRT + (uint64_t)plane * p.lr_plane;
  bool lr_ok[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) lr_ok[mb] = mb * 16 + n < p.r;

  float m_run[RB], l_run[RB];
  f32x4 oacc[RB][DB], lacc[RB][MB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -1e30f;
    l_run[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[rb][db] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) lacc[rb][mb] = f32x4{0, 0, 0, 0};
  }
  __syncthreads();

  const uint64_t head_off = (uint64_t)g * kPage * D;
  const uint64_t page_elems = (uint64_t)p.Hkv * kPage * D;
  // Two segments: shared view positions [0, b) and own positions [0, S) at b + j.
  for (int seg = 0; seg < 2; ++seg) {
    const int nkeys = seg == 0 ? min(b, t_max + 1) : own_keys;
    const int vbase = seg == 0 ? 0 : b;         // view position of segment key 0
    const int seg_lim = seg == 0 ? b : S;       // keys beyond the segment are invalid
    const int pg_off = seg == 0 ? 0 : np_sh;
    for (int c = 0; c * 32 < nkeys; ++c) {
      const int key0 = c * 32;
      const int page = s_pages[pg_off + key0 / kPage];
      const int half = (key0 % kPage) / 32;
      const u16* kp = p.K + (uint64_t)page * page_elems + head_off + (uint64_t)(half * 32) * D;
      bf16x8 kf[2][KS], vf[DB], lf[MB];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[t][s] = ld8(kp + perm_key(n, t) * D + 32 * s + 8 * q);
      const u16* vp = p.VT + (uint64_t)page * page_elems + head_off + half * 32 + 8 * q;
#pragma unroll
      for (int db = 0; db < DB; ++db) vf[db] = ld8(vp + (db * 16 + n) * kPage);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        lf[mb] = lr_ok[mb] ? ld8(lrb + (uint64_t)page * p.r * kPage + (mb * 16 + n) * kPage +
                                 half * 32 + 8 * q)
                           : zero8();
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 s0 = {0, 0, 0, 0}, s1 = {0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          s0 = mfma(kf[0][s], qf[rb][s], s0);
          s1 = mfma(kf[1][s], qf[rb][s], s1);
        }
        float sc[8];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int kA = key0 + 8 * q + jj, kB = kA + 4;
          const bool okA = kA < seg_lim && vbase + kA <= tpos[rb];
          const bool okB = kB < seg_lim && vbase + kB <= tpos[rb];
          sc[jj] = okA ? s0[jj] * p.scale_log2 : -INFINITY;
          sc[jj + 4] = okB ? s1[jj] * p.scale_log2 : -INFINITY;
        }
        float mx = sc[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
        mx = xmax16_32(mx);
        const float m_new = fmaxf(m_run[rb], mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        float pv[8], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          pv[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
          ps += pv[i];
        }
        l_run[rb] = l_run[rb] * alpha + ps;
        m_run[rb] = m_new;
        const bf16x8 pt = pack8(pv);
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[rb][db] = mfma(vf[db], pt, oacc[rb][db] * alpha);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) lacc[rb][mb] = mfma(lf[mb], pt, lacc[rb][mb] * alpha);
      }
    }
  }

  // finalize: o = (oacc + lacc . B_i) / l, B_i applied once for the block's rows
  const int HD = p.Hkv * D;
  const u16* Bi = p.B + (uint64_t)p.ag_id[ai] * p.r * HD + g * D;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l = xsum16_32(l_run[rb]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int k = mb * 16 + 4 * q + jj;
        if (k < p.r) s_lr[w][n][k] = lacc[rb][mb][jj] * inv;
      }
    __syncthreads();
    const int rho = row_blk0 + w * 16 * RB + rb * 16 + n;
    if (rho < rows_total) {
      const int ti = rho / p.G;
      u16* op = p.o + ((uint64_t)(p.ag_row0[ai] + ti) * p.Hq + g * p.G + rho % p.G) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        float out[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) out[jj] = oacc[rb][db][jj] * inv;
        const int d0 = db * 16 + 4 * q;
        for (int k = 0; k < p.r; ++k) {
          const float lk = s_lr[w][n][k];
          const u16* br = Bi + (uint64_t)k * HD + d0;
          u32x2 bb = *reinterpret_cast<const u32x2*>(br);
          out[0] += lk * __uint_as_float(bb[0] << 16);
          out[1] += lk * __uint_as_float(bb[0] & 0xffff0000u);
          out[2] += lk * __uint_as_float(bb[1] << 16);
          out[3] += lk * __uint_as_float(bb[1] & 0xffff0000u);
        }
        u32x2 pk;
        pk[0] = (uint32_t)f2bf(out[0]) | ((uint32_t)f2bf(out[1]) << 16);
        pk[1] = (uint32_t)f2bf(out[2]) | ((uint32_t)f2bf(out[3]) << 16);
        *reinterpret_cast<u32x2*>(op + d0) = pk;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Host side: launch helpers, planning, timing
// ---------------------------------------------------------------------------

struct DevState {
  bool timing = false;
  std::vector<hipEvent_t> pool;
  struct Rec {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

struct TimedLaunch {
  DevState* st;
  hipStream_t stream;
  int kind;
  hipEvent_t a = nullptr, b = nullptr;
  TimedLaunch(const skv::Geometry& g, int k)
      : st((DevState*)g.dev), stream((hipStream_t)g.stream), kind(k) {
    if (st && st->timing) {
      a = st->get();
      b = st->get();
      if (a && b) (void)hipEventRecord(a, stream);
    }
  }
  int done(const char* what) {
    hipError_t e = hipGetLastError();
    if (a && b) {
      (void)hipEventRecord(b, stream);
      st->recs.push_back({kind, a, b});
    }
    if (e != hipSuccess) {
      set_err(what, e);
      return SKV_ERR_HIP;
    }
    return SKV_OK;
  }
};

int decode_group_limit(const skv::Geometry& g) {
  // agents per decode launch: rows <= 64, stacked low-rank rows <= 128,
  // and (row blocks x low-rank blocks) <= 8
  for (int ng = std::min(g.N, kMaxDecodeRows / g.G); ng >= 1; --ng) {
    int planes = g.mode == SKV_BASE_SHARED ? ng : 1;
    int rb = (ng * g.G + 15) / 16;
    rb = rb <= 1 ? 1 : (rb <= 2 ? 2 : 4);
    int mb = (planes * g.r + 15) / 16;
    mb = mb <= 1 ? 1 : (mb <= 2 ? 2 : (mb <= 4 ? 4 : 8));
    if (planes * g.r <= 128 && rb * mb <= 8) return ng;
  }
  return 0;
}

int w_of(const skv::Geometry& g) { return g.D + g.r + 4; }

template <int D, int RB, int MB>
void launch_split_t(const DecodeParams& p, int items, hipStream_t st) {
  size_t lds = (size_t)RB * 16 * p.W * sizeof(float);
  hipLaunchKernelGGL((decode_split_kernel<D, RB, MB>), dim3(items), dim3(256), lds, st, p);
}

template <int D>
bool launch_split_d(int rb, int mb, const DecodeParams& p, int items, hipStream_t st) {
  if (rb == 1 && mb == 1) launch_split_t<D, 1, 1>(p, items, st);
  else if (rb == 1 && mb == 2) launch_split_t<D, 1, 2>(p, items, st);
  else if (rb == 1 && mb == 4) launch_split_t<D, 1, 4>(p, items, st);
  else if (rb == 1 && mb == 8) launch_split_t<D, 1, 8>(p, items, st);
  else if (rb == 2 && mb == 1) launch_split_t<D, 2, 1>(p, items, st);
  else if (rb == 2 && mb == 2) launch_split_t<D, 2, 2>(p, items, st);
  else if (rb == 2 && mb == 4) launch_split_t<D, 2, 4>(p, items, st);
  else if (rb == 4 && mb == 1) launch_split_t<D, 4, 1>(p, items, st);
  else if (rb == 4 && mb == 2) launch_split_t<D, 4, 2>(p, items, st);
  else return false;
  return true;
}

}  // namespace

namespace skv {

int dev_check(const Geometry& g) {
  if (g.ps != kPage) return SKV_ERR_UNSUPPORTED;
  if (g.G > kMaxDecodeRows) return SKV_ERR_UNSUPPORTED;
  if (decode_group_limit(g) < 1) return SKV_ERR_UNSUPPORTED;
  return SKV_OK;
}

uint64_t dev_scratch_bytes(const Geometry& g) {
  return (uint64_t)kMaxItems * kMaxDecodeRows * w_of(g) * sizeof(float);
}

int dev_init(Geometry& g) {
  // Masked keys still enter the MFMA products with weight 0, so every byte of
  // the pools must hold a finite value: clear them once. Later contents are
  // appended rows or stale rows of freed pages, both finite.
  hipError_t e = hipMemsetAsync(g.arena, 0, g.scratch_off, (hipStream_t)g.stream);
  if (e != hipSuccess) {
    set_err("hipMemsetAsync", e);
    return SKV_ERR_HIP;
  }
  g.dev = new DevState();
  return SKV_OK;
}

void dev_fini(Geometry& g) {
  auto* st = (DevState*)g.dev;
  if (!st) return;
  for (auto& r : st->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (auto e : st->pool) (void)hipEventDestroy(e);
  delete st;
  g.dev = nullptr;
}

int dev_append(const Geometry& g, const AppendJob& job) {
  AppendParams p{};
  const uint64_t lay = (uint64_t)job.layer;
  p.K = (u16*)(g.arena + g.k_off) + lay * g.k_layer();
  p.VT = (u16*)(g.arena + g.vt_off) + lay * g.k_layer();
  p.LRT = (u16*)(g.arena + g.lrt_off) + lay * g.lr_layer();
  p.lr_plane = g.lr_plane();
  p.tbl = (int32_t*)(g.arena + g.tbl_off) + lay * g.tbl_layer();
  p.tbl_seq = (int)g.tbl_seq();
  p.k = job.k;
  p.v = job.v;
  p.x = job.x;
  p.Hkv = g.Hkv;
  p.D = g.D;
  p.r = g.r;
  p.hidden = g.hidden;
  p.do_kv = job.do_kv;
  p.do_lr = job.do_lr;
  p.update_tables = job.update_tables;
  p.n_spans = job.n_spans;
  memcpy(p.spans, job.spans, sizeof(Span) * job.n_spans);
  memcpy(p.ids, job.ids, sizeof(int32_t) * job.n_ids);
  p.kv_block0[0] = 0;
  p.lr_block0[0] = 0;
  for (int s = 0; s < job.n_spans; ++s) {
    const Span& sp = job.spans[s];
    p.kv_block0[s + 1] = p.kv_block0[s] + (job.do_kv ? sp.n_pages * g.Hkv : 0);
    int nb = 0;
    p.lr_kind[s] = 0;
    if (job.do_lr) {
      if (!job.x) {
        p.lr_kind[s] = 0;
        nb = sp.n_pages;
      } else if (sp.n <= 8) {
        p.lr_kind[s] = 1;
        nb = sp.n;
      } else {
        p.lr_kind[s] = 2;
        nb = (sp.n + kLrTile - 1) / kLrTile;
      }
    }
    p.lr_block0[s + 1] = p.lr_block0[s] + nb;
  }
  const int blocks = p.kv_block0[job.n_spans] + p.lr_block0[job.n_spans];
  if (blocks == 0 && !job.update_tables) return SKV_OK;
  TimedLaunch t(g, job.do_kv ? 0 : 1);
  hipLaunchKernelGGL(append_kernel, dim3(std::max(blocks, 1)), dim3(256), 0,
                     (hipStream_t)g.stream, p);
  ++*g.launches;
  return t.done("append_kernel");
}

int dev_attn_decode(const Geometry& g, const AttnJob& job) {
  const int ng = decode_group_limit(g);
  hipStream_t st = (hipStream_t)g.stream;
  const int W = w_of(g);
  float* part = (float*)(g.arena + g.scratch_off);
  for (int a0 = 0; a0 < job.n; a0 += ng) {
    const int n = std::min(ng, job.n - a0);
    DecodeParams p{};
    const uint64_t lay = (uint64_t)job.layer;
    p.K = (const u16*)(g.arena + g.k_off) + lay * g.k_layer();
    p.VT = (const u16*)(g.arena + g.vt_off) + lay * g.k_layer();
    p.LRT = (const u16*)(g.arena + g.lrt_off) + lay * g.lr_layer();
    p.lr_plane = g.lr_plane();
    p.tbl = (const int32_t*)(g.arena + g.tbl_off) + lay * g.tbl_layer();
    p.tbl_seq = (int)g.tbl_seq();
    p.q = job.q + (uint64_t)job.ag[a0].q_row0 * g.Hq * g.D;
    p.part = part;
    p.Hkv = g.Hkv;
    p.Hq = g.Hq;
    p.G = g.G;
    p.r = g.r;
    p.R = n * g.G;
    p.W = W;
    p.n = n;
    p.n_planes = 0;
    int max_b = 0, own_keys = 0;
    for (int i = 0; i < n; ++i) {
      const AttnAgent& a = job.ag[a0 + i];
      p.ag_id[i] = a.agent;
      p.ag_b[i] = a.b;
      p.ag_S[i] = a.S;
      int pidx = -1;
      for (int k = 0; k < p.n_planes; ++k)
        if (p.planes[k] == a.plane) pidx = k;
      if (pidx < 0) {
        pidx = p.n_planes;
        p.planes[p.n_planes++] = a.plane;
      }
      p.ag_pidx[i] = pidx;
      max_b = std::max(max_b, a.b);
      own_keys += a.S;
    }
    p.max_b = max_b;
    // split plan: about 2 workgroups per CU over all KV heads, 256-key granularity
    const int target_per_head = std::max(1, 512 / g.Hkv);
    const int keys = max_b + own_keys;
    int split = ((keys + target_per_head - 1) / target_per_head + 255) / 256 * 256;
    split = std::max(split, 256);
    int items_per_head = 0;
    for (;;) {
      int ns = (max_b + split - 1) / split;
      int no = 0;
      for (int i = 0; i < n; ++i) no += (p.ag_S[i] + split - 1) / split;
      items_per_head = ns + no;
      if ((uint64_t)items_per_head * g.Hkv <= (uint64_t)kMaxItems &&
          items_per_head <= kMaxMergeSlots)
        break;
      split *= 2;
    }
    if (split / kPage > kMaxItemPages) {
      snprintf(g_err, sizeof g_err, "decode view too long for the split plan (%d keys)", keys);
      return SKV_ERR_UNSUPPORTED;
    }
    p.split = split;
    p.n_shared = (max_b + split - 1) / split;
    p.own0[0] = 0;
    for (int i = 0; i < n; ++i) p.own0[i + 1] = p.own0[i] + (p.ag_S[i] + split - 1) / split;
    p.items_per_head = items_per_head;
    p.scale_log2 = 1.4426950408889634f / sqrtf((float)g.D);
    int rb = (p.R + 15) / 16;
    rb = rb <= 1 ? 1 : (rb <= 2 ? 2 : 4);
    int mb = (p.n_planes * g.r + 15) / 16;
    mb = mb <= 1 ? 1 : (mb <= 2 ? 2 : (mb <= 4 ? 4 : 8));
    const int items = items_per_head * g.Hkv;
    {
      TimedLaunch t(g, 2);
      bool ok = g.D == 128 ? launch_split_d<128>(rb, mb, p, items, st)
                           : launch_split_d<64>(rb, mb, p, items, st);
      if (!ok) {
        snprintf(g_err, sizeof g_err, "no decode kernel for rb=%d mb=%d", rb, mb);
        return SKV_ERR_UNSUPPORTED;
      }
      ++*g.launches;
      int rc = t.done("decode_split_kernel");
      if (rc != SKV_OK) return rc;
    }
    MergeParams mp{};
    mp.part = part;
    mp.B = job.B;
    mp.o = job.o + (uint64_t)job.ag[a0].q_row0 * g.Hq * g.D;
    mp.Hkv = g.Hkv;
    mp.Hq = g.Hq;
    mp.G = g.G;
    mp.D = g.D;
    mp.r = g.r;
    mp.R = p.R;
    mp.W = W;
    mp.n = n;
    for (int i = 0; i < n; ++i) mp.ag_id[i] = p.ag_id[i];
    for (int i = 0; i <= n; ++i) mp.own0[i] = p.own0[i];
    mp.n_shared = p.n_shared;
    mp.items_per_head = items_per_head;
    {
      TimedLaunch t(g, 3);
      hipLaunchKernelGGL(decode_merge_kernel, dim3(n * g.Hkv), dim3(256), 0, st, mp);
      ++*g.launches;
      int rc = t.done("decode_merge_kernel");
      if (rc != SKV_OK) return rc;
    }
  }
  return SKV_OK;
}

int dev_attn_prefill(const Geometry& g, const AttnJob& job) {
  PrefillParams p{};
  const uint64_t lay = (uint64_t)job.layer;
  p.K = (const u16*)(g.arena + g.k_off) + lay * g.k_layer();
  p.VT = (const u16*)(g.arena + g.vt_off) + lay * g.k_layer();
  p.LRT = (const u16*)(g.arena + g.lrt_off) + lay * g.lr_layer();
  p.lr_plane = g.lr_plane();
  p.tbl = (const int32_t*)(g.arena + g.tbl_off) + lay * g.tbl_layer();
  p.tbl_seq = (int)g.tbl_seq();
  p.q = job.q;
  p.B = job.B;
  p.o = job.o;
  p.Hkv = g.Hkv;
  p.Hq = g.Hq;
  p.G = g.G;
  p.r = g.r;
  p.n = job.n;
  p.blk0[0] = 0;
  for (int i = 0; i < job.n; ++i) {
    const AttnAgent& a = job.ag[i];
    if ((a.b + kPage - 1) / kPage + (a.S + kPage - 1) / kPage > kMaxViewPages) {
      snprintf(g_err, sizeof g_err, "view of %d rows exceeds the prefill limit", a.b + a.S);
      return SKV_ERR_UNSUPPORTED;
    }
    p.ag_id[i] = a.agent;
    p.ag_b[i] = a.b;
    p.ag_S[i] = a.S;
    p.ag_plane[i] = a.plane;
    p.ag_nq[i] = a.n_q;
    p.ag_row0[i] = a.q_row0;
    p.blk0[i + 1] = p.blk0[i] + (a.n_q * g.G + kPrefRows - 1) / kPrefRows;
  }
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)g.D);
  const int blocks = p.blk0[job.n] * g.Hkv;
  hipStream_t st = (hipStream_t)g.stream;
  TimedLaunch t(g, 4);
  const int mb = (g.r + 15) / 16;
  if (g.D == 128) {
    if (mb == 1) hipLaunchKernelGGL((prefill_kernel<128, 1>), dim3(blocks), dim3(256), 0, st, p);
    else hipLaunchKernelGGL((prefill_kernel<128, 2>), dim3(blocks), dim3(256), 0, st, p);
  } else {
    if (mb == 1) hipLaunchKernelGGL((prefill_kernel<64, 1>), dim3(blocks), dim3(256), 0, st, p);
    else hipLaunchKernelGGL((prefill_kernel<64, 2>), dim3(blocks), dim3(256), 0, st, p);
  }
  ++*g.launches;
  return t.done("prefill_kernel");
}

int dev_sync(const Geometry& g) {
  hipError_t e = hipStreamSynchronize((hipStream_t)g.stream);
  if (e != hipSuccess) {
    set_err("hipStreamSynchronize", e);
    return SKV_ERR_HIP;
  }
  return SKV_OK;
}

int dev_set_timing(Geometry& g, bool enable) {
  auto* st = (DevState*)g.dev;
  st->timing = enable;
  return SKV_OK;
}

int dev_collect_timing(Geometry& g, skv_kernel_times* out) {
  auto* st = (DevState*)g.dev;
  *out = skv_kernel_times{};
  hipError_t e = hipStreamSynchronize((hipStream_t)g.stream);
  if (e != hipSuccess) {
    set_err("hipStreamSynchronize", e);
    return SKV_ERR_HIP;
  }
  for (auto& r : st->recs) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
      out->ms[r.kind] += ms;
      out->launches[r.kind] += 1;
    }
    st->pool.push_back(r.a);
    st->pool.push_back(r.b);
  }
  st->recs.clear();
  return SKV_OK;
}

const char* dev_last_error() { return g_err; }

}  // namespace skv
