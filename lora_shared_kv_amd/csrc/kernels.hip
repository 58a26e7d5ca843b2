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
//   prefill_kernel      one workgroup per (KV head, agent, 256 query rows):
//                       the same MFMA tile scheme over the agent's whole view
//                       with a causal mask, pages staged in LDS for the whole
//                       workgroup, two wave groups alternating MFMA and
//                       softmax phases; B_i applied once per query row.
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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "backend.h"
#include "plan.h"

namespace skv {
// Written by the probe kernels only on an impossible value; external linkage,
// so the compiler must keep the work that feeds it.
__device__ unsigned int probe_sink[4];
// One word per wave of the launch-pattern probe's streaming launch (at most
// four waves in each of kPlanCUs workgroups), read by the small launch after it.
__device__ unsigned int probe_part[4 * kPlanCUs];
}  // namespace skv

// Static device scratch of skv_decode_step_static (callers that cannot
// allocate): the decode partial rows, kStaticScratchBytes, one copy per device
// for the life of the process. Host code never passes this name to a kernel:
// it takes the array's device address per device with hipGetSymbolAddress.
static __device__ __align__(256) float scratch[skv::kStaticScratchBytes / sizeof(float)];

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

constexpr int kPage = skv::kPlanPage;  // rows per page in the GPU build
using skv::kMaxDecodeRows;
using skv::kMaxItems;
using skv::kMaxMergeSlots;
using skv::kMaxViewPages;
using skv::kMaxItemChunks;
constexpr int kCUs = skv::kPlanCUs;

char g_err[256] = "";
void set_err(const char* what, hipError_t e) {
  snprintf(g_err, sizeof g_err, "%s: %s", what, hipGetErrorString(e));
}

__device__ __forceinline__ float bf2f(u16 b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ u16 f2bf(float f) { return __builtin_bit_cast(u16, (__bf16)f); }

__device__ __forceinline__ bf16x8 ld8(const u16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ bf16x8 ld8_nt(const u16* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0}); }

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max of three floats in one instruction. fmaxf would first quiet each
// operand that could be a signalling NaN (one extra instruction per operand);
// the scores here are finite or -inf.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// s_waitcnt WAIT, then a bare s_barrier; no LDS access moves across either.
template <int WAIT>
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(WAIT);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// s_waitcnt for every LDS and scalar-memory operation alone (vector-memory
// and export counters at their maxima)
constexpr int kWaitLdsOnly = 15 | (7 << 4) | (3 << 14);

// Zero the first nm of the eight bf16 values of x (value 2k is the low half
// of 32-bit word k). nm <= 0 keeps all of them, nm >= 8 zeroes all.
__device__ __forceinline__ bf16x8 zero_leading(bf16x8 x, int nm) {
  u32x4 u = __builtin_bit_cast(u32x4, x);
#pragma unroll
  for (int k = 0; k < 4; ++k) u[k] &= (2 * k < nm ? 0u : 0x0000ffffu) | (2 * k + 1 < nm ? 0u : 0xffff0000u);
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ bf16x8 pack8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)p[i];
  return r;
}

// Reductions over the four lanes n, n + 16, n + 32, n + 48 (the lane groups
// that hold one MFMA column): v_permlane16_swap / v_permlane32_swap with both
// operands = v return, per lane, v at the lane and at the lane 16 (32) apart,
// as plain VALU ops.
__device__ __forceinline__ float xpair16(float v, float (*op)(float, float)) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xpair32(float v, float (*op)(float, float)) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float fmax_op(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float add_op(float a, float b) { return a + b; }
__device__ __forceinline__ float xmax16_32(float v) { return xpair32(xpair16(v, fmax_op), fmax_op); }
__device__ __forceinline__ float xsum16_32(float v) { return xpair32(xpair16(v, add_op), add_op); }

// Whole-wave reductions without LDS: DPP quad permutes (lanes xor 1, xor 2),
// the 8-lane and 16-lane mirrors (which pair the halves of each group), then
// the two permlane swaps. Every lane ends with the result.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = op(v, dppf<0xb1>(v));   // quad_perm [1, 0, 3, 2]
  v = op(v, dppf<0x4e>(v));   // quad_perm [2, 3, 0, 1]
  v = op(v, dppf<0x141>(v));  // row_half_mirror
  v = op(v, dppf<0x140>(v));  // row_mirror
  v = xpair16(v, op);
  return xpair32(v, op);
}
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, fmax_op); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, add_op); }

// Row of the permuted 16-key score tile t (0/1) that lane row m loads:
// keys 8*(m/4) + m%4 for tile 0 and 8*(m/4) + 4 + m%4 for tile 1, so the C
// tile entry j of lane group q is key 8q + j (tile 0) or 8q + 4 + j (tile 1).
__device__ __forceinline__ int perm_key(int m, int t) { return 8 * (m >> 2) + 4 * t + (m & 3); }

// Operand-ordered page tiles. One (page, KV head) tile holds 64 keys x D
// values of K (or of V) in the order the MFMA operand loads consume them, so
// every wave-wide 16-byte-per-lane load reads 1 KB of contiguous memory.
//   K tile: load (half h, score tile t, k-step s) lane (n, q) gets
//     K[32h + perm_key(n, t)][32s + 8q .. 32s + 8q + 7]
//     at element ((h * 2 + t) * (D / 32) + s) * 512 + (n + 16q) * 8.
//   V tile: load (half h, d-block db) lane (n, q) gets
//     V[32h + 8q .. 32h + 8q + 7][16db + n]  (eight keys of one column)
//     at element (h * (D / 16) + db) * 512 + (n + 16q) * 8.
template <int D>
__device__ __forceinline__ int k_tile_off(int key, int d) {
  const int h = key >> 5, kk = key & 31;
  const int n = 4 * (kk >> 3) + (kk & 3), t = (kk & 7) >> 2;
  const int s = d >> 5, q = (d & 31) >> 3, e = d & 7;
  return ((h * 2 + t) * (D / 32) + s) * 512 + (n + 16 * q) * 8 + e;
}
template <int D>
__device__ __forceinline__ int v_tile_off(int key, int d) {
  const int h = key >> 5, kk = key & 31;
  const int q = kk >> 3, e = kk & 7;
  const int db = d >> 4, n = d & 15;
  return (h * (D / 16) + db) * 512 + (n + 16 * q) * 8 + e;
}

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

constexpr int kLrTile = 16;  // rows per MFMA low-rank block

template <int D, int NTA>
__device__ void append_kv_tile(const AppendParams& p, int s, int blk, char* smem) {
  const skv::Span& sp = p.spans[s];
  const int pi = blk / p.Hkv, h = blk % p.Hkv;
  const int page_idx = sp.first_page + pi;
  const int page = p.ids[sp.ids_off + pi];
  const int lo = (pi == 0) ? sp.pos0 % kPage : 0;
  const int end = sp.pos0 + sp.n;
  const int hi = (page_idx == (end - 1) / kPage) ? (end - 1) % kPage + 1 : kPage;
  const int rows = hi - lo;
  const int src0 = sp.src_row + (page_idx * kPage + lo - sp.pos0);
  constexpr int VPR = D / 8;  // 16-byte vectors per row
  // K: eight consecutive d of one key stay contiguous in the tile
  u16* kdst = p.K + ((uint64_t)page * p.Hkv + h) * kPage * D;
  for (int i = threadIdx.x; i < rows * VPR; i += NTA) {
    const int rr = i / VPR, c = i % VPR;
    const u16* src = p.k + ((uint64_t)(src0 + rr) * p.Hkv + h) * D + c * 8;
    *reinterpret_cast<u32x4*>(kdst + k_tile_off<D>(lo + rr, c * 8)) = *reinterpret_cast<const u32x4*>(src);
  }
  // V: eight consecutive keys of one column are contiguous; stage the rows in
  // LDS, then write whole 8-key groups as vectors and partial groups by element
  u16* vs = reinterpret_cast<u16*>(smem);  // [64][D + 8]
  constexpr int ld = D + 8;
  for (int i = threadIdx.x; i < rows * VPR; i += NTA) {
    const int rr = i / VPR, c = i % VPR;
    const u16* src = p.v + ((uint64_t)(src0 + rr) * p.Hkv + h) * D + c * 8;
    const u32x4 val = *reinterpret_cast<const u32x4*>(src);
    u16* dst = vs + (lo + rr) * ld + c * 8;
    *reinterpret_cast<u32x2*>(dst) = u32x2{val[0], val[1]};
    *reinterpret_cast<u32x2*>(dst + 4) = u32x2{val[2], val[3]};
  }
  __syncthreads();
  u16* vdst = p.VT + ((uint64_t)page * p.Hkv + h) * D * kPage;
  const int g0 = lo >> 3, g1 = (hi + 7) >> 3;  // 8-key groups touched
  for (int i = threadIdx.x; i < (g1 - g0) * D; i += NTA) {
    const int grp = g0 + i / D, d = i % D;
    const int k0 = grp * 8;
    if (k0 >= lo && k0 + 8 <= hi) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)vs[(k0 + 2 * e) * ld + d] | ((uint32_t)vs[(k0 + 2 * e + 1) * ld + d] << 16);
      *reinterpret_cast<u32x4*>(vdst + v_tile_off<D>(k0, d)) = u32x4{w[0], w[1], w[2], w[3]};
    } else {
      for (int key = max(k0, lo); key < min(k0 + 8, hi); ++key) vdst[v_tile_off<D>(key, d)] = vs[key * ld + d];
    }
  }
}

template <int NTA>
__device__ void append_kv_block(const AppendParams& p, int s, int blk, char* smem) {
  if (p.D == 128)
    append_kv_tile<128, NTA>(p, s, blk, smem);
  else
    append_kv_tile<64, NTA>(p, s, blk, smem);
}

template <int NTA>
__device__ void append_lr_zero_block(const AppendParams& p, int s, int pi) {
  const skv::Span& sp = p.spans[s];
  const int page_idx = sp.first_page + pi;
  const int page = p.ids[sp.ids_off + pi];
  const int lo = (pi == 0) ? sp.pos0 % kPage : 0;
  const int end = sp.pos0 + sp.n;
  const int hi = (page_idx == (end - 1) / kPage) ? (end - 1) % kPage + 1 : kPage;
  u16* dst = p.LRT + sp.plane * p.lr_plane + (uint64_t)page * p.r * kPage;
  const int rows = hi - lo;
  for (int i = threadIdx.x; i < p.r * rows; i += NTA) {
    int k = i / rows, rr = i % rows;
    dst[k * kPage + lo + rr] = 0;
  }
}

// One low-rank row as a block-wide dot product, for spans of a few rows (a
// decode step appends one row per agent). Each thread takes 8 consecutive
// hidden columns at a time with 16-byte loads of x and of the matching A rows,
// so all of a thread's loads are independent and in flight together.
template <int R, int NTA, int RG = R>
__device__ void append_lr_dot_rows(const AppendParams& p, int s, int row, char* smem) {
  const skv::Span& sp = p.spans[s];
  const int H = p.hidden;
  const u16* x = p.x + (uint64_t)(sp.src_row + row) * H;
  constexpr int VG = RG >= 8 ? RG / 8 : 1;  // 16-byte vectors per A row and rank group (r = 4 reads 8 bytes)
  float* red = reinterpret_cast<float*>(smem);  // [waves][R]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // ranks in groups of RG, one pass over the columns each (every rank's sum
  // keeps the same order)
#pragma unroll
  for (int k0 = 0; k0 < R; k0 += RG) {
    float acc[RG];
#pragma unroll
    for (int k = 0; k < RG; ++k) acc[k] = 0.f;
#pragma unroll 2
    for (int u8 = threadIdx.x; u8 < H / 8; u8 += NTA) {
      const u32x4 xv = *reinterpret_cast<const u32x4*>(x + u8 * 8);
      const u16* arow = sp.a + (uint64_t)u8 * 8 * R + k0;
      u32x4 av[8][VG];
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int v = 0; v < VG; ++v) {
          if (R >= 8) {
            av[j][v] = *reinterpret_cast<const u32x4*>(arow + j * R + 8 * v);
          } else {
            u32x2 t = *reinterpret_cast<const u32x2*>(arow + j * R);
            av[j][v] = u32x4{t[0], t[1], 0u, 0u};
          }
        }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t xw = xv[j / 2];
        const float xf = __uint_as_float((j & 1) ? (xw & 0xffff0000u) : (xw << 16));
#pragma unroll
        for (int k = 0; k < RG; ++k) {
          const uint32_t aw = av[j][k / 8][(k % 8) / 2];
          acc[k] += xf * __uint_as_float((k & 1) ? (aw & 0xffff0000u) : (aw << 16));
        }
      }
    }
#pragma unroll
    for (int k = 0; k < RG; ++k) {
      float v = acc[k];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      if (lane == 0) red[w * R + k0 + k] = v;
    }
  }
  __syncthreads();
  if (threadIdx.x < R) {
    const int k = threadIdx.x;
    float v = 0.f;
    for (int ww = 0; ww < NTA / 64; ++ww) v += red[ww * R + k];
    const int pos = sp.pos0 + row;
    const int page = p.ids[sp.ids_off + pos / kPage - sp.first_page];
    p.LRT[sp.plane * p.lr_plane + (uint64_t)page * R * kPage + k * kPage + pos % kPage] = f2bf(v);
  }
}

// LEAN: rank 32 in two groups of 16 (for kernels with a tight register budget)
template <int NTA, bool LEAN = false>
__device__ void append_lr_dot_block(const AppendParams& p, int s, int row, char* smem) {
  switch (p.r) {
    case 4: append_lr_dot_rows<4, NTA>(p, s, row, smem); break;
    case 8: append_lr_dot_rows<8, NTA>(p, s, row, smem); break;
    case 16: append_lr_dot_rows<16, NTA>(p, s, row, smem); break;
    default: append_lr_dot_rows<32, NTA, LEAN ? 16 : 32>(p, s, row, smem); break;
  }
}

// Up to 16 low-rank rows with MFMA: C[row][rank] = X[row][:] . A[:][rank].
// The four waves split the hidden columns into slabs of HS 64-column sections
// (wave w takes slabs w, w + 4, ...) and keep two slabs' loads in flight: the
// slab's rows of A (a row per lane and section: NV 16-byte vectors, or 8
// bytes when NV = 0 for rank 4) and the wave's X fragments. Every load is
// unconditional, so the compiler's waits count exactly: lanes past the last
// row read the span's first row (their output rows are never stored), and a
// section past the last column reads the last one (its products are skipped).
// A wave stages each 64-column section of A transposed in its own LDS region
// (ranks padded to a multiple of 16) and reads the MFMA operand back from it;
// only its own lanes touch the region, and a wave's LDS operations complete in
// program order. The four partial tiles are added through LDS at the end.
constexpr int kLrStage = 64 + 4;  // u16 per staged rank row of a wave's region

template <int NV, int HS>
__device__ void append_lr_mfma_block(const AppendParams& p, int s, int tile, char* smem) {
  constexpr int R = NV == 0 ? 4 : 8 * NV;  // rank
  constexpr int NB = (R + 15) / 16;        // 16-rank blocks
  const skv::Span& sp = p.spans[s];
  const int H = p.hidden;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int row = tile * kLrTile + n;  // A-operand row of this lane
  const u16* xrow = p.x + (uint64_t)(sp.src_row + (row < sp.n ? row : 0)) * H;
  u16* const at = reinterpret_cast<u16*>(smem) + w * 32 * kLrStage;  // [NB*16][kLrStage]
  const int nslab = (H + 64 * HS - 1) / (64 * HS);
  const int mine = w < nslab ? (nslab - 1 - w) / 4 + 1 : 0;
  struct Slab {
    u32x4 a[HS][NV == 0 ? 1 : NV];  // [section][vector]
    bf16x8 x[2 * HS];                // [section * 2 + k-step]
  };
  auto load = [&](int i, Slab& sl) {
    const int c0 = 64 * HS * (w + 4 * i);
#pragma unroll
    for (int h = 0; h < HS; ++h) {
      const int c = min(c0 + 64 * h, H - 64);  // H is a multiple of 64
      const u16* arow = sp.a + (uint64_t)(c + lane) * R;
      if constexpr (NV == 0) {
        const u32x2 t = *reinterpret_cast<const u32x2*>(arow);
        sl.a[h][0] = u32x4{t[0], t[1], 0u, 0u};
      } else {
#pragma unroll
        for (int v = 0; v < NV; ++v) sl.a[h][v] = *reinterpret_cast<const u32x4*>(arow + 8 * v);
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) sl.x[2 * h + ks] = ld8(xrow + c + 32 * ks + 8 * q);
    }
  };
  f32x4 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0, 0, 0, 0};
  // staged rank rows the A vectors do not cover (padding up to NB*16) hold zeros
  constexpr int kCovered = NV == 0 ? 8 : 8 * NV;
#pragma unroll
  for (int k = kCovered; k < NB * 16; ++k) at[k * kLrStage + lane] = 0;
  auto compute = [&](int i, const Slab& sl) {
    const int c0 = 64 * HS * (w + 4 * i);
#pragma unroll
    for (int h = 0; h < HS; ++h) {
      if (c0 + 64 * h >= H) break;
#pragma unroll
      for (int v = 0; v < (NV == 0 ? 1 : NV); ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 8 * v + 2 * e;
          const uint32_t word = k < R ? sl.a[h][v][e] : 0u;
          at[k * kLrStage + lane] = (u16)(word & 0xffffu);
          at[(k + 1) * kLrStage + lane] = (u16)(word >> 16);
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bf16x8 ab = *reinterpret_cast<const bf16x8*>(at + (nb * 16 + n) * kLrStage + 32 * ks + 8 * q);
          acc[nb] = mfma(sl.x[2 * h + ks], ab, acc[nb]);
        }
      // the next section's transposed writes follow these reads in program order
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  };
  if (mine > 0) {
    Slab A, Bf;
    load(0, A);
    int i = 0;
    // sched_barrier keeps each prefetch ahead of the wait for the slab in use
    for (; i + 2 < mine; i += 2) {
      load(i + 1, Bf);
      __builtin_amdgcn_sched_barrier(0);
      compute(i, A);
      load(i + 2, A);
      __builtin_amdgcn_sched_barrier(0);
      compute(i + 1, Bf);
    }
    if (mine - i == 2) {
      load(i + 1, Bf);
      __builtin_amdgcn_sched_barrier(0);
      compute(i, A);
      compute(i + 1, Bf);
    } else {
      compute(i, A);
    }
  }
  // waves 1..3 hand their partial tiles to wave 0 (added in wave order)
  __syncthreads();  // every wave is done with its staging region
  float* const red = reinterpret_cast<float*>(smem);  // [3][64 lanes][8]
  if (w > 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<f32x4*>(red + ((w - 1) * 64 + lane) * 8 + 4 * nb) = acc[nb];
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int ww = 0; ww < 3; ++ww)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] += *reinterpret_cast<const f32x4*>(red + (ww * 64 + lane) * 8 + 4 * nb);
  // C tile: lane holds rank 16nb + n, rows 4q + j of the tile
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int k = nb * 16 + n;
    if (k < R) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = tile * kLrTile + 4 * q + j;
        if (rr < sp.n) {
          const int pos = sp.pos0 + rr;
          const int page = p.ids[sp.ids_off + pos / kPage - sp.first_page];
          p.LRT[sp.plane * p.lr_plane + (uint64_t)page * R * kPage + k * kPage + pos % kPage] =
              f2bf(acc[nb][j]);
        }
      }
    }
  }
}

// Work of block b of an append job (block 0 also writes the new page-table
// entries). smem must hold at least 64 * (128 + 8) bf16. KV and MFMA_LR say
// whether the kernel carries the K/V tile copies and the MFMA low-rank tiles:
// launches whose jobs never hold such blocks leave that code out, which keeps
// them small (the host checks the jobs it gives them). NTA threads of the
// block run it (the first NTA; the MFMA low-rank tiles take four waves). HS:
// 64-column sections per slab of the MFMA low-rank tiles at ranks up to 16
// (2 for kernels with a tight register budget, whose dot-product rows then
// take rank 32 in two passes).
// KV / LR: compile the K/V copies / the low-rank rows (a launch whose jobs
// never carry one leaves its code, and its registers, out).
template <bool KV = true, bool MFMA_LR = true, int NTA = 256, int HS = 4, bool LR = true>
__device__ void append_block(const AppendParams& p, int b, char* smem) {
  static_assert(!MFMA_LR || NTA == 256, "the MFMA low-rank tiles are written for four waves");
  if (b == 0 && p.update_tables) {
    for (int s = 0; s < p.n_spans; ++s) {
      const skv::Span& sp = p.spans[s];
      int32_t* t = p.tbl + sp.seq_slot * p.tbl_seq + sp.first_page;
      for (int i = threadIdx.x; i < sp.n_pages; i += NTA) t[i] = p.ids[sp.ids_off + i];
    }
  }
  const int n_kv = p.kv_block0[p.n_spans];
  if (b >= n_kv + p.lr_block0[p.n_spans]) return;
  if (b < n_kv) {
    if constexpr (KV) {
      int s = 0;
      while (b >= p.kv_block0[s + 1]) ++s;
      append_kv_block<NTA>(p, s, b - p.kv_block0[s], smem);
    }
    return;
  }
  if constexpr (!LR) return;
  b -= n_kv;
  int s = 0;
  while (b >= p.lr_block0[s + 1]) ++s;
  const int sub = b - p.lr_block0[s];
  if (p.lr_kind[s] == 0)
    append_lr_zero_block<NTA>(p, s, sub);
  else if (p.lr_kind[s] == 1)
    append_lr_dot_block<NTA, HS == 2>(p, s, sub, smem);
  else if constexpr (MFMA_LR) {
    if (p.r == 4)
      append_lr_mfma_block<0, HS>(p, s, sub, smem);
    else if (p.r == 8)
      append_lr_mfma_block<1, HS>(p, s, sub, smem);
    else if (p.r == 16)
      append_lr_mfma_block<2, HS>(p, s, sub, smem);
    else
      append_lr_mfma_block<4, 2>(p, s, sub, smem);
  }
}

__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  __shared__ __attribute__((aligned(16))) char smem[64 * (128 + 8) * 2];
  append_block(p, blockIdx.x, smem);
}

// Block counts of an append job, per span: K/V tiles and low-rank blocks.
void plan_append(const skv::Geometry& g, const skv::AppendJob& job, AppendParams& p) {
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
  memcpy(p.spans, job.spans, sizeof(skv::Span) * job.n_spans);
  memcpy(p.ids, job.ids, sizeof(int32_t) * job.n_ids);
  p.kv_block0[0] = 0;
  p.lr_block0[0] = 0;
  for (int s = 0; s < job.n_spans; ++s) {
    const skv::Span& sp = job.spans[s];
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
}

int append_blocks(const AppendParams& p) {
  return p.kv_block0[p.n_spans] + p.lr_block0[p.n_spans];
}

// ---------------------------------------------------------------------------
// Decode: split pass
// ---------------------------------------------------------------------------

// Decode work is cut from one flattened key sequence per KV head: the shared
// prefix [0, max_b), then each listed agent's own suffix, every segment padded
// to a multiple of 32 keys. Equal slices of it ("items") go to workgroups, so
// the grid is balanced whatever the mix of shared and own keys. Each item
// streams its chunks once for all query rows of the group; a row only takes
// keys of its own view (shared keys below its b_i, its own suffix keys).
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
  int ag_lrb[SKV_MAX_AGENTS];     // adapter activation offset (view position)
  int lr_offsets;                 // some agent of the group has a nonzero offset
  int n_planes;
  int planes[SKV_MAX_AGENTS];     // stacked low-rank planes of this group
  int seg_off[SKV_MAX_AGENTS + 1];  // flattened offset of each own suffix; seg_off[n] = total
  int shared_len;                 // flattened length of the shared segment (max_b padded)
  int shared_run;                 // first id of the shared pages when they are consecutive, else -1
  int head_chunks;     // C: 32-key chunks of one head's flattened sequence
  int items_per_head;  // I: item j takes chunks [j C / I, (j + 1) C / I)
  float scale_log2;
  int n_app;        // leading blocks that write the step's low-rank rows and table entries
  AppendParams app;
};

// LDS slots of wave state the split pass's fold uses: one per wave where they
// fit (one fold stage), else two (pairwise folds).
template <int D, int RB, int MB>
constexpr int split_fold_slots() {
  constexpr int slot = RB * ((D / 16 + MB) * 64 * 16 + 2 * 64 * 4);
  return 4 * slot <= 128 * 1024 ? 4 : 2;
}

template <int D, int RB, int MB>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p) {
  constexpr int KS = D / 32, DB = D / 16;
  __shared__ int32_t s_cpage[kMaxItemChunks];   // page id of each chunk of the item
  __shared__ int32_t s_ckey[kMaxItemChunks];    // (segment << 24) | first key of the chunk in its segment
  extern __shared__ __attribute__((aligned(16))) float s_buf[];  // the waves' states (fold), or append staging

  if ((int)blockIdx.x < p.n_app) {
    // fused decode step: write the new low-rank rows and page-table entries;
    // the items below read only keys cached before this step
    append_block<false, false>(p.app, blockIdx.x, reinterpret_cast<char*>(s_buf));
    return;
  }
  const int item = blockIdx.x - p.n_app;
  const int g = item / p.items_per_head;
  const int j = item % p.items_per_head;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, q = lane >> 4;
  const int c_lo = (int)((int64_t)j * p.head_chunks / p.items_per_head);
  const int c_hi = (int)((int64_t)(j + 1) * p.head_chunks / p.items_per_head);
  const int f0 = 32 * c_lo;
  const int n_ck = c_hi - c_lo;

  // chunk descriptors: segment (0 = shared, 1 + a = agent a's suffix), first key,
  // page. Shared pages whose ids run consecutively need no table read, which
  // would otherwise sit in front of the item's first chunk loads.
  for (int c = threadIdx.x; c < n_ck; c += blockDim.x) {
    const int fc = f0 + 32 * c;
    int seg = 0, key0 = fc;
    if (fc >= p.shared_len) {
      int a = 0;
      while (fc >= p.seg_off[a + 1]) ++a;
      seg = 1 + a;
      key0 = fc - p.seg_off[a];
    }
    int page;
    if (seg == 0 && p.shared_run >= 0) {
      page = p.shared_run + key0 / kPage;
    } else {
      const int32_t* table = p.tbl + (seg == 0 ? 0 : 1 + p.ag_id[seg - 1]) * p.tbl_seq;
      page = table[key0 / kPage];
    }
    s_cpage[c] = page;
    s_ckey[c] = (seg << 24) | key0;
  }

  // Low-rank A-operand row of this lane in block mb: stacked row sr = 16mb + n
  // is rank sr % r of plane sr / r. For an own-suffix chunk the other agents'
  // planes hold don't-care rows: their products only reach rows that are
  // masked out for that chunk, or stacked entries a row never keeps. A lane
  // past the last plane reads a valid row and masks it to zero. Set up before
  // the query loads: the first chunk loads need these addresses, and the wait
  // for them must not include the query loads.
  uint32_t lr_mask[MB];
  const u16* lr_row[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int sr = mb * 16 + n;
    const int pi = sr / p.r, k = sr % p.r;
    const bool ok = pi < p.n_planes;
    lr_mask[mb] = ok ? 0xffffffffu : 0u;
    lr_row[mb] = p.LRT + (uint64_t)p.planes[ok ? pi : 0] * p.lr_plane + (ok ? k : 0) * kPage;
  }
  // per-lane query rows: Q^T B-operand slices, agent and base length of the row
  bf16x8 qf[RB][KS];
  int row_agent[RB], row_b[RB], row_S[RB], row_lrb[RB];
  // Every load here is unconditional (a padding lane reads agent 0's row and
  // drops it): loads under a divergent condition would leave the compiler's
  // count of loads in flight unknown at the join, and the first chunk loads
  // would then wait for all of them.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int rho = rb * 16 + n;
    const bool ok = rho < p.R;
    const int a = ok ? rho / p.G : 0;
    const int b_a = p.ag_b[a], S_a = p.ag_S[a], lrb_a = p.ag_lrb[a];
    row_agent[rb] = ok ? a : -1;
    row_b[rb] = ok ? b_a : 0;
    row_S[rb] = ok ? S_a : 0;
    row_lrb[rb] = ok ? lrb_a : 0;
    const u16* qp = p.q + ((uint64_t)a * p.Hq + g * p.G + (ok ? rho % p.G : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 v = ld8(qp + 32 * s + 8 * q);
      qf[rb][s] = ok ? v : zero8();
    }
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
  // the chunk table is in LDS; the query loads stay in flight (a full
  // workgroup fence here would hold the first chunk loads behind them)
  stage_barrier<kWaitLdsOnly>();

  const uint64_t head_off = (uint64_t)g * kPage * D;  // offset of head g inside a page
  const uint64_t page_elems = (uint64_t)p.Hkv * kPage * D;

  // Two 32-key chunk buffers per wave (one for 64 query rows, below): the loop
  // is unrolled by two so the buffers never need copying, and every prefetch
  // is unconditional (the tail is peeled), so the compiler keeps the next
  // chunk's loads in flight while the current chunk is consumed. K and V^T are
  // streamed once, so their loads are non-temporal.
  struct Chunk {
    bf16x8 k[2][KS], v[DB];
    u32x4 l[MB];  // raw low-rank rows; the lane mask is applied where they are used
  };
  auto load = [&](int c, Chunk& ch) {
    const int page = s_cpage[c];
    const int half = ((s_ckey[c] & 0xffffff) % kPage) / 32;
    const u16* kp = p.K + (uint64_t)page * page_elems + head_off + half * (2 * KS * 512) + lane * 8;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int s = 0; s < KS; ++s) ch.k[t][s] = ld8_nt(kp + (t * KS + s) * 512);
    const u16* vp = p.VT + (uint64_t)page * page_elems + head_off + half * (DB * 512) + lane * 8;
#pragma unroll
    for (int db = 0; db < DB; ++db) ch.v[db] = ld8_nt(vp + db * 512);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      ch.l[mb] = *reinterpret_cast<const u32x4*>(lr_row[mb] + (uint64_t)page * p.r * kPage +
                                                 half * 32 + 8 * q);
  };
  auto compute = [&](int c, const Chunk& ch) {
    const int meta = s_ckey[c];
    const int seg = meta >> 24, key0 = meta & 0xffffff;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      // keys of this chunk visible to the lane's row: shared keys below b_i,
      // or the row's own agent's suffix keys
      const int lim = seg == 0 ? row_b[rb] : (row_agent[rb] == seg - 1 ? row_S[rb] : 0);
      f32x4 s0 = {0, 0, 0, 0}, s1 = {0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        s0 = mfma(ch.k[0][s], qf[rb][s], s0);
        s1 = mfma(ch.k[1][s], qf[rb][s], s1);
      }
      float sc[8];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int kA = key0 + 8 * q + jj, kB = kA + 4;
        sc[jj] = kA < lim ? s0[jj] * p.scale_log2 : -INFINITY;
        sc[jj + 4] = kB < lim ? s1[jj] * p.scale_log2 : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[i]);
      mx = xmax16_32(mx);
      const float m_new = fmaxf(m_run[rb], mx);
      float pv[8], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sc[i] - m_new);
        ps += pv[i];
      }
      // rescale the accumulators only when some row's running max grew
      // (rare once the maxima settle); otherwise the scale factor is 1
      if (__any(m_new > m_run[rb])) {
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) lacc[rb][mb] *= alpha;
        m_run[rb] = m_new;
      }
      l_run[rb] += ps;
      const bf16x8 pt = pack8(pv);
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[rb][db] = mfma(ch.v[db], pt, oacc[rb][db]);
      // keys of the lane's eight that lie before its row's adapter activation
      // (view position: the shared key, or b_i + own key) take no low-rank term
      bf16x8 ptl = pt;
      if (p.lr_offsets) {
        const int nm = row_lrb[rb] - (seg == 0 ? 0 : row_b[rb]) - key0 - 8 * q;
        if (__any(nm > 0)) ptl = zero_leading(pt, nm);
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        lacc[rb][mb] = mfma(__builtin_bit_cast(bf16x8, ch.l[mb] & lr_mask[mb]), ptl, lacc[rb][mb]);
    }
  };
  const int n_chunks = w < n_ck ? (n_ck - w + 3) / 4 : 0;  // this wave's chunks: w, w + 4, ...
  if constexpr (RB >= 4) {
    // 64 query rows: their accumulators leave no registers for a second chunk
    // buffer, so each chunk is loaded, then used
    Chunk A;
    for (int i = 0; i < n_chunks; ++i) {
      load(w + 4 * i, A);
      __builtin_amdgcn_sched_barrier(0);
      compute(w + 4 * i, A);
    }
  } else if (n_chunks > 0) {
    Chunk A, Bf;
    load(w, A);
    int i = 0;
    // sched_barrier keeps each prefetch ahead of the wait for the buffer in use
    for (; i + 2 < n_chunks; i += 2) {
      load(w + 4 * (i + 1), Bf);
      __builtin_amdgcn_sched_barrier(0);
      compute(w + 4 * i, A);
      load(w + 4 * (i + 2), A);
      __builtin_amdgcn_sched_barrier(0);
      compute(w + 4 * (i + 1), Bf);
    }
    if (n_chunks - i == 2) {
      load(w + 4 * (i + 1), Bf);
      __builtin_amdgcn_sched_barrier(0);
      compute(w + 4 * i, A);
      compute(w + 4 * (i + 1), Bf);
    } else {
      compute(w + 4 * i, A);
    }
  }

  // Fold the four waves' states through LDS and write the item's partial rows
  // (o, o_lr, m, l) for the merge. Each lane exchanges exactly the accumulator
  // quads it holds (MFMA layout), so slots are written and read conflict-free.
  //  - one stage, where a slot per wave fits in LDS: every wave puts its state,
  //    then wave w combines quads w, w + 4, ... of the four slots, each slot
  //    weighted by 2^(m_s - M) with M the largest of the slots' maxima, and
  //    stores them; wave 0 also writes each row's m and l;
  //  - else pairwise (waves 2 and 3 into 0 and 1, then 1 into 0), and wave 0
  //    writes the rows.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) l_run[rb] = xsum16_32(l_run[rb]);
  constexpr int NQ = DB + MB;  // accumulator quads per lane and row block
  constexpr int NS = split_fold_slots<D, RB, MB>();
  f32x4* const s_st = reinterpret_cast<f32x4*>(s_buf);                   // [NS][RB][NQ][64]
  float* const s_ml = reinterpret_cast<float*>(s_st + NS * RB * NQ * 64);  // [NS][RB][2][64]
  auto put = [&](int slot) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4* const st = s_st + (slot * RB + rb) * NQ * 64 + lane;
#pragma unroll
      for (int db = 0; db < DB; ++db) st[db * 64] = oacc[rb][db];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) st[(DB + mb) * 64] = lacc[rb][mb];
      s_ml[((slot * RB + rb) * 2) * 64 + lane] = m_run[rb];
      s_ml[((slot * RB + rb) * 2 + 1) * 64 + lane] = l_run[rb];
    }
  };
  const int W = p.W;
  float* const dst = p.part + (uint64_t)item * p.R * W;
  // the stacked low-rank entries of quad j (j >= DB) that belong to the row's own plane
  auto put_lr = [&](float* row, int rho, int j, const f32x4& v) {
    const int pidx = p.ag_pidx[rho / p.G];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int sr = (j - DB) * 16 + 4 * q + jj;
      if (sr / p.r == pidx) row[D + sr % p.r] = v[jj];
    }
  };
  if constexpr (NS == 4) {
    put(w);
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rho = rb * 16 + n;
      float ms[4], ws[4];
      float M = -INFINITY;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        ms[sl] = s_ml[((sl * RB + rb) * 2) * 64 + lane];
        M = fmaxf(M, ms[sl]);
      }
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) ws[sl] = __builtin_amdgcn_exp2f(ms[sl] - M);
      if (rho >= p.R) continue;
      float* const row = dst + rho * W;
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        if ((j & 3) != w) continue;
        f32x4 acc = s_st[rb * NQ * 64 + j * 64 + lane] * ws[0];
#pragma unroll
        for (int sl = 1; sl < 4; ++sl) acc += s_st[(sl * RB + rb) * NQ * 64 + j * 64 + lane] * ws[sl];
        if (j < DB)
          *reinterpret_cast<f32x4*>(row + j * 16 + 4 * q) = acc;
        else
          put_lr(row, rho, j, acc);
      }
      if (w == 0 && q == 0) {
        float l = 0.f;
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) l += s_ml[((sl * RB + rb) * 2 + 1) * 64 + lane] * ws[sl];
        row[D + p.r] = M;
        row[D + p.r + 1] = l;
      }
    }
  } else {
    auto fold = [&](int slot) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const f32x4* const st = s_st + (slot * RB + rb) * NQ * 64 + lane;
        const float mo = s_ml[((slot * RB + rb) * 2) * 64 + lane];
        const float lo = s_ml[((slot * RB + rb) * 2 + 1) * 64 + lane];
        const float mc = fmaxf(m_run[rb], mo);
        const float a = __builtin_amdgcn_exp2f(m_run[rb] - mc), b = __builtin_amdgcn_exp2f(mo - mc);
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[rb][db] = oacc[rb][db] * a + st[db * 64] * b;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) lacc[rb][mb] = lacc[rb][mb] * a + st[(DB + mb) * 64] * b;
        l_run[rb] = l_run[rb] * a + lo * b;
        m_run[rb] = mc;
      }
    };
    if (w >= 2) put(w - 2);
    __syncthreads();
    if (w < 2) fold(w);
    if (w == 1) put(1);
    __syncthreads();
    if (w != 0) return;
    fold(1);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int rho = rb * 16 + n;
      if (rho >= p.R) continue;
      float* const row = dst + rho * W;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(row + db * 16 + 4 * q) = oacc[rb][db];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) put_lr(row, rho, DB + mb, lacc[rb][mb]);
      if (q == 0) {
        row[D + p.r] = m_run[rb];
        row[D + p.r + 1] = l_run[rb];
      }
    }
  }
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
  int items_per_head;
  // fused decode step: each agent's new token enters as one more softmax term
  int step;
  const u16* q;       // [n][Hq][D] of this group
  const u16* k_new;   // [n][Hkv][D] of this group
  const u16* v_new;   // [n][Hkv][D] of this group
  const u16* LRT;     // layer base of plane 0 (holds the new low-rank rows)
  uint64_t lr_plane;
  int new_page[SKV_MAX_AGENTS], new_slot[SKV_MAX_AGENTS], plane[SKV_MAX_AGENTS];
  int new_lr_on[SKV_MAX_AGENTS];  // the new token lies at or after the agent's adapter activation
  float scale_log2;
  int n_rows;       // leading blocks merge rows; the n_app after them copy the new K/V rows
  int n_app;
  AppendParams app;
};

// One workgroup per query row (agent, query head). Merges the row's partial
// softmax states from every item of its KV head: M = max m_s, weights
// w_s = 2^(m_s - M) / sum_s 2^(m_s - M) l_s, o = sum_s w_s o_s and
// o_lr = sum_s w_s o_lr,s (a fused step adds the new token's own term);
// then applies B_i once: o[d] += sum_k o_lr[k] B_i[k][g*D + d], in bf16.
// Every global load of the row (partial rows, the B_i slice, the new token)
// is issued up front and unconditionally, with indices past the end clamped
// and their terms dropped, so the row waits on memory once; B_i is staged in
// LDS for the final product.
constexpr int kMergeVec = 8;  // slots per thread held in registers

// NT threads per row: 256, or 1024 when the row has more slots than 256
// threads hold in one batch (few KV heads: many items per head), so that four
// times the loads are in flight.
template <int D, int NT>
__global__ __launch_bounds__(NT) void decode_merge_kernel(MergeParams p) {
  constexpr int kGroups = NT / 32;  // slot groups at most (an element quad row has >= 17 quads)
  extern __shared__ __attribute__((aligned(16))) char s_app[];  // append blocks' staging
  if ((int)blockIdx.x >= p.n_rows) {
    // fused decode step: copy the new K/V rows into the pages; the rows merged
    // here take the new token from the step's inputs instead
    append_block<true, false, NT, 4, false>(p.app, blockIdx.x - p.n_rows, s_app);
    return;
  }
  __shared__ float s_w[kMaxMergeSlots];
  __shared__ f32x4 s_red[kGroups][40];
  __shared__ float s_v[128 + 32];
  __shared__ float s_sm[40];  // maxima [NT/64], sums [NT/64], new score
  __shared__ u32x4 s_b[32 * 128 / 8];  // B_i slice [r][D] bf16
  const int row_id = blockIdx.x;
  const int hh = row_id % p.G;
  const int g = (row_id / p.G) % p.Hkv;
  const int a = row_id / (p.G * p.Hkv);
  const int rho = a * p.G + hh;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int I = p.items_per_head, W = p.W, r = p.r;
  const int E = D + r;
  auto slot_row = [&](int s) { return p.part + ((uint64_t)(g * I + s) * p.R + rho) * W; };
  // --- loads: per-slot (m, l), this thread's element quads, B_i, the new token
  const int ts = max(min(t, I - 1), 0);
  float m_ld = 0.f, l_ld = 0.f;
  const int NQ = E / 4;
  const int NG = min(kGroups, NT / NQ);
  const int qd = t % NQ, sg = min(t / NQ, NG - 1);
  const bool quad_thread = t < NQ * NG;
  f32x4 vals[kMergeVec];
  if (I > 0) {  // uniform: no slots when nothing was cached before a fused step
    m_ld = slot_row(ts)[E];
    l_ld = slot_row(ts)[E + 1];
#pragma unroll
    for (int i = 0; i < kMergeVec; ++i)
      vals[i] = *reinterpret_cast<const f32x4*>(slot_row(min(sg + i * NG, I - 1)) + 4 * qd);
  }
  const int HD = p.Hkv * D;
  constexpr int BV = D / 8;  // 16-byte vectors per B_i row slice
  const u16* bsl = p.B + (uint64_t)p.ag_id[a] * r * HD + g * D;
  constexpr int NBV = (32 * BV + NT - 1) / NT;  // B_i vectors per thread (rank up to 32)
  u32x4 bvec[NBV];
#pragma unroll
  for (int i = 0; i < NBV; ++i) {
    const int v = min(t + NT * i, r * BV - 1);
    bvec[i] = *reinterpret_cast<const u32x4*>(bsl + (uint64_t)(v / BV) * HD + 8 * (v % BV));
  }
  float dot = 0.f, nv = 0.f;
  if (p.step) {
    // the new token's score q . k_new (two elements per lane of wave 0) and its
    // value element t (its v row, then its low-rank row)
    const u16* qr = p.q + ((uint64_t)a * p.Hq + g * p.G + hh) * D;
    const u16* kr = p.k_new + ((uint64_t)a * p.Hkv + g) * D;
    const int dl = (2 * lane) % D;
    const uint32_t qw = *reinterpret_cast<const uint32_t*>(qr + dl), kw = *reinterpret_cast<const uint32_t*>(kr + dl);
    const float vv = bf2f(p.v_new[((uint64_t)a * p.Hkv + g) * D + min(t, D - 1)]);
    const float lv = bf2f(p.LRT[(uint64_t)p.plane[a] * p.lr_plane + (uint64_t)p.new_page[a] * r * kPage +
                                min(max(t - D, 0), r - 1) * kPage + p.new_slot[a]]);
    if (2 * lane < D)
      dot = __uint_as_float(qw << 16) * __uint_as_float(kw << 16) +
            __uint_as_float(qw & 0xffff0000u) * __uint_as_float(kw & 0xffff0000u);
    nv = t < D ? vv : (t < E && p.new_lr_on[a] ? lv : 0.f);
  }
  // --- softmax statistics
  constexpr int NWV = NT / 64;  // waves
  const float m_s = t < I ? m_ld : -1e30f, l_s = t < I ? l_ld : 0.f;
  float M = wave_max(m_s);
  if (p.step && w == 0) {
    dot = wave_sum(dot);
    if (lane == 0) s_sm[2 * NWV] = dot * p.scale_log2;
  }
  if (lane == 0) s_sm[w] = M;
#pragma unroll
  for (int i = 0; i < NBV; ++i)
    if (t + NT * i < r * BV) s_b[t + NT * i] = bvec[i];
  __syncthreads();
  const float m_new = p.step ? s_sm[2 * NWV] : -1e30f;
  M = m_new;
#pragma unroll
  for (int i = 0; i < NWV; ++i) M = fmaxf(M, s_sm[i]);
  // slots beyond the first blockDim.x are folded in below through s_w
  const float e_s = t < I ? __builtin_amdgcn_exp2f(m_s - M) : 0.f;
  if (t < I) s_w[t] = e_s;
  float L = e_s * l_s;
  for (int s = t + blockDim.x; s < I; s += blockDim.x) {
    const float e = __builtin_amdgcn_exp2f(slot_row(s)[E] - M);
    s_w[s] = e;
    L += e * slot_row(s)[E + 1];
  }
  L = wave_sum(L);
  if (lane == 0) s_sm[NWV + w] = L;
  __syncthreads();
  const float e_new = p.step ? __builtin_amdgcn_exp2f(m_new - M) : 0.f;
  float den = e_new;
#pragma unroll
  for (int i = 0; i < NWV; ++i) den += s_sm[NWV + i];
  const float inv = 1.f / den;
  // --- weighted sums: element quads x slot groups
  if (quad_thread) {
    f32x4 acc = {0, 0, 0, 0};
    if (I > 0) {
#pragma unroll
      for (int i = 0; i < kMergeVec; ++i) {
        const int s = sg + i * NG;
        acc += (s < I ? s_w[s] : 0.f) * vals[i];
      }
    }
    for (int s = sg + kMergeVec * NG; s < I; s += NG) acc += s_w[s] * *reinterpret_cast<const f32x4*>(slot_row(s) + 4 * qd);
    s_red[sg][qd] = acc;
  }
  __syncthreads();
  if (t < E) {
    float acc = 0.f;
    for (int gg = 0; gg < NG; ++gg) acc += s_red[gg][t / 4][t % 4];
    s_v[t] = (acc + e_new * nv) * inv;
  }
  __syncthreads();
  if (t < D) {
    const u16* bl = reinterpret_cast<const u16*>(s_b);
    float out = s_v[t];
    for (int k = 0; k < r; ++k) out += s_v[D + k] * bf2f(bl[k * D + t]);
    p.o[((uint64_t)a * p.Hq + g * p.G + hh) * D + t] = f2bf(out);
  }
}

// ---------------------------------------------------------------------------
// Prefill
// ---------------------------------------------------------------------------

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
  int ag_lrb[SKV_MAX_AGENTS];    // adapter activation offset (view position)
  int blk0[SKV_MAX_AGENTS + 1];  // prefix sums of query blocks per agent
  float scale_log2;
  // key-range split: workgroup w takes block w % nblk and the range w / nblk
  // of its pages; with ksplit > 1 it writes partial rows (W floats: o, o_lr,
  // m, l) to part for the merge instead of the output
  int ksplit, nblk, W;
  float* part;
};

// LDS image of one page of one KV head: the K tile and the V^T tile (64 x D
// each, in operand order) and the page's low-rank rows (up to 32 ranks x 64
// keys, in operand order).
template <int D>
constexpr int prefill_page_elems() { return 2 * 64 * D + 32 * 64; }

// Copy one 1 KB operand block into LDS with a buffer load that writes LDS:
// every lane moves 16 bytes from byte offset off + 16 lane of the buffer,
// landing at dst + 16 lane (the data of a wave is placed contiguously from the
// LDS base it is given). Reads past the buffer's size return zeros. A buffer
// load counts only in the vector-memory counter, so waits for LDS reads that
// follow it stay exact.
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit records
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRsrcWord3);
}
__device__ __forceinline__ void dma_block(__amdgpu_buffer_rsrc_t r, int off, u16* dst_wave, int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)dst_wave, 16, off + lane * 16,
                                           0, 0, 0);
}
// The same with each lane's own source offset (a gather into the wave's
// contiguous 1 KB of LDS).
__device__ __forceinline__ void dma_lanes(__amdgpu_buffer_rsrc_t r, int off_lane, u16* dst_wave) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3)))*)dst_wave, 16, off_lane, 0, 0,
                                           0);
}

// LDS (address space 3) views of the page ring: 32-bit addresses, so a read's
// constant offset goes into the instruction's offset field.
typedef __attribute__((address_space(3))) const u16 lds_u16;
typedef __attribute__((address_space(3))) const bf16x8 lds_frag;

// Suffix prefill: a workgroup of NW waves takes 16 NW RB query rows (rows =
// query position x query head of one KV head) and streams the view's pages once: each page's K,
// V^T and low-rank rows are copied to LDS by the whole workgroup through a ring
// of three buffers (the copies of the next two pages run during this page's
// compute), and every wave reads the MFMA operands of its 16 RB rows from LDS,
// so one K/V tile read serves RB row blocks. Scores stay in registers as in
// decode (S^T = K Q^T with permuted K rows); causal and segment masks are
// applied per key, except on 32-key halves every row of the wave sees whole.
template <int D, int MB, int RB, int NW, bool LRO>
__global__ __launch_bounds__(64 * NW) void prefill_kernel(PrefillParams p) {
  constexpr int KS = D / 32, DB = D / 16;
  constexpr int ROWS = NW * 16 * RB;
  constexpr int PE = prefill_page_elems<D>();
  constexpr int KB = D / 8 / NW;  // 1 KB blocks of a K (or V^T) page tile each wave copies
  static_assert(KB * NW * 8 == D, "page tile blocks must split evenly over the waves");
  extern __shared__ __attribute__((aligned(16))) u16 s_kv[];  // [3][PE]
  __shared__ int32_t s_pages[kMaxViewPages];
  __shared__ float s_lr[NW][16][33];
  // This lane's address in page buffer buf (elements lane_elems past its
  // start), formed with one add and hidden from the optimiser by an empty asm:
  // every operand read below is this address plus a constant the read
  // encodes. Left visible, the compiler kept an address register per fragment
  // and spent two adds on every read.
  auto lane_ptr = [&](int buf, int lane_elems) {
    lds_u16* ptr = (lds_u16*)(s_kv + buf * PE) + lane_elems;
    asm volatile("" : "+v"(ptr));
    return ptr;
  };
  const int split = blockIdx.x / p.nblk;
  const int bid = blockIdx.x % p.nblk;  // blocks of one KV head share blockIdx mod Hkv (and an XCD)
  const int g = bid % p.Hkv;
  int qb = bid / p.Hkv;
  int ai = 0;
  while (qb >= p.blk0[ai + 1]) ++ai;
  qb -= p.blk0[ai];
  const int b = p.ag_b[ai], S = p.ag_S[ai], nq = p.ag_nq[ai];
  const int Lv = b + S;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, q = lane >> 4;
  const int rows_total = nq * p.G;
  const int row_blk0 = qb * ROWS;
  // highest view position among this block's rows
  const int last_row = min(row_blk0 + ROWS, rows_total) - 1;
  const int t_max = Lv - nq + last_row / p.G;

  const int np_sh = (min(b, t_max + 1) + kPage - 1) / kPage;
  const int own_keys = max(0, min(S, t_max + 1 - b));
  const int np_own = (own_keys + kPage - 1) / kPage;
  // this workgroup's pages [p_lo, p_hi) of the block's view; below, page
  // indices are local to the range (p_lo + i is the view's page)
  const int p_lo = (int)((int64_t)split * (np_sh + np_own) / p.ksplit);
  const int p_hi = (int)((int64_t)(split + 1) * (np_sh + np_own) / p.ksplit);
  const int n_pages = p_hi - p_lo;
  const int32_t* tsh = p.tbl;
  const int32_t* tow = p.tbl + (1 + p.ag_id[ai]) * p.tbl_seq;
  for (int i = threadIdx.x; i < n_pages; i += blockDim.x)
    s_pages[i] = p_lo + i < np_sh ? tsh[p_lo + i] : tow[p_lo + i - np_sh];

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
  const u16* lrb = p.LRT + (uint64_t)p.ag_plane[ai] * p.lr_plane;
  // lowest view position among the wave's valid rows: a key at or below it is
  // visible to all of them
  int tmin = 0x7fffffff;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
    if (tpos[rb] >= 0) tmin = min(tmin, tpos[rb]);
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) tmin = min(tmin, __shfl_xor(tmin, o));
  tmin = __builtin_amdgcn_readfirstlane(tmin);
  // Low-rank A-operand rows: stacked row k = 16 mb + n holds rank k when
  // k < r. With r < 16 the row k = r is all bf16 ones, so its accumulator
  // entry collects each query row's softmax denominator from the same bf16 P.
  const bool ones_row = p.r < 16;
  // The score scale in a VGPR, read here once: a value the compiler would
  // reload from the kernel arguments inside the page loop would leave a
  // scalar load in flight there, and every LDS wait would then count to zero.
  float scale_log2 = p.scale_log2;
  asm volatile("" : "+v"(scale_log2));
  uint32_t lr_mask[MB];
  u32x4 lr_ones[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    lr_mask[mb] = mb * 16 + n < p.r ? 0xffffffffu : 0u;
    const uint32_t one = ones_row && mb * 16 + n == p.r ? 0x3f803f80u : 0u;
    lr_ones[mb] = u32x4{one, one, one, one};
  }
  // A page's low-rank rows sit in LDS in operand order, RP = 16 MB ranks
  // (the ranks past r hold zeros): 16-byte slot h 4RP + q RP + k holds rank k,
  // keys 32h + 8q .. 32h + 8q + 7, so the sixteen lanes of one q read
  // consecutive slots. (Rank rows 128 bytes apart, as in the cache, put eight
  // ranks on two groups of banks.) This lane's operand of block mb: rank
  // 16 mb + n (lanes past the last rank read the last one; masked above),
  // half h at a constant 4RP slots further.
  constexpr int RP = 16 * MB;
  int lr_elems[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) lr_elems[mb] = 2 * 64 * D + 8 * (q * RP + min(mb * 16 + n, p.r - 1));
  auto lr_lane = [&](int mb, int buf) { return lane_ptr(buf, lr_elems[mb]); };

  // With LRO (some agent has an adapter activation offset), the low-rank rows
  // of keys before the agent's offset are masked out of the A operand; the
  // ones row is added after the mask, so the denominators still see every key.
  // lr_keep(i, h): mask of the lane's eight keys of page i, half h.
  const int lr_on_at = p.ag_lrb[ai];
  auto lr_keep = [&](int i, int h) -> u32x4 {
    const int ia = p_lo + i;
    const int pstart = ia >= np_sh ? b + (ia - np_sh) * kPage : ia * kPage;  // view position of the page
    const int nm = lr_on_at - (pstart + 32 * h + 8 * q);
    u32x4 m;
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = (2 * k < nm ? 0u : 0x0000ffffu) | (2 * k + 1 < nm ? 0u : 0xffff0000u);
    return m;
  };
  u32x4 keep_lr[2] = {u32x4{~0u, ~0u, ~0u, ~0u}, u32x4{~0u, ~0u, ~0u, ~0u}};

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
  __syncthreads();  // s_pages

  const uint64_t head_off = (uint64_t)g * kPage * D;
  const uint64_t page_elems = (uint64_t)p.Hkv * kPage * D;
  // Page copies into LDS are issued by the first wave group (waves [0, NW/2)):
  // each of its waves moves KC of the K tile's 1 KB blocks, as many of the
  // V^T tile's, and the low-rank block w (waves past the block count repeat
  // block 0, the same bytes to the same place). A low-rank block is 64 slots
  // of the operand order above: each lane fetches the 16 bytes of its slot
  // from the page's rank rows (offset k 128 + 64 h + 16 q); ranks past r lie
  // past the page's rows and land as zeros.
  constexpr int NG = NW / 2;       // waves per group
  constexpr int KC = D / 8 / NG;   // 1 KB blocks of a K (or V^T) tile per copying wave
  static_assert(KC * NG * 8 == D, "page tile blocks must split evenly over a wave group");
  constexpr int NC = 2 * KC + 1;   // copies one copying wave issues per page
  constexpr int lr_blocks = RP / 8;  // 1 KB blocks of the low-rank slots
  static_assert(lr_blocks <= NG, "one low-rank block per copying wave");
  const int lb = w < lr_blocks ? w : 0;
  int lr_src;  // this lane's source offset in the page's low-rank rows
  {
    const int sl = 64 * lb + lane, hh = sl / (4 * RP), rem = sl % (4 * RP);
    lr_src = (rem % RP) * 128 + 64 * hh + 16 * (rem / RP);
  }
  struct PageSrc {
    __amdgpu_buffer_rsrc_t k, v, l;
  };
  auto page_src = [&](int page) {
    return PageSrc{byte_rsrc(p.K + (uint64_t)page * page_elems + head_off, 64 * D * 2),
                   byte_rsrc(p.VT + (uint64_t)page * page_elems + head_off, 64 * D * 2),
                   byte_rsrc(lrb + (uint64_t)page * p.r * kPage, p.r * kPage * 2)};
  };
  auto copy_one = [&](int c, const PageSrc& src, u16* dst) {
    if (c < KC) {
      const int blk = w * KC + c;
      dma_block(src.k, blk * 1024, dst + blk * 512, lane);
    } else if (c < 2 * KC) {
      const int blk = w * KC + c - KC;
      dma_block(src.v, blk * 1024, dst + 64 * D + blk * 512, lane);
    } else {
      dma_lanes(src.l, lr_src, dst + 2 * 64 * D + lb * 512);
    }
  };
  auto copy_page = [&](int page, int buf) {
    const PageSrc src = page_src(page);
#pragma unroll
    for (int c = 0; c < NC; ++c) copy_one(c, src, s_kv + buf * PE);
  };
  // s_waitcnt for every vector-memory operation of the wave (expcnt and
  // lgkmcnt left at their maxima)
  constexpr int kWaitCopies = (7 << 4) | (15 << 8);
  // s_waitcnt for every LDS and scalar-memory operation (vmcnt and expcnt at
  // their maxima)
  constexpr int kWaitLgkm = 15 | (7 << 4) | (3 << 14);

  // Two wave groups, waves [0, NW/2) and [NW/2, NW): wave w and wave w + NW/2
  // run on the same SIMD. Each wave alternates an MFMA phase (O^T, L^T += the
  // previous page's V^T P^T, LR^T P^T; then S^T = K Q^T for the next page) with a
  // softmax phase (the page's P from S). The second group runs one phase behind
  // the first, so on every SIMD one wave issues MFMAs while the other works on
  // the vector ALU and the exponential unit; a barrier separates the phases.
  //
  // Page j sits in LDS buffer j % 3. The first group reads it in phases 2j and
  // 2j + 2, the second in phases 2j + 1 and 2j + 3. The first group issues the
  // copy of page j + 1 inside its MFMA phase 2j (the buffer last held page
  // j - 2, read for the last time in phase 2j - 1) and waits for it at the end
  // of phase 2j + 1.
  const bool lead = w < NG;
  f32x4 sacc[RB][4];
  bf16x8 pt[RB][2];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int t = 0; t < 4; ++t) sacc[rb][t] = f32x4{0, 0, 0, 0};
    pt[rb][0] = pt[rb][1] = bf16x8{};
  }

  // MFMA phase j for the first and the last page: the V^T and low-rank
  // products of page j - 1 (from its P), then the scores of page j
  auto mfma_phase = [&](int j) {
    if (j >= 1) {
      lds_u16* kv = lane_ptr((j - 1) % 3, lane * 8);
      // O^T += V^T P^T and L^T += LR^T P^T; with a spare low-rank row, that
      // row is all ones and accumulates the row sums
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bf16x8 vf = *reinterpret_cast<lds_frag*>(kv + 64 * D + (h * DB + db) * 512);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma(vf, pt[rb][h], oacc[rb][db]);
        }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4 raw =
              __builtin_bit_cast(u32x4, *reinterpret_cast<lds_frag*>(lr_lane(mb, (j - 1) % 3) + h * 32 * RP));
          const u32x4 keep = LRO ? lr_keep(j - 1, h) : u32x4{~0u, ~0u, ~0u, ~0u};
          const bf16x8 lf = __builtin_bit_cast(bf16x8, (raw & lr_mask[mb] & keep) | lr_ones[mb]);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) lacc[rb][mb] = mfma(lf, pt[rb][h], lacc[rb][mb]);
        }
    }
    if (j < n_pages) {
      lds_u16* kv = lane_ptr(j % 3, lane * 8);
      // S^T = K Q^T for the page's 64 keys and the RB row blocks, one 16-key
      // score tile (half h, tile t: index 2h + t) at a time
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        bf16x8 kf[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[s] = *reinterpret_cast<lds_frag*>(kv + (ht * KS + s) * 512);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          f32x4 acc = {0, 0, 0, 0};
#pragma unroll
          for (int s = 0; s < KS; ++s) acc = mfma(kf[s], qf[rb][s], acc);
          sacc[rb][ht] = acc;
        }
      }
    }
  };

  // The same MFMA phase for 1 <= j < n_pages, as one sequence of NF operand
  // fragments (V^T tiles, low-rank rows, K tiles), each feeding RB MFMAs. A
  // wave reads LDS at a bounded rate (about 32 bytes a clock), so the first PF
  // V^T tiles of page j - 1 are read during the wave's softmax phase of that
  // page (which uses no LDS) into vpre; the rest are read kAhead fragments
  // before their use, starting with the first MFMA, so that the wave's reads
  // run during the whole phase and their latency hides behind the MFMAs of
  // the fragments before them. With
  // WC set, the copies of the page src into buffer dst ride along, one per
  // fragment.
  constexpr int NV = 2 * DB, NL = 2 * MB, NK = 4 * KS, NF = NV + NL + NK;
  constexpr int PF = NV / 2;
  constexpr int kAhead = PF;  // reads in flight: at most 15 are counted
  static_assert(NC <= NF, "copies ride along the fragments");
  static_assert(PF % RB == 0 && kAhead <= 15, "prefetch split");
  bf16x8 vpre[PF];
  auto frag_load = [&](int f, lds_u16* kvp, lds_u16* const* kvl, lds_u16* kvc) -> bf16x8 {
    if (f < NV)  // V^T tile: half h = f / DB, column block db = f % DB
      return *reinterpret_cast<lds_frag*>(kvp + 64 * D + f * 512);
    if (f < NV + NL) {  // low-rank rows: block mb, half h
      const int mb = (f - NV) >> 1, h = (f - NV) & 1;
      return *reinterpret_cast<lds_frag*>(kvl[mb] + h * 32 * RP);
    }
    // K tile (ht, s), taken chunk-major (s outer) so that consecutive MFMAs
    // update different score tiles
    const int ks = f - NV - NL, ht = ks % 4, s = ks / 4;
    return *reinterpret_cast<lds_frag*>(kvc + (ht * KS + s) * 512);
  };
  auto frag_use = [&](int f, bf16x8 x) {
    if (f < NV) {
      const int h = f / DB, db = f % DB;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = mfma(x, pt[rb][h], oacc[rb][db]);
    } else if (f < NV + NL) {
      const int mb = (f - NV) >> 1, h = (f - NV) & 1;
      const bf16x8 lf =
          __builtin_bit_cast(bf16x8, (__builtin_bit_cast(u32x4, x) & lr_mask[mb] & keep_lr[h]) | lr_ones[mb]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) lacc[rb][mb] = mfma(lf, pt[rb][h], lacc[rb][mb]);
    } else {
      const int ks = f - NV - NL, ht = ks % 4, s = ks / 4;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[rb][ht] = mfma(x, qf[rb][s], s == 0 ? f32x4{0, 0, 0, 0} : sacc[rb][ht]);
    }
  };
  auto mfma_phase_full = [&](int j, auto wc, int src_page, int dst_buf) {
    constexpr bool WC = decltype(wc)::value;
    if (LRO) {
      keep_lr[0] = lr_keep(j - 1, 0);
      keep_lr[1] = lr_keep(j - 1, 1);
    }
    lds_u16* kvp = lane_ptr((j - 1) % 3, lane * 8);
    lds_u16* kvc = lane_ptr(j % 3, lane * 8);
    lds_u16* kvl[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) kvl[mb] = lr_lane(mb, (j - 1) % 3);
    PageSrc src{};
    if (WC) src = page_src(src_page);
    u16* dst = s_kv + dst_buf * PE;
    bf16x8 fr[NF];
#pragma unroll
    for (int f = 0; f < PF; ++f) fr[f] = vpre[f];
    // program order is kept (sched_barrier) so that the reads leave in the
    // order of use and each wait covers just the fragment needed
#pragma unroll
    for (int f = PF; f < kAhead && f < NF; ++f) {
      fr[f] = frag_load(f, kvp, kvl, kvc);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int g = f + kAhead;
      if (g >= PF && g < NF) fr[g] = frag_load(g, kvp, kvl, kvc);
      frag_use(f, fr[f]);
      if (WC && f < NC) copy_one(f, src, dst);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax phase of page i: online softmax per row block. Lane (n, q) holds
  // keys 32h + 8q + 4t + j (score i = 8h + 4t + j), which in half h is the
  // B-operand slice P^T needs. Scores are scaled inside the exponent's FMA and
  // the running max m is kept in the scaled (log2) domain. m is raised only
  // when some score exceeds it by more than kSlack (then the accumulators are
  // rescaled), so P stays below 2^kSlack and a page needs no cross-lane
  // reduction unless its max grows that far; the normalisation at the end
  // divides by the sum of the same P, so the result does not depend on m.
  constexpr float kSlack = 8.f;
  auto softmax_phase = [&](int i) {
    lds_u16* kvi = lane_ptr(i % 3, lane * 8) + 64 * D;  // V^T tile of page i
    const int ia = p_lo + i;                         // the view's page
    const bool own = ia >= np_sh;
    const int pg_key0 = (own ? ia - np_sh : ia) * kPage;  // first key of the page in its segment
    const int vbase = own ? b : 0;                       // view position of segment key 0
    const int seg_lim = own ? S : b;                     // keys beyond the segment are invalid
    // every row of the wave sees all 64 keys of the page
    const bool whole = pg_key0 + 64 <= seg_lim && vbase + pg_key0 + 63 <= tmin;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (!whole) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = pg_key0 + 32 * (e >> 3) + 8 * q + (e & 7);
          if (!(key < seg_lim && vbase + key <= tpos[rb])) sacc[rb][e >> 2][e & 3] = -INFINITY;
        }
      }
      // max over the lane's 16 scores as a tree (short dependency chain)
      const f32x4* sa = sacc[rb];
      const float m0 = max3f(sa[0][0], sa[0][1], sa[0][2]), m1 = max3f(sa[0][3], sa[1][0], sa[1][1]);
      const float m2 = max3f(sa[1][2], sa[1][3], sa[2][0]), m3 = max3f(sa[2][1], sa[2][2], sa[2][3]);
      const float m4 = max3f(sa[3][0], sa[3][1], sa[3][2]);
      const float mx = max3f(max3f(m0, m1, m2), max3f(m3, m4, sa[3][3]), -INFINITY);
      if (__any(mx * scale_log2 > m_run[rb] + kSlack)) {
        const float m_new = fmaxf(m_run[rb], xmax16_32(mx) * scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[rb][db] *= alpha;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) lacc[rb][mb] *= alpha;
        m_run[rb] = m_new;
      }
      // this row block's share of the V^T prefetch, each read followed by a
      // few of the exponentials' instructions (a wave's LDS reads issue at a
      // bounded rate, so a burst of them would stall the wave)
      constexpr int PV = PF / RB;
#pragma unroll
      for (int f = rb * PV; f < (rb + 1) * PV; ++f) vpre[f] = *reinterpret_cast<lds_frag*>(kvi + f * 512);
      float pv[16];
#pragma unroll
      for (int e = 0; e < 16; ++e)
        pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[rb][e >> 2][e & 3], scale_log2, -m_run[rb]));
#pragma unroll
      for (int f = 0; f < PV; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
      if (!ones_row) {
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) ps += pv[e];
        l_run[rb] += ps;
      }
      pt[rb][0] = pack8(pv);
      pt[rb][1] = pack8(pv + 8);
    }
    // the prefetched tiles have landed long before the phase ends; waiting
    // for them here keeps the count of LDS reads in flight in the MFMA phase
    // within what the counter tracks
    __builtin_amdgcn_s_waitcnt(kWaitLgkm);
  };

  using CopyOn = std::integral_constant<bool, true>;
  using CopyOff = std::integral_constant<bool, false>;
  if (lead) {
    if (n_pages > 0) copy_page(s_pages[0], 0);
    if (n_pages > 1) copy_page(s_pages[1], 1);
  }
  __builtin_amdgcn_s_waitcnt(kWaitCopies);
  __builtin_amdgcn_s_barrier();
  // Iteration j holds phases 2j and 2j + 1, each closed by a barrier; the
  // groups run separate loops so that each keeps its phase order fixed. The
  // first iteration has no products of a previous page and the last no
  // scores, so both are peeled off the steady loops.
  if (n_pages > 0) {
    if (lead) {
      mfma_phase(0);
      __builtin_amdgcn_s_barrier();
      int pid = s_pages[min(2, n_pages - 1)];
      softmax_phase(0);
      int next_page = __builtin_amdgcn_readfirstlane(pid);  // the page the next iteration copies
      // nothing of the prologue stays in flight on the LDS/scalar counter,
      // so the waits inside the loop can count LDS reads alone
      __builtin_amdgcn_s_waitcnt(kWaitLgkm);
      __builtin_amdgcn_s_barrier();
      for (int j = 1; j < n_pages; ++j) {
        // at j = n_pages - 1 this copies the last page once more into the
        // free buffer n_pages % 3 (it held page n_pages - 3); it is never read
        mfma_phase_full(j, CopyOn{}, next_page, (j + 1) % 3);
        __builtin_amdgcn_s_barrier();
        pid = s_pages[min(j + 2, n_pages - 1)];
        softmax_phase(j);
        next_page = __builtin_amdgcn_readfirstlane(pid);
        __builtin_amdgcn_s_waitcnt(kWaitCopies);  // this wave's copies of page j + 1 have landed
        __builtin_amdgcn_s_barrier();             // ... and every other wave's
      }
      mfma_phase(n_pages);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_s_barrier();
    } else {
      __builtin_amdgcn_s_barrier();
      mfma_phase(0);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm);
      __builtin_amdgcn_s_barrier();
      for (int j = 1; j < n_pages; ++j) {
        softmax_phase(j - 1);
        __builtin_amdgcn_s_barrier();
        mfma_phase_full(j, CopyOff{}, 0, 0);
        __builtin_amdgcn_s_barrier();
      }
      softmax_phase(n_pages - 1);
      __builtin_amdgcn_s_barrier();
      mfma_phase(n_pages);
      __builtin_amdgcn_s_barrier();
    }
  }
  __syncthreads();

  if (p.ksplit > 1) {
    // partial state of this key range for the merge: o and o_lr unnormalised,
    // the reference max m (log2 units) and the denominator l
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float l = ones_row ? __shfl(lacc[rb][0][0], n + 4 * p.r) : xsum16_32(l_run[rb]);
      const int pr = w * 16 * RB + rb * 16 + n;
      if (row_blk0 + pr < rows_total) {
        float* pp = p.part + ((uint64_t)blockIdx.x * ROWS + pr) * p.W;
#pragma unroll
        for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4*>(pp + db * 16 + 4 * q) = oacc[rb][db];
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int k = mb * 16 + 4 * q + jj;
            if (k < p.r) pp[D + k] = lacc[rb][mb][jj];
          }
        if (q == 0) {
          pp[D + p.r] = m_run[rb];
          pp[D + p.r + 1] = l;
        }
      }
    }
    return;
  }

  // finalize: o = (oacc + lacc . B_i) / l, B_i applied once for the block's rows
  const int HD = p.Hkv * D;
  const u16* Bi = p.B + (uint64_t)p.ag_id[ai] * p.r * HD + g * D;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    // denominator: the ones row's entry (lane (n, r / 4), entry 0 since r is a
    // multiple of 4), else the lanes' partial sums
    const float l = ones_row ? __shfl(lacc[rb][0][0], n + 4 * p.r) : xsum16_32(l_run[rb]);
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

// prefill workgroup shape: waves, and 16-row blocks per wave
constexpr int kPrefNW = 8;
constexpr int kPrefRB = 2;
constexpr int kMaxPrefillSplit = 8;  // key ranges a prefill row block is split into, at most

// Merge of a split prefill: one wave per query row combines the partial rows
// of its key ranges (s = 0 .. ksplit - 1 at part[((s nblk + block) 256 + row)
// W]): M = max m_s, w_s = 2^(m_s - M), o = sum w_s o_s / sum w_s l_s and
// likewise o_lr; then o += o_lr B_i[:, g D:(g + 1) D] once, in bf16.
struct PrefillMergeParams {
  const float* part;
  const u16* B;
  u16* o;
  int Hkv, Hq, G, r, W, ksplit, nblk, n;
  int ag_id[SKV_MAX_AGENTS], ag_nq[SKV_MAX_AGENTS], ag_row0[SKV_MAX_AGENTS];
  int blk0[SKV_MAX_AGENTS + 1];
};

template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillMergeParams p) {
  constexpr int ROWS = kPrefNW * 16 * kPrefRB, EPL = D / 64;  // rows per block, elements per lane
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.nblk * ROWS) return;
  const int bid = row / ROWS, pr = row % ROWS;
  const int g = bid % p.Hkv;
  int qb = bid / p.Hkv;
  int ai = 0;
  while (qb >= p.blk0[ai + 1]) ++ai;
  qb -= p.blk0[ai];
  const int rho = qb * ROWS + pr;
  if (rho >= p.ag_nq[ai] * p.G) return;  // the whole wave leaves together
  auto prow = [&](int s) { return p.part + (((uint64_t)s * p.nblk + bid) * ROWS + pr) * p.W; };
  // Every load is issued here, before the reductions, and unconditionally
  // (indices clamped into range; the clamped values are weighted by zero or
  // never read), so the compiler's waits count each group exactly: the
  // partial rows first, then the first eight rows of B_i's column slice.
  const float m_l = prow(min(lane, p.ksplit - 1))[D + p.r];
  const float l_l = prow(min(lane, p.ksplit - 1))[D + p.r + 1];
  float po[kMaxPrefillSplit][EPL], plr[kMaxPrefillSplit];
#pragma unroll
  for (int s = 0; s < kMaxPrefillSplit; ++s) {
    const float* pp = prow(min(s, p.ksplit - 1));
#pragma unroll
    for (int e = 0; e < EPL; ++e) po[s][e] = pp[lane + 64 * e];
    plr[s] = pp[D + min(lane, p.r - 1)];
  }
  const int HD = p.Hkv * D;
  const u16* Bi = p.B + (uint64_t)p.ag_id[ai] * p.r * HD + g * D;
  u16 b8[8][EPL];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < EPL; ++e) b8[k][e] = Bi[(uint64_t)min(k, p.r - 1) * HD + lane + 64 * e];
  const float m_s = lane < p.ksplit ? m_l : -1e30f;
  const float l_s = lane < p.ksplit ? l_l : 0.f;
  const float M = wave_max(m_s);
  const float w_s = lane < p.ksplit ? __builtin_amdgcn_exp2f(m_s - M) : 0.f;
  const float L = wave_sum(w_s * l_s);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float acc[EPL], acc_lr = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxPrefillSplit; ++s) {
    const float ws = __shfl(w_s, s);  // zero past the last range
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] += ws * po[s][e];
    acc_lr += ws * plr[s];  // meaningful in lanes below r
  }
  float out[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) out[e] = acc[e] * inv;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float lk = __shfl(acc_lr, k) * inv;
    if (k < p.r) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) out[e] += lk * bf2f(b8[k][e]);
    }
  }
  for (int k = 8; k < p.r; ++k) {
    const float lk = __shfl(acc_lr, k) * inv;
#pragma unroll
    for (int e = 0; e < EPL; ++e) out[e] += lk * bf2f(Bi[(uint64_t)k * HD + lane + 64 * e]);
  }
  u16* op = p.o + ((uint64_t)(p.ag_row0[ai] + rho / p.G) * p.Hq + g * p.G + rho % p.G) * D;
#pragma unroll
  for (int e = 0; e < EPL; ++e) op[lane + 64 * e] = f2bf(out[e]);
}

// ---------------------------------------------------------------------------
// Front end: q, k, v projections with rotary embedding, written into pages
// ---------------------------------------------------------------------------

// The rows X of one append job (some agents' new tokens, consecutive rows of
// the call) against the stacked projection weights W [(Hq + 2 Hkv) D][hidden]
// (query heads, then key heads, then value heads): Y^T = W X^T on bf16 MFMA
// with fp32 accumulation (LRAgent review, "What carries the argument": one pass
// over X gives q, k and the base value, whose adapter term stays the rank-r
// rows X A_i). A wave owns 64 output features of one head, d in [32u, 32u + 32)
// and the same range shifted by D/2, so both members of every rotary pair
// (d, d + D/2) sit in the same lane of its C tiles, and TM tokens. A workgroup
// of four waves takes four such units and shares one X tile: X is copied to LDS
// in MFMA-operand order (each 1 KB fragment is one buffer-to-LDS copy), W goes
// from memory to registers, both two 64-column stages ahead of the MFMAs. The
// epilogue rotates q and k, writes q to the caller's rows and k, v into their
// pages in the K / V^T tile order. Blocks after the GEMM blocks compute the
// low-rank rows bf16(X A_i) with the append code and write the page tables.
struct ProjectParams {
  AppendParams app;  // spans and page ids of the job's rows, low-rank rows, table entries
  const u16* x;      // [rows of the call][hidden]
  const u16* w;      // packed weights (pack_qkv_kernel)
  u16* q;            // [rows of the call][Hq][D]
  int row0, rows;    // this job's rows of the call: [row0, row0 + rows)
  int n_units;       // 64-feature units: (Hq + 2 Hkv) D / 64
  int tok_tiles;     // TM-row tiles of the job
  int n_gemm;        // GEMM tiles: unit groups of four x token tiles
  int per_xcd;       // GEMM tiles per XCD; the GEMM part of the grid is 8 per_xcd blocks
  int Hq, Hkv, hidden;
  int rope;                           // rotate q and k
  int view_off[skv::kMaxJobSpans];    // view position of own row 0 of each span's agent (its b_i)
  double inv_freq[64];                // theta^(-2i/D), i < D/2
};
static_assert(sizeof(ProjectParams) <= 4096, "kernel arguments");

// Epilogue of the projection for one wave: C tiles acc[c][jj] hold 16-token
// tile c (tokens t0 + 16 c + n) and feature tile jj of unit hu of head `head`;
// tiles jj and jj + NJ/2 are the two members of the rotary pairs (feature
// tiles jp and jp + 2 of the unit: jp = pp, or `half` when a wave holds half a
// unit). Rotates q and k, writes q to the caller's rows and k, v into their
// pages in the K / V^T tile order (bf16, round to nearest even).
template <int D, int NC, int NJ>
__device__ __forceinline__ void project_epilogue(const ProjectParams& p, const f32x4 (&acc)[NC][NJ], int t0,
                                                 int head, int hu, int half) {
  const int lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int part = head < p.Hq ? 0 : (head < p.Hq + p.Hkv ? 1 : 2);  // q, k, v
  const int hh = part == 0 ? head : (part == 1 ? head - p.Hq : head - p.Hq - p.Hkv);
  constexpr double kTwoPi = 6.283185307179586;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int t = t0 + 16 * c + n;
    if (t >= p.rows) continue;
    const int row = p.row0 + t;
    int s = 0;
    while (s + 1 < p.app.n_spans && row >= p.app.spans[s + 1].src_row) ++s;
    const skv::Span& sp = p.app.spans[s];
    const int pos = sp.pos0 + row - sp.src_row;  // own row index
    const int page = p.app.ids[sp.ids_off + pos / kPage - sp.first_page];
    const int slot_in_page = pos % kPage;
    const double view = (double)(p.view_off[s] + pos);
#pragma unroll
    for (int pp = 0; pp < NJ / 2; ++pp) {
      // rotary pair: tiles jj = pp and pp + NJ/2 are feature tiles jp and jp + 2
      const int jp = NJ == 2 ? half : pp;
      const int dlo = 32 * hu + 16 * jp + 4 * qd;  // element 0 of the low half; the high half is + D/2
      float lo[4], hi[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = acc[c][pp][e];
        hi[e] = acc[c][pp + NJ / 2][e];
      }
      if (part < 2 && p.rope) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // angle in fp64, reduced to [-pi, pi] before the fp32 sine and cosine
          double a = view * p.inv_freq[dlo + e];
          a -= rint(a * (1.0 / kTwoPi)) * kTwoPi;
          float sn, cs;
          sincosf((float)a, &sn, &cs);
          const float l = lo[e], h = hi[e];
          lo[e] = l * cs - h * sn;
          hi[e] = l * sn + h * cs;
        }
      }
      if (part == 2) {
        u16* vt = p.app.VT + ((uint64_t)page * p.Hkv + hh) * kPage * D;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vt[v_tile_off<D>(slot_in_page, dlo + e)] = f2bf(lo[e]);
          vt[v_tile_off<D>(slot_in_page, dlo + D / 2 + e)] = f2bf(hi[e]);
        }
      } else {
        const u32x2 vlo{(uint32_t)f2bf(lo[0]) | ((uint32_t)f2bf(lo[1]) << 16),
                        (uint32_t)f2bf(lo[2]) | ((uint32_t)f2bf(lo[3]) << 16)};
        const u32x2 vhi{(uint32_t)f2bf(hi[0]) | ((uint32_t)f2bf(hi[1]) << 16),
                        (uint32_t)f2bf(hi[2]) | ((uint32_t)f2bf(hi[3]) << 16)};
        u16 *dl, *dh;
        if (part == 0) {
          dl = p.q + ((uint64_t)row * p.Hq + hh) * D + dlo;
          dh = dl + D / 2;
        } else {
          u16* kt = p.app.K + ((uint64_t)page * p.Hkv + hh) * kPage * D;
          dl = kt + k_tile_off<D>(slot_in_page, dlo);
          dh = kt + k_tile_off<D>(slot_in_page, dlo + D / 2);
        }
        *reinterpret_cast<u32x2*>(dl) = vlo;
        *reinterpret_cast<u32x2*>(dh) = vhi;
      }
    }
  }
}


// Few rows (a decode step, up to 16): split K. A workgroup takes half a unit
// (one rotary-paired pair of 16-feature tiles) and the 16-row tile, and its
// four waves take a quarter of the hidden columns each, with rings of three
// slots of their own (two stages in flight ahead of the MFMAs); the partial
// sums meet in LDS at the end. Eight times as many workgroups stream W as with
// four units per workgroup: the weight stream of a few rows is bound by how
// many CUs pull on it.
constexpr int kSplitSlots = 3;
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void project_split_kernel(
    ProjectParams p) {
  constexpr int NS = kSplitSlots;
  constexpr int SLOT = (2 + 4) * 512;  // u16 per ring slot: 2 X fragments, then 4 W fragments
  static_assert(4 * NS * SLOT * 2 >= 64 * (128 + 8) * 2, "the low-rank blocks stage rows in the same LDS");
  extern __shared__ __attribute__((aligned(16))) u16 s_pr[];
  const int b = blockIdx.x;
  if (b >= 8 * p.per_xcd) {
    append_block(p.app, b - 8 * p.per_xcd, reinterpret_cast<char*>(s_pr));
    return;
  }
  // Block b runs on XCD b % 8: each XCD takes a contiguous run of tiles.
  const int lb = (b % 8) * p.per_xcd + b / 8;
  if (lb >= p.n_gemm) return;
  const int ug = lb;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int unit = ug / 2;
  const int half = ug % 2;  // feature tiles half and half + 2 of the unit
  const bool active = unit < p.n_units;
  constexpr int UPH = D / 64;  // units per head
  const int uc = active ? unit : p.n_units - 1;
  const int head = uc / UPH, hu = uc % UPH;
  const int H = p.hidden, nk = H / 64;
  const int kbeg = wave * nk / 4;  // this wave's stages [kbeg, kbeg + kcnt)
  const int kcnt = (wave + 1) * nk / 4 - kbeg;
  u16* const ring = s_pr + wave * NS * SLOT;
  // W is packed (pack_qkv_kernel): the unit's eight fragments of a stage are
  // 8 KB of contiguous memory, so each copy is 1 KB contiguous and a wave
  // streams its unit's weights front to back.
  const __amdgpu_buffer_rsrc_t wr = byte_rsrc(p.w + (uint64_t)uc * nk * 8 * 512, nk * 8 * 1024);
  // X fragment ks: lane (n, qd) copies token n, columns 32 ks + 8 qd + [0, 8).
  // Rows past the job read as zero (buffer bounds).
  const __amdgpu_buffer_rsrc_t xr = byte_rsrc(p.x + (uint64_t)p.row0 * H, p.rows * H * 2);
  const int xoff0 = (n * H + 8 * qd) * 2;

  // tile jj of the wave is feature tile half + 2 jj
  f32x4 acc[1][2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) acc[0][jj] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Copies of stage s into ring slot s % NS: the two X fragments, then the
  // wave's four W fragments. Stages past the end copy the last one again, so
  // every stage issues the same copies and the wait below holds.
  auto issue = [&](int s) {
    if (kcnt == 0) return;
    const int sc = kbeg + (s < kcnt ? s : kcnt - 1);
    u16* slot = ring + (s % NS) * SLOT;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (void __attribute__((address_space(3)))*)(slot + ks * 512), 16,
                                               xoff0 + (64 * sc + 32 * ks) * 2, 0, 0, 0);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int j = half + 2 * jj;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (void __attribute__((address_space(3)))*)(slot + (2 + 2 * jj + ks) * 512),
                                                 16, ((sc * 8 + 2 * j + ks) * 64 + lane) * 16, 0, 0, 0);
      }
  };
  // Before stage s: stages s .. s + NS - 2 are in flight (six copies each);
  // with no more than NS - 2 stages' worth outstanding, stage s has landed.
  // Every wave reads only its own ring.
  constexpr int kAfter = (NS - 2) * 6;
  constexpr int kWaitStage = (kAfter & 15) | ((kAfter >> 4) << 14) | (7 << 4) | (15 << 8);
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(s);
  for (int s = 0; s < kcnt; ++s) {
    __builtin_amdgcn_s_waitcnt(kWaitStage);
    issue(s + NS - 1);
    const u16* slot = ring + (s % NS) * SLOT;
    bf16x8 bx[2], aw[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        aw[ks][jj] = *reinterpret_cast<const bf16x8*>(slot + (2 + 2 * jj + ks) * 512 + lane * 8);
      bx[ks] = *reinterpret_cast<const bf16x8*>(slot + ks * 512 + lane * 8);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        acc[0][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[ks][jj], bx[ks], acc[0][jj], 0, 0, 0);
    // every LDS read of the stage first, then the MFMAs (the first ones wait
    // only for their own operands)
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): no copy outlives the wave
  // waves 1..3 hand their partial sums to wave 0 (added in wave order)
  __syncthreads();  // every wave is done with its ring
  float* red = reinterpret_cast<float*>(s_pr);  // [3][64 lanes][8]
  if (wave > 0) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) *reinterpret_cast<f32x4*>(red + ((wave - 1) * 64 + lane) * 8 + 4 * jj) = acc[0][jj];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[0][jj] += *reinterpret_cast<const f32x4*>(red + (w * 64 + lane) * 8 + 4 * jj);
  if (!active) return;
  project_epilogue<D, 1, 2>(p, acc, 0, head, hu, half);
}

// Calls of hundreds of rows and more: a workgroup takes 128 tokens and NH
// half units (32 output features each: feature tiles h and h + 2 of a unit,
// the two members of its rotary pairs) and streams both operands through LDS
// (per 64-column stage, X 16 KB and W 4 NH KB; X token-major, each copy
// reading whole cache lines). NH = 4 (two units) gives each byte copied twice
// the flops of the four-unit, 32-row tile; NH = 3 makes 4/3 as many tiles,
// for calls whose two-unit tiles would leave CUs idle. Compute wave w takes
// tokens 64 (w / NH) .. + 63 and half unit w % NH, two waves per SIMD, so one
// wave's LDS reads run under the other's MFMAs. Four copy waves, one per SIMD,
// issue the stage's buffer-to-LDS copies: a wave that issues copies waits
// while the CU's address and data units take them, and none of that wait
// falls on the compute waves. A ring of NS slots keeps the copies NS - 2
// stages ahead of the stage whose operands are read. Blocks after the GEMM
// blocks compute the low-rank rows with the append code (four waves; the
// others end at once, and a barrier waits only for waves that have not ended).
constexpr int kWideRows = 128;  // tokens per tile of the wide form

template <int D, int NS, int NH>
__global__ __launch_bounds__(64 * (2 * NH + 4)) void project_wide_kernel(ProjectParams p) {
  static_assert(NH == 3 || NH == 4, "three or four half units per tile");
  constexpr int CW = 2 * NH;               // compute waves
  constexpr int SLOT = (16 + 4 * NH) * 512;  // u16 per ring slot: 16 X copies, then 4 W fragments per half unit
  constexpr int NCP = 4 + NH;              // copies per copy wave and stage
  static_assert(NS * SLOT * 2 >= 64 * (128 + 8) * 2, "the low-rank blocks stage rows in the same LDS");
  static_assert(NS >= 4, "stage s + 1 is read while stage s + NS - 1 is copied into the slot of stage s - 1");
  extern __shared__ __attribute__((aligned(16))) u16 s_pw[];
  const int b = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= 8 * p.per_xcd) {
    if (wave >= 4) return;  // a wave-uniform exit
    append_block<false, true, 256, 2>(p.app, b - 8 * p.per_xcd, reinterpret_cast<char*>(s_pw));
    return;
  }
  // block b runs on XCD b % 8; token tile fastest, so the token tiles of one
  // column of half units read W through one L2
  const int lb = (b % 8) * p.per_xcd + b / 8;
  if (lb >= p.n_gemm) return;
  const int ct = lb / p.tok_tiles, tt = lb % p.tok_tiles;
  const int H = p.hidden, nk = H / 64;
  // Before the MFMAs of stage s, the copy waves wait until their copies of
  // stage s + 1 have landed (later stages may remain in flight) and the
  // compute waves until every LDS read they issued has returned. The barrier
  // then publishes stage s + 1 and retires the reads of the slot the next
  // copies overwrite. It is a bare barrier: a workgroup fence would wait for
  // every copy in flight.
  if (wave >= CW) {
    const int cw = wave - CW;
    // X copy xi (tokens 8 xi .. 8 xi + 7 of the tile): lane l writes LDS
    // bytes 16 l of the copy, token 8 xi + l / 8, the 16-byte chunk
    // (l % 8) ^ (token % 8) of the token's 64 columns. Each eight lanes read
    // one token's 128 contiguous bytes (a single cache line), and the XOR
    // swizzle keeps the compute waves' operand reads free of bank conflicts.
    // Rows past the job read as zero (buffer bounds).
    const __amdgpu_buffer_rsrc_t xr = byte_rsrc(p.x + (uint64_t)p.row0 * H, p.rows * H * 2);
    const int xt = lane >> 3, xc = (lane & 7) ^ (xt & 7);  // token in the copy, chunk it reads
    const int xoff0 = ((tt * kWideRows + xt) * H + 8 * xc) * 2;
    // W copy wi = 4 hs + 2 jj + ks: k-step ks of feature tile half + 2 jj of
    // the tile's half unit hs (packed: 1 KB contiguous per copy); a half unit
    // past the last reads the last unit
    const __amdgpu_buffer_rsrc_t wr = byte_rsrc(p.w, p.n_units * nk * 8 * 1024);
    // Stages past the end copy the last one again, so every stage issues the
    // same copies and the wait counts hold.
    auto issue = [&](int s) {
      const int sc = s < nk ? s : nk - 1;
      u16* slot = s_pw + (s % NS) * SLOT;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int xi = cw + 4 * i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (void __attribute__((address_space(3)))*)(slot + xi * 512), 16,
                                                 xoff0 + (8 * xi * H + 64 * sc) * 2, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < NH; ++i) {
        const int wi = cw + 4 * i, gh = NH * ct + (wi >> 2);
        const int u = min(gh >> 1, p.n_units - 1);
        const int f = 2 * ((gh & 1) + 2 * ((wi >> 1) & 1)) + (wi & 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (void __attribute__((address_space(3)))*)(slot + (16 + wi) * 512),
                                                 16, ((u * nk + sc) * 8 + f) * 1024 + lane * 16, 0, 0, 0);
      }
    };
    constexpr int kFirst = (NS - 2) * NCP, kAfter = (NS - 3) * NCP;
    constexpr int kWaitFirst = (kFirst & 15) | ((kFirst >> 4) << 14) | (7 << 4) | (15 << 8);
    constexpr int kWaitCopies = (kAfter & 15) | ((kAfter >> 4) << 14) | (7 << 4) | (15 << 8);
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s);
    stage_barrier<kWaitFirst>();  // stage 0 has landed
    for (int s = 0; s < nk; ++s) {
      stage_barrier<kWaitCopies>();  // stage s + 1 has landed
      issue(s + NS - 1);  // into the slot of stage s - 1, whose reads ended before the last barrier
    }
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): no copy outlives the wave
    return;
  }
  const int rh = wave / NH, hs = wave % NH;
  const int gh = NH * ct + hs;
  const int unit = gh >> 1, half = gh & 1;
  f32x4 acc[4][2];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[c][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
  // B operand (token 16 c' + n, columns 32 ks + 8 qd of the stage, c' the
  // wave's token tile 4 rh + c): the swizzled 16-byte chunk 4 ks + qd
  const int n = lane & 15, qd = lane >> 4;
  int xrd[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) xrd[ks] = (64 * rh + n) * 64 + (((4 * ks + qd) ^ (n & 7)) << 3);
  // Operands of one stage in registers, two sets: the reads of stage s + 1
  // are in flight while stage s's MFMAs issue.
  struct Ops {
    bf16x8 bx[2][4], aw[2][2];
  };
  auto read = [&](int s, Ops& o) {
    const u16* slot = s_pw + (s % NS) * SLOT;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        o.aw[ks][jj] = *reinterpret_cast<const bf16x8*>(slot + (16 + 4 * hs + 2 * jj + ks) * 512 + lane * 8);
#pragma unroll
      for (int c = 0; c < 4; ++c) o.bx[ks][c] = *reinterpret_cast<const bf16x8*>(slot + xrd[ks] + c * 16 * 64);
    }
  };
  auto mma = [&](const Ops& o) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o.aw[ks][jj], o.bx[ks][c], acc[c][jj], 0, 0, 0);
  };
  constexpr int kWaitReads = 15 | (7 << 4) | (3 << 14);  // lgkmcnt(0)
  Ops oa, ob;
  stage_barrier<kWaitReads>();
  read(0, oa);
  // Stage nk (read in the last round) is a copy of stage nk - 1 that is
  // never used.
  for (int s = 0; s < nk; s += 2) {
    stage_barrier<kWaitReads>();
    read(s + 1, ob);
    mma(oa);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // the reads first, then the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    if (s + 1 == nk) break;
    stage_barrier<kWaitReads>();
    read(s + 2, oa);
    mma(ob);
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
  }
  if (unit >= p.n_units) return;
  constexpr int UPH = D / 64;  // units per head
  project_epilogue<D, 4, 2>(p, acc, tt * kWideRows + 64 * rh, unit / UPH, unit % UPH, half);
}

// Calls of a thousand rows and more: 256 tokens x two units (128 features)
// per workgroup, so each byte copied serves 4/3 the flops of the 128-token
// tile (X 32 KB and W 16 KB per 64-column stage for 4 MFLOP). Compute wave w
// takes tokens 64 (w / 2) .. + 63 and the whole unit w % 2 (feature tiles 0-3;
// tiles j and j + 2 are rotary pairs); with 64 accumulator registers it reads
// one stage at a time, the k-step 1 operands under the k-step 0 MFMAs. Four
// copy waves keep the copies of a three-slot ring two stages ahead.
constexpr int kTallRows = 256;  // tokens per tile of the tall form
template <int D>
__global__ __launch_bounds__(64 * 12) void project_tall_kernel(ProjectParams p) {
  constexpr int NS = 3;
  constexpr int SLOT = 48 * 512;  // u16 per ring slot: 32 X copies, then 8 W fragments of each unit
  constexpr int NCP = 12;         // copies per copy wave and stage
  extern __shared__ __attribute__((aligned(16))) u16 s_pt[];
  const int b = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= 8 * p.per_xcd) {
    if (wave >= 4) return;  // a wave-uniform exit
    append_block<false, true, 256, 2>(p.app, b - 8 * p.per_xcd, reinterpret_cast<char*>(s_pt));
    return;
  }
  const int lb = (b % 8) * p.per_xcd + b / 8;
  if (lb >= p.n_gemm) return;
  const int ct = lb / p.tok_tiles, tt = lb % p.tok_tiles;
  const int H = p.hidden, nk = H / 64;
  if (wave >= 8) {
    const int cw = wave - 8;
    // X copy xi (tokens 8 xi .. 8 xi + 7 of the tile) as in the wide form:
    // token-major, XOR-swizzled 16-byte chunks, whole cache lines per copy
    const __amdgpu_buffer_rsrc_t xr = byte_rsrc(p.x + (uint64_t)p.row0 * H, p.rows * H * 2);
    const int xt = lane >> 3, xc = (lane & 7) ^ (xt & 7);
    const int xoff0 = ((tt * kTallRows + xt) * H + 8 * xc) * 2;
    const __amdgpu_buffer_rsrc_t wr = byte_rsrc(p.w, p.n_units * nk * 8 * 1024);
    auto issue = [&](int s) {
      const int sc = s < nk ? s : nk - 1;
      u16* slot = s_pt + (s % NS) * SLOT;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int xi = cw + 4 * i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (void __attribute__((address_space(3)))*)(slot + xi * 512), 16,
                                                 xoff0 + (8 * xi * H + 64 * sc) * 2, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int fi = cw + 4 * i;  // fragment fi % 8 of unit fi / 8 of the tile
        const int u = min(2 * ct + (fi >> 3), p.n_units - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (void __attribute__((address_space(3)))*)(slot + (32 + fi) * 512),
                                                 16, ((u * nk + sc) * 8 + (fi & 7)) * 1024 + lane * 16, 0, 0, 0);
      }
    };
    // before stage s: its copies have landed (stage s + 1 may be in flight)
    constexpr int kAfter = (NS - 2) * NCP;
    constexpr int kWaitCopies = (kAfter & 15) | ((kAfter >> 4) << 14) | (7 << 4) | (15 << 8);
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s);
    for (int s = 0; s < nk; ++s) {
      stage_barrier<kWaitCopies>();
      issue(s + NS - 1);  // into the slot of stage s - 1, whose reads ended before this barrier
    }
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): no copy outlives the wave
    return;
  }
  const int rh = wave >> 1, u2 = wave & 1;
  const int unit = 2 * ct + u2;
  f32x4 acc[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[c][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int n = lane & 15, qd = lane >> 4;
  int xrd[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) xrd[ks] = (64 * rh + n) * 64 + (((4 * ks + qd) ^ (n & 7)) << 3);
  constexpr int kWaitReads = 15 | (7 << 4) | (3 << 14);  // lgkmcnt(0)
  for (int s = 0; s < nk; ++s) {
    stage_barrier<kWaitReads>();
    const u16* slot = s_pt + (s % NS) * SLOT;
    bf16x8 bx[2][4], aw[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        aw[ks][j] = *reinterpret_cast<const bf16x8*>(slot + (32 + 8 * u2 + 2 * j + ks) * 512 + lane * 8);
#pragma unroll
      for (int c = 0; c < 4; ++c) bx[ks][c] = *reinterpret_cast<const bf16x8*>(slot + xrd[ks] + c * 16 * 64);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc[c][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aw[ks][j], bx[ks][c], acc[c][j], 0, 0, 0);
    // k-step 0's reads, then its MFMAs with k-step 1's reads among them, then k-step 1's MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
  }
  if (unit >= p.n_units) return;
  constexpr int UPH = D / 64;  // units per head
  project_epilogue<D, 4, 4>(p, acc, tt * kTallRows + 64 * rh, unit / UPH, unit % UPH, 0);
}

// Packs W [(Hq + 2 Hkv) D][hidden] for project_kernel: for 64-feature unit u
// (head u / (D / 64), d in [32 hu, 32 hu + 32) and that + D/2), 64-column
// stage s, fragment f = 2 j + ks and lane l = n + 16 qd, the 16 bytes at
// ((u * nk + s) * 8 + f) * 1024 + 16 l hold W[row][64 s + 32 ks + 8 qd .. + 8]
// with row = head D + 32 hu + 16 (j & 1) + (D/2)(j >> 1) + n: the order in which
// one wave's MFMA A operands are read. One block per (unit, stage).
struct PackParams {
  const u16* w;
  u16* out;
  int D, H;
};
__global__ __launch_bounds__(256) void pack_qkv_kernel(PackParams p) {
  const u16* __restrict__ w = p.w;
  u16* __restrict__ out = p.out;
  const int D = p.D, H = p.H;
  const int nk = H / 64, uph = D / 64;
  const int u = blockIdx.x / nk, s = blockIdx.x % nk;
  const int head = u / uph, hu = u % uph;
  for (int v = threadIdx.x; v < 512; v += blockDim.x) {
    const int f = v >> 6, l = v & 63, j = f >> 1, ks = f & 1, n = l & 15, qd = l >> 4;
    const int row = head * D + 32 * hu + 16 * (j & 1) + (D / 2) * (j >> 1) + n;
    const u32x4 val = *reinterpret_cast<const u32x4*>(w + (uint64_t)row * H + 64 * s + 32 * ks + 8 * qd);
    *reinterpret_cast<u32x4*>(out + ((uint64_t)blockIdx.x * 8 + f) * 512 + l * 8) = val;
  }
}

// ---------------------------------------------------------------------------
// Measurement probes (roofline calibration; not part of the attention path)
// ---------------------------------------------------------------------------


// Grid-stride non-temporal 16-byte reads, eight in flight per lane.
__global__ __launch_bounds__(256) void probe_stream_kernel(const u32x4* __restrict__ src, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  if ((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) == 0x9e3779b9u) skv::probe_sink[threadIdx.x & 3] = acc[0];
}

// Back-to-back v_mfma_f32_16x16x32_bf16 on eight independent accumulators.
__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters) {
  const uint32_t lane = threadIdx.x & 63;
  const bf16x8 a = __builtin_bit_cast(bf16x8, u32x4{0x3a003a00u + lane, 0x3a003a00u, 0x3a003a00u, 0x3a003a00u});
  const bf16x8 b = __builtin_bit_cast(bf16x8, u32x4{0x3a003a00u, 0x3a003a00u + lane, 0x3a003a00u, 0x3a003a00u});
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mfma(a, b, acc[j]);
  }
  f32x4 t = acc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) t += acc[j];
  if (t[0] + t[1] + t[2] + t[3] == 1234.5f) skv::probe_sink[threadIdx.x & 3] = __float_as_uint(t[0]);
}

// The same issue loop on operand data: each wave takes eight A and eight B
// fragments (16 bytes a lane each) from src, so consecutive MFMAs see
// different bit patterns, as the operands of attention do. The matrix pipe's
// power draw depends on them, and under a sustained load the power limit sets
// the clock: constant operands run faster than real data.
__global__ __launch_bounds__(256) void probe_mfma_data_kernel(const u32x4* __restrict__ src, int iters) {
  const uint32_t lane = threadIdx.x & 63;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = __builtin_bit_cast(bf16x8, src[j * 64 + lane]);
    b[j] = __builtin_bit_cast(bf16x8, src[(8 + j) * 64 + lane]);
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mfma(a[j], b[j], acc[j]);
  }
  f32x4 t = acc[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) t += acc[j];
  if (t[0] + t[1] + t[2] + t[3] == 1234.5f) skv::probe_sink[threadIdx.x & 3] = __float_as_uint(t[0]);
}

// The launch-pattern probe's pair: a one-workgroup-per-CU streaming read of a
// layer-sized buffer that leaves one word per wave, then a small launch of
// single-row workgroups that reads those words (so it is ordered after the
// read, as a merge is after its split pass).
__global__ __launch_bounds__(256) void probe_layer_kernel(const u32x4* __restrict__ src, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  u32x4 acc = {0, 0, 0, 0};
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t a = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) a ^= __shfl_xor(a, o);
  if ((threadIdx.x & 63) == 0) skv::probe_part[(blockIdx.x * 4 + (threadIdx.x >> 6)) % (4 * kCUs)] = a;
}

__global__ __launch_bounds__(256) void probe_tail_kernel() {
  uint32_t a = skv::probe_part[(blockIdx.x * 256 + threadIdx.x) % (4 * kCUs)];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) a ^= __shfl_xor(a, o);
  if (a == 0x9e3779b9u) skv::probe_sink[threadIdx.x & 3] = a;
}

// ---------------------------------------------------------------------------
// Host side: launch helpers, planning, timing
// ---------------------------------------------------------------------------

struct DevState {
  int timing = 0;  // bit mask of kernel kinds to time
  float* scratch_static = nullptr;  // device address of `scratch` on this context's device
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

// Launch on the context stream. When timing is on for this kernel kind the
// dispatch itself records start/stop events (hipExtLaunchKernelGGL), so the
// measured interval is the kernel's own execution.
template <typename Kernel, typename Params>
int launch(const skv::Geometry& g, int kind, Kernel kernel, dim3 grid, size_t lds,
           const Params& params, const char* what, int threads = 256) {
  auto* st = (DevState*)g.dev;
  hipStream_t stream = (hipStream_t)g.stream;
  hipEvent_t a = nullptr, b = nullptr;
  if (st && kind >= 0 && (st->timing >> kind & 1)) {
    a = st->get();
    b = st->get();
  }
  if (a && b) {
    hipExtLaunchKernelGGL(kernel, grid, dim3(threads), (uint32_t)lds, stream, a, b, 0, params);
    st->recs.push_back({kind, a, b});
  } else {
    hipLaunchKernelGGL(kernel, grid, dim3(threads), lds, stream, params);
  }
  ++*g.launches;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_err(what, e);
    return SKV_ERR_HIP;
  }
  return SKV_OK;
}

int group_limit(const skv::Geometry& g) { return skv::decode_group_limit(g.N, g.G, g.mode, g.r); }

int w_of(const skv::Geometry& g) { return g.D + g.r + 4; }

template <int D, int RB, int MB>
int launch_split_t(const skv::Geometry& g, const DecodeParams& p, int items, bool timed) {
  constexpr int DB = D / 16, NQ = DB + MB;
  size_t lds = (size_t)split_fold_slots<D, RB, MB>() * RB * (NQ * 64 * 16 + 2 * 64 * 4);  // wave states
  if (p.n_app > 0) lds = std::max(lds, (size_t)64 * (128 + 8) * 2);  // append blocks' staging
  return launch(g, timed ? 2 : -1, decode_split_kernel<D, RB, MB>, dim3(p.n_app + items), lds, p,
                "decode_split_kernel");
}

// Prefill workgroups: eight waves of two 16-row blocks each (two waves per
// SIMD, accumulators in VGPRs), 256 query rows per workgroup.
constexpr int prefill_rows(int) { return kPrefNW * 16 * kPrefRB; }

template <int D, int MB, bool LRO>
int launch_prefill(const skv::Geometry& g, const PrefillParams& p, int blocks) {
  const size_t lds = (size_t)3 * prefill_page_elems<D>() * sizeof(u16);
  // the page ring exceeds the default dynamic LDS limit (set once per process;
  // the attribute holds for every device)
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(prefill_kernel<D, MB, kPrefRB, kPrefNW, LRO>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) {
    set_err("hipFuncSetAttribute(prefill_kernel)", attr);
    return SKV_ERR_HIP;
  }
  return launch(g, 4, prefill_kernel<D, MB, kPrefRB, kPrefNW, LRO>, dim3(blocks), lds, p, "prefill_kernel",
                64 * kPrefNW);
}

template <int D, int MB>
int launch_prefill_o(const skv::Geometry& g, const PrefillParams& p, int blocks, bool lro) {
  return lro ? launch_prefill<D, MB, true>(g, p, blocks) : launch_prefill<D, MB, false>(g, p, blocks);
}

// Prefill of few row blocks: each block's key range is split over ksplit
// workgroups so that the launch fills the CUs; a merge launch combines the
// partial rows and applies B_i. The partials use the decode scratch (the two
// kinds of call are ordered on the stream).
constexpr int kMinSplitPages = 4;  // pages per workgroup below which a split does not pay

int prefill_split(int nblk, int min_view_pages) {
  int ks = 1;
  while (ks < kMaxPrefillSplit && 2 * ks * nblk <= kCUs && min_view_pages >= 2 * ks * kMinSplitPages) ks *= 2;
  return ks;
}

template <int D>
int launch_split_d(const skv::Geometry& g, int rb, int mb, const DecodeParams& p, int items, bool timed) {
  if (rb == 1 && mb == 1) return launch_split_t<D, 1, 1>(g, p, items, timed);
  if (rb == 1 && mb == 2) return launch_split_t<D, 1, 2>(g, p, items, timed);
  if (rb == 1 && mb == 4) return launch_split_t<D, 1, 4>(g, p, items, timed);
  if (rb == 1 && mb == 8) return launch_split_t<D, 1, 8>(g, p, items, timed);
  if (rb == 2 && mb == 1) return launch_split_t<D, 2, 1>(g, p, items, timed);
  if (rb == 2 && mb == 2) return launch_split_t<D, 2, 2>(g, p, items, timed);
  if (rb == 2 && mb == 4) return launch_split_t<D, 2, 4>(g, p, items, timed);
  if (rb == 4 && mb == 1) return launch_split_t<D, 4, 1>(g, p, items, timed);
  if (rb == 4 && mb == 2) return launch_split_t<D, 4, 2>(g, p, items, timed);
  snprintf(g_err, sizeof g_err, "no decode kernel for rb=%d mb=%d", rb, mb);
  return SKV_ERR_UNSUPPORTED;
}

}  // namespace

namespace skv {

int dev_check(const Geometry& g) {
  if (g.ps != kPage) return SKV_ERR_UNSUPPORTED;
  if (g.G > kMaxDecodeRows) return SKV_ERR_UNSUPPORTED;
  if (group_limit(g) < 1) return SKV_ERR_UNSUPPORTED;
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
  // the static scratch's device address on the current device, once per device
  static std::mutex mu;
  static float* addr[64] = {};
  int dev = 0;
  e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= 64) {
    set_err("hipGetDevice", e);
    return SKV_ERR_HIP;
  }
  float* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
      e = hipGetSymbolAddress((void**)&addr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        addr[dev] = nullptr;
        set_err("hipGetSymbolAddress(scratch)", e);
        return SKV_ERR_HIP;
      }
    }
    ptr = addr[dev];
  }
  auto* st = new DevState();
  st->scratch_static = ptr;
  g.dev = st;
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
  plan_append(g, job, p);
  const int blocks = append_blocks(p);
  if (blocks == 0 && !job.update_tables) return SKV_OK;
  return launch(g, job.do_kv ? 0 : 1, append_kernel, dim3(std::max(blocks, 1)), 0, p, "append_kernel");
}

// The GEMM part takes the split form up to 16 rows (a decode step) and the
// wide or tall form beyond (the wide form measured 1.2-1.9x faster than 32-
// and 64-row tiles of four units from 24 to 2,048 rows at the llama3 and qwen3
// shapes; the tall form 1.08-1.3x faster than the wide one where it is taken).
constexpr int kProjectSplitRows = 16;
template <int D>
int launch_project_split(const Geometry& g, const ProjectParams& p) {
  const size_t lds = (size_t)4 * kSplitSlots * 6 * 512 * sizeof(u16);
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(project_split_kernel<D>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) {
    set_err("hipFuncSetAttribute(project_split_kernel)", attr);
    return SKV_ERR_HIP;
  }
  const int grid = 8 * p.per_xcd + append_blocks(p.app);
  return launch(g, 5, project_split_kernel<D>, dim3(grid), lds, p, "project_split_kernel");
}

constexpr int kWideSlots = 4;  // ring slots of the wide form
template <int D, int NH>
int launch_project_wide(const Geometry& g, const ProjectParams& p) {
  const size_t lds = (size_t)kWideSlots * (16 + 4 * NH) * 512 * sizeof(u16);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(project_wide_kernel<D, kWideSlots, NH>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) {
    set_err("hipFuncSetAttribute(project_wide_kernel)", attr);
    return SKV_ERR_HIP;
  }
  const int grid = 8 * p.per_xcd + append_blocks(p.app);
  return launch(g, 5, project_wide_kernel<D, kWideSlots, NH>, dim3(grid), lds, p, "project_wide_kernel",
                64 * (2 * NH + 4));
}

template <int D>
int launch_project_tall(const Geometry& g, const ProjectParams& p) {
  const size_t lds = (size_t)3 * 48 * 512 * sizeof(u16);
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(project_tall_kernel<D>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) {
    set_err("hipFuncSetAttribute(project_tall_kernel)", attr);
    return SKV_ERR_HIP;
  }
  const int grid = 8 * p.per_xcd + append_blocks(p.app);
  return launch(g, 5, project_tall_kernel<D>, dim3(grid), lds, p, "project_tall_kernel", 64 * 12);
}

// nh: 3 or 4 half units per 128-token tile, or 0 for the tall form
template <int D>
int launch_project(const Geometry& g, const ProjectParams& p, bool split, int nh) {
  if (split) return launch_project_split<D>(g, p);
  if (nh == 0) return launch_project_tall<D>(g, p);
  return nh == 3 ? launch_project_wide<D, 3>(g, p) : launch_project_wide<D, 4>(g, p);
}

int dev_pack_qkv(const Geometry& g, const uint16_t* w, uint16_t* out) {
  const int units = (g.Hq + 2 * g.Hkv) * g.D / 64;
  return launch(g, 5, pack_qkv_kernel, dim3(units * (g.hidden / 64)), 0, PackParams{w, out, g.D, g.hidden},
                "pack_qkv_kernel");
}

int dev_project(const Geometry& g, const ProjectJob& job) {
  const AppendJob& a = job.app;
  if (g.hidden % 64 != 0 || a.n_spans < 1) {
    set_err("project", hipErrorInvalidValue);
    return SKV_ERR_UNSUPPORTED;
  }
  // k and v come from the GEMM: the append part of the launch writes only the
  // low-rank rows and the table entries (its K/V copy blocks would read job.k).
  AppendJob aj = a;
  aj.do_kv = false;
  aj.k = aj.v = nullptr;
  ProjectParams p{};
  plan_append(g, aj, p.app);
  p.x = job.x;
  p.w = job.w;
  p.q = job.q;
  p.row0 = a.spans[0].src_row;
  p.rows = a.spans[a.n_spans - 1].src_row + a.spans[a.n_spans - 1].n - p.row0;
  p.n_units = (g.Hq + 2 * g.Hkv) * g.D / 64;
  // up to 16 rows: half a unit per workgroup (split K); more rows: tiles of
  // 128 tokens and three or four half units, whichever moves fewer bytes per
  // CU (rounds of workgroups over the CUs, the low-rank blocks included, x
  // bytes per tile: 16 + 4 NH KB a stage)
  const int nk = g.hidden / 64;
  const bool split = p.rows <= kProjectSplitRows;
  if (!split && (int64_t)p.n_units * nk * 8 * 1024 >= ((int64_t)1 << 31)) {
    set_err("project: packed weights of 2 GiB or more", hipErrorInvalidValue);
    return SKV_ERR_UNSUPPORTED;
  }
  int nh = 4;
  if (split) {
    p.tok_tiles = 1;
    p.n_gemm = 2 * p.n_units;
  } else {
    // rounds of workgroups over the CUs x KB copied per stage of a tile:
    // 128 tokens x 3 half units 28, x 4 half units 32, 256 tokens x 4 48
    const int64_t app = append_blocks(p.app);
    const int64_t tt128 = (p.rows + kWideRows - 1) / kWideRows, tt256 = (p.rows + kTallRows - 1) / kTallRows;
    const int64_t c4 = ((2 * p.n_units + 3) / 4 * tt128 + app + kCUs - 1) / kCUs * 32;
    const int64_t c3 = ((2 * p.n_units + 2) / 3 * tt128 + app + kCUs - 1) / kCUs * 28;
    const int64_t ct = ((2 * p.n_units + 3) / 4 * tt256 + app + kCUs - 1) / kCUs * 48;
    if (c3 < c4 && c3 <= ct) nh = 3;
    if (ct < c4 && ct < c3) nh = 0;
    p.tok_tiles = (int)(nh == 0 ? tt256 : tt128);
    p.n_gemm = (nh == 0 ? (p.n_units + 1) / 2 : (2 * p.n_units + nh - 1) / nh) * p.tok_tiles;
  }
  p.per_xcd = (p.n_gemm + 7) / 8;
  p.Hq = g.Hq;
  p.Hkv = g.Hkv;
  p.hidden = g.hidden;
  p.rope = job.theta != 0.f;
  for (int s = 0; s < a.n_spans; ++s) p.view_off[s] = job.view_off[s];
  for (int i = 0; i < g.D / 2; ++i) p.inv_freq[i] = p.rope ? std::pow((double)job.theta, -2.0 * i / g.D) : 0.0;
  return g.D == 128 ? launch_project<128>(g, p, split, nh) : launch_project<64>(g, p, split, nh);
}

// Decode for the agents of job, in groups that fit one launch. With app (a
// fused decode step) each group's split launch also writes the group's new
// rows and the merge adds the new tokens.
static int decode_impl(const Geometry& g, const AttnJob& job, const AppendJob* app, float* part, bool timed) {
  const int ng = group_limit(g);
  const int W = w_of(g);
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
    int max_b = 0;
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
      p.ag_lrb[i] = a.lr_begin;
      if (a.lr_begin > 0) p.lr_offsets = 1;
      max_b = std::max(max_b, a.b);
    }
    // A fused step writes the group's new rows: the low-rank rows (and new
    // page-table entries) from leading blocks of the split launch, which the
    // merge reads back for the new token; the K/V rows from trailing blocks of
    // the merge launch, which takes them from the inputs.
    AppendJob sub{};
    AppendParams kv_app{};
    int n_kv_app = 0;
    if (app) {
      sub.layer = app->layer;
      sub.k = app->k;
      sub.v = app->v;
      sub.x = app->x;
      for (int i = 0; i < n; ++i) {
        Span sp = app->spans[a0 + i];
        for (int t = 0; t < sp.n_pages; ++t) sub.ids[sub.n_ids + t] = app->ids[sp.ids_off + t];
        sp.ids_off = sub.n_ids;
        sub.n_ids += sp.n_pages;
        sub.spans[sub.n_spans++] = sp;
      }
      sub.do_kv = false;
      sub.do_lr = app->do_lr;
      sub.update_tables = app->update_tables;
      plan_append(g, sub, p.app);
      p.n_app = append_blocks(p.app);
      if (p.n_app == 0 && sub.update_tables) p.n_app = 1;  // the table update rides on block 0
      sub.do_kv = app->do_kv;
      sub.do_lr = false;
      sub.update_tables = false;
      plan_append(g, sub, kv_app);
      n_kv_app = append_blocks(kv_app);
      // the split launch's append code has no K/V copies and no MFMA low-rank
      // tiles, the merge launch's no low-rank rows at all
      bool fits = p.app.kv_block0[p.app.n_spans] == 0 && kv_app.lr_block0[kv_app.n_spans] == 0;
      for (int s = 0; s < p.app.n_spans; ++s) fits = fits && p.app.lr_kind[s] != 2;
      if (!fits) {
        snprintf(g_err, sizeof g_err, "decode step: an agent appends more than one row");
        return SKV_ERR_UNSUPPORTED;
      }
    }
    // flattened key sequence per KV head: shared prefix, then each own suffix,
    // each padded to whole 32-key chunks
    p.shared_len = (max_b + 31) / 32 * 32;
    p.shared_run = job.shared_run;
    p.seg_off[0] = p.shared_len;
    for (int i = 0; i < n; ++i) p.seg_off[i + 1] = p.seg_off[i] + (p.ag_S[i] + 31) / 32 * 32;
    const int chunks = p.seg_off[n] / 32;
    // items per KV head: the same plan the runtime has checked the call against
    const int items_per_head = skv::decode_items_per_head(chunks, p.n_app, g.Hkv);
    if (items_per_head < 0) {
      snprintf(g_err, sizeof g_err, "decode view too long for the split plan (%d keys)", p.seg_off[n]);
      return SKV_ERR_UNSUPPORTED;
    }
    p.head_chunks = chunks;
    p.items_per_head = items_per_head;
    p.scale_log2 = 1.4426950408889634f / sqrtf((float)g.D);
    int rb = (p.R + 15) / 16;
    rb = rb <= 1 ? 1 : (rb <= 2 ? 2 : 4);
    int mb = (p.n_planes * g.r + 15) / 16;
    mb = mb <= 1 ? 1 : (mb <= 2 ? 2 : (mb <= 4 ? 4 : 8));
    const int items = items_per_head * g.Hkv;
    int rc = SKV_OK;
    if (p.n_app + items > 0)
      rc = g.D == 128 ? launch_split_d<128>(g, rb, mb, p, items, timed) : launch_split_d<64>(g, rb, mb, p, items, timed);
    if (rc != SKV_OK) return rc;
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
    mp.items_per_head = items_per_head;
    if (app) {
      mp.step = 1;
      mp.q = p.q;
      mp.k_new = app->k + (uint64_t)a0 * g.Hkv * g.D;
      mp.v_new = app->v + (uint64_t)a0 * g.Hkv * g.D;
      mp.LRT = p.LRT;
      mp.lr_plane = g.lr_plane();
      for (int i = 0; i < n; ++i) {
        const Span& sp = app->spans[a0 + i];
        mp.new_page[i] = app->ids[sp.ids_off];
        mp.new_slot[i] = sp.pos0 % kPage;
        mp.plane[i] = sp.plane;
        const AttnAgent& ag = job.ag[a0 + i];
        mp.new_lr_on[i] = ag.b + ag.S >= ag.lr_begin;  // the new token's view position
      }
      mp.scale_log2 = p.scale_log2;
      mp.app = kv_app;
      mp.n_app = n_kv_app;
    }
    mp.n_rows = n * g.Hkv * g.G;
    const size_t mlds = mp.n_app ? (size_t)64 * (128 + 8) * 2 : 0;
    const int kind = timed ? 3 : -1;
    // a row's slots beyond what 256 threads hold in one batch: 1024 threads per row
    const bool wide = items_per_head > kMergeVec * std::min(8, 256 / ((g.D + g.r) / 4));
    const dim3 mgrid(mp.n_rows + mp.n_app);
    if (g.D == 128)
      rc = wide ? launch(g, kind, decode_merge_kernel<128, 1024>, mgrid, mlds, mp, "decode_merge_kernel", 1024)
                : launch(g, kind, decode_merge_kernel<128, 256>, mgrid, mlds, mp, "decode_merge_kernel");
    else
      rc = wide ? launch(g, kind, decode_merge_kernel<64, 1024>, mgrid, mlds, mp, "decode_merge_kernel", 1024)
                : launch(g, kind, decode_merge_kernel<64, 256>, mgrid, mlds, mp, "decode_merge_kernel");
    if (rc != SKV_OK) return rc;
  }
  return SKV_OK;
}

static_assert(sizeof(DecodeParams) <= 4096, "kernel arguments too large");
static_assert(sizeof(MergeParams) <= 4096, "kernel arguments too large");
static_assert(sizeof(AppendParams) <= 4096, "kernel arguments too large");
static_assert(sizeof(PrefillParams) <= 4096, "kernel arguments too large");

// Time `reps` launches of a probe with dispatch events; return the shortest
// interval in milliseconds (or a negative HIP error).
template <typename Kernel, typename... Args>
static double probe_best_ms(hipStream_t st, int reps, dim3 grid, Kernel kernel, Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -1.0;
  double best = 1e30;
  for (int r = 0; r < reps; ++r) {
    hipExtLaunchKernelGGL(kernel, grid, dim3(256), 0, st, a, b, 0, args...);
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(b) != hipSuccess) {
      best = -1.0;
      break;
    }
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, a, b);
    best = std::min(best, (double)ms);
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return best;
}

int dev_probe_stream_read(const void* src, uint64_t bytes, int reps, void* stream, double* gbs) {
  const double ms = probe_best_ms((hipStream_t)stream, reps, dim3(16384), probe_stream_kernel,
                                  (const u32x4*)src, (size_t)(bytes / 16));
  if (ms <= 0) {
    set_err("probe_stream_kernel", hipGetLastError());
    return SKV_ERR_HIP;
  }
  *gbs = (double)bytes / (ms * 1e-3) / 1e9;
  return SKV_OK;
}

int dev_probe_mfma_bf16(void* stream, double* tflops) {
  constexpr int kIters = 2048, kBlocks = 2 * kCUs;  // two waves per SIMD
  const double ms = probe_best_ms((hipStream_t)stream, 3, dim3(kBlocks), probe_mfma_kernel, kIters);
  if (ms <= 0) {
    set_err("probe_mfma_kernel", hipGetLastError());
    return SKV_ERR_HIP;
  }
  const double flops = (double)kBlocks * 4 * kIters * 8 * (16.0 * 16 * 32 * 2);
  *tflops = flops / (ms * 1e-3) / 1e12;
  return SKV_OK;
}

// `steps` steps of `layers` layers: per layer one probe_layer_kernel over that
// layer's bytes, then (with_tail) one probe_tail_kernel of tail_blocks
// workgroups; one untimed step first; ms per step, the best of three runs.
static double probe_pattern_ms(hipStream_t st, const char* src, uint64_t layer_bytes, int layers, int steps,
                               int tail_blocks, bool with_tail) {
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -1.0;
  const size_t n = (size_t)(layer_bytes / 16);
  double best = 1e30;
  for (int run = 0; run < 3 && best > 0; ++run) {
    for (int s = -1; s < steps; ++s) {
      if (s == 0) (void)hipEventRecord(a, st);
      for (int l = 0; l < layers; ++l) {
        hipLaunchKernelGGL(probe_layer_kernel, dim3(kCUs), dim3(256), 0, st,
                           (const u32x4*)(src + (uint64_t)l * layer_bytes), n);
        if (with_tail) hipLaunchKernelGGL(probe_tail_kernel, dim3(tail_blocks), dim3(256), 0, st);
      }
    }
    (void)hipEventRecord(b, st);
    if (hipGetLastError() != hipSuccess || hipEventSynchronize(b) != hipSuccess) {
      best = -1.0;
      break;
    }
    float ms = 0.f;
    (void)hipEventElapsedTime(&ms, a, b);
    best = std::min(best, (double)ms / steps);
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return best;
}

int dev_probe_launch_pattern(const void* src, uint64_t layer_bytes, int layers, int steps, int tail_blocks,
                             void* stream, double* ms_pattern, double* ms_stream) {
  const hipStream_t st = (hipStream_t)stream;
  const double pat = probe_pattern_ms(st, (const char*)src, layer_bytes, layers, steps, tail_blocks, true);
  const double str = pat > 0 ? probe_pattern_ms(st, (const char*)src, layer_bytes, layers, steps, tail_blocks, false)
                             : -1.0;
  if (pat <= 0 || str <= 0) {
    set_err("probe_layer_kernel / probe_tail_kernel", hipGetLastError());
    return SKV_ERR_HIP;
  }
  *ms_pattern = pat;
  *ms_stream = str;
  return SKV_OK;
}

int dev_probe_mfma_bf16_data(const void* src, void* stream, double* tflops) {
  // long enough (about 10 ms) for the clock to settle under the power limit
  constexpr int kIters = 65536, kBlocks = 2 * kCUs;  // two waves per SIMD
  const double ms = probe_best_ms((hipStream_t)stream, 3, dim3(kBlocks), probe_mfma_data_kernel,
                                  (const u32x4*)src, kIters);
  if (ms <= 0) {
    set_err("probe_mfma_data_kernel", hipGetLastError());
    return SKV_ERR_HIP;
  }
  const double flops = (double)kBlocks * 4 * kIters * 8 * (16.0 * 16 * 32 * 2);
  *tflops = flops / (ms * 1e-3) / 1e12;
  return SKV_OK;
}

float* arena_partials(const Geometry& g) { return (float*)(g.arena + g.scratch_off); }

int dev_attn_decode(const Geometry& g, const AttnJob& job) {
  return decode_impl(g, job, nullptr, arena_partials(g), true);
}

int dev_decode_step(const Geometry& g, const AttnJob& job, const AppendJob& app) {
  return decode_impl(g, job, &app, arena_partials(g), true);
}

// The partial rows go to the static scratch (the runtime has checked that the
// call's largest launch fits it); nothing is allocated and no events recorded.
int dev_decode_step_static(const Geometry& g, const AttnJob& job, const AppendJob& app) {
  auto* st = (DevState*)g.dev;
  return decode_impl(g, job, &app, st->scratch_static, false);
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
  const int mb = (g.r + 15) / 16;
  const int rows = prefill_rows(mb);
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
    p.ag_lrb[i] = a.lr_begin;
    p.blk0[i + 1] = p.blk0[i] + (a.n_q * g.G + rows - 1) / rows;
  }
  p.scale_log2 = 1.4426950408889634f / sqrtf((float)g.D);
  const int nblk = p.blk0[job.n] * g.Hkv;
  if (nblk == 0) return SKV_OK;
  int min_view_pages = 1 << 30;
  for (int i = 0; i < job.n; ++i)
    min_view_pages = std::min(min_view_pages, (job.ag[i].b + job.ag[i].S + kPage - 1) / kPage);
  const int ks = prefill_split(nblk, min_view_pages);
  static_assert((uint64_t)kCUs * prefill_rows(1) <= (uint64_t)kMaxItems * kMaxDecodeRows,
                "split prefill partials fit the decode scratch");
  p.ksplit = ks;
  p.nblk = nblk;
  p.W = w_of(g);
  p.part = (float*)(g.arena + g.scratch_off);
  bool lro = false;  // some agent's adapter activation offset lies inside its view
  for (int i = 0; i < job.n; ++i) lro |= job.ag[i].lr_begin > 0;
  const int blocks = nblk * ks;
  int rc;
  if (g.D == 128)
    rc = mb == 1 ? launch_prefill_o<128, 1>(g, p, blocks, lro) : launch_prefill_o<128, 2>(g, p, blocks, lro);
  else
    rc = mb == 1 ? launch_prefill_o<64, 1>(g, p, blocks, lro) : launch_prefill_o<64, 2>(g, p, blocks, lro);
  if (rc != SKV_OK || ks == 1) return rc;
  PrefillMergeParams mp{};
  mp.part = p.part;
  mp.B = job.B;
  mp.o = job.o;
  mp.Hkv = g.Hkv;
  mp.Hq = g.Hq;
  mp.G = g.G;
  mp.r = g.r;
  mp.W = p.W;
  mp.ksplit = ks;
  mp.nblk = nblk;
  mp.n = job.n;
  for (int i = 0; i <= job.n; ++i) mp.blk0[i] = p.blk0[i];
  for (int i = 0; i < job.n; ++i) {
    mp.ag_id[i] = p.ag_id[i];
    mp.ag_nq[i] = p.ag_nq[i];
    mp.ag_row0[i] = p.ag_row0[i];
  }
  const dim3 grid((nblk * rows + 3) / 4);
  return g.D == 128 ? launch(g, 4, prefill_merge_kernel<128>, grid, 0, mp, "prefill_merge_kernel")
                    : launch(g, 4, prefill_merge_kernel<64>, grid, 0, mp, "prefill_merge_kernel");
}

int dev_sync(const Geometry& g) {
  hipError_t e = hipStreamSynchronize((hipStream_t)g.stream);
  if (e != hipSuccess) {
    set_err("hipStreamSynchronize", e);
    return SKV_ERR_HIP;
  }
  return SKV_OK;
}

int dev_set_timing(Geometry& g, int mask) {
  auto* st = (DevState*)g.dev;
  st->timing = mask;
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
