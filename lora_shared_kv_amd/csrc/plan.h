// Launch plans of the GPU build and their limits, shared by the host runtime
// and the HIP backend. The runtime checks every attention call against these
// limits before it enqueues anything (SKV_ERR_UNSUPPORTED otherwise), and the
// backend builds its launches from the same functions, so a call that passes
// the check runs whole. The CPU-only build applies the same checks, which
// lets the limits be tested without a GPU.
#pragma once

#include <algorithm>
#include <cstdio>

#include "backend.h"

namespace skv {

constexpr int kDecodeChunk = 32;       // keys per decode chunk (one MFMA score tile pair)
constexpr int kMaxDecodeRows = 64;     // query rows (agents x G) per decode launch
constexpr int kMaxItems = 2048;        // decode work items per launch (the partial rows' capacity)
constexpr int kMaxMergeSlots = 1024;   // items per KV head (the merge keeps one weight per item in LDS)
constexpr int kMaxItemChunks = 512;    // chunks per decode item (the item's chunk table in LDS)
constexpr int kPlanPage = 64;          // rows per page of the GPU build
constexpr int kMaxViewPages = 4096;    // prefill: pages of one view (its page list in LDS)
constexpr int kPlanCUs = 256;          // compute units a decode launch fills

// Agents per decode launch: query rows <= 64, stacked low-rank ranks <= 128,
// and (16-row blocks x 16-rank blocks) <= 8. 0 if no agent fits.
inline int decode_group_limit(int N, int G, int mode, int r) {
  for (int ng = std::min(N, kMaxDecodeRows / G); ng >= 1; --ng) {
    const int planes = mode == SKV_BASE_SHARED ? ng : 1;
    int rb = (ng * G + 15) / 16;
    rb = rb <= 1 ? 1 : (rb <= 2 ? 2 : 4);
    int mb = (planes * r + 15) / 16;
    mb = mb <= 1 ? 1 : (mb <= 2 ? 2 : (mb <= 4 ? 4 : 8));
    if (planes * r <= 128 && rb * mb <= 8) return ng;
  }
  return 0;
}

// 32-key chunks per KV head of one decode launch over agents ag[0..n): the
// shared prefix up to the largest b_i, then each agent's own suffix, each
// padded to whole chunks.
inline long decode_group_chunks(const AttnAgent* ag, int n) {
  long max_b = 0, own = 0;
  for (int i = 0; i < n; ++i) {
    max_b = std::max<long>(max_b, ag[i].b);
    own += (ag[i].S + kDecodeChunk - 1) / kDecodeChunk;
  }
  return (max_b + kDecodeChunk - 1) / kDecodeChunk + own;
}

// Items per KV head of the split pass of a decode launch over `chunks` chunks
// per head, with n_app leading append blocks: as many as leave one CU per
// workgroup, each a balanced run of whole chunks, at most kMaxItemChunks each.
// 0 when nothing is cached yet (the merge alone takes the new token); -1 when
// the launch would exceed the item capacities.
inline int decode_items_per_head(long chunks, int n_app, int Hkv) {
  if (chunks <= 0) return 0;
  long I = std::min<long>(chunks, std::max(1, (kPlanCUs - n_app) / Hkv));
  I = std::max<long>(I, (chunks + kMaxItemChunks - 1) / kMaxItemChunks);
  if (I * Hkv > kMaxItems || I > kMaxMergeSlots) return -1;
  return (int)I;
}

// SKV_OK if every launch of a decode call (step: a fused decode step, whose
// split launches carry one leading append block per agent) fits the plan.
inline int plan_check_decode(const Geometry& g, const AttnJob& job, bool step, char* msg, size_t cap) {
  const int ng = decode_group_limit(g.N, g.G, g.mode, g.r);
  if (ng < 1) {
    snprintf(msg, cap, "no decode plan for this shape");
    return SKV_ERR_UNSUPPORTED;
  }
  for (int a0 = 0; a0 < job.n; a0 += ng) {
    const int n = std::min(ng, job.n - a0);
    const long chunks = decode_group_chunks(job.ag + a0, n);
    if (decode_items_per_head(chunks, step ? n : 0, g.Hkv) < 0) {
      snprintf(msg, cap, "decode views too long for one launch (%ld chunks of %d keys per KV head)", chunks,
               kDecodeChunk);
      return SKV_ERR_UNSUPPORTED;
    }
  }
  return SKV_OK;
}

// Bytes of decode partial rows the largest launch of a decode call writes:
// items x (agents x G) rows x (d + r + 4) fp32 values.
inline uint64_t decode_partial_bytes(const Geometry& g, const AttnJob& job, bool step) {
  const int ng = decode_group_limit(g.N, g.G, g.mode, g.r);
  uint64_t most = 0;
  for (int a0 = 0; ng > 0 && a0 < job.n; a0 += ng) {
    const int n = std::min(ng, job.n - a0);
    const int I = decode_items_per_head(decode_group_chunks(job.ag + a0, n), step ? n : 0, g.Hkv);
    if (I > 0) most = std::max(most, (uint64_t)I * g.Hkv * n * g.G * (g.D + g.r + 4) * sizeof(float));
  }
  return most;
}

// Size of the library's static device scratch (the partial rows of the
// decode entry point that allocates nothing, skv_decode_step_static).
constexpr uint64_t kStaticScratchBytes = 16ull << 20;

// SKV_OK if every agent's view of a prefill call fits the prefill kernel's
// page list (4096 pages of 64 rows: 262,144 rows, shared and own pages
// counted separately).
inline int plan_check_prefill(const AttnJob& job, char* msg, size_t cap) {
  for (int i = 0; i < job.n; ++i) {
    const AttnAgent& a = job.ag[i];
    const long pages = (a.b + kPlanPage - 1) / kPlanPage + (long)(a.S + kPlanPage - 1) / kPlanPage;
    if (pages > kMaxViewPages) {
      snprintf(msg, cap, "agent %d: a view of %d rows exceeds the prefill limit (%d pages of %d rows)", a.agent,
               a.b + a.S, kMaxViewPages, kPlanPage);
      return SKV_ERR_UNSUPPORTED;
    }
  }
  return SKV_OK;
}

// SKV_OK if the front end can stream the packed projection weights: the wide
// form addresses them with 32-bit byte offsets, so they must stay below 2 GiB.
inline int plan_check_project(const Geometry& g, char* msg, size_t cap) {
  const uint64_t bytes = (uint64_t)(g.Hq + 2 * g.Hkv) * g.D * g.hidden * 2;
  if (bytes >= (1ull << 31)) {
    snprintf(msg, cap, "packed projection weights of %llu bytes (the front end takes less than 2 GiB)",
             (unsigned long long)bytes);
    return SKV_ERR_UNSUPPORTED;
  }
  return SKV_OK;
}

}  // namespace skv
