// Internal interface between the host runtime (runtime.cpp) and a device
// backend. The HIP backend (kernels.hip) runs the work on the GPU; the null
// backend (backend_null.cpp) accepts every job without touching memory, so the
// host metadata (lengths, page tables, validation) can be tested on a CPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "skv.h"

namespace skv {

constexpr int kMaxJobPages = 64;  // page ids carried by one append launch
constexpr int kMaxJobSpans = 16;  // row spans carried by one append launch

struct Geometry {
  int L, Hq, Hkv, G, D, hidden, r, N, mode, ps, max_pages, planes;
  char* arena;  // device address of the arena
  uint64_t k_off, vt_off, lrt_off, tbl_off, scratch_off, scratch_bytes, arena_bytes;
  void* stream;            // hipStream_t
  void* dev;               // backend state (dev_init / dev_fini)
  int64_t* launches;       // incremented once per device launch

  // element strides (bf16 elements) of the pools
  uint64_t k_page() const { return (uint64_t)Hkv * ps * D; }              // one page, all heads
  uint64_t k_layer() const { return (uint64_t)max_pages * k_page(); }
  uint64_t lr_page() const { return (uint64_t)r * ps; }
  uint64_t lr_layer() const { return (uint64_t)max_pages * lr_page(); }
  uint64_t lr_plane() const { return (uint64_t)L * lr_layer(); }
  uint64_t tbl_seq() const { return (uint64_t)max_pages; }                // int32 entries
  uint64_t tbl_layer() const { return (uint64_t)(N + 1) * tbl_seq(); }
};

// Rows [pos0, pos0 + n) of one sequence at one layer. The pages holding them
// are page indices first_page .. first_page + n_pages - 1 of the sequence,
// with ids ids[ids_off .. ids_off + n_pages) of the job.
struct Span {
  int32_t seq_slot;   // 0 = shared sequence, 1 + a = agent a
  int32_t pos0, n;
  int32_t src_row;    // first row of this span in the job's k / v / x
  int32_t first_page, n_pages, ids_off;
  int32_t plane;      // low-rank plane written by this span
  const uint16_t* a;  // [hidden][r] down-projection for this span (low-rank part)
};

struct AppendJob {
  int layer;
  bool do_kv, do_lr, update_tables;
  const uint16_t* k;  // [rows][Hkv][D]
  const uint16_t* v;
  const uint16_t* x;  // [rows][hidden]; nullptr = zero low-rank rows
  int n_spans;
  Span spans[kMaxJobSpans];
  int n_ids;
  int32_t ids[kMaxJobPages];
};

struct AttnAgent {
  int32_t agent, b, S, plane, n_q, q_row0;
  int32_t lr_begin;  // view positions below it take no low-rank term
};

struct AttnJob {
  int layer;
  int n;
  // First page id when the shared pages every view of the job reads are one
  // run of consecutive ids (shared page i is shared_run + i), else -1.
  int32_t shared_run = -1;
  AttnAgent ag[SKV_MAX_AGENTS];
  const uint16_t* q;  // [sum n_q][Hq][D]
  const uint16_t* B;  // [N][r][Hkv*D]
  uint16_t* o;        // [sum n_q][Hq][D]
};

// Front end: the projections of one append job's rows (app: spans with
// src_row indexing x and q, pages, low-rank rows, table update; app.k and
// app.v are unused): q, k, v = x W^T, rotary embedding (base theta, 0 = none)
// on q and k at view position view_off[span] + own row index. q goes to the
// caller's rows, k and v into the job's pages.
struct ProjectJob {
  AppendJob app;
  const uint16_t* x;  // [rows of the call][hidden]
  const uint16_t* w;  // packed projection weights (skv_pack_qkv)
  uint16_t* q;        // [rows of the call][Hq][D]
  float theta;
  int32_t view_off[kMaxJobSpans];
};

// Backend entry points. Each returns an skv_status.
int dev_check(const Geometry& g);             // SKV_ERR_UNSUPPORTED if the shape is not handled
uint64_t dev_scratch_bytes(const Geometry& g);  // device scratch the backend needs in the arena
int dev_init(Geometry& g);
void dev_fini(Geometry& g);
int dev_append(const Geometry& g, const AppendJob& job);
int dev_attn_decode(const Geometry& g, const AttnJob& job);
int dev_project(const Geometry& g, const ProjectJob& job);
int dev_pack_qkv(const Geometry& g, const uint16_t* w, uint16_t* out);
// Fused decode step: job holds lengths before the step; app appends one row
// per agent (in the same order as job.ag).
int dev_decode_step(const Geometry& g, const AttnJob& job, const AppendJob& app);
// The same with the partial rows in the library's static device scratch
// (kStaticScratchBytes, one array per device): no device memory is allocated,
// no timing events are recorded.
int dev_decode_step_static(const Geometry& g, const AttnJob& job, const AppendJob& app);
int dev_attn_prefill(const Geometry& g, const AttnJob& job);
int dev_sync(const Geometry& g);
int dev_set_timing(Geometry& g, int mask);
int dev_collect_timing(Geometry& g, skv_kernel_times* out);
const char* dev_last_error();
// measurement probes (no context): see skv_probe_stream_read / skv_probe_mfma_bf16 /
// skv_probe_mfma_bf16_data / skv_probe_launch_pattern
int dev_probe_stream_read(const void* src, uint64_t bytes, int reps, void* stream, double* gbs);
int dev_probe_mfma_bf16(void* stream, double* tflops);
int dev_probe_mfma_bf16_data(const void* src, void* stream, double* tflops);
int dev_probe_launch_pattern(const void* src, uint64_t layer_bytes, int layers, int steps, int tail_blocks,
                             void* stream, double* ms_pattern, double* ms_stream);

}  // namespace skv
