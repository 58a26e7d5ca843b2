// Host runtime of the shared-prefix multi-LoRA attention library: the C ABI
// declared in include/skv.h. It validates every call, owns the metadata of
// the paged store (lengths, page tables, low-rank coverage, free pages), and
// turns each call into backend jobs. It never allocates device memory and
// never waits for the GPU except in skv_sync / skv_collect_timing.
//
// Store model (readings of the pages; see include/skv.h for the sources):
//   one shared sequence per layer holds base-weight K/V computed once
//   (LRAgent review Fig. 2; paperlayer summary of arXiv 2609.17109 Sec. 2),
//   agent i's view is SHARED[0:b_i] ++ OWN_i[0:S_i], pages are page_size
//   rows, a new page takes the lowest free id of its layer, and a crop frees
//   the pages lying wholly beyond the new length (paperlayer Sec. 3.2: a
//   paged cache is the route to physical sharing; RoleKV "How we built it":
//   crop at a handoff).
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <initializer_list>
#include <set>
#include <string>
#include <vector>

#include "backend.h"
#include "plan.h"

namespace {

using skv::AppendJob;
using skv::AttnJob;
using skv::Geometry;
using skv::Span;

struct Layer {
  std::set<int32_t> free;                   // free page ids; *begin() is the lowest
  std::vector<std::vector<int32_t>> tbl;    // [1 + N] page ids per sequence slot
  std::vector<int> len;                     // [1 + N] rows per sequence slot
  std::vector<int> lr_shared;               // [planes] low-rank rows over the shared sequence
  std::vector<int> lr_own;                  // [N] low-rank rows over each agent's own rows
};

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Device tensors are read and written with 16-byte vector accesses.
bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if ((uintptr_t)p & 15) return false;
  return true;
}
uint64_t align256(uint64_t x) { return (x + 255) & ~uint64_t(255); }

bool valid_config(const skv_config* c) {
  if (!c) return false;
  auto pow2 = [](int x) { return x > 0 && (x & (x - 1)) == 0; };
  return c->n_layers >= 1 && c->n_kv_heads >= 1 && c->n_q_heads >= c->n_kv_heads &&
         c->n_q_heads % c->n_kv_heads == 0 && (c->head_dim == 64 || c->head_dim == 128) &&
         (c->rank == 4 || c->rank == 8 || c->rank == 16 || c->rank == 32) && c->n_agents >= 1 &&
         c->n_agents <= SKV_MAX_AGENTS &&
         (c->mode == SKV_BASE_SHARED || c->mode == SKV_BASE_LR_SHARED) && c->hidden >= 64 &&
         c->hidden % 64 == 0 && pow2(c->page_size) && c->page_size >= 4 &&
         c->page_size <= 1024 && c->max_pages >= 1;
}

Geometry geometry_of(const skv_config* c) {
  Geometry g{};
  g.L = c->n_layers;
  g.Hq = c->n_q_heads;
  g.Hkv = c->n_kv_heads;
  g.G = c->n_q_heads / c->n_kv_heads;
  g.D = c->head_dim;
  g.hidden = c->hidden;
  g.r = c->rank;
  g.N = c->n_agents;
  g.mode = c->mode;
  g.ps = c->page_size;
  g.max_pages = c->max_pages;
  g.planes = c->mode == SKV_BASE_SHARED ? c->n_agents : 1;
  uint64_t off = 0;
  g.k_off = off;
  off = align256(off + 2 * (uint64_t)g.L * g.k_layer());
  g.vt_off = off;
  off = align256(off + 2 * (uint64_t)g.L * g.k_layer());
  g.lrt_off = off;
  off = align256(off + 2 * (uint64_t)g.planes * g.lr_plane());
  g.tbl_off = off;
  off = align256(off + 4 * (uint64_t)g.L * g.tbl_layer());
  g.scratch_off = off;
  g.scratch_bytes = align256(skv::dev_scratch_bytes(g));
  off += g.scratch_bytes;
  g.arena_bytes = off;
  return g;
}

}  // namespace

struct skv_ctx {
  Geometry g{};
  std::vector<Layer> layers;
  std::vector<int> base_len;
  std::vector<int> lr_begin;  // per agent: first view position with the adapter term on
  skv_counters counters{};
  std::string err;

  int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    err = buf;
    return code;
  }
  int plane_of(int agent) const { return g.mode == SKV_BASE_SHARED ? agent : 0; }
  static int slot_of(int seq) { return seq + 1; }  // SHARED -> 0, agent a -> 1 + a
  bool seq_ok(int seq) const { return seq == SKV_SHARED || (seq >= 0 && seq < g.N); }
  int min_len(int slot) const {
    int m = layers[0].len[slot];
    for (auto& l : layers) m = std::min(m, l.len[slot]);
    return m;
  }
  int max_base() const {
    int m = 0;
    for (int b : base_len) m = std::max(m, b);
    return m;
  }
  // Release pages of (layer, slot) whose index is >= ceil(new_len / ps).
  void free_beyond(Layer& l, int slot, int new_len) {
    size_t keep = (size_t)ceil_div(new_len, g.ps);
    auto& t = l.tbl[slot];
    for (size_t i = keep; i < t.size(); ++i) {
      l.free.insert(t[i]);
      counters.pages_freed++;
    }
    if (t.size() > keep) t.resize(keep);
  }
};

namespace {

// Split rows [pos0, pos0 + n) of a sequence into spans that fit the job limits
// and append them to jobs (opening new jobs when a job is full).
void add_spans(const skv_ctx* c, std::vector<AppendJob>& jobs, const AppendJob& proto,
               const std::vector<int32_t>& table, int slot, int pos0, int n, int src_row,
               int plane, const uint16_t* a) {
  const int ps = c->g.ps;
  int done = 0;
  while (done < n) {
    if (jobs.empty() || jobs.back().n_spans == skv::kMaxJobSpans ||
        jobs.back().n_ids == skv::kMaxJobPages) {
      jobs.push_back(proto);
    }
    AppendJob& j = jobs.back();
    int p = pos0 + done;
    int first_page = p / ps;
    int room = skv::kMaxJobPages - j.n_ids;
    // rows until the end of the last page that still fits in this job
    int last_row_excl = (first_page + room) * ps;
    int take = std::min(n - done, last_row_excl - p);
    int n_pages = ceil_div(p + take, ps) - first_page;
    Span s{};
    s.seq_slot = slot;
    s.pos0 = p;
    s.n = take;
    s.src_row = src_row + done;
    s.first_page = first_page;
    s.n_pages = n_pages;
    s.ids_off = j.n_ids;
    s.plane = plane;
    s.a = a;
    for (int i = 0; i < n_pages; ++i) j.ids[j.n_ids++] = table[first_page + i];
    j.spans[j.n_spans++] = s;
    done += take;
  }
}

// Bounds checks on what a launch will touch, run on the host before each
// launch (no device traps): every page id inside the pool; every span's rows
// inside the pages the job carries for it, those pages being the ones its
// sequence's table holds (or will hold) at those positions. A failure is a
// broken invariant of the store's metadata; the call fails before anything
// is enqueued.
using TableOf = std::function<const std::vector<int32_t>&(int slot)>;

bool job_in_bounds(const skv_ctx* c, const AppendJob& j, const TableOf& table_of, char* msg, size_t cap) {
  const Geometry& g = c->g;
  if (j.n_spans < 0 || j.n_spans > skv::kMaxJobSpans || j.n_ids < 0 || j.n_ids > skv::kMaxJobPages) {
    snprintf(msg, cap, "job with %d spans and %d page ids", j.n_spans, j.n_ids);
    return false;
  }
  for (int i = 0; i < j.n_ids; ++i)
    if (j.ids[i] < 0 || j.ids[i] >= g.max_pages) {
      snprintf(msg, cap, "page id %d outside the pool of %d pages", j.ids[i], g.max_pages);
      return false;
    }
  for (int s = 0; s < j.n_spans; ++s) {
    const Span& sp = j.spans[s];
    const bool ok = sp.seq_slot >= 0 && sp.seq_slot <= g.N && sp.pos0 >= 0 && sp.n > 0 && sp.src_row >= 0 &&
                    sp.first_page == sp.pos0 / g.ps && sp.n_pages == ceil_div(sp.pos0 + sp.n, g.ps) - sp.first_page &&
                    sp.ids_off >= 0 && sp.ids_off + sp.n_pages <= j.n_ids && sp.plane >= 0 && sp.plane < g.planes;
    if (!ok) {
      snprintf(msg, cap, "span %d (rows %d..%d of slot %d) does not fit its pages", s, sp.pos0, sp.pos0 + sp.n,
               sp.seq_slot);
      return false;
    }
    {
      const std::vector<int32_t>& t = table_of(sp.seq_slot);
      for (int i = 0; i < sp.n_pages; ++i)
        if (sp.first_page + i >= (int)t.size() || t[sp.first_page + i] != j.ids[sp.ids_off + i]) {
          snprintf(msg, cap, "span %d: page %d of slot %d is not the table's", s, sp.first_page + i, sp.seq_slot);
          return false;
        }
    }
  }
  return true;
}

// Every page of each listed agent's view (shared pages below b, own pages
// below S) is in its table and inside the pool.
bool views_in_bounds(const skv_ctx* c, const AttnJob& job, char* msg, size_t cap) {
  const Geometry& g = c->g;
  const Layer& l = c->layers[job.layer];
  for (int i = 0; i < job.n; ++i) {
    const skv::AttnAgent& a = job.ag[i];
    const std::vector<int32_t>* ts[2] = {&l.tbl[0], &l.tbl[1 + a.agent]};
    const int need[2] = {ceil_div(a.b, g.ps), ceil_div(a.S, g.ps)};
    for (int k = 0; k < 2; ++k) {
      if ((int)ts[k]->size() < need[k]) {
        snprintf(msg, cap, "agent %d: %d pages in its %s table, the view needs %d", a.agent, (int)ts[k]->size(),
                 k ? "own" : "shared", need[k]);
        return false;
      }
      for (int p = 0; p < need[k]; ++p)
        if ((*ts[k])[p] < 0 || (*ts[k])[p] >= g.max_pages) {
          snprintf(msg, cap, "agent %d: page id %d outside the pool", a.agent, (*ts[k])[p]);
          return false;
        }
    }
  }
  return true;
}

int run_jobs(skv_ctx* c, const std::vector<AppendJob>& jobs, const TableOf& table_of) {
  char msg[256];
  for (auto& j : jobs)
    if (!job_in_bounds(c, j, table_of, msg, sizeof msg)) return c->fail(SKV_ERR_STATE, "bounds check: %s", msg);
  for (auto& j : jobs) {
    int rc = skv::dev_append(c->g, j);
    if (rc != SKV_OK) return c->fail(rc, "device append failed: %s", skv::dev_last_error());
  }
  return SKV_OK;
}

// Checks shared by the calls that append own rows to listed agents, in the
// order every call follows (arguments, then state, then pages): layer,
// distinct agents, counts; for a call with rows, arg_err (the caller's
// pointer and argument checks, nullptr if they passed); then low-rank rows
// level with base rows. total gets the row count.
int check_agent_rows(skv_ctx* c, int layer, int n, const int* agents, const int* counts, long* total,
                     const char* arg_err) {
  const Geometry& g = c->g;
  *total = 0;
  if (layer < 0 || layer >= g.L) return c->fail(SKV_ERR_ARG, "layer %d out of range", layer);
  if (n < 0 || n > g.N) return c->fail(SKV_ERR_ARG, "agent count %d", n);
  if (n == 0) return SKV_OK;
  if (!agents || !counts) return c->fail(SKV_ERR_ARG, "null agents or counts");
  uint32_t seen = 0;
  for (int i = 0; i < n; ++i) {
    int a = agents[i];
    if (a >= 0 && a < g.N && (seen >> a & 1u)) return c->fail(SKV_ERR_ARG, "duplicate agent %d", a);
    if (a >= 0 && a < g.N) seen |= 1u << a;
  }
  long tot = 0;
  for (int i = 0; i < n; ++i) {
    int a = agents[i];
    if (a < 0 || a >= g.N || counts[i] < 0)
      return c->fail(SKV_ERR_ARG, "agent list entry %d (count %d)", a, counts[i]);
    tot += counts[i];
  }
  if (tot == 0) return SKV_OK;
  if (arg_err) return c->fail(SKV_ERR_ARG, "%s", arg_err);
  const Layer& l = c->layers[layer];
  for (int i = 0; i < n; ++i) {
    int slot = 1 + agents[i];
    if (l.lr_own[agents[i]] != l.len[slot])
      return c->fail(SKV_ERR_STATE, "agent %d low-rank rows (%d) lag base rows (%d)", agents[i],
                     l.lr_own[agents[i]], l.len[slot]);
  }
  *total = tot;
  return SKV_OK;
}

// Pages and jobs of a checked agent-row append. The pages are taken from the
// free list now; finish_agent_rows commits them or gives them back.
struct AgentRows {
  std::vector<std::vector<int32_t>> tables;
  std::vector<int32_t> taken;
  std::vector<AppendJob> jobs;
  int need = 0;
};

int plan_agent_rows(skv_ctx* c, int layer, int n, const int* agents, const int* counts,
                    const skv_bf16* k, const skv_bf16* v, const skv_bf16* x, const skv_bf16* A,
                    AgentRows& ar) {
  const Geometry& g = c->g;
  Layer& l = c->layers[layer];
  for (int i = 0; i < n; ++i) {
    int slot = 1 + agents[i];
    ar.need += ceil_div(l.len[slot] + counts[i], g.ps) - (int)l.tbl[slot].size();
  }
  if (ar.need > (int)l.free.size())
    return c->fail(SKV_ERR_OOM, "layer %d: %d pages needed, %d free", layer, ar.need,
                   (int)l.free.size());
  ar.tables.resize(n);
  for (int i = 0; i < n; ++i) {
    int slot = 1 + agents[i];
    ar.tables[i] = l.tbl[slot];
    int want = ceil_div(l.len[slot] + counts[i], g.ps) - (int)ar.tables[i].size();
    for (int p = 0; p < want; ++p) {
      int32_t id = *l.free.begin();
      l.free.erase(l.free.begin());
      ar.tables[i].push_back(id);
      ar.taken.push_back(id);
    }
  }
  AppendJob proto{};
  proto.layer = layer;
  proto.do_kv = true;
  proto.do_lr = true;
  proto.update_tables = true;
  proto.k = k;
  proto.v = v;
  proto.x = x;
  const uint64_t a_stride = (uint64_t)g.hidden * g.r;
  int row = 0;
  for (int i = 0; i < n; ++i) {
    int a = agents[i];
    const uint16_t* ap = nullptr;
    if (x) ap = g.mode == SKV_BASE_SHARED ? A + a_stride * a : A;
    add_spans(c, ar.jobs, proto, ar.tables[i], 1 + a, l.len[1 + a], counts[i], row, c->plane_of(a), ap);
    row += counts[i];
  }
  return SKV_OK;
}

// Table lookup for the bounds checks of a planned agent-row append: the
// planned tables of the listed agents, the current ones of other sequences.
TableOf planned_tables(const skv_ctx* c, int layer, int n, const int* agents, const AgentRows& ar) {
  return [c, layer, n, agents, &ar](int s) -> const std::vector<int32_t>& {
    for (int i = 0; i < n; ++i)
      if (agents[i] + 1 == s) return ar.tables[i];
    return c->layers[layer].tbl[s];
  };
}

int finish_agent_rows(skv_ctx* c, int layer, int n, const int* agents, const int* counts, long total,
                      bool lr_from_x, AgentRows& ar, int rc) {
  Layer& l = c->layers[layer];
  if (rc != SKV_OK) {
    for (int32_t p : ar.taken) l.free.insert(p);
    return rc;
  }
  for (int i = 0; i < n; ++i) {
    int slot = 1 + agents[i];
    l.tbl[slot] = std::move(ar.tables[i]);
    l.len[slot] += counts[i];
    l.lr_own[agents[i]] += counts[i];
  }
  c->counters.pages_alloc += ar.need;
  c->counters.base_rows_own += total;
  (lr_from_x ? c->counters.lr_rows : c->counters.lr_zero_rows) += total;
  return SKV_OK;
}

}  // namespace

extern "C" {

size_t skv_arena_bytes(const skv_config* cfg) {
  if (!valid_config(cfg)) return 0;
  return (size_t)geometry_of(cfg).arena_bytes;
}

int skv_create(const skv_config* cfg, void* dev_arena, size_t arena_bytes, void* stream,
               skv_ctx** out) {
  if (!out) return SKV_ERR_ARG;
  *out = nullptr;
  if (!valid_config(cfg) || !dev_arena || ((uintptr_t)dev_arena & 255)) return SKV_ERR_ARG;
  Geometry g = geometry_of(cfg);
  if (arena_bytes < g.arena_bytes) return SKV_ERR_ARG;
  int rc = skv::dev_check(g);
  if (rc != SKV_OK) return rc;
  auto* c = new skv_ctx();
  c->g = g;
  c->g.arena = (char*)dev_arena;
  c->g.stream = stream;
  c->g.launches = &c->counters.launches;
  rc = skv::dev_init(c->g);
  if (rc != SKV_OK) {
    delete c;
    return rc;
  }
  c->layers.resize(g.L);
  for (auto& l : c->layers) {
    for (int p = 0; p < g.max_pages; ++p) l.free.insert(l.free.end(), p);
    l.tbl.assign(g.N + 1, {});
    l.len.assign(g.N + 1, 0);
    l.lr_shared.assign(g.planes, 0);
    l.lr_own.assign(g.N, 0);
  }
  c->base_len.assign(g.N, 0);
  c->lr_begin.assign(g.N, 0);
  *out = c;
  return SKV_OK;
}

void skv_destroy(skv_ctx* c) {
  if (!c) return;
  skv::dev_fini(c->g);
  delete c;
}

int skv_append_base(skv_ctx* c, int layer, int seq, int n, const skv_bf16* k, const skv_bf16* v) {
  if (!c) return SKV_ERR_ARG;
  if (layer < 0 || layer >= c->g.L) return c->fail(SKV_ERR_ARG, "layer %d out of range", layer);
  if (!c->seq_ok(seq)) return c->fail(SKV_ERR_ARG, "sequence %d out of range", seq);
  if (n < 0) return c->fail(SKV_ERR_ARG, "negative row count");
  if (n == 0) return SKV_OK;
  if (!k || !v) return c->fail(SKV_ERR_ARG, "null k or v");
  if (!aligned16({k, v})) return c->fail(SKV_ERR_ARG, "k and v must be 16-byte aligned");
  Layer& l = c->layers[layer];
  const int slot = skv_ctx::slot_of(seq);
  const int cur = l.len[slot];
  const int need = ceil_div(cur + n, c->g.ps) - (int)l.tbl[slot].size();
  if (need > (int)l.free.size())
    return c->fail(SKV_ERR_OOM, "layer %d: %d pages needed, %d free", layer, need,
                   (int)l.free.size());
  std::vector<int32_t> table = l.tbl[slot];
  std::vector<int32_t> taken;
  for (int i = 0; i < need; ++i) {
    int32_t p = *l.free.begin();
    l.free.erase(l.free.begin());
    table.push_back(p);
    taken.push_back(p);
  }
  AppendJob proto{};
  proto.layer = layer;
  proto.do_kv = true;
  proto.update_tables = true;
  proto.k = k;
  proto.v = v;
  std::vector<AppendJob> jobs;
  add_spans(c, jobs, proto, table, slot, cur, n, 0, 0, nullptr);
  int rc = run_jobs(c, jobs, [&](int s) -> const std::vector<int32_t>& { return s == slot ? table : l.tbl[s]; });
  if (rc != SKV_OK) {
    for (int32_t p : taken) l.free.insert(p);
    return rc;
  }
  l.tbl[slot] = std::move(table);
  l.len[slot] = cur + n;
  c->counters.pages_alloc += need;
  (seq == SKV_SHARED ? c->counters.base_rows_shared : c->counters.base_rows_own) += n;
  return SKV_OK;
}

int skv_append_lowrank(skv_ctx* c, int layer, int seq, int plane, int n, const skv_bf16* x,
                       const skv_bf16* A) {
  if (!c) return SKV_ERR_ARG;
  if (layer < 0 || layer >= c->g.L) return c->fail(SKV_ERR_ARG, "layer %d out of range", layer);
  if (!c->seq_ok(seq)) return c->fail(SKV_ERR_ARG, "sequence %d out of range", seq);
  if (seq == SKV_SHARED) {
    if (plane < 0 || plane >= c->g.planes) return c->fail(SKV_ERR_ARG, "plane %d", plane);
  } else if (plane != c->plane_of(seq)) {
    return c->fail(SKV_ERR_ARG, "agent %d writes plane %d, not %d", seq, c->plane_of(seq), plane);
  }
  if (n < 0) return c->fail(SKV_ERR_ARG, "negative row count");
  if (x && !A) return c->fail(SKV_ERR_ARG, "x given without A");
  if (!aligned16({x, x ? A : nullptr})) return c->fail(SKV_ERR_ARG, "x and A must be 16-byte aligned");
  if (n == 0) return SKV_OK;
  Layer& l = c->layers[layer];
  const int slot = skv_ctx::slot_of(seq);
  int& cov = seq == SKV_SHARED ? l.lr_shared[plane] : l.lr_own[seq];
  if (cov + n > l.len[slot])
    return c->fail(SKV_ERR_STATE, "low-rank rows %d..%d run ahead of %d base rows", cov, cov + n,
                   l.len[slot]);
  AppendJob proto{};
  proto.layer = layer;
  proto.do_lr = true;
  proto.x = x;
  std::vector<AppendJob> jobs;
  add_spans(c, jobs, proto, l.tbl[slot], slot, cov, n, 0, plane, A);
  int rc = run_jobs(c, jobs, [&](int s) -> const std::vector<int32_t>& { return l.tbl[s]; });
  if (rc != SKV_OK) return rc;
  cov += n;
  (x ? c->counters.lr_rows : c->counters.lr_zero_rows) += n;
  return SKV_OK;
}

int skv_append_agents(skv_ctx* c, int layer, int n, const int* agents, const int* counts,
                      const skv_bf16* k, const skv_bf16* v, const skv_bf16* x,
                      const skv_bf16* A) {
  if (!c) return SKV_ERR_ARG;
  if (x && !A) return c->fail(SKV_ERR_ARG, "x given without A");
  const char* arg_err = (!k || !v) ? "null k or v"
                        : !aligned16({k, v, x, x ? A : nullptr}) ? "k, v, x and A must be 16-byte aligned"
                                                                 : nullptr;
  long total = 0;
  int rc = check_agent_rows(c, layer, n, agents, counts, &total, arg_err);
  if (rc != SKV_OK || total == 0) return rc;
  AgentRows ar;
  rc = plan_agent_rows(c, layer, n, agents, counts, k, v, x, A, ar);
  if (rc != SKV_OK) return rc;
  rc = run_jobs(c, ar.jobs, planned_tables(c, layer, n, agents, ar));
  return finish_agent_rows(c, layer, n, agents, counts, total, x != nullptr, ar, rc);
}

// The first id of the shared pages the job's views read, when they are one
// run of consecutive ids, else -1 (the decode then looks each page up).
static int32_t shared_run(const skv_ctx* c, const Layer& l, const AttnJob& job) {
  int max_b = 0;
  for (int i = 0; i < job.n; ++i) max_b = std::max(max_b, (int)job.ag[i].b);
  const int pages = ceil_div(max_b, c->g.ps);
  const std::vector<int32_t>& t = l.tbl[0];
  if (pages == 0 || (int)t.size() < pages) return -1;
  for (int i = 1; i < pages; ++i)
    if (t[i] != t[0] + i) return -1;
  return t[0];
}

static int validate_attend(skv_ctx* c, int layer, int n, const int* agents, const int* base_len,
                           const int* suffix_len, const int* n_q, const void* q, const void* B,
                           const void* o, AttnJob& job) {
  const Geometry& g = c->g;
  if (layer < 0 || layer >= g.L) return c->fail(SKV_ERR_ARG, "layer %d out of range", layer);
  if (n < 1 || n > g.N) return c->fail(SKV_ERR_ARG, "agent count %d", n);
  if (!agents || !base_len || !suffix_len || !q || !B || !o)
    return c->fail(SKV_ERR_ARG, "null argument");
  if (!aligned16({q, B, o})) return c->fail(SKV_ERR_ARG, "q, B and o must be 16-byte aligned");
  const Layer& l = c->layers[layer];
  uint32_t seen = 0;
  for (int i = 0; i < n; ++i) {
    int a = agents[i];
    if (a >= 0 && a < g.N && (seen >> a & 1u)) return c->fail(SKV_ERR_ARG, "duplicate agent %d", a);
    if (a >= 0 && a < g.N) seen |= 1u << a;
  }
  job.layer = layer;
  job.n = n;
  int row = 0;
  for (int i = 0; i < n; ++i) {
    int a = agents[i];
    if (a < 0 || a >= g.N) return c->fail(SKV_ERR_ARG, "agent id %d", a);
    int b = c->base_len[a], S = l.len[1 + a];
    if (base_len[i] != b || suffix_len[i] != S)
      return c->fail(SKV_ERR_STATE,
                     "agent %d: caller lengths (b=%d, S=%d) differ from the cache (b=%d, S=%d)", a,
                     base_len[i], suffix_len[i], b, S);
    int nq = n_q ? n_q[i] : 1;
    if (b + S < 1 || nq < 1 || nq > b + S)
      return c->fail(SKV_ERR_ARG, "agent %d: %d queries over a view of %d", a, nq, b + S);
    int p = c->plane_of(a);
    if (l.lr_shared[p] < b || l.lr_own[a] < S)
      return c->fail(SKV_ERR_STATE, "agent %d: low-rank rows do not cover the view", a);
    job.ag[i] = skv::AttnAgent{a, b, S, p, nq, row, c->lr_begin[a]};
    row += nq;
  }
  job.q = (const uint16_t*)q;
  job.B = (const uint16_t*)B;
  job.o = (uint16_t*)o;
  job.shared_run = shared_run(c, l, job);
  return SKV_OK;
}

int skv_attn_prefill(skv_ctx* c, int layer, int n, const int* agents, const int* base_len,
                     const int* suffix_len, const int* n_q, const skv_bf16* q, const skv_bf16* B,
                     skv_bf16* o) {
  if (!c) return SKV_ERR_ARG;
  if (!n_q) return c->fail(SKV_ERR_ARG, "null n_q");
  AttnJob job;
  int rc = validate_attend(c, layer, n, agents, base_len, suffix_len, n_q, q, B, o, job);
  if (rc != SKV_OK) return rc;
  char msg[256];
  if ((rc = skv::plan_check_prefill(job, msg, sizeof msg)) != SKV_OK) return c->fail(rc, "%s", msg);
  if (!views_in_bounds(c, job, msg, sizeof msg)) return c->fail(SKV_ERR_STATE, "bounds check: %s", msg);
  rc = skv::dev_attn_prefill(c->g, job);
  if (rc != SKV_OK) return c->fail(rc, "device prefill failed: %s", skv::dev_last_error());
  return SKV_OK;
}

int skv_attn_decode(skv_ctx* c, int layer, int n, const int* agents, const int* base_len,
                    const int* suffix_len, const skv_bf16* q, const skv_bf16* B, skv_bf16* o) {
  if (!c) return SKV_ERR_ARG;
  AttnJob job;
  int rc = validate_attend(c, layer, n, agents, base_len, suffix_len, nullptr, q, B, o, job);
  if (rc != SKV_OK) return rc;
  char msg[256];
  if ((rc = skv::plan_check_decode(c->g, job, false, msg, sizeof msg)) != SKV_OK) return c->fail(rc, "%s", msg);
  if (!views_in_bounds(c, job, msg, sizeof msg)) return c->fail(SKV_ERR_STATE, "bounds check: %s", msg);
  rc = skv::dev_attn_decode(c->g, job);
  if (rc != SKV_OK) return c->fail(rc, "device decode failed: %s", skv::dev_last_error());
  return SKV_OK;
}

// Fused decode step; with scratch_static the launches keep their partial
// rows in the library's static device scratch instead of the arena.
static int decode_step(skv_ctx* c, int layer, int n, const int* agents, const int* base_len,
                       const int* suffix_len, const skv_bf16* k, const skv_bf16* v, const skv_bf16* x,
                       const skv_bf16* A, const skv_bf16* q, const skv_bf16* B, skv_bf16* o,
                       bool scratch_static) {
  if (!c) return SKV_ERR_ARG;
  const Geometry& g = c->g;
  if (layer < 0 || layer >= g.L) return c->fail(SKV_ERR_ARG, "layer %d out of range", layer);
  if (n < 1 || n > g.N) return c->fail(SKV_ERR_ARG, "agent count %d", n);
  if (!agents || !base_len || !suffix_len || !k || !v || !q || !B || !o)
    return c->fail(SKV_ERR_ARG, "null argument");
  if (x && !A) return c->fail(SKV_ERR_ARG, "x given without A");
  if (!aligned16({k, v, x, x ? A : nullptr, q, B, o}))
    return c->fail(SKV_ERR_ARG, "device pointers must be 16-byte aligned");
  Layer& l = c->layers[layer];
  uint32_t seen = 0;
  for (int i = 0; i < n; ++i) {
    int a = agents[i];
    if (a < 0 || a >= g.N || (seen >> a & 1u)) return c->fail(SKV_ERR_ARG, "agent list entry %d", a);
    seen |= 1u << a;
  }
  AttnJob job{};
  job.layer = layer;
  job.n = n;
  int need = 0;
  for (int i = 0; i < n; ++i) {
    int a = agents[i];
    int b = c->base_len[a], S = l.len[1 + a];
    if (base_len[i] != b || suffix_len[i] != S)
      return c->fail(SKV_ERR_STATE,
                     "agent %d: caller lengths (b=%d, S=%d) differ from the cache (b=%d, S=%d)", a,
                     base_len[i], suffix_len[i], b, S);
    int p = c->plane_of(a);
    if (l.lr_own[a] != S)
      return c->fail(SKV_ERR_STATE, "agent %d low-rank rows (%d) lag base rows (%d)", a, l.lr_own[a], S);
    if (l.lr_shared[p] < b)
      return c->fail(SKV_ERR_STATE, "agent %d: low-rank rows do not cover the view", a);
    job.ag[i] = skv::AttnAgent{a, b, S, p, 1, i, c->lr_begin[a]};
    need += ceil_div(S + 1, g.ps) - (int)l.tbl[1 + a].size();
  }
  job.shared_run = shared_run(c, l, job);
  if (need > (int)l.free.size())
    return c->fail(SKV_ERR_OOM, "layer %d: %d pages needed, %d free", layer, need, (int)l.free.size());
  char msg[256];
  int rc = skv::plan_check_decode(g, job, true, msg, sizeof msg);
  if (rc != SKV_OK) return c->fail(rc, "%s", msg);
  if (scratch_static && skv::decode_partial_bytes(g, job, true) > skv::kStaticScratchBytes)
    return c->fail(SKV_ERR_UNSUPPORTED, "decode partial rows (%llu bytes) exceed the static scratch (%llu bytes)",
                   (unsigned long long)skv::decode_partial_bytes(g, job, true),
                   (unsigned long long)skv::kStaticScratchBytes);
  std::vector<std::vector<int32_t>> tables(n);
  std::vector<int32_t> taken;
  for (int i = 0; i < n; ++i) {
    int slot = 1 + agents[i];
    tables[i] = l.tbl[slot];
    if (ceil_div(l.len[slot] + 1, g.ps) > (int)tables[i].size()) {
      int32_t id = *l.free.begin();
      l.free.erase(l.free.begin());
      tables[i].push_back(id);
      taken.push_back(id);
    }
  }
  AppendJob app{};
  app.layer = layer;
  app.do_kv = true;
  app.do_lr = true;
  app.update_tables = true;
  app.k = k;
  app.v = v;
  app.x = x;
  const uint64_t a_stride = (uint64_t)g.hidden * g.r;
  for (int i = 0; i < n; ++i) {
    int a = agents[i];
    const int pos = l.len[1 + a];
    Span sp{};
    sp.seq_slot = 1 + a;
    sp.pos0 = pos;
    sp.n = 1;
    sp.src_row = i;
    sp.first_page = pos / g.ps;
    sp.n_pages = 1;
    sp.ids_off = app.n_ids;
    sp.plane = c->plane_of(a);
    sp.a = x ? (g.mode == SKV_BASE_SHARED ? A + a_stride * a : A) : nullptr;
    app.ids[app.n_ids++] = tables[i][sp.first_page];
    app.spans[app.n_spans++] = sp;
  }
  job.q = q;
  job.B = B;
  job.o = o;
  const TableOf step_tables = [&](int s) -> const std::vector<int32_t>& {
    for (int i = 0; i < n; ++i)
      if (agents[i] + 1 == s) return tables[i];
    return l.tbl[s];
  };
  if (!views_in_bounds(c, job, msg, sizeof msg) || !job_in_bounds(c, app, step_tables, msg, sizeof msg)) {
    for (int32_t p : taken) l.free.insert(p);
    return c->fail(SKV_ERR_STATE, "bounds check: %s", msg);
  }
  rc = scratch_static ? skv::dev_decode_step_static(g, job, app) : skv::dev_decode_step(g, job, app);
  if (rc != SKV_OK) {
    for (int32_t p : taken) l.free.insert(p);
    return c->fail(rc, "device decode step failed: %s", skv::dev_last_error());
  }
  for (int i = 0; i < n; ++i) {
    int slot = 1 + agents[i];
    l.tbl[slot] = std::move(tables[i]);
    l.len[slot] += 1;
    l.lr_own[agents[i]] += 1;
  }
  c->counters.pages_alloc += (int64_t)taken.size();
  c->counters.base_rows_own += n;
  (x ? c->counters.lr_rows : c->counters.lr_zero_rows) += n;
  return SKV_OK;
}

int skv_decode_step(skv_ctx* c, int layer, int n, const int* agents, const int* base_len,
                    const int* suffix_len, const skv_bf16* k, const skv_bf16* v, const skv_bf16* x,
                    const skv_bf16* A, const skv_bf16* q, const skv_bf16* B, skv_bf16* o) {
  return decode_step(c, layer, n, agents, base_len, suffix_len, k, v, x, A, q, B, o, false);
}

int skv_decode_step_static(skv_ctx* c, int layer, int n, const int* agents, const int* base_len,
                           const int* suffix_len, const skv_bf16* k, const skv_bf16* v, const skv_bf16* x,
                           const skv_bf16* A, const skv_bf16* q, const skv_bf16* B, skv_bf16* o) {
  return decode_step(c, layer, n, agents, base_len, suffix_len, k, v, x, A, q, B, o, true);
}

int skv_pack_qkv(skv_ctx* c, const skv_bf16* w_qkv, skv_bf16* w_packed) {
  if (!c) return SKV_ERR_ARG;
  if (!w_qkv || !w_packed) return c->fail(SKV_ERR_ARG, "null w_qkv or w_packed");
  if (!aligned16({w_qkv, w_packed})) return c->fail(SKV_ERR_ARG, "w_qkv and w_packed must be 16-byte aligned");
  const Geometry& g = c->g;
  const uint64_t bytes = 2ull * (g.Hq + 2 * g.Hkv) * g.D * g.hidden;
  const uintptr_t a = (uintptr_t)w_qkv, b = (uintptr_t)w_packed;
  if (a < b + bytes && b < a + bytes) return c->fail(SKV_ERR_ARG, "w_qkv and w_packed overlap");
  int rc = skv::dev_pack_qkv(g, (const uint16_t*)w_qkv, (uint16_t*)w_packed);
  if (rc != SKV_OK) return c->fail(rc, "device pack failed: %s", skv::dev_last_error());
  return SKV_OK;
}

int skv_project_append(skv_ctx* c, int layer, int n, const int* agents, const int* counts,
                       const skv_bf16* x, const skv_bf16* w_packed, const skv_bf16* A, float rope_theta,
                       skv_bf16* q_out) {
  if (!c) return SKV_ERR_ARG;
  const char* arg_err = (!x || !w_packed || !q_out) ? "null x, w_packed or q_out"
                        : !aligned16({x, w_packed, A, q_out}) ? "device pointers must be 16-byte aligned"
                        : !(rope_theta == 0.f || (rope_theta > 1.f && rope_theta < 1e30f))
                            ? "rotary base must be 0 or above 1 (and finite)"
                            : nullptr;
  long total = 0;
  int rc = check_agent_rows(c, layer, n, agents, counts, &total, arg_err);
  if (rc != SKV_OK || total == 0) return rc;
  {
    char msg[160];
    rc = skv::plan_check_project(c->g, msg, sizeof msg);
    if (rc != SKV_OK) return c->fail(rc, "%s", msg);
  }
  AgentRows ar;
  rc = plan_agent_rows(c, layer, n, agents, counts, nullptr, nullptr, A ? x : nullptr, A, ar);
  if (rc != SKV_OK) return rc;
  {
    char msg[256];
    const TableOf tabs = planned_tables(c, layer, n, agents, ar);
    for (const AppendJob& j : ar.jobs)
      if (!job_in_bounds(c, j, tabs, msg, sizeof msg))
        return finish_agent_rows(c, layer, n, agents, counts, total, A != nullptr, ar,
                                 c->fail(SKV_ERR_STATE, "bounds check: %s", msg));
  }
  for (const AppendJob& j : ar.jobs) {
    skv::ProjectJob pj{};
    pj.app = j;
    pj.app.do_kv = false;  // k and v are written by the projection itself
    pj.x = (const uint16_t*)x;
    pj.w = (const uint16_t*)w_packed;
    pj.q = (uint16_t*)q_out;
    pj.theta = rope_theta;
    for (int s = 0; s < j.n_spans; ++s) pj.view_off[s] = c->base_len[j.spans[s].seq_slot - 1];
    rc = skv::dev_project(c->g, pj);
    if (rc != SKV_OK) {
      rc = c->fail(rc, "device projection failed: %s", skv::dev_last_error());
      break;
    }
  }
  return finish_agent_rows(c, layer, n, agents, counts, total, A != nullptr, ar, rc);
}

int skv_set_lr_begin(skv_ctx* c, int agent, int pos) {
  if (!c) return SKV_ERR_ARG;
  if (agent < 0 || agent >= c->g.N) return c->fail(SKV_ERR_ARG, "agent id %d", agent);
  if (pos < 0) return c->fail(SKV_ERR_ARG, "negative activation offset %d", pos);
  c->lr_begin[agent] = pos;
  return SKV_OK;
}

int skv_crop(skv_ctx* c, int seq, int new_len) {
  if (!c) return SKV_ERR_ARG;
  if (!c->seq_ok(seq)) return c->fail(SKV_ERR_ARG, "sequence %d out of range", seq);
  if (new_len < 0) return c->fail(SKV_ERR_ARG, "negative length");
  const int shared_min = c->min_len(0);
  if (seq == SKV_SHARED) {
    if (new_len < c->max_base() || new_len > shared_min)
      return c->fail(SKV_ERR_STATE, "shared crop to %d outside [%d, %d]", new_len, c->max_base(),
                     shared_min);
    for (auto& l : c->layers) {
      c->counters.rows_cropped += l.len[0] - new_len;
      l.len[0] = new_len;
      for (auto& cov : l.lr_shared) cov = std::min(cov, new_len);
      c->free_beyond(l, 0, new_len);
    }
    return SKV_OK;
  }
  const int slot = skv_ctx::slot_of(seq);
  int& b = c->base_len[seq];
  bool no_own = true;
  for (auto& l : c->layers) no_own = no_own && l.len[slot] == 0;
  if (no_own && new_len >= b) {
    if (new_len > shared_min)
      return c->fail(SKV_ERR_STATE, "attach at %d beyond shared length %d", new_len, shared_min);
    b = new_len;
    return SKV_OK;
  }
  int own;
  if (new_len < b) {
    own = 0;
  } else {
    own = new_len - b;
    if (own > c->min_len(slot))
      return c->fail(SKV_ERR_STATE, "crop to %d beyond the view (b=%d, min S=%d)", new_len, b,
                     c->min_len(slot));
  }
  for (auto& l : c->layers) {
    c->counters.rows_cropped += l.len[slot] - own;
    l.len[slot] = own;
    l.lr_own[seq] = std::min(l.lr_own[seq], own);
    c->free_beyond(l, slot, own);
  }
  if (new_len < b) b = new_len;
  return SKV_OK;
}

int skv_get_lens(const skv_ctx* c, int layer, int* P, int* base_len, int* suffix_len,
                 int* lr_shared, int* lr_own) {
  if (!c || layer < 0 || layer >= c->g.L) return SKV_ERR_ARG;
  const Layer& l = c->layers[layer];
  if (P) *P = l.len[0];
  for (int a = 0; a < c->g.N; ++a) {
    if (base_len) base_len[a] = c->base_len[a];
    if (suffix_len) suffix_len[a] = l.len[1 + a];
    if (lr_own) lr_own[a] = l.lr_own[a];
  }
  if (lr_shared)
    for (int p = 0; p < c->g.planes; ++p) lr_shared[p] = l.lr_shared[p];
  return SKV_OK;
}

int skv_get_pages(const skv_ctx* c, int layer, int seq, int32_t* ids, int cap) {
  if (!c || layer < 0 || layer >= c->g.L || !c->seq_ok(seq) || cap < 0) return SKV_ERR_ARG;
  const auto& t = c->layers[layer].tbl[skv_ctx::slot_of(seq)];
  for (int i = 0; i < (int)t.size() && i < cap; ++i) ids[i] = t[i];
  return (int)t.size();
}

int skv_get_pools(const skv_ctx* c, skv_pools* out) {
  if (!c || !out) return SKV_ERR_ARG;
  out->k_off = c->g.k_off;
  out->vt_off = c->g.vt_off;
  out->lrt_off = c->g.lrt_off;
  out->tables_off = c->g.tbl_off;
  out->scratch_off = c->g.scratch_off;
  out->scratch_bytes = c->g.scratch_bytes;
  out->arena_bytes = c->g.arena_bytes;
  out->planes = c->g.planes;
  return SKV_OK;
}

int skv_get_counters(const skv_ctx* c, skv_counters* out) {
  if (!c || !out) return SKV_ERR_ARG;
  *out = c->counters;
  return SKV_OK;
}

int skv_set_timing(skv_ctx* c, int enable) {
  if (!c) return SKV_ERR_ARG;
  return skv::dev_set_timing(c->g, enable);
}

int skv_collect_timing(skv_ctx* c, skv_kernel_times* out) {
  if (!c || !out) return SKV_ERR_ARG;
  int rc = skv::dev_collect_timing(c->g, out);
  if (rc != SKV_OK) return c->fail(rc, "timing: %s", skv::dev_last_error());
  return SKV_OK;
}

int skv_sync(skv_ctx* c) {
  if (!c) return SKV_ERR_ARG;
  int rc = skv::dev_sync(c->g);
  if (rc != SKV_OK) return c->fail(rc, "sync: %s", skv::dev_last_error());
  return SKV_OK;
}

const char* skv_last_error(const skv_ctx* c) { return c ? c->err.c_str() : "null context"; }

int skv_probe_stream_read(const void* src, uint64_t bytes, int reps, void* stream, double* gbs) {
  if (!src || !gbs || bytes < (1u << 20) || bytes % 16 || reps < 1) return SKV_ERR_ARG;
  return skv::dev_probe_stream_read(src, bytes, reps, stream, gbs);
}

int skv_probe_mfma_bf16(void* stream, double* tflops) {
  if (!tflops) return SKV_ERR_ARG;
  return skv::dev_probe_mfma_bf16(stream, tflops);
}

int skv_probe_mfma_bf16_data(const void* src, uint64_t bytes, void* stream, double* tflops) {
  if (!src || !tflops || bytes < (16u << 10)) return SKV_ERR_ARG;
  return skv::dev_probe_mfma_bf16_data(src, stream, tflops);
}

int skv_probe_launch_pattern(const void* src, uint64_t layer_bytes, int layers, int steps, int tail_blocks,
                             void* stream, double* ms_pattern, double* ms_stream) {
  if (!src || !ms_pattern || !ms_stream || layer_bytes < (1u << 20) || layer_bytes % 16 || layers < 1 ||
      layers > 1024 || steps < 1 || steps > 1000 || tail_blocks < 1 || tail_blocks > 65535)
    return SKV_ERR_ARG;
  return skv::dev_probe_launch_pattern(src, layer_bytes, layers, steps, tail_blocks, stream, ms_pattern, ms_stream);
}

}  // extern "C"
