/*
 * skv.h - shared-prefix multi-LoRA attention over one paged context cache.
 *
 * Several LoRA agents share one backbone. The base K/V of a shared context is
 * computed once with base weights and stored once; every agent attends over
 * that shared prefix followed by its own suffix. Agent i's value for token j is
 * V_base[j] + (X_j A_i) B_i, and the library applies it as
 *     O = P V_base + (P V_lr) B_i,
 * keeping only the rank-r rows V_lr = X A in the cache, so no agent's
 * full-width adapter value cache is ever formed.
 *
 * Sources (web pages; cited by page and part):
 *   LRAgent review (pith.science, arXiv 2602.01053), "What carries the
 *     argument": the value decomposition Y_i = X W0 + (X A_i) B_i (the paper's
 *     Eq. 3) and the reorder O = P V_base + (P V_lr) B, with B applied once
 *     per query block (its Eq. 12); Figs. 2-3: BaseShared (one LR cache per
 *     agent) and BaseLRShared (shared A, one LR cache).
 *   paperlayer summary of arXiv 2609.17109, Sec. 2: prefix KV computed once
 *     with adapters disabled, specialist takes over at a boundary b;
 *     Sec. 3.2: a paged cache is the route to physically shared storage.
 *   RoleKV write-up (devpost), "What it does" / "How we built it": one shared
 *     KV cache, crop and recompute at a role handoff; "Challenges": pass the
 *     adapter offsets explicitly or the adapter silently turns off.
 *
 * Conventions
 *   - All tensors are bf16 (passed as uint16_t bit patterns), row-major and
 *     contiguous, and live in DEVICE memory: k, v, x, A, B, q, o. Each starts
 *     at a 16-byte-aligned address (the kernels use 16-byte vector accesses);
 *     a misaligned pointer is rejected with SKV_ERR_ARG.
 *   - Small integer arrays (agents, lengths, counts) live in HOST memory.
 *   - Hq = n_q_heads, Hkv = n_kv_heads, G = Hq / Hkv, d = head_dim,
 *     r = rank, N = n_agents. Query head h reads KV head floor(h / G).
 *   - A sequence id is SKV_SHARED (-1) or an agent id 0..N-1. Agent i's view
 *     at a layer is SHARED[0:b_i] followed by OWN_i[0:S_i]; b_i is the same on
 *     every layer, S_i is per layer.
 *   - Low-rank planes: BaseShared keeps one plane per agent (plane i holds
 *     X A_i); BaseLRShared keeps plane 0 only (X A with the shared A). Agent
 *     i's own rows always use plane_of(i) = (mode == BaseShared ? i : 0).
 *   - Softmax scale is 1/sqrt(d). A query at view position t sees view
 *     positions 0..t (decode appends the token, then attends).
 *   - Every call validates on the host before it enqueues anything, and is
 *     all-or-nothing: on error the cache state is unchanged. Device work is
 *     enqueued on the stream given at create and no call waits for the GPU
 *     (except skv_sync). Faults in device work surface at skv_sync.
 *   - Ownership: the caller owns every device buffer and the arena, and keeps
 *     them alive until the stream work that uses them has completed. The
 *     library never allocates device memory; it carves its pools, page tables
 *     and scratch out of the arena. Host metadata belongs to the library.
 *     One host thread per context.
 */
#ifndef SKV_H
#define SKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKV_SHARED (-1)
#define SKV_MAX_AGENTS 16

enum skv_mode { SKV_BASE_SHARED = 0, SKV_BASE_LR_SHARED = 1 };

enum skv_status {
  SKV_OK = 0,
  SKV_ERR_ARG = -1,         /* bad argument (range, null pointer, shape)            */
  SKV_ERR_STATE = -2,       /* lengths disagree with the cache, LR rows missing,    */
                            /* crop out of range                                    */
  SKV_ERR_OOM = -3,         /* page pool of a layer exhausted                       */
  SKV_ERR_UNSUPPORTED = -4, /* configuration the device code does not handle        */
  SKV_ERR_HIP = -5          /* a HIP runtime call failed                            */
};

typedef uint16_t skv_bf16; /* bf16 bit pattern */

typedef struct skv_config {
  int32_t n_layers;
  int32_t n_q_heads;   /* Hq, a multiple of n_kv_heads                                  */
  int32_t n_kv_heads;  /* Hkv                                                            */
  int32_t head_dim;    /* d: 64 or 128                                                   */
  int32_t hidden;      /* width of X (input of A), a multiple of 64                      */
  int32_t rank;        /* r: 4, 8, 16 or 32                                              */
  int32_t n_agents;    /* N: 1..SKV_MAX_AGENTS                                           */
  int32_t mode;        /* SKV_BASE_SHARED or SKV_BASE_LR_SHARED                          */
  int32_t page_size;   /* rows per page, a power of two (the GPU build requires 64)     */
  int32_t max_pages;   /* pages per layer in the pool (shared by all sequences)         */
} skv_config;

typedef struct skv_ctx skv_ctx;

/* Bytes of device memory skv_create needs for cfg (0 if cfg is invalid): the
 * K/V and low-rank pools, page tables and scratch. Sized up front so the store
 * is one physically shared allocation (paperlayer summary of arXiv
 * 2609.17109, Sec. 3.2 and Table 2: without a shared paged store the prefix
 * was copied per branch and peak memory fell only 5-12%). */
size_t skv_arena_bytes(const skv_config* cfg);

/* Create a context over a caller-owned device arena of at least
 * skv_arena_bytes(cfg) bytes (256-byte aligned). The configuration carries the
 * quantities the pages state the problem in: the rank r, shared-A versus
 * per-agent-A (LRAgent review, "The reading" and Figs. 2-3: BaseShared and
 * BaseLRShared), the agents, and the GQA head groups. stream is a hipStream_t
 * (NULL = default stream). Errors: ARG (bad config, small arena),
 * UNSUPPORTED (page_size or shape the device code does not handle). */
int skv_create(const skv_config* cfg, void* dev_arena, size_t arena_bytes, void* stream,
               skv_ctx** out);

/* Free host metadata (the counterpart of skv_create). Does not touch the
 * arena, which stays the caller's. NULL is allowed. */
void skv_destroy(skv_ctx* ctx);

/* a1 / a3: append n rows of base-weight K and V to the end of sequence seq at
 * one layer (LRAgent review Fig. 2: the base cache is computed once and
 * shared; RoleKV "What it does": a role switch only computes the new tokens).
 * k, v: device [n][Hkv][d]. New pages take the lowest free page ids of the
 * layer. n == 0 is a no-op. Errors: ARG, OOM (nothing is appended). */
int skv_append_base(skv_ctx* ctx, int layer, int seq, int n, const skv_bf16* k,
                    const skv_bf16* v);

/* a2: append n low-rank rows bf16(X A) (fp32 accumulation, round to nearest
 * even) to plane `plane` of sequence seq at one layer, after the rows it
 * already holds (LRAgent review, "What carries the argument": the adapter
 * term is stored as the rank-r intermediate X A; Fig. 3: BaseShared fills it
 * for every context token the agent has not processed, BaseLRShared once).
 * x: device [n][hidden] or NULL for adapter-off zero rows (paperlayer Sec. 2:
 * prefix computed with adapters disabled); A: device [hidden][r] (ignored
 * when x is NULL). For SKV_SHARED, plane is 0..planes-1; for an agent, plane
 * must be plane_of(agent). LR rows may not run ahead of base rows.
 * Errors: ARG, STATE. */
int skv_append_lowrank(skv_ctx* ctx, int layer, int seq, int plane, int n, const skv_bf16* x,
                       const skv_bf16* A);

/* a2 + a3 batched: for each listed agent, append counts[i] own rows of base
 * K/V and their low-rank rows in one launch. agents/counts: host [n]. k, v:
 * device [sum counts][Hkv][d]; x: device [sum counts][hidden] or NULL (zero LR
 * rows); A: device [N][hidden][r] in BaseShared (A_i indexed by agent id) or
 * [hidden][r] in BaseLRShared. Each agent's own LR rows must be level with its
 * base rows before the call. Errors: ARG, STATE, OOM (nothing is appended). */
int skv_append_agents(skv_ctx* ctx, int layer, int n, const int* agents, const int* counts,
                      const skv_bf16* k, const skv_bf16* v, const skv_bf16* x,
                      const skv_bf16* A);

/* Front-end weights: reorder the stacked projection weights w_qkv (device
 * [(Hq + 2 Hkv) d][hidden]; rows = the Hq query heads, then the Hkv key heads,
 * then the Hkv value heads, d rows each, so that q = x w_q^T etc.) into
 * w_packed (device, the same size, not overlapping), the layout
 * skv_project_append streams: for 64-row unit u (head u / (d/64), rows
 * 32 (u % (d/64)) + [0, 32) and the same + d/2 of that head), 64-column step
 * s, and m = 0..7, lane l = 0..63, the 8 elements at
 * ((u * hidden/64 + s) * 8 + m) * 512 + 8 l are
 *   w_qkv[head d + 32 (u % (d/64)) + 16 (m/2 % 2) + (d/2)(m/4) + l % 16]
 *        [64 s + 32 (m % 2) + 8 (l / 16) .. + 8],
 * so each matrix-core operand read is 1 KB of contiguous memory. Done once
 * per layer when the weights are loaded; enqueued on the context stream.
 * Errors: ARG. */
int skv_pack_qkv(skv_ctx* ctx, const skv_bf16* w_qkv, skv_bf16* w_packed);

/* Front end fused with a2 + a3: for each listed agent, project counts[i] new
 * input rows into q, k and the base v with one GEMM against the base weights,
 * rotate q and k, and append k, v and the low-rank rows bf16(X A_i) to the
 * agent's own pages in the same launch (LRAgent review, "What carries the
 * argument": the base value and the rank-r rows X A_i come from the same X;
 * the base K/V is computed with the base weights for every agent).
 *   x: device [sum counts][hidden], agent blocks in call order.
 *   w_packed: the layer's weights as packed by skv_pack_qkv.
 *   A: as in skv_append_agents, or NULL for adapter-off zero low-rank rows.
 *   rope_theta: rotary base, 0 = no rotation, else above 1 and finite
 *     (ARG otherwise). Rotary embedding in the
 *     rotate-half form: for head vector u and view position t, each pair
 *     (u[j], u[j + d/2]), j < d/2, turns by the angle t * theta^(-2j/d). The
 *     view position of own row s of agent i is b_i + s (the shared prefix
 *     keeps positions 0 .. b_i - 1).
 *   q_out: device [sum counts][Hq][d], written (bf16, rotated).
 * q, k and v are rounded once to bf16 from fp32 accumulation. Each agent's
 * own low-rank rows must be level with its base rows before the call.
 * Errors: ARG, STATE, OOM, and UNSUPPORTED when the packed weights
 * ((Hq + 2 Hkv) d hidden bf16 values) reach 2 GiB (nothing is appended). */
int skv_project_append(skv_ctx* ctx, int layer, int n, const int* agents, const int* counts,
                       const skv_bf16* x, const skv_bf16* w_packed, const skv_bf16* A,
                       float rope_theta, skv_bf16* q_out);

/* a4: suffix prefill attention at one layer. For each listed agent i (host
 * arrays agents/base_len/suffix_len/n_q of length n), the queries are the last
 * n_q[i] positions of its view, already appended. base_len[i] and
 * suffix_len[i] must equal the cache's b_i and S_i at this layer (RoleKV
 * "Challenges": offsets are passed explicitly and checked). Each query at
 * view position t computes softmax(q K[0..t]^T / sqrt(d)) over the view and
 * o = P V_base + (P V_lr) B_i[:, g*d:(g+1)*d] (LRAgent review, "What carries
 * the argument"), with B_i applied once per query block.
 * q, o: device [sum n_q][Hq][d] (agent blocks in call order). B: device
 * [N][r][Hkv*d] indexed by agent id. Agents must be distinct.
 * Errors: ARG, STATE (lengths differ, LR rows do not cover the view). */
int skv_attn_prefill(skv_ctx* ctx, int layer, int n, const int* agents, const int* base_len,
                     const int* suffix_len, const int* n_q, const skv_bf16* q,
                     const skv_bf16* B, skv_bf16* o);

/* a5 + a6: decode attention, one query per listed agent at the last position
 * of its view: the same result as skv_attn_prefill with n_q[i] = 1. The
 * shared prefix is streamed from HBM once per KV head for all listed agents'
 * query rows, split over the GPU, and the partial softmax states are merged
 * before B_i is applied. q, o: device [n][Hq][d]. Errors: as prefill. */
int skv_attn_decode(skv_ctx* ctx, int layer, int n, const int* agents, const int* base_len,
                    const int* suffix_len, const skv_bf16* q, const skv_bf16* B, skv_bf16* o);

/* a2 + a3 + a5 + a6 fused for one decode token per listed agent: append the
 * agent's new row (base K/V and its low-rank row X A, as skv_append_agents
 * with counts of 1) at the end of its own suffix, then attend from that new
 * position over SHARED[0:b_i] ++ OWN_i[0:S_i + 1] (as skv_attn_decode).
 * Results equal the two separate calls up to fp32 summation order. On the
 * GPU it is two launches: the split pass over the keys already cached plus
 * the writes of the new rows, then the merge, which adds the new token as
 * one more softmax term and applies B_i.
 * base_len / suffix_len: b_i and S_i BEFORE the step (checked; each agent's
 * own low-rank rows must be level with its base rows). k, v: device
 * [n][Hkv][d]; x: device [n][hidden] or NULL (zero low-rank rows); A as in
 * skv_append_agents; q, o: device [n][Hq][d]; B: device [N][r][Hkv*d].
 * Errors: ARG, STATE, OOM (nothing is appended). */
int skv_decode_step(skv_ctx* ctx, int layer, int n, const int* agents, const int* base_len,
                    const int* suffix_len, const skv_bf16* k, const skv_bf16* v,
                    const skv_bf16* x, const skv_bf16* A, const skv_bf16* q, const skv_bf16* B,
                    skv_bf16* o);

/* skv_decode_step for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same arguments, results and errors, but the split pass's partial rows go to
 * the library's static device scratch instead of the arena. The scratch is one
 * array of 16 MiB per GPU the library runs on, held until the process ends;
 * this call allocates nothing and records no timing events. Every call on one
 * GPU shares that array: calls on the same stream are ordered, calls that
 * overlap on one GPU (other streams, other contexts) race. Extra error:
 * UNSUPPORTED when a launch's partial rows (split items x agents x G rows x
 * (d + r + 4) fp32 values) exceed 16 MiB; nothing is appended then. */
int skv_decode_step_static(skv_ctx* ctx, int layer, int n, const int* agents, const int* base_len,
                           const int* suffix_len, const skv_bf16* k, const skv_bf16* v,
                           const skv_bf16* x, const skv_bf16* A, const skv_bf16* q,
                           const skv_bf16* B, skv_bf16* o);

/* Adapter activation offset of one agent (RoleKV, "What it does": an
 * activated adapter switches on after the role's header, and everything
 * before it is processed with the base weights; "Challenges we ran into": the
 * offset is passed explicitly). From the next attention call on, view
 * positions j < pos of the agent take no low-rank term:
 * V_i[j] = V_base[j] + [j >= pos] (X_j A) B_i. The rows stay cached (in
 * BaseLRShared they are the shared plane's rows other agents use). 0 (the
 * default) turns the adapter on everywhere; pos may lie beyond the view.
 * Host metadata only. Errors: ARG (agent out of range, pos < 0). */
int skv_set_lr_begin(skv_ctx* ctx, int agent, int pos);

/* a7: set a view length on every layer (RoleKV "How we built it": crop at a
 * handoff; paperlayer Sec. 2: takeover boundary). Host metadata only.
 *   seq = agent i with no own rows and new_len >= b_i: (re)attach, b_i = new_len
 *         (new_len <= shared length on every layer).
 *   seq = agent i, b_i <= new_len <= b_i + min_l S_i: own rows truncated.
 *   seq = agent i, new_len < b_i: own rows dropped, b_i = new_len.
 *   seq = SKV_SHARED: max_i b_i <= new_len <= shared length on every layer.
 * Pages lying wholly beyond a new length are freed. Freed pages keep their
 * bytes. Errors: ARG, STATE. */
int skv_crop(skv_ctx* ctx, int seq, int new_len);

/* Lengths at one layer, for checking the cache's state from outside (RoleKV
 * write-up, "How we built it": cache-equivalence and canonicalization tests;
 * "Challenges we ran into": the offsets a caller passes must match the
 * cache). Any output pointer may be NULL. base_len, suffix_len, lr_own: host
 * [N]; lr_shared: host [planes]. P receives the shared length. */
int skv_get_lens(const skv_ctx* ctx, int layer, int* P, int* base_len, int* suffix_len,
                 int* lr_shared, int* lr_own);

/* Page ids of seq at layer, in order, into host ids[cap]: with skv_get_pools,
 * the means to check that agents resolve the shared prefix to the same
 * physical pages (paperlayer summary of arXiv 2609.17109, App. C: physical
 * sharing is checked by the identity of the prefix tensors' storage). Returns
 * the count (which may exceed cap) or a negative error. */
int skv_get_pages(const skv_ctx* ctx, int layer, int seq, int32_t* ids, int cap);

/* Device pool layout, for byte-level inspection (the storage-identity check
 * of paperlayer App. C; the canonicalization test of RoleKV "How we built
 * it" compares a recomputed cache with a fresh one byte by byte):
 *   K  [layer][page][Hkv][64 * d]              bf16 tiles, see below
 *   V  [layer][page][Hkv][64 * d]              bf16 tiles, see below
 *   LRT[plane][layer][page][r][page_size]      bf16 (low-rank rows transposed)
 *   tables [layer][1 + N][max_pages]           int32 (slot 0 = SHARED)
 * A (page, head) tile stores its 64 rows in the order the GPU's matrix-core
 * operand loads read them, so each wave load is 1 KB of contiguous memory.
 * With key = slot in page (0..63), h = key / 32, kk = key % 32:
 *   K[key][c] sits at element ((h*2 + t)*(d/32) + c/32)*512 + (n + 16*q)*8 + c%8
 *     where n = 4*(kk/8) + kk%4, t = (kk%8)/4, q = (c%32)/8;
 *   V[key][c] sits at element (h*(d/16) + c/16)*512 + (c%16 + 16*(kk/8))*8 + kk%8.
 * Offsets are in bytes from the arena start. */
typedef struct skv_pools {
  uint64_t k_off, vt_off, lrt_off, tables_off, scratch_off, scratch_bytes, arena_bytes;
  int32_t planes;
} skv_pools;
int skv_get_pools(const skv_ctx* ctx, skv_pools* out);

/* Token accounting: rows appended to the shared and own sequences, low-rank
 * and zero low-rank rows, rows cropped, pages, launches (RoleKV write-up,
 * "Challenges we ran into": count the canonicalization tokens; "How we built
 * it": prefill, reuse and canonicalization tokens are logged per turn). */
typedef struct skv_counters {
  int64_t base_rows_shared, base_rows_own, lr_rows, lr_zero_rows, rows_cropped;
  int64_t pages_alloc, pages_freed, launches;
} skv_counters;
int skv_get_counters(const skv_ctx* ctx, skv_counters* out);

/* Kernel timing with HIP events recorded on the context stream around each
 * launch, while enabled. Kinds: 0 append K/V, 1 append low-rank, 2 decode
 * attention (split pass), 3 decode merge + B_i, 4 prefill attention (and the
 * merge launch of a prefill whose key ranges are split), 5 front-end
 * projection (skv_project_append) and weight packing. */
#define SKV_KERNEL_KINDS 6
typedef struct skv_kernel_times {
  double ms[SKV_KERNEL_KINDS];
  int64_t launches[SKV_KERNEL_KINDS];
} skv_kernel_times;
/* enable: bit mask of kernel kinds to time (bit k = kind k), 0 = off. */
int skv_set_timing(skv_ctx* ctx, int enable);
/* Waits for the stream, sums the recorded intervals, and clears them. */
int skv_collect_timing(skv_ctx* ctx, skv_kernel_times* out);

/* Wait for all work enqueued by this context; device faults surface here
 * (every other call validates on the host and only enqueues: RoleKV
 * "Challenges we ran into": no state that silently diverges from what the
 * caller passed). Errors: HIP. */
int skv_sync(skv_ctx* ctx);

/* Message of the last failed call on ctx ("" if none): which argument or
 * length disagreed with the cache (RoleKV "Challenges we ran into": a wrong
 * offset must fail loudly, not turn the adapter off). */
const char* skv_last_error(const skv_ctx* ctx);

/* Measurement probes (no context; the current device; synchronous on
 * `stream`, a hipStream_t, 0 = default). They calibrate the rooflines the
 * attention kernels are reported against and are not part of the path.
 * skv_probe_stream_read: reads the device buffer src (bytes: a multiple of 16,
 *   at least 1 MiB; caller-owned, contents irrelevant) once per repetition
 *   with non-temporal 16-byte loads from every CU; *gbs = the best of `reps`
 *   repetitions in GB/s (10^9 bytes/s).
 * skv_probe_mfma_bf16: a dense v_mfma_f32_16x16x32_bf16 issue loop, two waves
 *   per SIMD on every CU with independent accumulators; *tflops = the
 *   achieved dense bf16 rate (10^12 flop/s, 2 flops per multiply-add).
 * skv_probe_mfma_bf16_data: the same issue loop on operand data: every wave
 *   takes its eight A and eight B fragments from the first 16 KiB of the
 *   device buffer src (bytes >= 16 KiB; caller-owned, e.g. normal draws in
 *   bf16), so consecutive MFMAs see different bit patterns as attention's
 *   do; runs about 10 ms per repetition so that the clock settles under the
 *   power limit; *tflops = the best of three.
 * skv_probe_launch_pattern: the launch pattern of a decode step without its
 *   arithmetic. src holds `layers` consecutive buffers of layer_bytes bytes
 *   (a multiple of 16, at least 1 MiB; caller-owned, contents irrelevant).
 *   One step is, for every layer, a streaming read of that layer's buffer by
 *   one workgroup per CU (non-temporal 16-byte loads) followed by a small
 *   launch of tail_blocks workgroups that reads what the streaming launch
 *   left (ordered after it, as a merge is after its split pass). After one
 *   untimed step, `steps` steps are timed between two events; *ms_pattern =
 *   ms per step (best of three runs), *ms_stream = the same without the small
 *   launches. layers in [1, 1024], steps in [1, 1000], tail_blocks in
 *   [1, 65535].
 * Errors: ARG (NULL pointers, bad sizes), HIP, UNSUPPORTED (CPU-only build). */
int skv_probe_stream_read(const void* src, uint64_t bytes, int reps, void* stream, double* gbs);
int skv_probe_mfma_bf16(void* stream, double* tflops);
int skv_probe_mfma_bf16_data(const void* src, uint64_t bytes, void* stream, double* tflops);
int skv_probe_launch_pattern(const void* src, uint64_t layer_bytes, int layers, int steps, int tail_blocks,
                             void* stream, double* ms_pattern, double* ms_stream);

#ifdef __cplusplus
}
#endif
#endif /* SKV_H */
