#!/usr/bin/env python3
"""Multi-agent decode throughput of the shared-prefix multi-LoRA attention path.

Workload (default): Llama-3-8B-like attention, 32 layers, 32 query heads,
8 KV heads, head_dim 128, hidden 4096; 4 agents sharing one down-projection A
(rank 8, per-agent B_i); a 32,768-token shared prefix. One step is one decode
token per agent through all 32 layers: for each layer, the four agents' new
K/V rows and low-rank rows are appended (skv_append_agents) and decode
attention runs over the shared prefix plus each agent's suffix
(skv_attn_decode: split pass + merge with B_i). Inputs are synthetic, seeded,
and already resident in GPU memory when the timed region starts.

Prints one JSON line. `value` = decode tokens/s (agents x steps / wall time).
`roofline` is for the dominant kernel (the decode split pass): algorithmic
bytes per launch / its average duration from HIP events recorded around each
launch on the library's stream during the timed steps, against 8 TB/s.
`prefill` reports the suffix-prefill kernel (4 agents x 512 tokens at the same
prefix) against the bf16 MFMA dense peak. `cpu_baseline` times the fp64 CPU
oracle on a bounded sample of the same decode workload.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "multi-agent decode tokens/s + % HBM roofline at 32K shared prefix"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0

WORKLOADS = {
    # name: (layers, Hq, Hkv, d, hidden, r, agents, mode (1 BaseLRShared, 0 BaseShared), prefix)
    "llama3-8b-attn-32k": (32, 32, 8, 128, 4096, 8, 4, 1, 32768),
    "llama3-8b-attn-33k": (32, 32, 8, 128, 4096, 8, 4, 1, 33792),
    "llama3-8b-attn-66k": (32, 32, 8, 128, 4096, 8, 4, 1, 67584),
    # the other workloads' shapes (their decode and prefill legs, and the many-agent mixed step)
    "tiny-1l-d64-1k": (1, 14, 2, 64, 896, 8, 2, 0, 1024),
    "qwen2.5-1.5b-attn-1k": (28, 12, 2, 128, 1536, 16, 2, 0, 1024),
    "qwen2.5-1.5b-attn-2k": (28, 12, 2, 128, 1536, 16, 2, 0, 2048),
    "qwen2.5-1.5b-attn-4k": (28, 12, 2, 128, 1536, 16, 2, 0, 4096),
    "qwen2.5-1.5b-attn-8k": (28, 12, 2, 128, 1536, 16, 2, 0, 8192),
    "qwen3-1.7b-attn-8k": (28, 16, 8, 128, 2048, 16, 2, 0, 8192),
    "many-agent-28l-16k": (28, 16, 8, 128, 2048, 16, 8, 0, 16384),
    # one GPU's shard of the headline when its 8 KV heads are split over 8 GPUs
    # (one KV head, its 4 query heads; the low-rank rows and B_i columns of that head)
    "llama3-8b-attn-32k-kvshard8": (32, 4, 1, 128, 4096, 8, 4, 1, 32768),
}


def split_kernel_name(d, rows, planes, r):
    """Template arguments the library picks for the split pass (row blocks of 16
    stacked query rows, low-rank blocks of 16 stacked plane ranks)."""
    rb = (rows + 15) // 16
    rb = 1 if rb <= 1 else (2 if rb <= 2 else 4)
    mb = (planes * r + 15) // 16
    mb = 1 if mb <= 1 else (2 if mb <= 2 else (4 if mb <= 4 else 8))
    return f"decode_split_kernel<{d},{rb},{mb}>"


def decode_split_bytes(Hkv, d, r, hidden, prefix, suffixes, n_agents, Hq, bls=True):
    """Algorithmic bytes the split launch of one fused decode step must move:
    the shared K and V rows once per KV head, the shared low-rank rows (one
    plane, or one per agent), each agent's cached own K/V/low-rank rows, the
    queries, and the step's low-rank appends (x rows and A read, the rows
    written). suffixes are the own lengths before the step."""
    shared = 4 * Hkv * d * prefix + 2 * r * (prefix if bls else prefix * n_agents)
    own = sum(s * (4 * Hkv * d + 2 * r) for s in suffixes)
    append = n_agents * (2 * r + 2 * hidden) + 2 * hidden * r * (1 if bls else n_agents)
    return shared + own + 2 * n_agents * Hq * d + append


def decode_step_bytes(Hkv, d, r, hidden, prefix, suffixes, n_agents, Hq, bls=True):
    """Algorithmic bytes of one fused decode-step launch at one layer: the
    shared K and V rows once per KV head, the shared low-rank rows (one plane,
    or one per agent), each agent's cached own K/V/low-rank rows, the queries
    read and the outputs written, each agent's B_i, and the step's appends (new
    K/V/low-rank rows written, x rows and A read). suffixes are the own lengths
    before the step."""
    shared = 4 * Hkv * d * prefix + 2 * r * (prefix if bls else prefix * n_agents)
    own = sum(s * (4 * Hkv * d + 2 * r) for s in suffixes)
    qo = 4 * n_agents * Hq * d
    b_i = 2 * n_agents * r * Hkv * d
    append = n_agents * (4 * Hkv * d + 2 * r + 2 * hidden) + 2 * hidden * r * (1 if bls else n_agents)
    return shared + own + qo + b_i + append


def project_flops(Hq, Hkv, d, hidden, r, rows):
    """Algorithmic flops of one front-end call: x [rows][hidden] times the
    stacked q, k, v weights and the rank-r A."""
    return 2 * rows * hidden * ((Hq + 2 * Hkv) * d + r)


def project_bytes(Hq, Hkv, d, hidden, r, rows, planes):
    """Algorithmic bytes of one front-end call: the weights, x and A read once;
    q, k, v and the low-rank rows written once."""
    return 2 * ((Hq + 2 * Hkv) * d * hidden + rows * hidden + planes * hidden * r
                + rows * (Hq + 2 * Hkv) * d + rows * r)


def project_kernel_name(Hq, Hkv, d, rows):
    """Template arguments the library picks for a front-end call of one
    agent's rows: the split form up to 16 rows, else 128-token tiles of three
    or four half units or 256-token tiles of four, whichever gives the fewest
    rounds of workgroups over the 256 CUs (the low-rank blocks included) times
    bytes copied per tile and stage (28, 32 and 48 KB)."""
    if rows <= 16:
        return f"project_split_kernel<{d}>"
    units = (Hq + 2 * Hkv) * d // 64
    app = -(-rows // 16) if rows > 8 else rows
    t128, t256 = -(-rows // 128), -(-rows // 256)
    c4 = -(-(-(-2 * units // 4) * t128 + app) // 256) * 32
    c3 = -(-(-(-2 * units // 3) * t128 + app) // 256) * 28
    ct = -(-(-(-2 * units // 4) * t256 + app) // 256) * 48
    if ct < c4 and ct < c3:
        return f"project_tall_kernel<{d}>"
    nh = 3 if c3 < c4 and c3 <= ct else 4
    return f"project_wide_kernel<{d},4,{nh}>"


def frontend_timing(B, cfg, randn, reps=20):
    """Times skv_project_append on one layer (HIP events on the library's
    stream): one row per agent (the decode step's shape, bound by streaming the
    weights) and 512 rows of one agent (a suffix, bound by the matrix cores).
    For context, the same products as one hipBLASLt GEMM (torch.matmul, no
    rotation, no writes into pages)."""
    import torch
    Hq, Hkv, d, hidden, r, N, mode = (cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["hidden"],
                                      cfg["rank"], cfg["n_agents"], cfg["mode"])
    F = (Hq + 2 * Hkv) * d
    cfg = dict(cfg, max_pages=64)  # rows are cropped after every call
    arena = torch.zeros(B.skv_arena_bytes(cfg), dtype=torch.uint8, device="cuda")
    ctx = B.skv_create(cfg, arena)
    w = randn(F, hidden, var=1.0 / hidden)
    wp = torch.empty_like(w)
    B.skv_pack_qkv(ctx, w, wp)
    A = randn(*((N, hidden, r) if mode == 0 else (hidden, r)), var=1.0 / hidden)
    out = {}
    for name, agents, counts in (("decode_rows", list(range(N)), [1] * N), ("suffix_rows", [0], [512])):
        T = sum(counts)
        x = randn(T, hidden)
        q = torch.empty(T, Hq, d, dtype=torch.bfloat16, device="cuda")
        for _ in range(3):
            B.skv_project_append(ctx, 0, agents, counts, x, wp, A, 500000.0, q)
            for a in agents:
                B.skv_crop(ctx, a, 0)
        B.skv_set_timing(ctx, True, ["project"])
        B.skv_collect_timing(ctx)
        for _ in range(reps):
            B.skv_project_append(ctx, 0, agents, counts, x, wp, A, 500000.0, q)
            for a in agents:
                B.skv_crop(ctx, a, 0)
        ms, n = B.skv_collect_timing(ctx)["project"]
        B.skv_set_timing(ctx, False)
        us = 1e3 * ms / n
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            x @ w.t()
        e0.record()
        for _ in range(reps):
            x @ w.t()
        e1.record()
        torch.cuda.synchronize()
        gemm_us = 1e3 * e0.elapsed_time(e1) / reps
        fl = project_flops(Hq, Hkv, d, hidden, r, T)
        by = project_bytes(Hq, Hkv, d, hidden, r, T, N if mode == 0 else 1)
        rec = {"rows": T, "avg_launch_us": round(us, 3), "flops": fl, "bytes": by,
               "tflops": round(fl / us / 1e6, 1), "gbs": round(by / us / 1e3, 1),
               "kernel": project_kernel_name(Hq, Hkv, d, T),
               "hipblaslt_gemm_only_us": round(gemm_us, 3)}
        if T <= 16:
            rec.update(bound="hbm", peak=HBM_PEAK_GBS, unit="GB/s", frac=round(by / us / 1e3 / HBM_PEAK_GBS, 4))
        else:
            rec.update(bound="mfma", peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                       frac=round(fl / us / 1e6 / BF16_PEAK_TFLOPS, 4))
        out[name] = rec
    B.skv_destroy(ctx)
    return out


def prefill_flops(Hq, d, r, views, n_q):
    """Algorithmic flops of one prefill call: visible causal pairs only."""
    tot = 0
    for L, n in zip(views, n_q):
        pairs = n * (L - n) + n * (n + 1) // 2
        tot += Hq * ((4 * d + 2 * r) * pairs + 2 * r * d * n)
    return tot


def kernel_hash():
    """Hash of the kernel source's code with comments and blank lines removed, so
    that a comment edit does not orphan counters taken on the same code."""
    p = os.path.join(ROOT, "lora_shared_kv_amd", "csrc", "kernels.hip")
    src = open(p).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    code = "\n".join(l.rstrip() for l in src.splitlines() if l.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def load_traffic(name):
    """HBM traffic per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel source; otherwise None."""
    p = os.path.join(ROOT, "profiles", name)
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, budget_s=15.0):
    """The fp64 oracle, as it stands, on one layer of the same decode step."""
    import numpy as np
    from oracle.cache import CacheModel
    from oracle.attention import attention_outputs
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    L, Hq, Hkv, d, hidden, r, N, mode, prefix = cfg
    rng = np.random.default_rng(2024)
    c = CacheModel(1, Hq, Hkv, d, hidden, r, N, mode, 64, prefix // 64 + 64)
    c.append_base(0, -1, rng.standard_normal((prefix, Hkv, d)), rng.standard_normal((prefix, Hkv, d)))
    A = rng.standard_normal((hidden, r)) / np.sqrt(hidden)
    for lo in range(0, prefix, 4096):
        n = min(4096, prefix - lo)
        c.append_lowrank(0, -1, 0, n, rng.standard_normal((n, hidden)), A)
    for a in range(N):
        c.crop(a, prefix)
    Bm = rng.standard_normal((N, r, Hkv * d)) * np.sqrt(0.01 / r)

    def time_decode(budget):
        steps, t0 = 0, time.perf_counter()
        while True:
            k = rng.standard_normal((N, Hkv, d))
            c.append_agents(0, list(range(N)), [1] * N, k, k, rng.standard_normal((N, hidden)), A)
            q = rng.standard_normal((N, Hq, d))
            attention_outputs(c, 0, list(range(N)), [1] * N, q, Bm)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return steps, el

    steps, el = time_decode(budget_s)
    per_layer = el / steps
    tok_s = N / (per_layer * L)
    one_core = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            s1, e1 = time_decode(budget_s / 3)
        one_core = {"value": round(N / (e1 / s1 * L), 4), "unit": "tokens/s", "cores": 1,
                    "sample": f"{s1} decode steps of 1 layer timed for {e1:.1f} s with BLAS limited to one thread"}
        steps += s1
    except Exception as exc:  # threadpoolctl missing: report the all-threads figure only
        one_core = {"error": str(exc)}
    # the same oracle on a sample of one suffix prefill call (512 own tokens per
    # agent): a few query rows of each agent, scaled to the call's rows
    n_pre = 512
    kx = rng.standard_normal((N * n_pre, Hkv, d))
    c.append_agents(0, list(range(N)), [n_pre] * N, kx, kx, rng.standard_normal((N * n_pre, hidden)), A)
    qp = rng.standard_normal((N * n_pre, Hq, d))
    sample = [a * n_pre + i for a in range(N) for i in (0, n_pre // 2, n_pre - 1)]
    t1 = time.perf_counter()
    attention_outputs(c, 0, list(range(N)), [n_pre] * N, qp, Bm, rows=sample)
    call_s = (time.perf_counter() - t1) / len(sample) * N * n_pre
    view = prefix + steps + n_pre
    flops = prefill_flops(Hq, d, r, [view] * N, [n_pre] * N)
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count() or 1
    return {"value": round(tok_s, 4), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "nproc": nproc, "one_core": one_core,
            "sample": f"{steps} decode steps of 1 layer (4 agents, fp64, prefix {prefix}) timed for "
                      f"{el:.1f} s; per-layer time x {L} layers",
            "prefill": {"value": round(flops / call_s / 1e12, 6), "unit": "TFLOP/s",
                        "sample": f"{len(sample)} of the {N * n_pre} query rows of one prefill call "
                                  f"(4 agents x {n_pre} tokens, view {view}), time scaled to all rows"}}


def ttft_sweep(reps=5):
    """Time to the first token of a new role, reusing the cached context versus
    processing it again, on every layer of the attention path (appends,
    prefill, one decode step), median of `reps` runs.

    qwen3 shapes (28 layers, 16/8 heads, hidden 2048, rank 16), 8,192-token
    base prefix with adapters off: a specialist takes over at b = 8192 - k and
    recomputes the last k tokens with its adapter (k = 0: its first decode
    token is its own), against the native path in which it processes all 8,192
    tokens itself (paperlayer summary of arXiv 2609.17109, Sec. 3.1, Table 1).
    qwen2.5 shapes (28 layers, 12/2 heads, hidden 1536, rank 16), shared context
    of 1k-8k tokens: the next role computes only its 256-token turn over the
    shared cache, against a per-role cache that must prefill the whole context
    plus the turn (RoleKV, "Accomplishments that we're proud of": role-switch
    first-token latency over the 1k-8k sweep)."""
    import torch
    from lora_shared_kv_amd import skv as B
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(2025)

    def randn(*shape, var=1.0):
        t = torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)
        if var != 1.0:
            t.mul_(var ** 0.5)
        return t.to(torch.bfloat16)

    def one(name, prefix, lr_prefix, b_new, n_new):
        """Median ms of: agent 0 attached at b_new appends n_new own rows with its
        adapter and prefills them on every layer, then one decode step."""
        L, Hq, Hkv, d, hidden, r, N, mode, _ = WORKLOADS[name]
        max_pages = prefix // 64 + (n_new + 2) // 64 + 8
        cfg = dict(n_layers=L, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, hidden=hidden, rank=r, n_agents=N,
                   mode=mode, page_size=64, max_pages=max_pages)
        arena = torch.empty(B.skv_arena_bytes(cfg), dtype=torch.uint8, device=dev)
        ctx = B.skv_create(cfg, arena)
        A = randn(N, hidden, r, var=1.0 / hidden) if mode == 0 else randn(hidden, r, var=1.0 / hidden)
        Bw = randn(N, r, Hkv * d, var=0.01 / r)
        if b_new > 0:
            for l in range(L):
                for lo in range(0, prefix, 8192):
                    n = min(8192, prefix - lo)
                    B.skv_append_base(ctx, l, -1, randn(n, Hkv, d), randn(n, Hkv, d))
                    for pl in (range(N) if mode == 0 else [0]):
                        x = randn(n, hidden) if lr_prefix else None
                        B.skv_append_lowrank(ctx, l, -1, pl, n, x, (A[pl].contiguous() if mode == 0 else A)
                                             if lr_prefix else None)
        kt, vt, xt, qt = (randn(max(n_new, 1), Hkv, d), randn(max(n_new, 1), Hkv, d),
                          randn(max(n_new, 1), hidden), randn(max(n_new, 1), Hq, d))
        ot = torch.empty_like(qt)
        k1, v1, x1, q1 = randn(1, Hkv, d), randn(1, Hkv, d), randn(1, hidden), randn(1, Hq, d)
        o1 = torch.empty_like(q1)
        times = []
        for rep in range(reps + 1):
            B.skv_crop(ctx, 0, 0)
            B.skv_crop(ctx, 0, b_new)
            B.skv_sync(ctx)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for l in range(L):
                for lo in range(0, n_new, 8192):
                    n = min(8192, n_new - lo)
                    B.skv_append_agents(ctx, l, [0], [n], kt[lo:lo + n], vt[lo:lo + n], xt[lo:lo + n], A)
                if n_new:
                    B.skv_attn_prefill(ctx, l, [0], [b_new], [n_new], [n_new], qt[:n_new], Bw, ot[:n_new])
            for l in range(L):
                B.skv_decode_step(ctx, l, [0], [b_new], [n_new], k1, v1, x1, A, q1, Bw, o1)
            torch.cuda.synchronize()
            if rep:  # the first run warms the kernels up
                times.append(1e3 * (time.perf_counter() - t0))
        B.skv_destroy(ctx)
        del arena
        times.sort()
        return round(times[len(times) // 2], 3)

    rows = []
    P = 8192
    native = one("qwen3-1.7b-attn-8k", 0, False, 0, P)
    for k in (0, 160, 320):
        reuse = one("qwen3-1.7b-attn-8k", P, False, P - k, k)
        rows.append({"workload": "qwen3-1.7b-attn-8k", "context": P, "takeover_k": k, "reuse_ms": reuse,
                     "native_ms": native, "ratio": round(native / reuse, 2)})
    for P in (1024, 2048, 4096, 8192):
        name = f"qwen2.5-1.5b-attn-{P // 1024}k"
        reuse = one(name, P, True, P, 256)
        reprefill = one(name, 0, True, 0, P + 256)
        rows.append({"workload": name, "context": P, "turn_tokens": 256, "reuse_ms": reuse,
                     "reprefill_ms": reprefill, "ratio": round(reprefill / reuse, 2)})
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--reps", type=int, default=10,
                    help="timed repetitions of the K-step loop; value is the median repetition")
    ap.add_argument("--workload", default="llama3-8b-attn-32k", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-events", action="store_true",
                    help="time the decode steps without per-launch HIP events (no roofline)")
    ap.add_argument("--layout", default="shared", choices=["shared", "private", "fullshared"],
                    help="shared: the prefix once, in SHARED pages (the method); fullshared: the same pages, "
                         "but every agent uses one full cache (no low-rank rows, no B_i: the pages' "
                         "FullShared, which gives up the per-agent adapter term); private: every agent "
                         "holds its own copy of the prefix in its own pages (the Non-Shared comparison)")
    ap.add_argument("--adapters", default=None, choices=["BaseShared", "BaseLRShared"],
                    help="adapter mode instead of the workload's (BaseShared: one A_i per agent)")
    ap.add_argument("--ttft", action="store_true",
                    help="time one new agent's first token: its rows and prefill on every layer (the default)")
    ap.add_argument("--no-ttft", action="store_true", help="skip the time-to-first-token leg")
    ap.add_argument("--mixed", type=int, default=0, metavar="K",
                    help="also time K mixed steps: the first half of the agents append and prefill 512 "
                         "own tokens while the second half decode one token, on every layer")
    ap.add_argument("--frontend", action="store_true",
                    help="time the fused front end (skv_project_append) on one layer of the workload: "
                         "one row per agent (a decode step) and 512 rows of one agent (a suffix) (the default)")
    ap.add_argument("--no-frontend", action="store_true", help="skip the front-end leg")
    ap.add_argument("--no-launch-pattern", action="store_true",
                    help="skip the launch-pattern probe (the decode step's launches without their arithmetic)")
    ap.add_argument("--ttft-sweep", action="store_true",
                    help="only time the first token of a new role, reusing the cache versus re-prefilling it, "
                         "at the qwen3 8K takeover shapes and the qwen2.5 1k-8k contexts; prints one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    if args.ttft_sweep:
        rows = ttft_sweep()
        print(json.dumps({"metric": "time to first token after a role switch: cache reuse vs re-prefill "
                                    "(attention path, all layers)", "unit": "ms", "higher_is_better": False,
                          "n_gpus": 1, "data": "synthetic", "sweep": rows}), flush=True)
        return

    import torch
    from lora_shared_kv_amd import skv as B

    cfg = WORKLOADS[args.workload]
    L, Hq, Hkv, d, hidden, r, N, mode, prefix = cfg
    if args.adapters:
        mode = 1 if args.adapters == "BaseLRShared" else 0
    private = args.layout == "private"
    fullshared = args.layout == "fullshared"
    if fullshared:
        mode = 1  # one plane, which holds zero rows
    default_run = args.layout == "shared" and mode == cfg[7]
    G = Hq // Hkv
    total_steps = args.warmup + args.steps
    prefill_n = 512
    own_max = (args.warmup + (args.reps + 2) * args.steps + (0 if args.no_prefill else prefill_n) + args.mixed * (prefill_n + 1)
               + (0 if args.no_ttft else prefill_n + 1))
    if private:
        max_pages = N * ((prefix + own_max) // 64 + 2) + 4
    else:
        max_pages = prefix // 64 + 1 + N * (own_max // 64 + 2) + 4
    c = dict(n_layers=L, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, hidden=hidden, rank=r,
             n_agents=N, mode=mode, page_size=64, max_pages=max_pages)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    arena = torch.empty(B.skv_arena_bytes(c), dtype=torch.uint8, device=dev)
    ctx = B.skv_create(c, arena, stream)

    # measured ceilings on this machine (reported beside the vendor peaks): a
    # streaming read over 2 GiB (well past the 256 MB infinity cache) and a
    # dense bf16 MFMA issue loop
    probe_buf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    stream_gbs = B.skv_probe_stream_read(probe_buf, reps=5)
    del probe_buf
    mfma_tflops = B.skv_probe_mfma_bf16()
    # the same MFMA loop on normal draws as operands: the power limit sets the
    # clock of a sustained matrix load, and real operand data draws more power
    # than the constant operands above
    og = torch.Generator(device=dev)
    og.manual_seed(1004)
    operands = torch.randn(8192, generator=og, device=dev).to(torch.bfloat16)  # 16 KiB
    mfma_data_tflops = B.skv_probe_mfma_bf16_data(operands)
    del operands
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)

    gen = torch.Generator(device=dev)
    gen.manual_seed(1003)

    def randn(*shape, var=1.0):
        t = torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32)
        if var != 1.0:
            t.mul_(var ** 0.5)
        return t.to(torch.bfloat16)

    # ---- setup: the prefix's base K/V and low-rank rows, once in SHARED pages
    # (shared layout) or once per agent in its own pages (private layout) ----
    A = randn(N, hidden, r, var=1.0 / hidden) if mode == 0 else randn(hidden, r, var=1.0 / hidden)
    A_of = (lambda a: A[a].contiguous()) if mode == 0 else (lambda a: A)
    plane_of = (lambda a: a) if mode == 0 else (lambda a: 0)
    Bw = randn(N, r, Hkv * d, var=0.01 / r)
    if fullshared:
        Bw.zero_()  # no per-agent adapter term
    chunk = 8192
    xbuf = randn(chunk, hidden)
    for l in range(L):
        for lo in range(0, prefix, chunk):
            n = min(chunk, prefix - lo)
            k_rows, v_rows = randn(n, Hkv, d), randn(n, Hkv, d)
            x_rows = xbuf[:n].contiguous()
            if private:
                # the same context rows in every agent's own pages, each with its own adapter
                for a in range(N):
                    B.skv_append_base(ctx, l, a, k_rows, v_rows)
                    B.skv_append_lowrank(ctx, l, a, plane_of(a), n, x_rows, A_of(a))
            else:
                B.skv_append_base(ctx, l, -1, k_rows, v_rows)
                for pl in (range(N) if mode == 0 else [0]):
                    if fullshared:
                        B.skv_append_lowrank(ctx, l, -1, pl, n, None, None)
                    else:
                        B.skv_append_lowrank(ctx, l, -1, pl, n, x_rows, A_of(pl))
    if not private:
        for a in range(N):
            B.skv_crop(ctx, a, prefix)
    B.skv_sync(ctx)
    base0, own0 = (0, prefix) if private else (prefix, 0)
    cnt = B.skv_get_counters(ctx)
    page_kv = 64 * 4 * Hkv * d  # K and V bytes of one page of one layer
    memory = {"kv_pages": int(cnt["pages_alloc"] - cnt["pages_freed"]),
              "kv_bytes": int((cnt["pages_alloc"] - cnt["pages_freed"]) * page_kv),
              "lr_rows": int(cnt["lr_rows"]), "lr_bytes": int(cnt["lr_rows"]) * 2 * r,
              "arena_bytes": int(arena.numel())}
    agents = list(range(N))
    kin = [randn(N, Hkv, d) for _ in range(L)]
    vin = [randn(N, Hkv, d) for _ in range(L)]
    xin = [randn(N, hidden) for _ in range(L)]
    qin = [randn(N, Hq, d) for _ in range(L)]
    out = [torch.empty(N, Hq, d, dtype=torch.bfloat16, device=dev) for _ in range(L)]
    # Device addresses and C int arrays are marshalled once; the step loop only
    # updates the suffix lengths it passes (and the library checks them).
    ptr = lambda ts: [t.data_ptr() for t in ts]
    kp, vp, xp, qp, op = ptr(kin), ptr(vin), ptr(xin), ptr(qin), ptr(out)
    if fullshared:
        xp = [0] * L  # zero low-rank rows for the new tokens too
    Ap, Bp = A.data_ptr(), Bw.data_ptr()
    ag = B.int_array(agents)
    ones = B.int_array([1] * N)
    bl = B.int_array([base0] * N)
    sl = B.int_array([own0] * N)
    S = [own0] * N

    def step():
        # one fused decode step per layer: append each agent's new row, attend
        for a in range(N):
            sl[a] = S[a]
        for l in range(L):
            B.skv_decode_step(ctx, l, ag, bl, sl, kp[l], vp[l], xp[l], Ap, qp[l], Bp, op[l])
        for a in range(N):
            S[a] += 1

    for _ in range(args.warmup):
        step()
    B.skv_sync(ctx)
    torch.cuda.synchronize()

    # ---- timed region: REPS repetitions of K decode steps (no events), each
    # bracketed by device synchronisation; value = the median repetition ----
    reps_ms = []
    for _ in range(args.reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        reps_ms.append(1e3 * (time.perf_counter() - t0))
    srt = sorted(reps_ms)
    med_ms = srt[len(srt) // 2] if len(srt) % 2 else 0.5 * (srt[len(srt) // 2 - 1] + srt[len(srt) // 2])
    ms_per_step = med_ms / args.steps
    value = N * args.steps / (med_ms / 1e3)
    spread = {"reps": args.reps, "ms_per_step_min": round(srt[0] / args.steps, 4),
              "ms_per_step_max": round(srt[-1] / args.steps, 4),
              "tokens_per_s_min": round(N * args.steps / (srt[-1] / 1e3), 2),
              "tokens_per_s_max": round(N * args.steps / (srt[0] / 1e3), 2)}
    # algorithmic bytes of one step over all layers (at the views of the timed
    # repetitions' middle step) against the median step time
    mid_S = S[0] - (args.reps * args.steps) // 2
    step_bytes = L * decode_step_bytes(Hkv, d, r, hidden, base0, [mid_S] * N, N, Hq, bls=mode == 1)
    step_gbs = step_bytes / (ms_per_step / 1e3) / 1e9
    step_roofline = {"bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4), "measured_peak": round(stream_gbs, 1),
                     "frac_of_measured": round(step_gbs / stream_gbs, 4),
                     "algorithmic_bytes_per_step": int(step_bytes), "launches_per_step": 2 * L}

    # ---- second timed region: the same steps with HIP events recorded by the
    # dispatch of each decode launch on the library's stream -> roofline ----
    suffix_hist = []
    times = {}
    if not args.no_events:
        B.skv_set_timing(ctx, True, ["decode_split", "decode_merge"])
        # an untimed pass first fills the library's pool of events: creating
        # them inside the measured pass would slow the host below the GPU's
        # pace, and a launch that reaches an idle GPU has its start event
        # stamped before the dispatch latency
        for _ in range(args.steps):
            step()
        B.skv_collect_timing(ctx)
        # The timed launches dispatch their own start and stop events, which
        # costs the host more per launch than the GPU spends on a layer; a
        # launch that finds the GPU idle would then have its dispatch latency
        # inside its interval. A spin kernel ahead of the pass holds the GPU
        # while the host queues every launch of it, so they run back to back.
        ev_steps = min(args.steps, 8)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(1 << 20)
        e1.record()
        e1.synchronize()
        spin_cycles = int((1 << 20) * 40.0 / max(e0.elapsed_time(e1), 1e-3))  # about 40 ms
        torch.cuda._sleep(spin_cycles)
        for _ in range(ev_steps):
            suffix_hist.append(S[0])
            step()
        times = B.skv_collect_timing(ctx)
        B.skv_set_timing(ctx, False)
    split_ms, split_n = times.get("decode_split", (0.0, 0))
    roofline = None
    if split_n:
        bytes_avg = sum(decode_split_bytes(Hkv, d, r, hidden, base0, [s] * N, N, Hq, bls=mode == 1)
                        for s in suffix_hist) / len(suffix_hist)
        avg_split_s = split_ms / 1e3 / split_n
        achieved = bytes_avg / avg_split_s / 1e9
        traffic = load_traffic("decode_split_traffic.json")
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "measured_peak": round(stream_gbs, 1),
                    "frac_of_measured": round(achieved / stream_gbs, 4),
                    "kernel": split_kernel_name(d, N * G, N if mode == 0 else 1, r),
                    "algorithmic_bytes_per_launch": int(bytes_avg),
                    "avg_launch_us": round(avg_split_s * 1e6, 3)}
    torch.cuda.synchronize()
    memory["peak_allocated_bytes"] = int(torch.cuda.max_memory_allocated(dev))
    memory["peak_note"] = ("torch allocator peak over setup and the decode steps: the arena (sized for this "
                           "layout's pages) plus the per-layer inputs and outputs")
    per_kernel = {k: {"ms_total": round(v[0], 3), "launches": v[1],
                      "avg_us": round(1e3 * v[0] / max(v[1], 1), 3)} for k, v in times.items() if v[1]}

    # ---- suffix prefill: 4 agents x 512 tokens on every layer, same prefix ----
    prefill = None
    if not args.no_prefill:
        kp = randn(N * prefill_n, Hkv, d)
        xp = randn(N * prefill_n, hidden)
        qp = randn(N * prefill_n, Hq, d)
        op = torch.empty_like(qp)
        for l in range(L):
            B.skv_append_agents(ctx, l, agents, [prefill_n] * N, kp, kp, xp, A)
        B.skv_sync(ctx)
        Ssuf = S[0] + prefill_n
        B.skv_set_timing(ctx, True)
        B.skv_collect_timing(ctx)
        for l in range(L):
            B.skv_attn_prefill(ctx, l, agents, [base0] * N, [Ssuf] * N, [prefill_n] * N, qp, Bw, op)
        pt = B.skv_collect_timing(ctx)
        B.skv_set_timing(ctx, False)
        # one call per layer: the prefill launch, plus a merge launch when its key
        # ranges are split
        pms = pt["prefill"][0]
        pn = L
        fl = prefill_flops(Hq, d, r, [base0 + Ssuf] * N, [prefill_n] * N)
        tf = fl / (pms / 1e3 / pn) / 1e12
        prefill = {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                   "frac": round(tf / BF16_PEAK_TFLOPS, 4), "kernel": f"prefill_kernel<{d},{(r + 15) // 16},2,8,false>",
                   "measured_peak": round(mfma_tflops, 1), "frac_of_measured": round(tf / mfma_tflops, 4),
                   "measured_peak_data": round(mfma_data_tflops, 1),
                   "frac_of_measured_data": round(tf / mfma_data_tflops, 4),
                   "flops_per_launch": fl, "avg_launch_ms": round(pms / pn, 4),
                   "ms_all_layers": round(pms, 3), "n_q_per_agent": prefill_n,
                   "view": base0 + Ssuf}
        S = [Ssuf] * N

    # ---- mixed steps (the many-agent turn): half the agents prefill 512 own
    # tokens while the other half decode one token each, on every layer ----
    mixed = None
    if args.mixed and N >= 2 and not args.no_prefill:
        grp_p, grp_d = agents[:N // 2], agents[N // 2:]
        np_ = len(grp_p)
        kx, vx, xx = randn(np_ * prefill_n, Hkv, d), randn(np_ * prefill_n, Hkv, d), randn(np_ * prefill_n, hidden)
        qx = randn(np_ * prefill_n, Hq, d)
        ox = torch.empty_like(qx)
        nd = len(grp_d)
        kd, vd, xd, qd = randn(nd, Hkv, d), randn(nd, Hkv, d), randn(nd, hidden), randn(nd, Hq, d)
        od = torch.empty_like(qd)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.mixed):
            for l in range(L):
                B.skv_append_agents(ctx, l, grp_p, [prefill_n] * np_, kx, vx, xx, A)
                B.skv_attn_prefill(ctx, l, grp_p, [base0] * np_, [S[a] + prefill_n for a in grp_p],
                                   [prefill_n] * np_, qx, Bw, ox)
                B.skv_decode_step(ctx, l, grp_d, [base0] * nd, [S[a] for a in grp_d], kd, vd, xd, A, qd, Bw, od)
            for a in grp_p:
                S[a] += prefill_n
            for a in grp_d:
                S[a] += 1
        torch.cuda.synchronize()
        mixed = {"ms_per_step": round(1e3 * (time.perf_counter() - t0) / args.mixed, 3), "steps": args.mixed,
                 "prefill_agents": np_, "prefill_tokens": prefill_n, "decode_agents": nd}

    # ---- time to first token of one new agent (agent 0 starts over): its rows
    # and its prefill on every layer, then one decode step. Shared layout: its
    # 512-token suffix over the cached prefix. Private layout: it must first
    # build its own copy of the prefix, so its rows and queries cover the whole
    # context ----
    ttft = None
    if not args.no_ttft:
        a0 = [0]
        n_new = prefill_n + (prefix if private else 0)
        B.skv_crop(ctx, 0, 0 if private else prefix)
        B.skv_sync(ctx)
        kt, vt, xt = randn(n_new, Hkv, d), randn(n_new, Hkv, d), randn(n_new, hidden)
        qt = randn(n_new, Hq, d)
        ot = torch.empty_like(qt)
        k1, v1, x1, q1 = randn(1, Hkv, d), randn(1, Hkv, d), randn(1, hidden), randn(1, Hq, d)
        o1 = torch.empty_like(q1)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(L):
            for lo in range(0, n_new, chunk):
                n = min(chunk, n_new - lo)
                B.skv_append_agents(ctx, l, a0, [n], kt[lo:lo + n], vt[lo:lo + n], xt[lo:lo + n], A)
            B.skv_attn_prefill(ctx, l, a0, [base0], [n_new], [n_new], qt, Bw, ot)
        for l in range(L):
            B.skv_decode_step(ctx, l, a0, [base0], [n_new], k1, v1, x1, A, q1, Bw, o1)
        torch.cuda.synchronize()
        ttft = {"ms": round(1e3 * (time.perf_counter() - t0), 3), "rows_appended_per_layer": n_new + 1,
                "queries_prefilled_per_layer": n_new}

    frontend = None
    if not args.no_frontend:
        frontend = frontend_timing(B, dict(c, n_layers=1), randn, reps=20)

    # ---- the decode step's launch pattern without its arithmetic: per layer a
    # streaming read of the split pass's algorithmic bytes by one workgroup per
    # CU, then a small launch of one workgroup per query row ordered after it.
    # Its step time bounds what any two-launch-per-layer decode step can reach
    # on this machine ----
    launch_pattern = None
    if not args.no_launch_pattern and not args.no_events:
        # the split pass's algorithmic bytes at the timed repetitions' middle step
        lb = (decode_split_bytes(Hkv, d, r, hidden, base0, [mid_S] * N, N, Hq, bls=mode == 1) + 15) // 16 * 16
        buf = torch.empty(L * lb, dtype=torch.uint8, device=dev)
        pat_ms, str_ms = B.skv_probe_launch_pattern(buf, lb, L, steps=20, tail_blocks=N * Hq)
        del buf
        ceiling = N / (pat_ms / 1e3)
        launch_pattern = {"layer_bytes": lb, "layers": L, "tail_blocks": N * Hq,
                          "ms_per_step": round(pat_ms, 4), "ms_per_step_stream_only": round(str_ms, 4),
                          "stream_only_gbs": round(L * lb / (str_ms / 1e3) / 1e9, 1),
                          "tokens_per_s_ceiling": round(ceiling, 1),
                          "frac_of_ceiling": round(value / ceiling, 4)}

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "timing": spread,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "layers": L, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": d, "hidden": hidden, "rank": r, "agents": N,
                   "mode": "BaseLRShared" if mode == 1 else "BaseShared",
                   "layout": args.layout, "shared_prefix": prefix,
                   "decode_tokens_per_step": N, "global_batch": N, "seq_len": prefix,
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "step_roofline": step_roofline,
        "kernels": per_kernel,
        "prefill": prefill,
        "memory": memory,
        "cpu_baseline": None,
    }
    if ttft is not None:
        res["ttft"] = ttft
    if frontend is not None:
        res["frontend"] = frontend
    if mixed is not None:
        res["mixed"] = mixed
    if launch_pattern is not None:
        res["launch_pattern"] = launch_pattern
    if not args.no_cpu_baseline and default_run:
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
