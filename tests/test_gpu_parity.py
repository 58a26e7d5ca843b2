"""GPU parity: libskv.so against the fp64 oracle on the same seeded inputs.

Bar (per attention call): max |o_gpu - o_ref| <= 2e-2 and
||o_gpu - o_ref||_2 / ||o_ref||_2 <= 1e-2, with bf16 inputs and fp32
accumulation on the GPU. Cache layout, page ids and crop results are compared
bit-exactly; low-rank rows within one bf16 ulp of bf16(X A).
"""
import numpy as np
import pytest

import synth
from synth import BASE_LR_SHARED, BASE_SHARED, Schedule, Shape, bf16_bits_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(torch_cuda):
    return torch_cuda


def log(msg):
    print(msg, flush=True)


def _runner():
    import gpu_runner
    return gpu_runner


def mini(shape, prefix, own, decode_steps=2, seed=7, attach=None, nq_extra=0, peaked=1.0,
         zero_vbase=False, lr="x", decode_without_append=False):
    sc = Schedule(shape, seed, n_layers=1, peaked=peaked, zero_vbase=zero_vbase)
    sc.draw_adapters()
    sc.shared_prefix(prefix, lr=lr)
    agents = list(range(shape.n_agents))
    for a in agents:
        sc.attach(a, attach[a] if attach else prefix)
    if any(own):
        ag = [a for a in agents if own[a] > 0]
        sc.own_rows(0, ag, [own[a] for a in ag])
    pre = [a for a in agents if own[a] + nq_extra > 0]
    if pre:
        sc.attend("prefill", 0, pre, [min(own[a] + nq_extra, sc.b[a] + sc.S[0][a]) for a in pre],
                  tag="prefill")
    if decode_without_append:
        sc.attend("decode", 0, agents, [1] * len(agents), tag="decode-noappend")
    for t in range(decode_steps):
        sc.own_rows(0, agents, [1] * len(agents))
        sc.attend("decode", 0, agents, [1] * len(agents), tag=f"decode{t}")
    return sc


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------

def test_tiny_fused_decode_steps():
    R = _runner()
    sc = synth.tiny_schedule(fused=True)
    _, _, res = R.run_parity(sc, log=log)
    assert len(res) == 2 + 16


@pytest.mark.parametrize("prefix,steps", [(33792, 3), (32768, 70)])
def test_llama3_fused_decode_steps(prefix, steps):
    # 70 steps from a page-aligned prefix cross into a second own page
    R = _runner()
    sc = synth.llama3_schedule(prefix=prefix, decode=steps, fused=True)
    R.run_parity(sc, log=log)


def test_fused_step_edge_cases():
    """Empty view (the first token is the whole view), zero low-rank rows,
    agents at different boundaries, groups larger than one launch."""
    R = _runner()
    for shape, prefix, attach in [
        (Shape("e", 1, 8, 2, 128, 256, 8, 3, BASE_SHARED, 0), 0, [0, 0, 0]),
        (Shape("e", 1, 8, 2, 64, 256, 16, 3, BASE_SHARED, 0), 200, [200, 131, 64]),
        (Shape("e", 1, 16, 4, 64, 256, 8, 16, BASE_LR_SHARED, 0), 90, None),
    ]:
        sc = Schedule(shape, 11, n_layers=1)
        sc.draw_adapters()
        if prefix:
            sc.shared_prefix(prefix)
        agents = list(range(shape.n_agents))
        for a in agents:
            sc.attach(a, attach[a] if attach else prefix)
        for t in range(3):
            sc.decode_step(0, agents, lr="zero" if t == 1 else "x", tag=f"step{t}")
        R.run_parity(sc, log=log)


def test_fused_step_cache_matches_separate_calls():
    """The fused step leaves the same cache bytes as append + decode."""
    import torch
    R = _runner()
    shape = Shape("e", 1, 16, 4, 128, 512, 16, 3, BASE_SHARED, 0)
    runs = []
    for fused in (False, True):
        sc = Schedule(shape, 5, n_layers=1)
        sc.draw_adapters()
        sc.shared_prefix(300)
        for a in range(3):
            sc.attach(a)
        for t in range(70):
            if fused:
                sc.decode_step(0, [0, 1, 2])
            else:
                sc.own_rows(0, [0, 1, 2], [1, 1, 1])
                sc.attend("decode", 0, [0, 1, 2], [1, 1, 1])
        gpu, orc, _ = R.run_parity(sc)
        runs.append([t.cpu().numpy() for t in _pool_views(gpu)])
    k0, v0, l0 = runs[0]
    k1, v1, l1 = runs[1]
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    d = np.abs(l0.view(np.uint16).astype(np.int32) - l1.view(np.uint16).astype(np.int32))
    assert d.max() <= 1     # low-rank rows: fp32 sums in a different order, at most 1 bf16 ulp


def test_tiny_full_schedule():
    R = _runner()
    sc = synth.tiny_schedule()
    _, _, res = R.run_parity(sc, log=log)
    assert len(res) == 2 + 16


@pytest.mark.parametrize("prefix", [1024, 2048, 4096])
def test_qwen25_turns_with_handoff(prefix):
    R = _runner()
    sc = synth.qwen25_schedule(prefix=prefix, decode_sample=[0, 1, 63, 127])
    R.run_parity(sc, log=log)


def test_qwen25_8k_prefix():
    R = _runner()
    sc = synth.qwen25_schedule(prefix=8192, turns=2, decode=8, decode_sample=[0, 7])
    R.run_parity(sc, log=log)


@pytest.mark.parametrize("takeover", [0, 160, 320])
def test_qwen3_takeover(takeover):
    R = _runner()
    sc = synth.qwen3_schedule(takeover=takeover, decode=6)
    R.run_parity(sc, log=log)


def test_llama3_suffix_prefill_at_32k():
    """The suffix prefill the throughput run times (4 agents x 512 own tokens over
    the 32,768-token shared prefix, llama3 shapes, one launch of 256 row blocks),
    on sampled query rows, then two fused decode steps on the same cache."""
    R = _runner()
    sc = synth.llama3_schedule(prefix=32768, prefill=512, decode=2, fused=True)
    samp = lambda ev: (list(range(0, sum(ev.n_q), 61)) + [sum(ev.n_q) - 1]) if ev.kind == "prefill" else None
    _, _, res = R.run_parity(sc, sample_rows=samp, log=log)
    assert sum(1 for r in res if r[1] == "prefill") == 1


def test_llama3_suffix_prefill_at_32k_every_row():
    """The timed suffix prefill (4 agents x 512 own tokens over the 32,768-token
    shared prefix, llama3 shapes, in its own launch shape), every one of its
    2,048 query rows against the oracle."""
    R = _runner()
    sc = synth.llama3_schedule(prefix=32768, prefill=512, decode=0, seed=1013)
    _, _, res = R.run_parity(sc, log=log)
    assert [r[1] for r in res] == ["prefill"]


@pytest.mark.parametrize("prefix,steps", [(33792, 3), (67584, 2)])
def test_llama3_long_prefix_decode(prefix, steps):
    R = _runner()
    sc = synth.llama3_schedule(prefix=prefix, decode=steps)
    R.run_parity(sc, log=log)


def test_llama3_kv_head_shard():
    """One GPU's share of the headline under KV-head sharding over 8 GPUs: one
    KV head and its 4 query heads (the 4 agents' 16 stacked rows unchanged),
    the shared A's low-rank rows and B_i's columns of that head: a 512-token
    suffix prefill per agent and fused decode steps over a 32,768-token shared
    prefix, every row."""
    R = _runner()
    shape = synth.LLAMA3.with_(n_q_heads=4, n_kv_heads=1, prefix=32768)
    sc = synth.Schedule(shape, 1031, n_layers=1)
    sc.draw_adapters()
    sc.shared_prefix(32768)
    agents = list(range(shape.n_agents))
    for a in agents:
        sc.attach(a)
    sc.own_rows(0, agents, [512] * 4)
    sc.attend("prefill", 0, agents, [512] * 4, tag="shard prefill")
    for t in range(3):
        sc.decode_step(0, agents, tag=f"shard step {t}")
    _, _, res = R.run_parity(sc, log=log)
    assert len(res) == 4


def test_many_agent_mixed_turns():
    """All six turns of the many-agent workload (one layer): four agents
    prefill 512 own tokens while four decode, then the lead agent crops 256
    own rows and re-appends them as canonical rows, so later turns crop agents
    that were cropped and re-appended before. Every query row is compared."""
    R = _runner()
    sc = synth.many_schedule(turns=6)
    _, _, res = R.run_parity(sc, log=log)
    assert len(res) == 12


# --------------------------------------------------------------------------
# shapes, ranks, modes and edge cases
# --------------------------------------------------------------------------

EDGE = [
    # name, shape, prefix, own, kwargs
    ("d64-G7-r8-BS", Shape("e", 1, 14, 2, 64, 896, 8, 2, BASE_SHARED, 0), 1000, [37, 70], {}),
    ("d128-G1-r4-BLS", Shape("e", 1, 4, 4, 128, 256, 4, 3, BASE_LR_SHARED, 0), 333, [1, 64, 129], {}),
    ("d128-G4-r32-BS", Shape("e", 1, 16, 4, 128, 512, 32, 3, BASE_SHARED, 0), 700, [65, 0, 3], {}),
    ("d64-G2-r16-BLS", Shape("e", 1, 4, 2, 64, 128, 16, 2, BASE_LR_SHARED, 0), 64, [64, 1], {}),
    ("hetero-b", Shape("e", 1, 8, 2, 128, 256, 8, 3, BASE_SHARED, 0), 900,
     [10, 40, 0], dict(attach=[900, 517, 130])),
    ("queries-into-shared", Shape("e", 1, 8, 2, 128, 256, 8, 2, BASE_SHARED, 0), 300, [5, 0],
     dict(nq_extra=40)),
    ("decode-at-shared-pos", Shape("e", 1, 8, 4, 64, 128, 8, 2, BASE_LR_SHARED, 0), 131, [0, 0],
     dict(decode_without_append=True, attach=[131, 77])),
    ("8agents-R32", Shape("e", 1, 16, 4, 128, 256, 16, 8, BASE_SHARED, 0), 500, [3] * 8, {}),
    ("16agents-R64-BLS", Shape("e", 1, 16, 4, 64, 256, 8, 16, BASE_LR_SHARED, 0), 257, [2] * 16, {}),
    ("16agents-BS-groups", Shape("e", 1, 8, 2, 64, 128, 16, 16, BASE_SHARED, 0), 190, [1] * 16, {}),
    # 64 stacked rows at head dim 128 (one buffered chunk per wave, pairwise fold), ranks 8 and 32
    ("16agents-R64-BLS-d128", Shape("e", 1, 16, 4, 128, 256, 8, 16, BASE_LR_SHARED, 0), 700, [2] * 16, {}),
    ("16agents-R64-BLS-d128-r32", Shape("e", 1, 16, 4, 128, 256, 32, 16, BASE_LR_SHARED, 0), 333,
     [1, 0] * 8, {}),
    # the remaining split-pass tile shapes (head dim, 16-row blocks, 16-rank blocks):
    # (64, 1, 8) eight planes of rank 16; (128, 2, 4) and (64, 2, 4) four planes over 32 rows;
    # (64, 2, 2) two planes over 32 rows; (64, 4, 2) rank 32 over 64 rows
    ("tiles-d64-1x8", Shape("e", 1, 4, 2, 64, 128, 16, 8, BASE_SHARED, 0), 300, [1, 0, 2, 0, 3, 0, 4, 0], {}),
    ("tiles-d128-2x4", Shape("e", 1, 16, 2, 128, 256, 16, 4, BASE_SHARED, 0), 260, [5, 0, 1, 3], {}),
    ("tiles-d64-2x4", Shape("e", 1, 8, 1, 64, 128, 16, 4, BASE_SHARED, 0), 190, [0, 2, 7, 1], {}),
    ("tiles-d64-2x2", Shape("e", 1, 16, 1, 64, 128, 16, 2, BASE_SHARED, 0), 450, [9, 2], {}),
    ("tiles-d64-4x2", Shape("e", 1, 16, 4, 64, 128, 32, 16, BASE_LR_SHARED, 0), 129, [1] * 16, {}),
    ("peaked-logits", Shape("e", 1, 8, 2, 128, 256, 16, 2, BASE_SHARED, 0), 1500, [100, 7],
     dict(peaked=4.0)),
    ("zero-lr-prefix", Shape("e", 1, 8, 2, 128, 256, 16, 2, BASE_SHARED, 0), 640, [33, 3],
     dict(lr="zero")),
    ("tiny-prefix-1", Shape("e", 1, 8, 2, 128, 256, 8, 2, BASE_SHARED, 0), 1, [1, 2], {}),
]


@pytest.mark.parametrize("name,shape,prefix,own,kw", EDGE, ids=[e[0] for e in EDGE])
def test_edge_cases(name, shape, prefix, own, kw):
    R = _runner()
    sc = mini(shape, prefix, own, **kw)
    R.run_parity(sc, log=lambda m: log(f"[{name}] {m}"))


@pytest.mark.parametrize("shape_name", ["llama3", "qwen3"])
def test_private_prefix_layout(shape_name):
    """The comparison layout in which every agent holds its own copy of the
    context in its own pages (b_i = 0, no shared rows): a 64-query prefill,
    then fused decode steps."""
    R = _runner()
    shape = synth.WORKLOADS[shape_name]
    sc = synth.Schedule(shape, 1011, n_layers=1)
    sc.draw_adapters()
    agents = list(range(shape.n_agents))
    sc.own_rows(0, agents, [2048] * len(agents))
    sc.attend("prefill", 0, agents, [64] * len(agents), tag="private prefill")
    for t in range(3):
        sc.decode_step(0, agents, tag=f"private step {t}")
    assert sc.b == [0] * shape.n_agents
    _, _, res = R.run_parity(sc, log=log)
    assert len(res) == 4


# head dim 64 at rank 8, and rank 32 (two 16-rank blocks in the prefill and decode tiles) at head dims 64
# and 128
OFFSET_SHAPES = {
    "d64-r8-BS": Shape("d64-r8", 1, 14, 2, 64, 896, 8, 2, BASE_SHARED, 0),
    "d64-r32-BLS": Shape("d64-r32", 1, 8, 2, 64, 256, 32, 3, BASE_LR_SHARED, 0),
    "d128-r32-BS": Shape("d128-r32", 1, 8, 4, 128, 256, 32, 2, BASE_SHARED, 0),
}


@pytest.mark.parametrize("shape_name", ["llama3", "qwen3", "d64-r8-BS", "d64-r32-BLS", "d128-r32-BS"])
def test_activation_offsets(shape_name):
    """Adapter activation offsets (RoleKV, "What it does": the adapter switches
    on after the role's header): 0, inside the shared prefix, inside the own
    suffix and beyond the view, through prefill, fused decode steps and a plain
    decode; the last agent's new tokens lie before its offset."""
    R = _runner()
    shape = OFFSET_SHAPES.get(shape_name) or synth.WORKLOADS[shape_name]
    N = shape.n_agents
    prefix, own = 4096, 256
    sc = synth.Schedule(shape, 1012, n_layers=1)
    sc.draw_adapters()
    sc.shared_prefix(prefix)
    agents = list(range(N))
    for a in agents:
        sc.attach(a)
    offsets = [0, 1000, prefix + 37, 1 << 20][:N] if N > 2 else [1000, prefix + 37]
    for a, t in zip(agents, offsets):
        sc.set_lr_begin(a, t)
    sc.own_rows(0, agents, [own] * N)
    sc.attend("prefill", 0, agents, [64] * N, tag="offsets prefill")
    for t in range(3):
        sc.decode_step(0, agents, tag=f"offsets step {t}")
    sc.own_rows(0, agents, [1] * N)
    sc.attend("decode", 0, agents, [1] * N, tag="offsets decode")
    _, _, res = R.run_parity(sc, log=log)
    assert len(res) == 5


@pytest.mark.parametrize("shape_name", ["llama3", "qwen3"])
def test_activation_offset_boundaries(shape_name):
    """V_base = 0, so the output is the adapter term alone, and each agent's
    offset sits a few keys before the end of its view: a key masked or kept
    by mistake changes the output by 10-100%, well past the tolerance."""
    R = _runner()
    shape = synth.WORKLOADS[shape_name]
    N = shape.n_agents
    prefix, own = 2048, 64
    sc = synth.Schedule(shape, 1013, n_layers=1, zero_vbase=True)
    sc.draw_adapters()
    sc.shared_prefix(prefix)
    agents = list(range(N))
    for a in agents:
        sc.attach(a)
    sc.own_rows(0, agents, [own] * N)
    L = prefix + own
    for a, back in zip(agents, [1, 2, 5, 9]):
        sc.set_lr_begin(a, L - back)
    sc.attend("prefill", 0, agents, [16] * N, tag="boundary prefill")
    sc.attend("decode", 0, agents, [1] * N, tag="boundary decode")
    for t in range(2):
        sc.decode_step(0, agents, tag=f"boundary step {t}")
    _, _, res = R.run_parity(sc, log=log)
    assert len(res) == 4


def test_h1_session_with_offsets_and_accounting():
    """A RoleKV-style session (RoleKV, "What it does" and "Challenges we ran
    into"): agents take turns; each turn's adapter switches on after a 5-token
    role header (its activation offset), the speaker appends and prefills its
    rows and decodes; at the hand-off (H1) it crops its last 20 rows and
    recomputes them as canonical rows (adapter off). Every attention call
    matches the oracle, and the library's token accounting (rows appended,
    low-rank rows, zero rows, rows cropped, pages) equals the oracle's
    exactly, recompute included."""
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = synth.WORKLOADS["llama3"]
    N = shape.n_agents
    sc = synth.Schedule(shape, 1021, n_layers=1)
    sc.draw_adapters()
    sc.shared_prefix(1500)
    agents = list(range(N))
    for a in agents:
        sc.attach(a)
    for t in range(2 * N):
        a = t % N
        end = sc.b[a] + sc.S[0][a]
        sc.set_lr_begin(a, end + 5)
        sc.own_rows(0, [a], [40])
        sc.attend("prefill", 0, [a], [16], tag=f"turn {t} prefill")
        for k in range(3):
            sc.decode_step(0, [a], tag=f"turn {t} step {k}")
        end = sc.b[a] + sc.S[0][a]
        sc.crop(a, end - 20)
        sc.own_rows(0, [a], [20], lr="zero")
    sc.attend("decode", 0, agents, [1] * N, tag="after the session")
    gpu, orc, res = R.run_parity(sc, log=log)
    assert len(res) == 2 * N * 4 + 1
    got = B.skv_get_counters(gpu.ctx)
    for k, v in orc.counters.items():
        assert got[k] == v, (k, got[k], v)
    assert orc.counters["rows_cropped"] == 2 * N * 20 and orc.counters["lr_zero_rows"] >= 2 * N * 20


@pytest.mark.parametrize("shape_name", ["llama3", "qwen3"])
def test_canonical_recompute_equals_fresh_appends(shape_name):
    """RoleKV ("How we built it": a hand-off crops the cache and recomputes the
    tokens canonically, which must equal a fresh base prefill of them).
    Context A: agent 0 appends 300 own rows with its adapter (x A), crops back
    to 100 (mid-page: three pages freed, the kept page holds stale slots), agent
    1 takes a freed page, then agent 0 re-appends the 200 tokens as canonical
    rows (the same base K/V, zero low-rank rows). Context B appends the same
    rows fresh, with no crop (so its page ids differ). Every live K/V byte and low-rank row is equal,
    decode and prefill outputs are equal bit for bit, and context A matches
    the oracle."""
    import torch
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = synth.WORKLOADS[shape_name]
    N, Hkv, d = shape.n_agents, shape.n_kv_heads, shape.head_dim
    dr = synth.Draws(4242)
    P = 1000
    kp, vp, xp = dr.normal((P, Hkv, d)), dr.normal((P, Hkv, d)), dr.normal((P, shape.hidden))
    if shape.mode == synth.BASE_SHARED:
        A = dr.normal((N, shape.hidden, shape.rank), 1.0 / shape.hidden)
    else:
        A = dr.normal((shape.hidden, shape.rank), 1.0 / shape.hidden)
    Bw = dr.normal((N, shape.rank, Hkv * d), 0.01 / shape.rank)
    ko, vo, xo = dr.normal((300, Hkv, d)), dr.normal((300, Hkv, d)), dr.normal((300, shape.hidden))
    k1, v1, x1 = dr.normal((80, Hkv, d)), dr.normal((80, Hkv, d)), dr.normal((80, shape.hidden))
    a_of = (lambda p: A[p]) if shape.mode == synth.BASE_SHARED else (lambda p: A)
    head = [synth.AppendBase(0, -1, kp, vp)] + [
        synth.AppendLowrank(0, -1, p, P, xp, a_of(p)) for p in range(synth.n_planes(shape))] + [
        synth.Crop(a, P) for a in range(N)] + [
        synth.AppendAgents(0, [1], [60], k1[:60], v1[:60], x1[:60], A)]
    evA = head + [synth.AppendAgents(0, [0], [300], ko, vo, xo, A), synth.Crop(0, P + 100),
                  synth.AppendAgents(0, [1], [20], k1[60:], v1[60:], x1[60:], A),
                  synth.AppendAgents(0, [0], [200], ko[100:], vo[100:], None, None)]
    evB = head + [synth.AppendAgents(0, [0], [100], ko[:100], vo[:100], xo[:100], A),
                  synth.AppendAgents(0, [0], [200], ko[100:], vo[100:], None, None),
                  synth.AppendAgents(0, [1], [20], k1[60:], v1[60:], x1[60:], A)]
    q_dec = dr.normal((2, shape.n_q_heads, d))
    q_pre = dr.normal((64, shape.n_q_heads, d))
    tail = [synth.Attend("decode", 0, [0, 1], [P, P], [300, 80], [1, 1], q_dec, Bw, "decode after hand-off"),
            synth.Attend("prefill", 0, [0], [P], [300], [64], q_pre, Bw, "prefill after hand-off")]
    sc = synth.Schedule(shape, 1, n_layers=1)
    sc.events = evA + tail
    gA, orc, resA = R.run_parity(sc, max_pages=64, log=log)
    gB = R.GpuRun(sc, max_pages=64)
    for ev in evB:
        gB.apply(ev)
    outB = [gB.apply(ev) for ev in tail]
    B.skv_sync(gB.ctx)
    # the same live bytes, read through each context's page tables
    ki, vi = k_tile_index(d), v_tile_index(d)
    pools = {}
    for name, g in (("A", gA), ("B", gB)):
        K, VT, LRT = (t.cpu().numpy().view(np.uint16) for t in _pool_views(g))
        rows = {}
        for seq, n in ((-1, P), (0, 300), (1, 80)):
            pages = B.skv_get_pages(g.ctx, 0, seq)
            kk = np.stack([K[0, pages[j // 64]][:, ki[j % 64]] for j in range(n)])
            vv = np.stack([VT[0, pages[j // 64]][:, vi[j % 64]] for j in range(n)])
            pl = 0 if seq == -1 or shape.mode == synth.BASE_LR_SHARED else seq
            lr = np.stack([LRT[pl, 0, pages[j // 64], :, j % 64] for j in range(n)])
            rows[seq] = (kk, vv, lr)
        pools[name] = rows
    for seq in (-1, 0, 1):
        for a, b in zip(pools["A"][seq], pools["B"][seq]):
            assert np.array_equal(a, b), seq
    assert np.all(pools["A"][0][2][100:] == 0)          # the recomputed tokens carry no low-rank term
    assert B.skv_get_lens(gA.ctx, 0) == B.skv_get_lens(gB.ctx, 0)
    # agent 1 took a page agent 0 freed, so the page ids differ between the contexts
    assert B.skv_get_pages(gA.ctx, 0, 1) != B.skv_get_pages(gB.ctx, 0, 1)
    assert [r[0] for r in resA] == ["decode after hand-off", "prefill after hand-off"]
    # bit-identical attention over the two caches
    oa = [gA.apply(ev) for ev in tail]
    for x, y in zip(oa, outB):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_lr_only_term():
    """V_base = 0: the output is only (P V_lr) B_i, about 10x smaller than usual."""
    R = _runner()
    shape = Shape("e", 1, 16, 4, 128, 512, 16, 3, BASE_SHARED, 0)
    sc = mini(shape, 700, [40, 9, 1], decode_steps=3, zero_vbase=True)

    def check(ev, got, ref):
        ma, rl = R.errors(got, ref)
        assert rl <= 1e-2, (ev.tag, rl)

    R.run_parity(sc, check=check, log=log)


def test_lr_contribution_difference():
    """The decode output with B_i minus the output with B_i = 0 matches the
    oracle's difference. This is the weaker check of the adapter term: each of
    the two bf16 outputs carries its own rounding, about ten times the adapter
    term's size, so the bar is 1e-2 of the difference plus that rounding floor.
    The adapter term itself is held to rel-L2 1e-2 by the V_base = 0 tests
    (test_lr_only_term, test_activation_offset_boundaries)."""
    import torch
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = Shape("e", 1, 32, 8, 128, 4096, 8, 4, BASE_LR_SHARED, 0)
    sc = mini(shape, 2000, [0, 0, 0, 0], decode_steps=1)
    gpu, orc, _ = R.run_parity(sc)
    ev = sc.events[-1]
    q = R.dev(ev.q)
    o1, o0 = torch.empty_like(q), torch.empty_like(q)
    B.skv_attn_decode(gpu.ctx, 0, ev.agents, ev.base_len, ev.suffix_len, q, R.dev(ev.b), o1)
    B.skv_attn_decode(gpu.ctx, 0, ev.agents, ev.base_len, ev.suffix_len, q,
                      R.dev(np.zeros_like(ev.b)), o0)
    import oracle
    f = bf16_bits_to_f64
    r1 = oracle.attention_outputs(orc, 0, ev.agents, ev.n_q, f(ev.q), f(ev.b))
    r0 = oracle.attention_outputs(orc, 0, ev.agents, ev.n_q, f(ev.q), np.zeros_like(f(ev.b)))
    dg = R.to_f64(o1) - R.to_f64(o0)
    dr = r1 - r0
    err = np.linalg.norm(dg - dr)
    # Each bf16 output carries a rounding error of at most 2^-8 of its value, and
    # the full outputs are about ten times the adapter term, so the difference of
    # two rounded outputs can be off by 2^-8 of the outputs' norm on top of the
    # kernel's own error.
    floor = 2.0 ** -8 * np.sqrt(np.linalg.norm(r1) ** 2 + np.linalg.norm(r0) ** 2)
    log(f"LR difference rel_l2={err / np.linalg.norm(dr):.3e} (rounding floor {floor / np.linalg.norm(dr):.3e})")
    assert err <= 1e-2 * np.linalg.norm(dr) + floor


# --------------------------------------------------------------------------
# layout, low-rank rows, determinism, sharing
# --------------------------------------------------------------------------

def k_tile_index(D):
    return _runner().k_tile_index(D)


def v_tile_index(D):
    return _runner().v_tile_index(D)


def _pool_views(gpu):
    return _runner().pool_views(gpu)


def test_cache_layout_bytes_and_lowrank_rows():
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = Shape("e", 1, 8, 2, 128, 512, 16, 2, BASE_SHARED, 0)
    sc = mini(shape, 333, [70, 5], decode_steps=2)
    gpu, orc, _ = R.run_parity(sc)
    K, VT, LRT = (t.cpu().numpy().view(np.uint16) for t in _pool_views(gpu))
    d = shape.head_dim
    ki, vi = k_tile_index(d), v_tile_index(d)
    for seq in [-1, 0, 1]:
        pages = B.skv_get_pages(gpu.ctx, 0, seq)
        assert pages == orc.pages(0, seq)
        n = orc.length[0][seq]
        kk = np.stack([K[0, pages[j // 64]][:, ki[j % 64]] for j in range(n)])
        vv = np.stack([VT[0, pages[j // 64]][:, vi[j % 64]] for j in range(n)])
        assert np.array_equal(bf16_bits_to_f64(kk), orc.k[0][seq].get(n)), seq
        assert np.array_equal(bf16_bits_to_f64(vv), orc.v[0][seq].get(n)), seq
        for p in orc._planes_of(seq):
            cov = orc.lr_cov[0][seq][p]
            lr = np.stack([LRT[p, 0, pages[j // 64], :, j % 64] for j in range(cov)])
            got = bf16_bits_to_f64(lr)
            ref = orc.lr[0][seq][p].get(cov)
            # within one bf16 ulp of the exact product
            ulp = np.maximum(np.abs(ref), 1e-30)
            ulp = 2.0 ** (np.floor(np.log2(ulp)) - 7)
            assert np.all(np.abs(got - ref) <= ulp), (seq, p, np.max(np.abs(got - ref) / ulp))


def test_one_hot_x_gives_rows_of_A_exactly():
    import torch
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = Shape("e", 1, 4, 2, 64, 128, 8, 1, BASE_SHARED, 0)
    sc = Schedule(shape, 3, n_layers=1)
    sc.draw_adapters()
    gpu = R.GpuRun(sc, max_pages=8)
    n = 70
    k = np.zeros((n, 2, 64), np.uint16)
    B.skv_append_base(gpu.ctx, 0, -1, R.dev(k), R.dev(k))
    x = np.zeros((n, 128), np.float32)
    for i in range(n):
        x[i, (5 * i) % 128] = 1.0
    xb = synth.f32_to_bf16_bits(x)
    a = sc.A[0][0]
    B.skv_append_lowrank(gpu.ctx, 0, -1, 0, n, R.dev(xb), R.dev(a))
    B.skv_sync(gpu.ctx)
    _, _, LRT = (t.cpu().numpy().view(np.uint16) for t in _pool_views(gpu))
    pages = B.skv_get_pages(gpu.ctx, 0, -1)
    for i in range(n):
        row = LRT[0, 0, pages[i // 64], :, i % 64]
        assert np.array_equal(row, a[(5 * i) % 128]), i


@pytest.mark.parametrize("hidden,rank,n", [(64, 4, 9), (192, 32, 17), (320, 16, 40), (192, 8, 31)])
def test_lowrank_rows_at_slab_edges(hidden, rank, n):
    """The MFMA low-rank tiles (16 rows each; the hidden columns go to the four
    waves in slabs) at hidden sizes that end inside a slab or give some waves
    no slab, at every rank, with row counts around the tile edges. Each row is
    within one bf16 ulp of the oracle's exact X A plus the fp32 sum's error
    bound gamma_k sum |x_k a_k| for the longest rounding chain k of the kernel
    (gpu_runner.lowrank_row_bound; near a cancellation this term exceeds an
    ulp of the small result)."""
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = Shape("e", 1, 4, 2, 64, hidden, rank, 1, BASE_SHARED, 0)
    sc = Schedule(shape, 11 + hidden + rank, n_layers=1)
    sc.draw_adapters()
    sc.shared_prefix(n)
    gpu, orc, _ = R.run_parity(sc)
    _, _, LRT = (t.cpu().numpy().view(np.uint16) for t in _pool_views(gpu))
    pages = B.skv_get_pages(gpu.ctx, 0, -1)
    ev = next(e for e in sc.events if isinstance(e, synth.AppendLowrank))
    ref = orc.lr[0][-1][0].get(n)
    got = bf16_bits_to_f64(np.stack([LRT[0, 0, pages[j // 64], :, j % 64] for j in range(n)]))
    bound = R.lowrank_row_bound(ref, bf16_bits_to_f64(ev.x), bf16_bits_to_f64(ev.a))
    assert got.shape == (n, rank)
    assert np.all(np.abs(got - ref) <= bound), np.max(np.abs(got - ref) / bound)


def test_decode_is_deterministic():
    import torch
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = Shape("e", 1, 32, 8, 128, 1024, 8, 4, BASE_LR_SHARED, 0)
    sc = mini(shape, 5000, [3, 3, 3, 3], decode_steps=1)
    gpu, _, _ = R.run_parity(sc)
    ev = sc.events[-1]
    q, b = R.dev(ev.q), R.dev(ev.b)
    outs = []
    for _ in range(3):
        o = torch.empty_like(q)
        B.skv_attn_decode(gpu.ctx, 0, ev.agents, ev.base_len, ev.suffix_len, q, b, o)
        outs.append(o.view(torch.int16).cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_agent_ops_never_touch_shared_pages():
    import torch
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = Shape("e", 1, 8, 2, 128, 256, 8, 2, BASE_SHARED, 0)
    sc = Schedule(shape, 5, n_layers=1)
    sc.draw_adapters()
    sc.shared_prefix(200)
    for a in range(2):
        sc.attach(a)
    gpu = R.GpuRun(sc, max_pages=64)
    for ev in sc.events:
        gpu.apply(ev)
    K, VT, LRT = _pool_views(gpu)
    sp = B.skv_get_pages(gpu.ctx, 0, -1)
    snap = [t[:, sp].clone() if t is not LRT else t[:, :, sp].clone() for t in (K, VT, LRT)]
    sc2_events_start = len(sc.events)
    sc.own_rows(0, [0, 1], [90, 13])
    sc.attend("prefill", 0, [0, 1], [90, 13])
    sc.crop(0, 250)
    sc.own_rows(0, [0], [77], lr="zero", batched=False)
    for ev in sc.events[sc2_events_start:]:
        gpu.apply(ev)
    B.skv_sync(gpu.ctx)
    after = [K[:, sp], VT[:, sp], LRT[:, :, sp]]
    for s0, s1 in zip(snap, after):
        assert torch.equal(s0, s1)
    # physical sharing: both agents' views resolve the shared prefix to the same pages
    assert B.skv_get_pages(gpu.ctx, 0, -1) == sp


@pytest.mark.parametrize("shape_name", ["llama3", "qwen3"])
def test_decode_over_scattered_shared_pages(shape_name):
    # The shared prefix grows after the agents took pages of their own, so its
    # page ids no longer run consecutively and the decode looks each shared
    # page up in the table; the agents attach at different lengths (one view
    # inside the first, consecutive run of pages, one past it), then decode
    # and the fused step run against the oracle.
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = synth.WORKLOADS[shape_name].with_(n_agents=2)
    sc = Schedule(shape, 41, n_layers=1)
    sc.draw_adapters()
    sc.shared_prefix(150)
    sc.attach(0, 150)
    sc.attach(1, 150)
    sc.own_rows(0, [0, 1], [70, 70])
    sc.shared_prefix(330)
    sc.attach(0, 100)   # drops its own rows; view inside the first, consecutive pages
    sc.attach(1, 150)   # drops its own rows ...
    sc.attach(1, 480)   # ... and attaches past them
    sc.own_rows(0, [0, 1], [5, 9])
    sc.attend("prefill", 0, [0, 1], [5, 9], tag="prefill")
    for t in range(3):
        sc.own_rows(0, [0, 1], [1, 1])
        sc.attend("decode", 0, [0, 1], [1, 1], tag=f"decode{t}")
    for t in range(3):
        sc.decode_step(0, [0, 1], tag=f"step{t}")
    gpu, _, res = R.run_parity(sc, max_pages=64, log=log)
    shared = B.skv_get_pages(gpu.ctx, 0, -1)
    assert any(shared[i + 1] != shared[i] + 1 for i in range(len(shared) - 1)), shared
    assert len(res) == 7


def test_maximum_sizes():
    # The plan's largest cases on a small head shape (8 KV heads of 64):
    #  - a prefill over a view of exactly 4,096 pages (262,144 keys, the page
    #    list a prefill workgroup holds in LDS), 64 queries at its end;
    #  - fused decode steps over a 520,000-key shared prefix: 16,250 chunks per
    #    KV head need 32 items per head at up to 508 chunks each (the chunk
    #    table's cap is 512), which with the step's two append blocks is more
    #    workgroups than CUs.
    R = _runner()
    shape = Shape("max", 1, 8, 8, 64, 128, 8, 2, BASE_SHARED, 0)
    view = 4096 * 64
    sc = Schedule(shape, 77, n_layers=1)
    sc.draw_adapters()
    sc.shared_prefix(520_000)
    sc.attach(0, view - 64)
    sc.attach(1, 520_000)
    sc.own_rows(0, [0], [64])
    sc.attend("prefill", 0, [0], [64], tag="prefill at the view limit")
    # per KV head: 16,250 shared chunks + agent 0's 3 own (65-66 rows) + agent 1's 1;
    # (256 CUs - 2 append blocks) / 8 heads = 31 items would need 525 chunks each
    for t in range(2):
        sc.decode_step(0, [0, 1], tag=f"step{t}")
    R.run_parity(sc, max_pages=520_000 // 64 + 16, log=log)


RANDOM_SHAPES = [
    Shape("rnd-d64-BS", 1, 8, 2, 64, 128, 8, 3, BASE_SHARED, 0),
    Shape("rnd-d128-BLS", 1, 8, 4, 128, 256, 16, 2, BASE_LR_SHARED, 0),
    Shape("rnd-d64-G4-BS", 1, 4, 1, 64, 128, 4, 4, BASE_SHARED, 0),
    Shape("rnd-d128-r32-BLS", 1, 16, 2, 128, 256, 32, 2, BASE_LR_SHARED, 0),
]


@pytest.mark.parametrize("seed", range(32))
def test_random_schedules(seed):
    # Seeded random interleavings of every operation on one store: own-row
    # appends, suffix prefills, decodes, fused decode steps, crops (inside the
    # suffix, into the shared prefix, then a re-attach) and activation offsets,
    # over lengths that start and end anywhere in a page; every attention call
    # is checked against the oracle.
    rng = np.random.RandomState(seed)
    R = _runner()
    shape = RANDOM_SHAPES[seed % len(RANDOM_SHAPES)]
    N = shape.n_agents
    sc = Schedule(shape, 3000 + seed, n_layers=1)
    sc.draw_adapters()
    P = int(rng.randint(0, 700))
    if P:
        sc.shared_prefix(P, lr="x" if rng.rand() < 0.7 else "zero")
    for a in range(N):
        sc.attach(a, int(rng.randint(0, P + 1)))
    view = lambda a: sc.b[a] + sc.S[0][a]
    subset = lambda: [a for a in range(N) if rng.rand() < 0.6] or [int(rng.randint(N))]
    for t in range(14):
        op = rng.choice(["own", "prefill", "decode", "step", "crop", "offset"], p=[.2, .2, .15, .25, .1, .1])
        if op == "own":
            ag = subset()
            sc.own_rows(0, ag, [int(rng.randint(1, 81)) for _ in ag])
        elif op == "prefill":
            ag = [a for a in subset() if view(a) > 0]
            if ag:
                sc.attend("prefill", 0, ag, [int(rng.randint(1, min(view(a), 48) + 1)) for a in ag], tag=f"prefill{t}")
        elif op == "decode":
            ag = subset()
            sc.own_rows(0, ag, [1] * len(ag))
            sc.attend("decode", 0, ag, [1] * len(ag), tag=f"decode{t}")
        elif op == "step":
            sc.decode_step(0, subset(), lr="x" if rng.rand() < 0.8 else "zero", tag=f"step{t}")
        elif op == "crop":
            a = int(rng.randint(N))
            sc.crop(a, int(rng.randint(0, view(a) + 1)))
            if sc.S[0][a] == 0 and rng.rand() < 0.5:
                sc.attach(a, int(rng.randint(sc.b[a], P + 1)))
        else:
            a = int(rng.randint(N))
            sc.set_lr_begin(a, int(rng.randint(0, view(a) + 50)))
    R.run_parity(sc, max_pages=256, log=lambda m: log(f"[seed {seed}] {m}"))


def test_length_mismatch_is_rejected_without_launch():
    import torch
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = Shape("e", 1, 8, 2, 64, 128, 8, 2, BASE_SHARED, 0)
    sc = mini(shape, 100, [4, 4], decode_steps=0)
    gpu, _, _ = R.run_parity(sc)
    before = B.skv_get_counters(gpu.ctx)["launches"]
    q = torch.zeros((2, 8, 64), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    bb = R.dev(sc.B[0])
    with pytest.raises(B.SkvError) as e:
        B.skv_attn_decode(gpu.ctx, 0, [0, 1], [100, 100], [4, 5], q, bb, o)
    assert e.value.code == "STATE"
    assert B.skv_get_counters(gpu.ctx)["launches"] == before


def test_prefill_equals_sequential_decodes():
    import torch
    from lora_shared_kv_amd import skv as B
    R = _runner()
    shape = Shape("e", 1, 8, 2, 128, 256, 8, 1, BASE_SHARED, 0)
    sc = mini(shape, 400, [20], decode_steps=0)
    gpu, _, _ = R.run_parity(sc)
    ev = sc.events[-1]
    q = R.dev(ev.q)
    o_pre = torch.empty_like(q)
    bb = R.dev(ev.b)
    B.skv_attn_prefill(gpu.ctx, 0, [0], [400], [20], [20], q, bb, o_pre)
    outs = []
    for i in range(19, -1, -1):
        B.skv_crop(gpu.ctx, 0, 400 + i + 1)
        o1 = torch.empty_like(q[i:i + 1])
        B.skv_attn_decode(gpu.ctx, 0, [0], [400], [i + 1], q[i:i + 1].contiguous(), bb, o1)
        outs.append((i, o1))
    for i, o1 in outs:
        d = (o1.float() - o_pre[i:i + 1].float()).abs().max().item()
        assert d <= 1e-2, (i, d)
