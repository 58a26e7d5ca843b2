"""GPU parity of the fused front end (skv_project_append) against the oracle.

The oracle side projects the same bf16 rows in float64 (oracle/frontend.py),
rotates q and k at the rows' view positions, and appends the bf16-rounded k, v
and the low-rank rows to its cache model. Bars:
  - q, and k, v as stored in the pages: within one bf16 ulp of the float64
    value (plus 1e-4 for fp32 summation), and the attention bar (max abs
    2e-2, relative L2 1e-2);
  - low-rank rows: within one bf16 ulp of X A, plus the fp32 sum's error bound
    gamma_k sum_k |x_k a_k| for the kernel's longest rounding chain k (which near a
    cancellation exceeds an ulp of the small result);
  - page ids and lengths: exactly the oracle's;
  - attention over the projected cache: the attention bar.
"""
import math

import numpy as np
import pytest

import synth
from synth import BASE_LR_SHARED, BASE_SHARED, Attend, Schedule, Shape, bf16_bits_to_f64
from oracle import frontend as fe
from oracle.run import apply_event

pytestmark = pytest.mark.gpu

MAX_ABS, MAX_REL_L2 = 2e-2, 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu(torch_cuda):
    return torch_cuda


def log(msg):
    print(msg, flush=True)


def _within_ulp(got, ref, what):
    err = np.abs(got - ref)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    worst = float(np.max(err / (ulp + 1e-4))) if err.size else 0.0
    assert worst <= 1.0, (what, worst)
    ma = float(np.max(err)) if err.size else 0.0
    rl = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert ma <= MAX_ABS and rl <= MAX_REL_L2, (what, ma, rl)
    return ma, rl


def run_case(shape, prefix, own_before, counts, theta, seed, with_a=True, attend=True):
    import torch
    import gpu_runner as R
    from lora_shared_kv_amd import skv as B
    N, Hq, Hkv, D, H, r = (shape.n_agents, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                           shape.hidden, shape.rank)
    agents = [a for a in range(N) if counts[a] > 0]
    cnt = [counts[a] for a in agents]
    log(f"case {shape.name} prefix={prefix} own={own_before} counts={counts} theta={theta} seed={seed}")
    sc = Schedule(shape, seed, n_layers=1)
    sc.draw_adapters()
    sc.shared_prefix(prefix)
    for a in range(N):
        sc.attach(a, prefix)
    if any(own_before):
        ag = [a for a in range(N) if own_before[a] > 0]
        sc.own_rows(0, ag, [own_before[a] for a in ag])
    max_pages = -(-prefix // 64) + sum(-(-(own_before[a] + counts[a]) // 64) + 1 for a in range(N)) + 8
    gpu, orc, _ = R.run_parity(sc, max_pages=max_pages)

    d = synth.Draws(seed + 101)
    T = sum(cnt)
    F = (Hq + 2 * Hkv) * D
    x = d.normal((T, H))
    w = d.normal((F, H), 1.0 / H)
    A = sc.A[0] if with_a else None
    q_out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device="cuda")
    wp = torch.empty((F, H), dtype=torch.bfloat16, device="cuda")
    B.skv_pack_qkv(gpu.ctx, R.dev(w), wp)
    B.skv_project_append(gpu.ctx, 0, agents, cnt, R.dev(x), wp, R.dev(A), theta, q_out)
    B.skv_sync(gpu.ctx)

    # oracle: view position of own row s of agent i is b_i + s
    pos = np.concatenate([prefix + own_before[a] + np.arange(counts[a]) for a in agents])
    x64, w64 = bf16_bits_to_f64(x), bf16_bits_to_f64(w)
    q, k, v = fe.project(x64, w64, Hq, Hkv, D, pos, theta)
    ma, rl = _within_ulp(R.to_f64(q_out), q, "q")
    log(f"  q: max_abs={ma:.3e} rel_l2={rl:.3e}")
    bf = lambda a: bf16_bits_to_f64(synth.f32_to_bf16_bits(a.astype(np.float32)))
    a64 = None if A is None else bf16_bits_to_f64(A)
    orc.append_agents(0, agents, cnt, bf(k), bf(v), x64 if with_a else None, a64)

    K, VT, LRT = (t.cpu().numpy().view(np.uint16) for t in R.pool_views(gpu))
    ki, vi = R.k_tile_index(D), R.v_tile_index(D)
    row = 0
    for a, c in zip(agents, cnt):
        pages = B.skv_get_pages(gpu.ctx, 0, a)
        assert pages == orc.pages(0, a), a
        lens = B.skv_get_lens(gpu.ctx, 0)
        assert lens == orc.lens(0), (lens, orc.lens(0))
        s0 = own_before[a]
        kk = np.stack([K[0, pages[j // 64]][:, ki[j % 64]] for j in range(s0, s0 + c)])
        vv = np.stack([VT[0, pages[j // 64]][:, vi[j % 64]] for j in range(s0, s0 + c)])
        _within_ulp(bf16_bits_to_f64(kk), k[row:row + c], f"k agent {a}")
        _within_ulp(bf16_bits_to_f64(vv), v[row:row + c], f"v agent {a}")
        plane = a if shape.mode == BASE_SHARED else 0
        lr = np.stack([LRT[plane, 0, pages[j // 64], :, j % 64] for j in range(s0, s0 + c)])
        got = bf16_bits_to_f64(lr)
        if with_a:
            ai = a64[a] if shape.mode == BASE_SHARED else a64
            ref = x64[row:row + c] @ ai
            # one bf16 ulp of the exact product, plus the fp32 summation's error
            # bound for the kernel's longest rounding chain, which near a
            # cancellation (|X A| much below sum |x_k a_k|) can exceed an ulp
            # of the small result
            bound = R.lowrank_row_bound(ref, x64[row:row + c], ai)
            assert np.all(np.abs(got - ref) <= bound), ("lr", a, float(np.max(np.abs(got - ref) / bound)))
        else:
            assert np.all(got == 0), ("zero lr rows", a)
        row += c

    if attend:
        q_att = synth.Draws(seed + 202).normal((T, Hq, D))
        ev = Attend("prefill", 0, agents, [prefix] * len(agents),
                    [own_before[a] + counts[a] for a in agents], cnt, q_att, sc.B[0], "after-project")
        o = gpu.apply(ev)
        ref = apply_event(orc, ev, None)
        ma, rl = R.errors(R.to_f64(o), ref)
        log(f"  attention after projection: max_abs={ma:.3e} rel_l2={rl:.3e}")
        assert ma <= MAX_ABS and rl <= MAX_REL_L2, (ma, rl)
    B.skv_sync(gpu.ctx)
    return gpu


LLAMA3_HEADS = Shape("llama3-8b-heads", 1, 32, 8, 128, 4096, 8, 4, BASE_LR_SHARED, 0)
QWEN25_HEADS = Shape("qwen2.5-1.5b-heads", 1, 12, 2, 128, 1536, 16, 2, BASE_SHARED, 0)
QWEN3_HEADS = Shape("qwen3-1.7b-heads", 1, 16, 8, 128, 2048, 16, 2, BASE_SHARED, 0)
TINY_HEADS = Shape("tiny-d64", 1, 14, 2, 64, 896, 8, 2, BASE_SHARED, 0)
SMALL = Shape("small-d128", 1, 8, 2, 128, 512, 16, 2, BASE_SHARED, 0)
MANY = Shape("many-agent-heads", 1, 16, 8, 128, 2048, 16, 8, BASE_SHARED, 0)
# head dim 64 with five 64-feature units: the last column of two-unit tiles holds one unit
ODD_UNITS = Shape("odd-units-d64", 1, 3, 1, 64, 256, 8, 2, BASE_SHARED, 0)
# head dim 64 with 96 units, so that a thousand rows take 256-token tiles
WIDE_D64 = Shape("wide-d64", 1, 64, 16, 64, 256, 8, 2, BASE_SHARED, 0)
# the llama3 heads with hidden 960: an odd number (15) of 64-column stages
ODD_STAGES = Shape("odd-stages", 1, 32, 8, 128, 960, 8, 4, BASE_LR_SHARED, 0)
# the largest packed weights the front end takes: (64 + 2 x 64) x 128 features x
# 43,648 columns x 2 bytes = 2,145,386,496 bytes, 2^18 below 2 GiB (32-bit byte
# offsets into the weights run up to there)
MAX_WEIGHTS = Shape("max-weights", 1, 64, 64, 128, 43648, 8, 2, BASE_SHARED, 0)


@pytest.mark.parametrize("name,shape,prefix,own,counts,theta", [
    # several 64-row tiles, agent boundaries inside tiles, partly filled pages
    ("llama3-ragged", LLAMA3_HEADS, 333, [0, 5, 0, 70], [70, 1, 130, 3], 500000.0),
    # 40 rows over three agents: one 64-row tile, agent boundaries inside it
    ("llama3-40-rows", LLAMA3_HEADS, 100, [3, 0, 64, 0], [17, 0, 20, 3], 500000.0),
    # the split form (16 rows or fewer), three agents in one tile
    ("llama3-split", LLAMA3_HEADS, 64, [0, 1, 0, 2], [5, 6, 0, 5], 500000.0),
    # one row per agent (16-row tiles), the decode step's shape
    ("qwen2.5-decode-rows", QWEN25_HEADS, 1000, [3, 0], [1, 1], 1000000.0),
    ("qwen3-takeover", QWEN3_HEADS, 160, [0, 0], [200, 64], 1000000.0),
    # head dim 64: one unit per head, a last workgroup with idle waves
    ("tiny-d64", TINY_HEADS, 1024, [0, 0], [100, 37], 10000.0),
    # head dim 64 in the split form
    ("tiny-d64-split", TINY_HEADS, 1024, [2, 0], [3, 4], 10000.0),
])
def test_project_append_matches_oracle(name, shape, prefix, own, counts, theta):
    run_case(shape, prefix, own, counts, theta, seed=11)


def test_project_append_without_rotation_or_adapter():
    run_case(SMALL, 64, [0, 10], [65, 63], 0.0, seed=12, with_a=False)


def test_project_append_long_call_at_large_positions():
    # 4200 rows: more pages than one launch carries, so several launches; view
    # positions near 64K check the fp64 angle reduction
    run_case(SMALL, 60000, [0, 0], [4200, 0], 500000.0, seed=13, attend=False)


def test_project_append_rejects_bad_rotary_base():
    import torch
    import gpu_runner as R
    from lora_shared_kv_amd import skv as B
    sc = Schedule(SMALL, 3, n_layers=1)
    sc.draw_adapters()
    gpu = R.GpuRun(sc, max_pages=8)
    x = torch.zeros((2, SMALL.hidden), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(((8 + 4) * 128, SMALL.hidden), dtype=torch.bfloat16, device="cuda")
    q = torch.empty((2, 8, 128), dtype=torch.bfloat16, device="cuda")
    for bad in (0.5, -3.0, math.inf, math.nan):
        with pytest.raises(B.SkvError):
            B.skv_project_append(gpu.ctx, 0, [0], [2], x, w, None, bad, q)
    assert B.skv_get_lens(gpu.ctx, 0)["S"][0] == 0


def test_packed_weights_follow_the_documented_layout():
    # the packing is a pure permutation: check it element by element against
    # the layout stated with skv_pack_qkv
    import torch
    import gpu_runner as R
    from lora_shared_kv_amd import skv as B
    for shape in (SMALL, TINY_HEADS):
        Hq, Hkv, D, H = shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.hidden
        sc = Schedule(shape, 5, n_layers=1)
        gpu = R.GpuRun(sc, max_pages=4)
        F = (Hq + 2 * Hkv) * D
        w = np.arange(F * H, dtype=np.int64).reshape(F, H) % 65521   # distinct-ish finite bf16 patterns
        wb = (w % 0x7F00).astype(np.uint16)
        wp = torch.empty((F, H), dtype=torch.bfloat16, device="cuda")
        B.skv_pack_qkv(gpu.ctx, R.dev(wb), wp)
        B.skv_sync(gpu.ctx)
        got = wp.cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)
        nk, uph = H // 64, D // 64
        u, s, m, l, e = np.meshgrid(np.arange(F // 64), np.arange(nk), np.arange(8), np.arange(64), np.arange(8),
                                    indexing="ij")
        row = (u // uph) * D + 32 * (u % uph) + 16 * ((m // 2) % 2) + (D // 2) * (m // 4) + l % 16
        col = 64 * s + 32 * (m % 2) + 8 * (l // 16) + e
        assert np.array_equal(got, wb[row, col].reshape(-1)), shape.name


def test_project_append_many_agents_decode_rows():
    # one row for each of eight agents (per-agent A), all in one 16-row tile
    run_case(MANY, 2000, [1, 0, 3, 0, 5, 0, 7, 0], [1] * 8, 1000000.0, seed=14)


def test_project_append_many_agents_suffix_rows():
    # 4 x 512 rows: 64-row tiles over the whole chip, agent boundaries on tile edges
    run_case(MANY, 4096, [0] * 8, [512, 0, 512, 0, 512, 0, 512, 0], 1000000.0, seed=15, attend=False)



def test_project_append_wide_tiles():
    # 555 rows over three agents (the wide form: 128-token tiles of two units):
    # agent boundaries inside tiles, a partly filled last tile, and a 5-row
    # agent whose low-rank rows take the dot-product blocks
    run_case(LLAMA3_HEADS, 200, [0, 7, 0, 64], [300, 5, 0, 250], 500000.0, seed=16)


def test_project_append_wide_tiles_odd_units():
    # 301 rows, head dim 64, five units: the last tile column has idle waves
    run_case(ODD_UNITS, 96, [0, 3], [260, 41], 10000.0, seed=17)


def test_project_append_wide_tiles_three_half_units():
    # 384 rows of the llama3 shapes: tiles of three half units (64 of them per
    # 128 tokens, so that every CU takes one), an agent boundary inside a tile
    run_case(LLAMA3_HEADS, 64, [0, 0, 9, 0], [200, 0, 184, 0], 500000.0, seed=18)


def test_project_append_tall_tiles():
    # 1,024 rows of the llama3 shapes: 256-token tiles of two units, with an
    # agent boundary inside a tile and a partly filled last tile
    run_case(LLAMA3_HEADS, 64, [0, 0, 0, 0], [600, 0, 424, 0], 500000.0, seed=19, attend=False)


def test_project_append_tall_tiles_d64():
    # head dim 64: 1,000 rows over two agents in 256-token tiles
    run_case(WIDE_D64, 128, [0, 5], [700, 300], 10000.0, seed=20, attend=False)


@pytest.mark.parametrize("counts", [[7, 0, 5, 0], [200, 0, 100, 0], [700, 0, 0, 324]],
                         ids=["split", "wide-3-half-units", "tall"])
def test_project_append_odd_stage_count(counts):
    # 15 stages of 64 hidden columns: the split form's quarters differ in
    # length, and the wide and tall forms end on an odd stage
    run_case(ODD_STAGES, 64, [0, 0, 0, 0], counts, 500000.0, seed=21, attend=False)


@pytest.mark.parametrize("counts", [[3, 3], [300, 0]], ids=["split", "wide"])
def test_project_append_largest_weights(counts):
    assert (64 + 2 * 64) * 128 * 43648 * 2 == 2_145_386_496 < 1 << 31
    run_case(MAX_WEIGHTS, 64, [0, 0], counts, 10000.0, seed=22, attend=False)
