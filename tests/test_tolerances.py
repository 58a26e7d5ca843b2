"""The derived tolerance of the low-rank rows, checked against an emulation.

gpu_runner.lowrank_row_bound bounds |bf16(fp32 sum) - X A| by one bf16 ulp of
X A plus gamma_k sum |x_k a_k| for the kernel's longest rounding chain k. Here
the worst case is emulated in numpy float32: each of four waves adds its slab
of products one at a time (every product its own rounding), the four partial
sums meet in sequence, and the result is rounded to bf16 with ties to even;
rows built to cancel (|X A| far below sum |x_k a_k|) are included. Every
element must lie inside the bound, and the bound must not be vacuous (it stays
within a few ulps for rows that do not cancel).
"""
import numpy as np
import pytest

import synth
from gpu_runner import lowrank_chain, lowrank_row_bound


def emulate(x, a, hs):
    """bf16(sum) with the kernel's worst-case fp32 rounding order (slabs of
    64*hs columns dealt to four waves in turn)."""
    H = x.shape[-1]
    nslab = -(-H // (64 * hs))
    part = np.zeros((4,) + (x.shape[0], a.shape[1]), np.float32)
    for w in range(4):
        cols = [c for s in range(w, nslab, 4) for c in range(64 * hs * s, min(64 * hs * (s + 1), H))]
        acc = np.zeros((x.shape[0], a.shape[1]), np.float32)
        for c in cols:
            acc = (acc + (x[:, c:c + 1].astype(np.float32) * a[c:c + 1, :].astype(np.float32))).astype(np.float32)
        part[w] = acc
    s = part[0]
    for w in range(1, 4):
        s = (s + part[w]).astype(np.float32)
    return synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(s))


@pytest.mark.parametrize("hidden,rank", [(64, 4), (192, 32), (896, 8), (1536, 16), (4096, 8)])
def test_emulated_rows_stay_inside_the_bound(hidden, rank):
    d = synth.Draws(31 + hidden + rank)
    x = synth.bf16_bits_to_f64(d.normal((24, hidden)))
    a = synth.bf16_bits_to_f64(d.normal((hidden, rank), 1.0 / hidden))
    # rows 16..23 nearly cancel: the second half of x repeats the first half negated
    h2 = hidden // 2
    x[16:, h2:2 * h2] = -x[16:, :h2]
    a[h2:2 * h2] = synth.bf16_bits_to_f64(synth.f32_to_bf16_bits(a[:h2] * (1 + 2.0 ** -6)))
    ref = x @ a
    bound = lowrank_row_bound(ref, x, a)
    for hs in (4, 2):
        got = emulate(x, a, hs)
        assert np.all(np.abs(got - ref) <= bound), (hs, float(np.max(np.abs(got - ref) / bound)))
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref[:16]), 1e-30))) - 7)
    assert np.median(bound[:16] / ulp) < 4.0


def test_chain_lengths():
    # one wave's share of whole slabs, plus the combining additions
    assert lowrank_chain(4096) == 1024 + 9
    assert lowrank_chain(896) == 256 + 9
    assert lowrank_chain(192) == 192 + 9
