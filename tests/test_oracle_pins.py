"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each pin compares the oracle with something other than itself: a library
routine (torch's scaled_dot_product_attention), brute force in pure Python
on views of at most 8 positions, closed forms, the decomposition identity
of the LRAgent review ("What carries the argument": O = P V_base + (P V_lr) B),
and invariants. The planted-mistake tests at the end patch a plausible bug
into the oracle and require that at least one pin fails.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from oracle.cache import CacheModel, OracleError, SHARED, BASE_SHARED, BASE_LR_SHARED
from synth import Draws, bf16_bits_to_f64

RTOL = 1e-12


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _small_cache(mode=BASE_SHARED, hq=6, hkv=2, d=64, r=4, n_agents=2, hidden=64,
                 prefix=5, own=(3, 2), seed=0, zero_vbase=False, ps=4):
    """A cache with a shared prefix, per-plane LR rows, and own suffixes."""
    rng = np.random.default_rng(seed)
    c = CacheModel(1, hq, hkv, d, hidden, r, n_agents, mode, ps, 256)
    planes = n_agents if mode == BASE_SHARED else 1
    A = rng.standard_normal((planes, hidden, r)) / math.sqrt(hidden)
    B = rng.standard_normal((n_agents, r, hkv * d)) * 0.3
    k = rng.standard_normal((prefix, hkv, d))
    v = np.zeros((prefix, hkv, d)) if zero_vbase else rng.standard_normal((prefix, hkv, d))
    x = rng.standard_normal((prefix, hidden))
    c.append_base(0, SHARED, k, v)
    for p in range(planes):
        c.append_lowrank(0, SHARED, p, prefix, x, A[p])
    for a in range(n_agents):
        c.crop(a, prefix)
        n = own[a]
        ka = rng.standard_normal((n, hkv, d))
        va = np.zeros((n, hkv, d)) if zero_vbase else rng.standard_normal((n, hkv, d))
        xa = rng.standard_normal((n, hidden))
        c.append_base(0, a, ka, va)
        c.append_lowrank(0, a, c.plane_of(a), n, xa, A[c.plane_of(a)])
    return c, A, B


# ---------------------------------------------------------------------------
# pins (plain functions so the planted-mistake tests can run them)
# ---------------------------------------------------------------------------

def pin_decomposition_identity():
    """P V_i == P V_base + (P LR) B_i (exact algebra; LRAgent review, Eq. 12)."""
    c, A, B = _small_cache(seed=1)
    rng = np.random.default_rng(2)
    for a in range(c.N):
        k, vb, lr = c.view(0, a)
        L = k.shape[0]
        q = rng.standard_normal((3, c.Hq, c.d))
        o_full = oracle.attention_outputs(c, 0, [a], [3], q, B)
        pos = [L - 3, L - 2, L - 1]
        o_base = oatt.attend_view(q, k, vb, pos)
        lr_heads = np.repeat(lr[:, None, :], c.Hkv, axis=1)
        o_lr = oatt.attend_view(q, k, lr_heads, pos)            # P . V_lr  [n][Hq][r]
        for h in range(c.Hq):
            g = h // c.G
            re = o_base[:, h] + o_lr[:, h] @ B[a][:, g * c.d:(g + 1) * c.d]
            assert np.allclose(o_full[:, h], re, rtol=1e-12, atol=1e-12)


def pin_b_zero_is_sdpa():
    """With B_i = 0 the output is plain GQA causal attention (torch SDPA, fp64)."""
    for mode in (BASE_SHARED, BASE_LR_SHARED):
        c, A, B = _small_cache(mode=mode, hq=8, hkv=2, seed=3)
        B0 = np.zeros_like(B)
        rng = np.random.default_rng(4)
        for a in range(c.N):
            k, vb, _ = c.view(0, a)
            L = k.shape[0]
            n = 3
            q = rng.standard_normal((n, c.Hq, c.d)) * 2.0
            o = oracle.attention_outputs(c, 0, [a], [n], q, B0)
            tq = torch.tensor(q).permute(1, 0, 2)[None]             # [1][Hq][n][d]
            tk = torch.tensor(k).permute(1, 0, 2)[None]
            tv = torch.tensor(vb).permute(1, 0, 2)[None]
            mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=mask, enable_gqa=True)[0].permute(1, 0, 2).numpy()
            assert np.allclose(o, ref, rtol=1e-11, atol=1e-12), np.abs(o - ref).max()


def pin_brute_force():
    """Pure-Python loops from the raw inputs on views of at most 8 positions."""
    rng = np.random.default_rng(5)
    hq, hkv, d, r, hidden, N = 4, 2, 64, 4, 64, 2
    G = hq // hkv
    for mode in (BASE_SHARED, BASE_LR_SHARED):
        c = CacheModel(1, hq, hkv, d, hidden, r, N, mode, 4, 64)
        planes = N if mode == BASE_SHARED else 1
        A = rng.standard_normal((planes, hidden, r)) / 8
        B = rng.standard_normal((N, r, hkv * d)) * 0.5
        P = 5
        K = rng.standard_normal((P, hkv, d)); V = rng.standard_normal((P, hkv, d))
        X = rng.standard_normal((P, hidden))
        c.append_base(0, SHARED, K, V)
        for p in range(planes):
            c.append_lowrank(0, SHARED, p, P, X, A[p])
        # agent 0 sees all 5 shared rows plus 3 own rows; agent 1 takes over at b=3
        c.crop(0, 5)
        c.crop(1, 3)
        own = {}
        for a, n in ((0, 3), (1, 4)):
            ka = rng.standard_normal((n, hkv, d)); va = rng.standard_normal((n, hkv, d))
            xa = rng.standard_normal((n, hidden))
            pa = a if mode == BASE_SHARED else 0
            c.append_base(0, a, ka, va)
            c.append_lowrank(0, a, pa, n, xa, A[pa])
            own[a] = (ka, va, xa, pa)
        for a, b, nq in ((0, 5, 2), (1, 3, 4)):
            ka, va, xa, pa = own[a]
            rows_k = [K[j] for j in range(b)] + [ka[j] for j in range(len(ka))]
            rows_v = [V[j] for j in range(b)] + [va[j] for j in range(len(va))]
            rows_x = [X[j] for j in range(b)] + [xa[j] for j in range(len(xa))]
            L = len(rows_k)
            assert L <= 8
            q = rng.standard_normal((nq, hq, d))
            got = oracle.attention_outputs(c, 0, [a], [nq], q, B)
            lr_rows = [[sum(rows_x[j][u] * A[pa][u, kk] for u in range(hidden)) for kk in range(r)]
                       for j in range(L)]
            for i in range(nq):
                t = L - nq + i
                for h in range(hq):
                    g = h // G
                    s = []
                    for j in range(t + 1):
                        acc = 0.0
                        for e in range(d):
                            acc += q[i, h, e] * rows_k[j][g, e]
                        s.append(acc / math.sqrt(d))
                    mx = max(s)
                    w = [math.exp(x - mx) for x in s]
                    tot = sum(w)
                    for e in range(d):
                        val = 0.0
                        for j in range(t + 1):
                            vij = rows_v[j][g, e] + sum(lr_rows[j][kk] * B[a][kk, g * d + e]
                                                        for kk in range(r))
                            val += w[j] / tot * vij
                        assert abs(val - got[i, h, e]) <= 1e-11 * max(1.0, abs(val)), (mode, a, i, h, e)


def pin_closed_forms():
    """L=1 gives V_i[0]; equal keys or q=0 give the mean of V_i; one-hot X gives a row of A."""
    rng = np.random.default_rng(6)
    hq, hkv, d, r, hidden = 4, 2, 64, 8, 64
    c = CacheModel(1, hq, hkv, d, hidden, r, 1, BASE_SHARED, 4, 64)
    A = rng.standard_normal((hidden, r))
    B = rng.standard_normal((1, r, hkv * d))
    x1 = np.zeros((1, hidden)); x1[0, 7] = 1.0
    k1 = rng.standard_normal((1, hkv, d)); v1 = rng.standard_normal((1, hkv, d))
    c.append_base(0, SHARED, k1, v1)
    c.append_lowrank(0, SHARED, 0, 1, x1, A)
    c.crop(0, 1)
    # one-hot X -> the LR row equals row 7 of A exactly
    _, _, lr = c.view(0, 0)
    assert np.array_equal(lr[0], A[7])
    # L = 1: o = V_base[0] + A[7] . B slice, independent of q
    q = rng.standard_normal((1, hq, d)) * 5
    o = oracle.attention_outputs(c, 0, [0], [1], q, B)
    for h in range(hq):
        g = h // 2
        expect = [v1[0, g, e] + sum(A[7, kk] * B[0, kk, g * d + e] for kk in range(r)) for e in range(d)]
        assert np.allclose(o[0, h], expect, rtol=1e-13, atol=1e-13)
    # equal keys: uniform weights -> mean of the materialised V rows
    c2 = CacheModel(1, hq, hkv, d, hidden, r, 1, BASE_SHARED, 4, 64)
    L = 6
    krow = rng.standard_normal((1, hkv, d))
    K = np.repeat(krow, L, axis=0)
    V = rng.standard_normal((L, hkv, d))
    X = rng.standard_normal((L, hidden))
    c2.append_base(0, SHARED, K, V)
    c2.append_lowrank(0, SHARED, 0, L, X, A)
    c2.crop(0, L)
    q = rng.standard_normal((1, hq, d))
    o = oracle.attention_outputs(c2, 0, [0], [1], q, B)
    for h in range(hq):
        g = h // 2
        for e in range(0, d, 7):
            m = sum(V[j, g, e] + sum(sum(X[j, u] * A[u, kk] for u in range(hidden)) * B[0, kk, g * d + e]
                                     for kk in range(r)) for j in range(L)) / L
            assert abs(o[0, h, e] - m) < 1e-11
    # q = 0 with distinct keys is also uniform
    c3 = CacheModel(1, hq, hkv, d, hidden, r, 1, BASE_SHARED, 4, 64)
    K3 = rng.standard_normal((L, hkv, d))
    c3.append_base(0, SHARED, K3, V)
    c3.append_lowrank(0, SHARED, 0, L, X, A)
    c3.crop(0, L)
    o3 = oracle.attention_outputs(c3, 0, [0], [1], np.zeros((1, hq, d)), B)
    assert np.allclose(o3, o, rtol=1e-12, atol=1e-12)


def pin_lr_only():
    """V_base = 0 and B_i = [I_r | 0] in every head slice: o[:r] = mean-weighted X A, o[r:] = 0."""
    rng = np.random.default_rng(7)
    hq, hkv, d, r, hidden = 4, 2, 64, 8, 64
    c = CacheModel(1, hq, hkv, d, hidden, r, 1, BASE_SHARED, 4, 64)
    A = rng.standard_normal((hidden, r))
    B = np.zeros((1, r, hkv * d))
    for g in range(hkv):
        B[0, :, g * d:g * d + r] = np.eye(r)
    L = 5
    X = rng.standard_normal((L, hidden))
    c.append_base(0, SHARED, rng.standard_normal((L, hkv, d)), np.zeros((L, hkv, d)))
    c.append_lowrank(0, SHARED, 0, L, X, A)
    c.crop(0, L)
    o = oracle.attention_outputs(c, 0, [0], [1], np.zeros((1, hq, d)), B)   # q = 0: uniform
    mean_lr = [sum(sum(X[j, u] * A[u, kk] for u in range(hidden)) for j in range(L)) / L for kk in range(r)]
    for h in range(hq):
        assert np.allclose(o[0, h, :r], mean_lr, rtol=1e-12, atol=1e-12)
        assert np.all(o[0, h, r:] == 0.0)


def pin_identical_adapters_and_permutation():
    """Agents with the same adapter and the same suffix rows agree; order permutes outputs."""
    rng = np.random.default_rng(8)
    hq, hkv, d, r, hidden, N = 4, 2, 64, 4, 64, 3
    c = CacheModel(1, hq, hkv, d, hidden, r, N, BASE_SHARED, 4, 64)
    A1 = rng.standard_normal((hidden, r)) / 8
    B1 = rng.standard_normal((r, hkv * d))
    B = np.stack([B1, B1, rng.standard_normal((r, hkv * d))])
    P = 6
    X = rng.standard_normal((P, hidden))
    c.append_base(0, SHARED, rng.standard_normal((P, hkv, d)), rng.standard_normal((P, hkv, d)))
    for p in range(N):
        c.append_lowrank(0, SHARED, p, P, X, A1 if p < 2 else A1 * 2)
    ko = rng.standard_normal((3, hkv, d)); vo = rng.standard_normal((3, hkv, d)); xo = rng.standard_normal((3, hidden))
    for a in range(N):
        c.crop(a, P)
        c.append_base(0, a, ko, vo)
        c.append_lowrank(0, a, a, 3, xo, A1 if a < 2 else A1 * 2)
    q1 = rng.standard_normal((2, hq, d))
    q = np.concatenate([q1, q1, q1])
    o = oracle.attention_outputs(c, 0, [0, 1, 2], [2, 2, 2], q, B)
    assert np.array_equal(o[0:2], o[2:4])
    assert not np.allclose(o[0:2], o[4:6])
    o_perm = oracle.attention_outputs(c, 0, [2, 0, 1], [2, 2, 2], q, B)
    assert np.array_equal(o_perm[0:2], o[4:6]) and np.array_equal(o_perm[2:4], o[0:2])


def pin_softmax_rows():
    s = _rand((7, 33), 9) * 30
    p = oatt.softmax_rows(s)
    assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert np.all(p >= 0)
    assert np.allclose(oatt.softmax_rows(s + 1000.0), p, rtol=1e-12, atol=1e-15)
    # weights follow exp differences: p_j / p_k = exp(s_j - s_k)
    assert abs(p[0, 1] / p[0, 2] - math.exp(s[0, 1] - s[0, 2])) < 1e-9 * math.exp(s[0, 1] - s[0, 2])


def pin_prefill_equals_decodes():
    """n prefill queries equal n decode calls on views cut after each query."""
    c, A, B = _small_cache(seed=11, own=(4, 3))
    rng = np.random.default_rng(12)
    q = rng.standard_normal((4, c.Hq, c.d))
    o_pre = oracle.attention_outputs(c, 0, [0], [4], q, B)
    b0 = c.base_len[0]
    for i in range(3, -1, -1):
        c.crop(0, b0 + i + 1)
        o1 = oracle.attention_outputs(c, 0, [0], [1], q[i:i + 1], B)
        assert np.allclose(o1[0], o_pre[i], rtol=1e-12, atol=1e-12)


PINS = [pin_decomposition_identity, pin_b_zero_is_sdpa, pin_brute_force, pin_closed_forms,
        pin_lr_only, pin_identical_adapters_and_permutation, pin_softmax_rows,
        pin_prefill_equals_decodes]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin
# ---------------------------------------------------------------------------

def _mut_gqa_modulo(h, group):
    return h % 2


def _mut_drop_lr(v_base, lr_rows, b_agent):
    return v_base.copy()


def _mut_wrong_head_slice(v_base, lr_rows, b_agent):
    L, hkv, d = v_base.shape
    out = np.empty_like(v_base)
    for g in range(hkv):
        gg = hkv - 1 - g
        out[:, g, :] = v_base[:, g, :] + lr_rows @ b_agent[:, gg * d:(gg + 1) * d]
    return out


def _mut_lr_sign(v_base, lr_rows, b_agent):
    L, hkv, d = v_base.shape
    out = np.empty_like(v_base)
    for g in range(hkv):
        out[:, g, :] = v_base[:, g, :] - lr_rows @ b_agent[:, g * d:(g + 1) * d]
    return out


def _make_attend_mut(kind):
    # the oracle's matrix form with one plausible mistake: the causal mask one
    # key short (a query does not see its own position), or a 1/d scale
    def attend(q, k, v, positions):
        n, hq, d = q.shape
        hkv = k.shape[1]
        group = hq // hkv
        scale = 1.0 / d if kind == "scale" else 1.0 / np.sqrt(d)
        pos = np.asarray(positions, dtype=np.int64)
        Lv = int(pos.max()) + 1
        after = np.arange(Lv)[None, :] > pos[:, None]
        if kind == "causal":
            after = np.arange(Lv)[None, :] >= np.maximum(pos[:, None], 1)
        o = np.empty((n, hq, v.shape[2]))
        for h in range(hq):
            g = oatt.kv_head_of(h, group)
            s = (q[:, h, :] @ k[:Lv, g, :].T) * scale
            s[after] = -np.inf
            o[:, h, :] = oatt.softmax_rows(s) @ v[:Lv, g, :]
        return o
    return attend


def _mut_softmax_no_norm(s):
    m = np.max(s, axis=-1, keepdims=True)
    return np.exp(s - m)


def _mut_view_wrong_plane(self, layer, agent):
    b = self.base_len[agent]
    s = self.length[layer][agent]
    p = self.plane_of(agent)
    q = 0 if self.mode == BASE_SHARED else p
    k = np.concatenate([self.k[layer][SHARED].get(b), self.k[layer][agent].get(s)])
    v = np.concatenate([self.v[layer][SHARED].get(b), self.v[layer][agent].get(s)])
    lr = np.concatenate([self.lr[layer][SHARED][q].get(b), self.lr[layer][agent][p].get(s)])
    return k, v, lr


MUTATIONS = {
    "gqa_modulo": (oatt, "kv_head_of", _mut_gqa_modulo),
    "drop_lr_term": (oatt, "materialize_values", _mut_drop_lr),
    "wrong_head_slice_of_B": (oatt, "materialize_values", _mut_wrong_head_slice),
    "lr_sign": (oatt, "materialize_values", _mut_lr_sign),
    "causal_off_by_one": (oatt, "attend_view", _make_attend_mut("causal")),
    "scale_1_over_d": (oatt, "attend_view", _make_attend_mut("scale")),
    "softmax_unnormalised": (oatt, "softmax_rows", _mut_softmax_no_norm),
    "view_reads_plane0": (CacheModel, "view", _mut_view_wrong_plane),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    obj, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(obj, attr, fn)
    caught = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name} passed every pin"


# ---------------------------------------------------------------------------
# state-model error semantics
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("mode", [BASE_SHARED, BASE_LR_SHARED])
def test_private_copies_equal_shared_prefix(mode):
    """The comparison layout in which every agent holds its own copy of the
    context in its own pages attends over the same rows as the shared prefix
    followed by the agent's suffix, so the outputs agree (the LRAgent review
    compares both layouts; only where the rows live differs)."""
    rng = np.random.default_rng(41)
    hq, hkv, d, r, N, hidden, P, own = 6, 2, 64, 4, 2, 64, 9, 3
    planes = N if mode == BASE_SHARED else 1
    A = rng.standard_normal((planes, hidden, r)) / math.sqrt(hidden)
    B = rng.standard_normal((N, r, hkv * d)) * 0.3
    k, v = rng.standard_normal((P, hkv, d)), rng.standard_normal((P, hkv, d))
    x = rng.standard_normal((P, hidden))
    ko, vo = rng.standard_normal((N, own, hkv, d)), rng.standard_normal((N, own, hkv, d))
    xo = rng.standard_normal((N, own, hidden))
    sh = CacheModel(1, hq, hkv, d, hidden, r, N, mode, 4, 256)
    pv = CacheModel(1, hq, hkv, d, hidden, r, N, mode, 4, 256)
    sh.append_base(0, SHARED, k, v)
    for p in range(planes):
        sh.append_lowrank(0, SHARED, p, P, x, A[p])
    for a in range(N):
        pl = sh.plane_of(a)
        sh.crop(a, P)
        sh.append_base(0, a, ko[a], vo[a])
        sh.append_lowrank(0, a, pl, own, xo[a], A[pl])
        pv.append_base(0, a, np.concatenate([k, ko[a]]), np.concatenate([v, vo[a]]))
        pv.append_lowrank(0, a, pl, P + own, np.concatenate([x, xo[a]]), A[pl])
    assert pv.base_len == [0] * N and sh.base_len == [P] * N
    q = rng.standard_normal((N * own, hq, d))
    o_sh = oracle.attention_outputs(sh, 0, list(range(N)), [own] * N, q, B)
    o_pv = oracle.attention_outputs(pv, 0, list(range(N)), [own] * N, q, B)
    assert np.allclose(o_sh, o_pv, rtol=RTOL, atol=RTOL)


def _offset_caches(mode, t, seed=43):
    """Two caches over the same base rows: in the first every position has its
    low-rank row X A; in the second the positions below t have zero rows
    (adapter off), the rest the same rows. Returns (with_rows, zero_rows, B, q)."""
    rng = np.random.default_rng(seed)
    hq, hkv, d, r, N, hidden, P, own = 4, 2, 64, 4, 2, 64, 7, 5
    planes = N if mode == BASE_SHARED else 1
    A = rng.standard_normal((planes, hidden, r)) / math.sqrt(hidden)
    B = rng.standard_normal((N, r, hkv * d)) * 0.5
    k, v = rng.standard_normal((P, hkv, d)), rng.standard_normal((P, hkv, d))
    x = rng.standard_normal((P, hidden))
    ko, vo = rng.standard_normal((N, own, hkv, d)), rng.standard_normal((N, own, hkv, d))
    xo = rng.standard_normal((N, own, hidden))
    caches = []
    for zero_before in (False, True):
        c = CacheModel(1, hq, hkv, d, hidden, r, N, mode, 4, 256)
        c.append_base(0, SHARED, k, v)
        for p_ in range(planes):
            if zero_before and t > 0:
                c.append_lowrank(0, SHARED, p_, min(t, P), None, None)
                if t < P:
                    c.append_lowrank(0, SHARED, p_, P - t, x[t:], A[p_])
            else:
                c.append_lowrank(0, SHARED, p_, P, x, A[p_])
        for a in range(N):
            pl = c.plane_of(a)
            c.crop(a, P)
            c.append_base(0, a, ko[a], vo[a])
            cut = min(max(t - P, 0), own) if zero_before else 0
            if cut:
                c.append_lowrank(0, a, pl, cut, None, None)
            if own - cut:
                c.append_lowrank(0, a, pl, own - cut, xo[a][cut:], A[pl])
        caches.append(c)
    q = rng.standard_normal((N * 3, hq, d))
    return caches[0], caches[1], B, q


@pytest.mark.parametrize("mode", [BASE_SHARED, BASE_LR_SHARED])
@pytest.mark.parametrize("t", [0, 3, 7, 9, 12, 40])
def test_activation_offset_equals_zero_rows(mode, t):
    """An adapter activation offset t (RoleKV, "What it does": the adapter is
    on only after the role's header) gives the outputs of a cache whose rows
    below t were appended with the adapter off (zero low-rank rows)."""
    with_rows, zero_rows, B, q = _offset_caches(mode, t)
    for a in range(with_rows.N):
        with_rows.set_lr_begin(a, t)
    ag = list(range(with_rows.N))
    o1 = oracle.attention_outputs(with_rows, 0, ag, [3] * len(ag), q, B)
    o0 = oracle.attention_outputs(zero_rows, 0, ag, [3] * len(ag), q, B)
    assert np.allclose(o1, o0, rtol=RTOL, atol=RTOL)
    if t == 0:  # no offset: the rows are on everywhere
        assert np.array_equal(with_rows.lr_begin, [0, 0])
    if t >= 12:  # offset past every view: plain base attention (B = 0)
        ob = oracle.attention_outputs(with_rows, 0, ag, [3] * len(ag), q, np.zeros_like(B))
        assert np.allclose(o1, ob, rtol=RTOL, atol=RTOL)


def test_activation_offset_rejects_bad_arguments():
    c, A, B = _small_cache()
    for agent, pos in ((-1, 0), (2, 0), (0, -1)):
        with pytest.raises(OracleError):
            c.set_lr_begin(agent, pos)


def test_errors_leave_state_unchanged():
    c = CacheModel(1, 4, 2, 64, 64, 4, 2, BASE_SHARED, 4, 3)
    k = np.zeros((9, 2, 64))
    c.append_base(0, SHARED, k[:8], k[:8])            # 2 pages
    with pytest.raises(OracleError) as e:
        c.append_base(0, 0, k, k)                       # needs 3 pages, 1 free
    assert e.value.code == "OOM"
    assert c.pages(0, 0) == [] and c.lens(0)["S"] == [0, 0]
    with pytest.raises(OracleError) as e:
        c.append_lowrank(0, SHARED, 0, 9, None, None)  # ahead of base rows
    assert e.value.code == "STATE"
    with pytest.raises(OracleError) as e:
        c.crop(0, 9)                                    # attach beyond P
    assert e.value.code == "STATE"
    c.crop(0, 6)
    with pytest.raises(OracleError) as e:
        c.crop(SHARED, 5)                               # below an agent's base length
    assert e.value.code == "STATE"
    with pytest.raises(OracleError) as e:
        c.validate_attend(0, [0], [6], [0], [1])        # LR rows missing over the view
    assert e.value.code == "STATE"
    c.append_lowrank(0, SHARED, 0, 8, None, None)
    c.validate_attend(0, [0], [6], [0], [1])
    with pytest.raises(OracleError) as e:
        c.validate_attend(0, [0], [5], [0], [1])        # caller's length disagrees
    assert e.value.code == "STATE"


def test_synth_bf16_rounding_is_rne():
    from synth import f32_to_bf16_bits
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    b = bf16_bits_to_f64(f32_to_bf16_bits(x))
    # 1+2^-8 is a tie -> even (1.0); 1+3*2^-8 is a tie -> even (1+2^-6... i.e. 1+4*2^-8)
    assert list(b) == [1.0, 1.0, 1.0 + 4 * 2 ** -8, -2.5, 1.0]
    d = Draws(3).normal((1000,))
    assert d.dtype == np.uint16
