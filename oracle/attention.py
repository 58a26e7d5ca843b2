"""Oracle arithmetic: materialise each agent's values, then plain causal softmax attention.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
CPU-baseline leg of the benchmark.

The method (LRAgent review, "What carries the argument") reaches exactly the
plain result by associativity: O = P (V_base + V_lr B) = P V_base + (P V_lr) B.
So the oracle computes the plain definition, in float64, with nothing
reordered or fused:

  1. V_i[j, g, :] = V_base[j, g, :] + (X_j A) B_i[:, g*d:(g+1)*d]
     (the LoRA value projection Y = X W0 + (X A) B, the review's statement of
     the paper's Eq. 3; B_i is r x (Hkv*d) and column slice g belongs to KV
     head g). With an activation offset t_i for agent i (RoleKV, "What it
     does": the adapter switches on after the role's header), the term is
     present only for j >= t_i.
  2. For a query at view position t and query head h, with KV head
     g = floor(h / G) (G = Hq / Hkv; the pages do not say how query heads map
     to KV heads, the reading taken is contiguous groups):
        s_j = q_h . K[j, g] / sqrt(d)  for 0 <= j <= t   (scale: the pages are
        silent; the reading is standard scaled dot-product attention)
        p = exp(s - max s) / sum exp(s - max s)
        o_h = sum_j p_j V_i[j, g]
     A query sees every view position up to and including its own (decode
     appends the new token, then attends).
"""
from __future__ import annotations

import numpy as np


def kv_head_of(h: int, group: int) -> int:
    """Query head h reads KV head floor(h / group)."""
    return h // group


def materialize_values(v_base: np.ndarray, lr_rows: np.ndarray, b_agent: np.ndarray) -> np.ndarray:
    """V_i = V_base + LR . B_i, head by head.

    v_base [L][Hkv][d], lr_rows [L][r] (the rank-r X A rows), b_agent [r][Hkv*d].
    """
    L, hkv, d = v_base.shape
    out = np.empty_like(v_base)
    for g in range(hkv):
        out[:, g, :] = v_base[:, g, :] + lr_rows @ b_agent[:, g * d:(g + 1) * d]
    return out


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row-wise softmax with the row maximum subtracted first."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attend_view(q: np.ndarray, k: np.ndarray, v: np.ndarray, positions) -> np.ndarray:
    """Causal softmax attention of queries at the given view positions.

    q [n][Hq][d], k [L][Hkv][d], v [L][Hkv][dv] (already materialised for this agent),
    positions: length-n view positions t (each query sees rows 0..t).
    Returns o [n][Hq][d] in float64.

    The definition in matrix form, one query head at a time: S = Q K^T / sqrt(d)
    over the view, keys after a query's position set to -inf, a softmax over
    each row, O = P V.
    """
    n, hq, d = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    scale = 1.0 / np.sqrt(d)
    pos = np.asarray(positions, dtype=np.int64)
    Lv = int(pos.max()) + 1
    after = np.arange(Lv)[None, :] > pos[:, None]   # key j lies after query i's position
    o = np.empty((n, hq, v.shape[2]))
    for h in range(hq):
        g = kv_head_of(h, group)
        s = (q[:, h, :] @ k[:Lv, g, :].T) * scale
        s[after] = -np.inf
        o[:, h, :] = softmax_rows(s) @ v[:Lv, g, :]
    return o


def attention_outputs(cache, layer, agents, n_q, q, b_all, rows=None):
    """Outputs of one attention call.

    cache: CacheModel; agents / n_q as passed to the library; q [sum n_q][Hq][d]
    (float64); b_all [N][r][Hkv*d] (float64). The queries of agent i are the
    last n_q[i] positions of its view. rows (optional) restricts the result to
    those row indices of the concatenated query list (others are NaN).
    Returns o [sum n_q][Hq][d].
    """
    tot = int(sum(n_q))
    out = np.full((tot,) + q.shape[1:], np.nan)
    want = set(range(tot)) if rows is None else set(int(r) for r in rows)
    off = 0
    for a, nq in zip(agents, n_q):
        idx = [i for i in range(nq) if off + i in want]
        if idx:
            k, vb, lr = cache.view(layer, a)
            lr = lr.copy()
            lr[:cache.lr_begin[a]] = 0.0  # positions before the adapter's activation
            L = k.shape[0]
            v = materialize_values(vb, lr, b_all[a])
            pos = [L - nq + i for i in idx]
            o = attend_view(q[[off + i for i in idx]], k, v, pos)
            for j, i in enumerate(idx):
                out[off + i] = o[j]
        off += nq
    return out
