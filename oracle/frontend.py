"""Oracle of the front end: the projections of a layer's input rows, with rotary
position embedding, before they enter the cache.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
CPU-baseline leg of the benchmark.

The LRAgent review ("What carries the argument") writes the value projection
of agent i as Y_i = X_i W_0 + (X_i A_i) B_i: the base term X W_0 is the cached
V_base, the rank-r rows X A_i are the low-rank cache. The same pass over X
gives the queries and keys (X W_q, X W_k). The pages do not describe position
encoding; the reading taken is rotary embedding in the rotate-half form, as in
the models the pages use, with its base theta passed by the caller (0 = none):
for a head vector u of size d and view position t, pairs (u_i, u_{i+d/2}),
i < d/2, rotate by the angle t * theta^(-2i/d).

Everything is float64; the results are rounded to bf16 where the cache and the
output store bf16 (round to nearest even).
"""
from __future__ import annotations

import numpy as np


def rope(u: np.ndarray, positions, theta: float) -> np.ndarray:
    """Rotary embedding of u [n][heads][d] at view positions [n] (float64)."""
    u = np.asarray(u, dtype=np.float64)
    if theta == 0:
        return u.copy()
    n, h, d = u.shape
    half = d // 2
    inv_freq = theta ** (-2.0 * np.arange(half) / d)             # [d/2]
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]  # [n][d/2]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    lo, hi = u[..., :half], u[..., half:]
    return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)


def project(x: np.ndarray, w_qkv: np.ndarray, n_q_heads: int, n_kv_heads: int, head_dim: int,
            positions, theta: float):
    """q, k, v of the rows x [n][hidden] (float64) with w_qkv [(Hq + 2 Hkv) d][hidden]
    (rows: the query heads, then the key heads, then the value heads). Returns
    float64 q [n][Hq][d] and k, v [n][Hkv][d], rotary embedding applied to q and k."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_qkv, dtype=np.float64)
    y = x @ w.T
    n = x.shape[0]
    nq = n_q_heads * head_dim
    nk = n_kv_heads * head_dim
    q = y[:, :nq].reshape(n, n_q_heads, head_dim)
    k = y[:, nq:nq + nk].reshape(n, n_kv_heads, head_dim)
    v = y[:, nq + nk:nq + 2 * nk].reshape(n, n_kv_heads, head_dim)
    return rope(q, positions, theta), rope(k, positions, theta), v
