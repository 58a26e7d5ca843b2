"""Pins of the front-end oracle (oracle/frontend.py) against things other than itself:
torch's linear layer (a library routine), explicit 2-D rotations written out in
pure Python, and the properties that define a rotary embedding (norms kept,
position 0 is the identity, dot products depend only on the position
difference)."""
import math

import numpy as np
import pytest
import torch

from oracle import frontend as fe


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_projection_without_rotation_is_a_linear_layer():
    hq, hkv, d, hidden, n = 4, 2, 16, 32, 5
    x = _rand((n, hidden), 1)
    w = _rand(((hq + 2 * hkv) * d, hidden), 2)
    q, k, v = fe.project(x, w, hq, hkv, d, np.arange(n), 0.0)
    y = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w)).numpy()
    assert np.allclose(q.reshape(n, -1), y[:, :hq * d], rtol=1e-12, atol=1e-12)
    assert np.allclose(k.reshape(n, -1), y[:, hq * d:(hq + hkv) * d], rtol=1e-12, atol=1e-12)
    assert np.allclose(v.reshape(n, -1), y[:, (hq + hkv) * d:], rtol=1e-12, atol=1e-12)


def test_rotation_matches_explicit_pairwise_rotation():
    d, theta = 8, 500000.0
    u = _rand((3, 2, d), 3)
    pos = [0, 7, 65537]
    got = fe.rope(u, pos, theta)
    for i, t in enumerate(pos):
        for h in range(2):
            for j in range(d // 2):
                a = t * theta ** (-2.0 * j / d)
                lo, hi = u[i, h, j], u[i, h, j + d // 2]
                assert math.isclose(got[i, h, j], lo * math.cos(a) - hi * math.sin(a), rel_tol=1e-9, abs_tol=1e-12)
                assert math.isclose(got[i, h, j + d // 2], lo * math.sin(a) + hi * math.cos(a),
                                    rel_tol=1e-9, abs_tol=1e-12)


@pytest.mark.parametrize("theta", [10000.0, 500000.0])
def test_rotation_properties(theta):
    d = 64
    a, b = _rand((1, 1, d), 4), _rand((1, 1, d), 5)
    assert np.array_equal(fe.rope(a, [0], theta), a)                       # position 0: identity
    ra = fe.rope(a, [1234], theta)
    half = d // 2
    assert np.allclose(ra[..., :half] ** 2 + ra[..., half:] ** 2,          # every pair keeps its norm
                       a[..., :half] ** 2 + a[..., half:] ** 2, rtol=1e-12)
    for t1, t2, s in ((3, 10, 100), (0, 4096, 31)):                        # relative position only
        d1 = np.sum(fe.rope(a, [t1], theta) * fe.rope(b, [t2], theta))
        d2 = np.sum(fe.rope(a, [t1 + s], theta) * fe.rope(b, [t2 + s], theta))
        assert math.isclose(d1, d2, rel_tol=1e-9, abs_tol=1e-9)
