"""The oracle's state model against the hand-worked page-table fixture and invariants."""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle.cache import CacheModel, OracleError, SHARED
from layout_fixture import check, load


class OracleBackend:
    def __init__(self, cfg):
        self.c = CacheModel(**cfg)

    def _rc(self, fn, *a):
        try:
            fn(*a)
            return "OK"
        except OracleError as e:
            return e.code

    def append_base(self, layer, seq, n):
        z = np.zeros((n, self.c.Hkv, self.c.d))
        return self._rc(self.c.append_base, layer, seq, z, z)

    def crop(self, seq, new_len):
        return self._rc(self.c.crop, seq, new_len)

    def pages(self, layer, seq):
        return self.c.pages(layer, seq)

    def lens(self, layer):
        return self.c.lens(layer)

    def base_len(self):
        return list(self.c.base_len)


def test_hand_worked_fixture():
    fx = load()
    check(OracleBackend(fx["config"]), fx)


def _invariants(c: CacheModel):
    for l in range(c.L):
        live = []
        for s in [SHARED] + list(range(c.N)):
            t = c.tables[l][s]
            assert len(t) == -(-c.length[l][s] // c.ps)
            live += t
        assert len(live) == len(set(live))
        assert set(live) | c.free[l] == set(range(c.max_pages))
        assert not (set(live) & c.free[l])
    for a in range(c.N):
        assert c.base_len[a] <= min(c.length[l][SHARED] for l in range(c.L))


ops = st.lists(st.tuples(st.sampled_from(["ab", "crop"]), st.integers(0, 1),
                         st.integers(-1, 2), st.integers(-1, 14)), max_size=60)


@settings(max_examples=150, deadline=None)
@given(ops)
def test_random_ops_keep_invariants(seq_ops):
    c = CacheModel(2, 4, 2, 64, 64, 4, 3, 0, 4, 12)
    for kind, layer, seq, n in seq_ops:
        try:
            if kind == "ab":
                z = np.zeros((max(n, 0), 2, 64))
                c.append_base(layer, seq, z, z)
            else:
                c.crop(seq, n)
        except OracleError:
            pass
        _invariants(c)
