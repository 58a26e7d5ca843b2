"""The C++ runtime's store metadata against the hand-worked fixture and the oracle.

Runs libskv_host.so (the host runtime linked with the null device backend) so
it needs no GPU: lengths, page ids, free lists, crop results and error codes
must equal the oracle's state model exactly.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

from lora_shared_kv_amd import skv as B
from oracle.cache import CacheModel, OracleError, SHARED
from layout_fixture import check, load

FAKE = 0x100000     # a non-null "device" address; the null backend never dereferences it


def make(cfg):
    n = B.skv_arena_bytes(cfg, "host")
    return B.skv_create(cfg, (1 << 24, n), None, "host")


class LibBackend:
    def __init__(self, cfg):
        self.ctx = make(cfg)
        self.N = cfg["n_agents"]

    def _rc(self, fn, *a, **kw):
        try:
            fn(self.ctx, *a, **kw)
            return "OK"
        except B.SkvError as e:
            return e.code

    def append_base(self, layer, seq, n):
        return self._rc(B.skv_append_base, layer, seq, FAKE, FAKE, n=n)

    def crop(self, seq, new_len):
        return self._rc(B.skv_crop, seq, new_len)

    def pages(self, layer, seq):
        return B.skv_get_pages(self.ctx, layer, seq)

    def lens(self, layer):
        return B.skv_get_lens(self.ctx, layer)

    def base_len(self):
        return B.skv_get_lens(self.ctx, 0)["b"]


def test_hand_worked_fixture_on_the_library():
    fx = load()
    check(LibBackend(fx["config"]), fx)


CFG = dict(n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, hidden=64, rank=4, n_agents=3,
           mode=0, page_size=4, max_pages=12)

op = st.one_of(
    st.tuples(st.just("base"), st.integers(0, 1), st.integers(-1, 2), st.integers(0, 9)),
    st.tuples(st.just("lr"), st.integers(0, 1), st.integers(-1, 2), st.integers(0, 3), st.integers(0, 9),
              st.booleans()),
    st.tuples(st.just("agents"), st.integers(0, 1), st.lists(st.integers(0, 2), min_size=0, max_size=3),
              st.lists(st.integers(0, 5), min_size=3, max_size=3), st.booleans()),
    st.tuples(st.just("project"), st.integers(0, 1), st.lists(st.integers(0, 2), min_size=0, max_size=3),
              st.lists(st.integers(0, 5), min_size=3, max_size=3), st.booleans()),
    st.tuples(st.just("crop"), st.integers(-1, 2), st.integers(-1, 16)),
    st.tuples(st.just("attend"), st.integers(0, 1), st.lists(st.integers(0, 2), min_size=1, max_size=3),
              st.integers(0, 2), st.integers(1, 3)),
    st.tuples(st.just("step"), st.integers(0, 1), st.lists(st.integers(0, 2), min_size=1, max_size=3,
                                                            unique=True), st.booleans()),
)


def _oracle_rc(fn, *a):
    try:
        fn(*a)
        return "OK"
    except OracleError as e:
        return e.code


@settings(max_examples=300, deadline=None)
@given(st.lists(op, max_size=50), st.sampled_from([0, 1]))
def test_random_ops_match_the_oracle(ops, mode):
    cfg = dict(CFG, mode=mode)
    ctx = make(cfg)
    orc = CacheModel(**cfg)
    Hkv, d, hidden, r = cfg["n_kv_heads"], cfg["head_dim"], cfg["hidden"], cfg["rank"]
    for o in ops:
        kind = o[0]
        if kind == "base":
            _, layer, seq, n = o
            z = np.zeros((n, Hkv, d))
            want = _oracle_rc(orc.append_base, layer, seq, z, z)
            try:
                B.skv_append_base(ctx, layer, seq, FAKE, FAKE, n=n); got = "OK"
            except B.SkvError as e:
                got = e.code
        elif kind == "lr":
            _, layer, seq, plane, n, with_x = o
            x = np.zeros((n, hidden)) if with_x else None
            a = np.zeros((hidden, r)) if with_x else None
            want = _oracle_rc(orc.append_lowrank, layer, seq, plane, n, x, a)
            try:
                B.skv_append_lowrank(ctx, layer, seq, plane, n, FAKE if with_x else None,
                                     FAKE if with_x else None); got = "OK"
            except B.SkvError as e:
                got = e.code
        elif kind == "agents":
            _, layer, agents, counts, with_x = o
            counts = counts[:len(agents)]
            tot = sum(counts)
            z = np.zeros((tot, Hkv, d))
            x = np.zeros((tot, hidden)) if with_x else None
            a = (np.zeros((cfg["n_agents"], hidden, r)) if mode == 0 else np.zeros((hidden, r))) if with_x else None
            want = _oracle_rc(orc.append_agents, layer, agents, counts, z, z, x, a)
            try:
                B.skv_append_agents(ctx, layer, agents, counts, FAKE, FAKE, FAKE if with_x else None,
                                    FAKE if with_x else None); got = "OK"
            except B.SkvError as e:
                got = e.code
        elif kind == "project":
            # the fused front end appends like skv_append_agents (its k, v come
            # from the projection; x feeds the low-rank rows when A is given)
            _, layer, agents, counts, with_a = o
            counts = counts[:len(agents)]
            tot = sum(counts)
            z = np.zeros((tot, Hkv, d))
            x = np.zeros((tot, hidden)) if with_a else None
            a = (np.zeros((cfg["n_agents"], hidden, r)) if mode == 0 else np.zeros((hidden, r))) if with_a else None
            want = _oracle_rc(orc.append_agents, layer, agents, counts, z, z, x, a)
            try:
                B.skv_project_append(ctx, layer, agents, counts, FAKE, FAKE, FAKE if with_a else None,
                                     10000.0, FAKE); got = "OK"
            except B.SkvError as e:
                got = e.code
        elif kind == "crop":
            _, seq, n = o
            want = _oracle_rc(orc.crop, seq, n)
            try:
                B.skv_crop(ctx, seq, n); got = "OK"
            except B.SkvError as e:
                got = e.code
        elif kind == "step":
            from oracle.run import decode_step
            _, layer, agents, with_x = o
            bl = [orc.base_len[a] for a in agents]
            sl = [orc.length[layer][a] for a in agents]
            n = len(agents)
            z = np.zeros((n, Hkv, d))
            x = np.zeros((n, hidden)) if with_x else None
            a = (np.zeros((cfg["n_agents"], hidden, r)) if mode == 0 else np.zeros((hidden, r))) if with_x else None
            want = _oracle_rc(decode_step, orc, layer, agents, bl, sl, z, z, x, a)
            try:
                B.skv_decode_step(ctx, layer, agents, bl, sl, FAKE, FAKE, FAKE if with_x else None,
                                  FAKE if with_x else None, FAKE, FAKE, FAKE); got = "OK"
            except B.SkvError as e:
                got = e.code
        else:
            _, layer, agents, perturb, nq = o
            bl = [orc.base_len[a] if 0 <= a < orc.N else 0 for a in agents]
            sl = [orc.length[layer][a] if 0 <= a < orc.N else 0 for a in agents]
            if perturb == 1 and bl:
                bl[0] += 1
            nqs = [nq] * len(agents)
            want = _oracle_rc(orc.validate_attend, layer, agents, bl, sl, nqs)
            try:
                B.skv_attn_prefill(ctx, layer, agents, bl, sl, nqs, FAKE, FAKE, FAKE); got = "OK"
            except B.SkvError as e:
                got = e.code
        assert got == want, (o, got, want)
        for layer in range(cfg["n_layers"]):
            lib_l = B.skv_get_lens(ctx, layer)
            assert lib_l == orc.lens(layer), (o, lib_l, orc.lens(layer))
            for seq in [SHARED] + list(range(cfg["n_agents"])):
                assert B.skv_get_pages(ctx, layer, seq) == orc.pages(layer, seq), (o, layer, seq)


def test_counters_account_for_every_row():
    cfg = dict(CFG, mode=0, n_layers=1)
    ctx = make(cfg)
    B.skv_append_base(ctx, 0, -1, FAKE, FAKE, n=10)
    for p in range(3):
        B.skv_append_lowrank(ctx, 0, -1, p, 10, FAKE, FAKE)
    B.skv_crop(ctx, 0, 10)
    B.skv_append_agents(ctx, 0, [0], [5], FAKE, FAKE, None, None)
    B.skv_crop(ctx, 0, 12)
    c = B.skv_get_counters(ctx)
    assert c["base_rows_shared"] == 10 and c["base_rows_own"] == 5
    assert c["lr_rows"] == 30 and c["lr_zero_rows"] == 5
    assert c["rows_cropped"] == 3
    assert c["pages_alloc"] == 3 + 2 and c["pages_freed"] == 1


def test_project_append_accounting_and_rotary_base_checks():
    cfg = dict(CFG, mode=0, n_layers=1, page_size=4, max_pages=12)
    ctx = make(cfg)
    B.skv_append_base(ctx, 0, -1, FAKE, FAKE, n=6)
    B.skv_crop(ctx, 0, 6)
    before = B.skv_get_counters(ctx)["launches"]
    B.skv_project_append(ctx, 0, [0, 2], [5, 3], FAKE, FAKE, FAKE, 500000.0, FAKE)
    c = B.skv_get_counters(ctx)
    assert c["launches"] == before + 1           # one fused launch for the whole call
    assert c["base_rows_own"] == 8 and c["lr_rows"] == 8
    assert B.skv_get_lens(ctx, 0)["S"] == [5, 0, 3] and B.skv_get_lens(ctx, 0)["lr_own"] == [5, 0, 3]
    B.skv_project_append(ctx, 0, [1], [2], FAKE, FAKE, None, 0.0, FAKE)
    assert B.skv_get_counters(ctx)["lr_zero_rows"] == 2
    for bad in (1.0, 0.5, -1.0, float("inf"), float("nan")):
        try:
            B.skv_project_append(ctx, 0, [1], [1], FAKE, FAKE, None, bad, FAKE)
            raise AssertionError(f"rotary base {bad} accepted")
        except B.SkvError as e:
            assert e.code == "ARG"
    for bad in ((None, FAKE), (FAKE, None), (FAKE, FAKE + 2)):   # null, or overlapping buffers
        try:
            B.skv_pack_qkv(ctx, bad[0], bad[1])
            raise AssertionError("bad pack arguments accepted")
        except B.SkvError as e:
            assert e.code == "ARG"
    B.skv_pack_qkv(ctx, FAKE, FAKE + (1 << 22))
    for args in ((None, FAKE, FAKE), (FAKE, None, FAKE), (FAKE, FAKE, None)):
        try:
            B.skv_project_append(ctx, 0, [1], [1], args[0], args[1], None, 0.0, args[2])
            raise AssertionError("null pointer accepted")
        except B.SkvError as e:
            assert e.code == "ARG"
    try:   # more pages than the pool holds: nothing appended
        B.skv_project_append(ctx, 0, [1], [100], FAKE, FAKE, None, 0.0, FAKE)
        raise AssertionError("overflow accepted")
    except B.SkvError as e:
        assert e.code == "OOM"
    assert B.skv_get_lens(ctx, 0)["S"] == [5, 2, 3]
