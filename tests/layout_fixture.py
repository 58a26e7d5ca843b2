"""Driver for the hand-worked page-table fixture (tests/golden/layout_ps4.json).

The same steps run through two independent implementations: the oracle's
state model and the C++ runtime (through the C ABI). Each backend is an
object with append_base(layer, seq, n) -> rc, crop(seq, new_len) -> rc,
pages(layer, seq), lens(layer) and base_len(); rc is one of
"OK", "ARG", "STATE", "OOM".
"""
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def load(name="layout_ps4.json"):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)


def check(backend, fx):
    for i, st in enumerate(fx["steps"]):
        if st["op"] == "append_base":
            rc = backend.append_base(st["layer"], st["seq"], st["n"])
        else:
            rc = backend.crop(st["seq"], st["new_len"])
        assert rc == st["rc"], (i, st, rc)
        for layer, seqs in st.get("expect", {}).items():
            for seq, pages in seqs.items():
                got = backend.pages(int(layer), int(seq))
                assert got == pages, (i, st, layer, seq, got)
        if "base_len" in st:
            assert backend.base_len() == st["base_len"], (i, backend.base_len())
        for layer, want in st.get("lens", {}).items():
            got = backend.lens(int(layer))
            for k, v in want.items():
                assert got[k] == v, (i, layer, k, got[k], v)
    fin = fx["final"]
    assert backend.base_len() == fin["base_len"]
    for layer, seqs in fin["tables"].items():
        for seq, pages in seqs.items():
            assert backend.pages(int(layer), int(seq)) == pages
    for layer, want in fin["lens"].items():
        got = backend.lens(int(layer))
        for k, v in want.items():
            assert got[k] == v
