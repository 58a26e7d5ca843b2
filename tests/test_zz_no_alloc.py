"""skv_decode_step_static (the entry point that allocates nothing: its decode
partial rows live in the library's static device scratch) against
skv_decode_step on identical contexts and inputs: two fused steps in a row,
the second over fewer agents and a shorter view (a smaller launch), each
compared element by element (the same kernels and summation order, so the
outputs must be identical) and with the oracle to the attention bar."""
import numpy as np
import pytest

import synth
from synth import BASE_LR_SHARED, Schedule, Shape

pytestmark = pytest.mark.gpu


def _run(shape, prefix, steps, seed, static):
    import torch
    import gpu_runner as R
    from lora_shared_kv_amd import skv as B
    sc = Schedule(shape, seed, n_layers=1)
    sc.draw_adapters()
    sc.shared_prefix(prefix)
    N = shape.n_agents
    for a in range(N):
        sc.attach(a)
    evs = [sc.decode_step(0, list(range(N)), tag="step 0"),
           sc.decode_step(0, list(range(N // 2)), tag="step 1 (half the agents)")]
    gpu = R.GpuRun(sc)
    orc = R.model_for(shape, 1, max_pages=gpu.cfg["max_pages"])
    outs = []
    fn = B.skv_decode_step_static if static else B.skv_decode_step
    for ev in sc.events:
        ref = R.apply_event(orc, ev)
        if isinstance(ev, synth.DecodeStep):
            q = R.dev(ev.q)
            o = torch.empty_like(q)
            fn(gpu.ctx, ev.layer, ev.agents, ev.base_len, ev.suffix_len, R.dev(ev.k), R.dev(ev.v), R.dev(ev.x),
               R.dev(ev.a), q, R.dev(ev.b), o)
            got = R.to_f64(o)
            ma, rl = R.errors(got, ref)
            print(f"{'static' if static else 'arena '} {ev.tag}: max_abs={ma:.3e} rel_l2={rl:.3e}", flush=True)
            assert ma <= R.MAX_ABS and rl <= R.MAX_REL_L2, (ev.tag, ma, rl)
            outs.append(o.view(torch.int16).cpu().numpy())
        else:
            gpu.apply(ev)
    B.skv_sync(gpu.ctx)
    return outs


@pytest.fixture(scope="module", autouse=True)
def _gpu(torch_cuda):
    return torch_cuda


@pytest.mark.parametrize("shape,prefix", [
    (Shape("llama3-heads", 1, 32, 8, 128, 4096, 8, 4, BASE_LR_SHARED, 0), 8000),
    (Shape("d64", 1, 8, 2, 64, 256, 16, 4, synth.BASE_SHARED, 0), 700),
])
def test_static_scratch_step_equals_arena_step(shape, prefix):
    a = _run(shape, prefix, 2, 77, static=False)
    s = _run(shape, prefix, 2, 77, static=True)
    assert len(a) == len(s) == 2
    for x, y in zip(a, s):
        assert np.array_equal(x, y)
