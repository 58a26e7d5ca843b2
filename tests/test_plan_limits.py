"""Every attention call is checked against the GPU launch plan on the host, before
anything is enqueued: a call past a plan limit returns UNSUPPORTED and leaves the
cache exactly as it was (no launch, no page taken, no length changed).

Runs on libskv_host.so (the host runtime with the null device backend), which
applies the same plan checks as the GPU build. The limits (plan.h):
  decode: per launch, items per KV head <= min(2048 / Hkv, 1024), each item at
    most 512 chunks of 32 keys, so a KV head's flattened view (shared prefix up
    to the largest b_i, then every own suffix, each padded to 32 keys) holds at
    most 32 * 512 * min(2048 / Hkv, 1024) keys;
  prefill: a view spans at most 4096 pages of 64 rows (shared and own pages
    counted separately);
  front end: the packed projection weights stay below 2 GiB.
"""
import pytest

from lora_shared_kv_amd import skv as B

FAKE = 0x100000  # a non-null "device" address; the null backend never dereferences it

# 64 KV heads: at most 32 items per head, 32 * 512 * 32 = 524,288 keys per launch
CFG = dict(n_layers=1, n_q_heads=64, n_kv_heads=64, head_dim=64, hidden=64, rank=4, n_agents=2,
           mode=0, page_size=64, max_pages=8200)
DECODE_KEYS = 32 * 512 * (2048 // 64)
PREFILL_ROWS = 4096 * 64


def make(shared_rows):
    n = B.skv_arena_bytes(CFG, "host")
    ctx = B.skv_create(CFG, (1 << 24, n), None, "host")
    B.skv_append_base(ctx, 0, -1, FAKE, FAKE, n=shared_rows)
    for plane in range(2):
        B.skv_append_lowrank(ctx, 0, -1, plane, shared_rows, None, None)
    return ctx


def state(ctx):
    return (B.skv_get_lens(ctx, 0), B.skv_get_counters(ctx),
            [B.skv_get_pages(ctx, 0, s) for s in (-1, 0, 1)])


def expect_unsupported(ctx, fn, *args):
    before = state(ctx)
    with pytest.raises(B.SkvError) as e:
        fn(ctx, *args)
    assert e.value.code == "UNSUPPORTED", e.value
    assert state(ctx) == before


@pytest.fixture(scope="module")
def ctx():
    return make(DECODE_KEYS + 64)


def test_decode_at_and_past_the_view_limit(ctx):
    B.skv_crop(ctx, 0, DECODE_KEYS)
    n0 = B.skv_get_counters(ctx)["launches"]
    B.skv_attn_decode(ctx, 0, [0], [DECODE_KEYS], [0], FAKE, FAKE, FAKE)
    assert B.skv_get_counters(ctx)["launches"] > n0
    B.skv_crop(ctx, 0, 0)
    B.skv_crop(ctx, 0, DECODE_KEYS + 1)  # one key past: one more chunk
    expect_unsupported(ctx, B.skv_attn_decode, 0, [0], [DECODE_KEYS + 1], [0], FAKE, FAKE, FAKE)


def test_fused_step_past_the_view_limit_takes_no_page(ctx):
    B.skv_crop(ctx, 0, 0)
    B.skv_crop(ctx, 0, DECODE_KEYS + 32)
    expect_unsupported(ctx, B.skv_decode_step, 0, [0], [DECODE_KEYS + 32], [0], FAKE, FAKE, FAKE, FAKE, FAKE,
                       FAKE, FAKE)
    # at the limit the step runs, appends the agent's row and takes its page
    B.skv_crop(ctx, 0, 0)
    B.skv_crop(ctx, 0, DECODE_KEYS)
    B.skv_decode_step(ctx, 0, [0], [DECODE_KEYS], [0], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert B.skv_get_lens(ctx, 0)["S"][0] == 1
    B.skv_crop(ctx, 0, DECODE_KEYS)


def test_decode_limit_counts_every_agent_of_a_launch(ctx):
    # two agents share one launch: the shared prefix once, plus each own suffix
    B.skv_crop(ctx, 0, 0)
    B.skv_crop(ctx, 1, 0)
    B.skv_crop(ctx, 0, DECODE_KEYS - 32)
    B.skv_crop(ctx, 1, DECODE_KEYS - 64)
    B.skv_append_agents(ctx, 0, [0, 1], [32, 1], FAKE, FAKE, None, None)
    # flattened: DECODE_KEYS - 32 shared keys + 32 + 32 (padded) own keys: one chunk too many
    expect_unsupported(ctx, B.skv_attn_decode, 0, [0, 1], [DECODE_KEYS - 32, DECODE_KEYS - 64], [32, 1], FAKE,
                       FAKE, FAKE)
    # each agent alone fits
    B.skv_attn_decode(ctx, 0, [0], [DECODE_KEYS - 32], [32], FAKE, FAKE, FAKE)
    B.skv_attn_decode(ctx, 0, [1], [DECODE_KEYS - 64], [1], FAKE, FAKE, FAKE)
    B.skv_crop(ctx, 0, 0)
    B.skv_crop(ctx, 1, 0)


def test_prefill_at_and_past_the_view_limit(ctx):
    B.skv_crop(ctx, 0, 0)
    B.skv_crop(ctx, 0, PREFILL_ROWS)
    B.skv_attn_prefill(ctx, 0, [0], [PREFILL_ROWS], [0], [16], FAKE, FAKE, FAKE)
    B.skv_crop(ctx, 0, 0)
    B.skv_crop(ctx, 0, PREFILL_ROWS + 1)
    expect_unsupported(ctx, B.skv_attn_prefill, 0, [0], [PREFILL_ROWS + 1], [0], [16], FAKE, FAKE, FAKE)
    # own pages count separately from shared pages
    B.skv_crop(ctx, 0, 0)
    B.skv_crop(ctx, 0, PREFILL_ROWS - 10)
    B.skv_append_agents(ctx, 0, [0], [20], FAKE, FAKE, None, None)
    expect_unsupported(ctx, B.skv_attn_prefill, 0, [0], [PREFILL_ROWS - 10], [20], [16], FAKE, FAKE, FAKE)
    B.skv_crop(ctx, 0, 0)


def test_misaligned_device_pointers_are_rejected(ctx):
    # the kernels use 16-byte vector accesses on every device tensor
    B.skv_crop(ctx, 0, 0)
    B.skv_crop(ctx, 0, 1000)
    before = state(ctx)
    calls = [
        (B.skv_append_base, (0, 0, FAKE + 2, FAKE), dict(n=4)),
        (B.skv_append_agents, (0, [0], [4], FAKE, FAKE + 8, None, None), {}),
        (B.skv_attn_decode, (0, [0], [1000], [0], FAKE, FAKE + 4, FAKE), {}),
        (B.skv_attn_prefill, (0, [0], [1000], [0], [4], FAKE + 2, FAKE, FAKE), {}),
        (B.skv_decode_step, (0, [0], [1000], [0], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2), {}),
    ]
    for fn, args, kw in calls:
        with pytest.raises(B.SkvError) as e:
            fn(ctx, *args, **kw)
        assert e.value.code == "ARG", (fn.__name__, e.value)
        assert state(ctx) == before
    B.skv_crop(ctx, 0, 0)


def test_static_scratch_limit():
    """skv_decode_step_static keeps the decode partial rows in a 16 MiB static
    array: a launch needing more is refused before anything is enqueued, while
    the arena-backed skv_decode_step takes the same call."""
    cfg = dict(n_layers=1, n_q_heads=64, n_kv_heads=64, head_dim=128, hidden=64, rank=32, n_agents=16,
               mode=1, page_size=64, max_pages=7200)
    n = B.skv_arena_bytes(cfg, "host")
    c = B.skv_create(cfg, (1 << 24, n), None, "host")
    P = 450_000  # 14,063 chunks per KV head: 28 items of <= 512 chunks, 64 heads
    B.skv_append_base(c, 0, -1, FAKE, FAKE, n=P)
    B.skv_append_lowrank(c, 0, -1, 0, P, None, None)
    agents = list(range(16))
    for a in agents:
        B.skv_crop(c, a, P)
    # 28 items x 64 heads x 16 rows x (128 + 32 + 4) x 4 bytes = 18.8 MB > 16 MiB
    before = state16(c)
    with pytest.raises(B.SkvError) as e:
        B.skv_decode_step_static(c, 0, agents, [P] * 16, [0] * 16, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert e.value.code == "UNSUPPORTED" and "static scratch" in str(e.value)
    assert state16(c) == before
    # one agent: 28 x 64 x 1 x 164 x 4 bytes = 1.2 MB fits
    B.skv_decode_step_static(c, 0, [0], [P], [0], FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    # the arena path takes the 16-agent call
    B.skv_decode_step(c, 0, agents, [P] * 16, [1] + [0] * 15, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def state16(c):
    return (B.skv_get_lens(c, 0), B.skv_get_counters(c), [B.skv_get_pages(c, 0, s) for s in range(-1, 16)])


def test_front_end_weight_limit():
    """The front end addresses the packed projection weights with 32-bit byte
    offsets: a geometry whose packed weights reach 2 GiB is refused before
    anything is planned, and the same call one column block smaller runs."""
    def ctx_for(hidden):
        cfg = dict(n_layers=1, n_q_heads=64, n_kv_heads=64, head_dim=128, hidden=hidden, rank=8, n_agents=2,
                   mode=1, page_size=64, max_pages=16)
        n = B.skv_arena_bytes(cfg, "host")
        return B.skv_create(cfg, (1 << 24, n), None, "host")
    big = 43712  # (64 + 128) * 128 * 43712 * 2 bytes >= 2 GiB
    assert (64 + 2 * 64) * 128 * big * 2 >= 1 << 31 > (64 + 2 * 64) * 128 * (big - 64) * 2
    c = ctx_for(big)
    before = state(c)
    with pytest.raises(B.SkvError) as e:
        B.skv_project_append(c, 0, [0], [32], FAKE, FAKE, FAKE, 0.0, FAKE)
    assert e.value.code == "UNSUPPORTED" and "2 GiB" in str(e.value)
    assert state(c) == before
    c = ctx_for(big - 64)
    B.skv_project_append(c, 0, [0], [32], FAKE, FAKE, FAKE, 0.0, FAKE)
    assert B.skv_get_lens(c, 0)["S"][0] == 32
