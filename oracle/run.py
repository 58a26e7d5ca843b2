"""Replay a schedule of synthetic events through the oracle.

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
CPU-baseline leg of the benchmark.
"""
from __future__ import annotations

import numpy as np

from synth import (AppendAgents, AppendBase, AppendLowrank, Attend, Crop, DecodeStep, Schedule,
                   SetLrBegin, bf16_bits_to_f64)

from .attention import attention_outputs
from .cache import CacheModel, OracleError, SHARED


def model_for(shape, n_layers, max_pages=None):
    if max_pages is None:
        max_pages = 1 << 20
    return CacheModel(n_layers, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.hidden,
                      shape.rank, shape.n_agents, shape.mode, shape.page_size, max_pages)


def decode_step(cache: CacheModel, layer, agents, base_len, suffix_len, k, v, x=None, a=None):
    """State part of a fused decode step: checks (lengths before the step, own
    low-rank rows level with base rows, low-rank rows over the shared view,
    then pages), then one appended row per agent. The attention that follows
    is an ordinary decode over the grown views."""
    cache._check_layer(layer)
    n = len(agents)
    if not (1 <= n <= cache.N) or len(base_len) != n or len(suffix_len) != n:
        raise OracleError("ARG", "agents")
    if x is not None and a is None:
        raise OracleError("ARG", "A missing")
    if len(set(agents)) != n or any(not (0 <= ag < cache.N) for ag in agents):
        raise OracleError("ARG", "agent list")
    need = 0
    for ag, b, S in zip(agents, base_len, suffix_len):
        if b != cache.base_len[ag] or S != cache.length[layer][ag]:
            raise OracleError("STATE", "caller lengths differ from the cache")
        p = cache.plane_of(ag)
        if cache.lr_cov[layer][ag][p] != S:
            raise OracleError("STATE", "own low-rank rows lag base rows")
        if cache.lr_cov[layer][SHARED][p] < b:
            raise OracleError("STATE", "low-rank rows do not cover the view")
        need += -(-(S + 1) // cache.ps) - len(cache.tables[layer][ag])
    if need > len(cache.free[layer]):
        raise OracleError("OOM", "page pool exhausted")
    cache.append_agents(layer, agents, [1] * n, k, v, x, a)


def apply_event(cache: CacheModel, ev, sample_rows=None):
    """Apply one event. Returns the float64 outputs for an Attend event, else None."""
    f = bf16_bits_to_f64
    if isinstance(ev, AppendBase):
        cache.append_base(ev.layer, ev.seq, f(ev.k), f(ev.v))
    elif isinstance(ev, AppendLowrank):
        x = None if ev.x is None else f(ev.x)
        a = None if ev.a is None else f(ev.a)
        cache.append_lowrank(ev.layer, ev.seq, ev.plane, ev.n, x, a)
    elif isinstance(ev, AppendAgents):
        x = None if ev.x is None else f(ev.x)
        a = None if ev.a is None else f(ev.a)
        cache.append_agents(ev.layer, ev.agents, ev.counts, f(ev.k), f(ev.v), x, a)
    elif isinstance(ev, Crop):
        cache.crop(ev.seq, ev.new_len)
    elif isinstance(ev, SetLrBegin):
        cache.set_lr_begin(ev.agent, ev.pos)
    elif isinstance(ev, DecodeStep):
        x = None if ev.x is None else f(ev.x)
        a = None if ev.a is None else f(ev.a)
        decode_step(cache, ev.layer, ev.agents, ev.base_len, ev.suffix_len, f(ev.k), f(ev.v), x, a)
        rows = None if sample_rows is None else sample_rows(ev)
        return attention_outputs(cache, ev.layer, ev.agents, ev.n_q, f(ev.q), f(ev.b), rows)
    elif isinstance(ev, Attend):
        cache.validate_attend(ev.layer, ev.agents, ev.base_len, ev.suffix_len, ev.n_q)
        rows = None if sample_rows is None else sample_rows(ev)
        return attention_outputs(cache, ev.layer, ev.agents, ev.n_q, f(ev.q), f(ev.b), rows)
    else:
        raise TypeError(type(ev))
    return None


def run_schedule(sc: Schedule, sample_rows=None, max_pages=None):
    """Run every event; return (cache, [(event, float64 outputs)] for attention events)."""
    cache = model_for(sc.s, sc.L, max_pages)
    outs = []
    for ev in sc.events:
        o = apply_event(cache, ev, sample_rows)
        if o is not None:
            outs.append((ev, o))
    return cache, outs
