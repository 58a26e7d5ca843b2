"""Seeded synthetic inputs for the shared-prefix multi-LoRA attention path.

This module is the only code that the CPU oracle and the GPU path have in
common. It holds no arithmetic of the method: it draws random bf16 tensors,
and it writes down *schedules* (which sequence gets which rows, which agents
attend, which crops happen, and the lengths each call must carry). Every
number the method computes from these inputs is computed separately by each
side.

Value recipe (all workloads): Q, K, V_base and the hidden states X are
N(0, 1); the down-projection A is N(0, 1/hidden) and the up-projection B is
N(0, 0.01/r), where the second parameter is the variance. Draws are float32
from numpy's PCG64 and are rounded to bf16 with round-to-nearest-even. With
these scales X.A is about N(0, 1) and the adapter value term has a standard
deviation near 0.1, against 1 for V_base.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Iterator, List, Optional, Sequence

import numpy as np

SHARED = -1
BASE_SHARED = 0        # per-agent A_i, one low-rank plane per agent
BASE_LR_SHARED = 1     # one shared A, a single low-rank plane

# ---------------------------------------------------------------------------
# bf16 bit helpers (input preparation only)
# ---------------------------------------------------------------------------


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


class Draws:
    """Deterministic stream of bf16 normal draws."""

    def __init__(self, seed: int):
        self.rng = np.random.default_rng(np.random.PCG64(seed))

    def normal(self, shape, var: float = 1.0) -> np.ndarray:
        x = self.rng.standard_normal(size=shape, dtype=np.float32)
        if var != 1.0:
            x = x * np.float32(np.sqrt(var))
        return f32_to_bf16_bits(x)


# ---------------------------------------------------------------------------
# Workload shapes
# ---------------------------------------------------------------------------


@dataclass(frozen=True)
class Shape:
    name: str
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    hidden: int
    rank: int
    n_agents: int
    mode: int
    prefix: int
    page_size: int = 64

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def with_(self, **kw) -> "Shape":
        return dataclasses.replace(self, **kw)


# The five workloads. Prefix lengths in "k" are multiples of 1024.
TINY = Shape("tiny-1L-14q2kv-d64", 1, 14, 2, 64, 896, 8, 2, BASE_SHARED, 1024)
QWEN25 = Shape("qwen2.5-1.5b-attn", 28, 12, 2, 128, 1536, 16, 2, BASE_SHARED, 8192)
QWEN3 = Shape("qwen3-1.7b-attn", 28, 16, 8, 128, 2048, 16, 2, BASE_SHARED, 8192)
LLAMA3 = Shape("llama3-8b-attn", 32, 32, 8, 128, 4096, 8, 4, BASE_LR_SHARED, 33792)
MANY = Shape("many-agent-28L-16q8kv", 28, 16, 8, 128, 2048, 16, 8, BASE_SHARED, 16384)

WORKLOADS = {"tiny": TINY, "qwen25": QWEN25, "qwen3": QWEN3, "llama3": LLAMA3, "many": MANY}
QWEN25_PREFIXES = (1024, 2048, 4096, 8192)
QWEN3_TAKEOVER = (0, 160, 320)
LLAMA3_PREFIXES = (33792, 67584)
HEADLINE_PREFIX = 32768


def plane_of(shape: Shape, agent: int) -> int:
    return agent if shape.mode == BASE_SHARED else 0


def n_planes(shape: Shape) -> int:
    return shape.n_agents if shape.mode == BASE_SHARED else 1


# ---------------------------------------------------------------------------
# Schedule events. Arrays are uint16 bf16 bit patterns.
# ---------------------------------------------------------------------------


@dataclass
class AppendBase:
    layer: int
    seq: int
    k: np.ndarray          # [n][Hkv][d]
    v: np.ndarray          # [n][Hkv][d]


@dataclass
class AppendLowrank:
    layer: int
    seq: int
    plane: int
    n: int
    x: Optional[np.ndarray]   # [n][hidden] or None for adapter-off (zero) rows
    a: Optional[np.ndarray]   # [hidden][r] or None with x


@dataclass
class AppendAgents:
    """One row block per listed agent, base K/V and low-rank rows together."""
    layer: int
    agents: List[int]
    counts: List[int]
    k: np.ndarray          # [sum counts][Hkv][d]
    v: np.ndarray
    x: Optional[np.ndarray]   # [sum counts][hidden] or None (zero rows)
    a: Optional[np.ndarray]   # [n_agents][hidden][r] (per-agent A) or [hidden][r] (shared A)


@dataclass
class Crop:
    seq: int
    new_len: int


@dataclass
class Attend:
    kind: str              # "prefill" or "decode"
    layer: int
    agents: List[int]
    base_len: List[int]
    suffix_len: List[int]
    n_q: List[int]         # all ones for decode
    q: np.ndarray          # [sum n_q][Hq][d]
    b: np.ndarray          # [n_agents][r][Hkv*d]
    tag: str = ""


@dataclass
class SetLrBegin:
    """Adapter activation offset of one agent (view position)."""
    agent: int
    pos: int


@dataclass
class DecodeStep:
    """One decode token per listed agent: append its row, then attend from it.
    base_len / suffix_len are the lengths before the step."""
    layer: int
    agents: List[int]
    base_len: List[int]
    suffix_len: List[int]
    k: np.ndarray          # [n][Hkv][d]
    v: np.ndarray
    x: Optional[np.ndarray]   # [n][hidden] or None (zero low-rank rows)
    a: Optional[np.ndarray]   # as AppendAgents.a
    q: np.ndarray          # [n][Hq][d]
    b: np.ndarray          # [n_agents][r][Hkv*d]
    tag: str = ""

    @property
    def n_q(self):
        return [1] * len(self.agents)

    kind = "step"


# ---------------------------------------------------------------------------
# Schedule builder: keeps the lengths each attention call must carry.
# ---------------------------------------------------------------------------


class Schedule:
    """Builds an event list and tracks the view lengths that the schedule implies."""

    def __init__(self, shape: Shape, seed: int, n_layers: Optional[int] = None,
                 peaked: float = 1.0, zero_vbase: bool = False):
        self.s = shape
        self.L = n_layers if n_layers is not None else shape.n_layers
        self.d = Draws(seed)
        self.peaked = peaked
        self.zero_vbase = zero_vbase
        N = shape.n_agents
        self.P = [0] * self.L
        self.S = [[0] * N for _ in range(self.L)]
        self.b = [0] * N
        self.A: List[np.ndarray] = []   # per layer: [N][hidden][r] or [hidden][r]
        self.B: List[np.ndarray] = []   # per layer: [N][r][Hkv*d]
        self.events: List[object] = []

    # -- weights --------------------------------------------------------------
    def draw_adapters(self):
        s = self.s
        for _ in range(self.L):
            if s.mode == BASE_SHARED:
                self.A.append(self.d.normal((s.n_agents, s.hidden, s.rank), 1.0 / s.hidden))
            else:
                self.A.append(self.d.normal((s.hidden, s.rank), 1.0 / s.hidden))
            self.B.append(self.d.normal((s.n_agents, s.rank, s.n_kv_heads * s.head_dim), 0.01 / s.rank))

    def a_for(self, layer: int, agent: int) -> np.ndarray:
        a = self.A[layer]
        return a[agent] if self.s.mode == BASE_SHARED else a

    # -- helpers --------------------------------------------------------------
    def _kv(self, n):
        s = self.s
        k = self.d.normal((n, s.n_kv_heads, s.head_dim))
        v = self.d.normal((n, s.n_kv_heads, s.head_dim))
        if self.zero_vbase:
            v = np.zeros_like(v)
        return k, v

    def _q(self, n):
        s = self.s
        q = self.d.normal((n, s.n_q_heads, s.head_dim))
        if self.peaked != 1.0:
            q = f32_to_bf16_bits(bf16_bits_to_f64(q).astype(np.float32) * np.float32(self.peaked))
        return q

    # -- ops ------------------------------------------------------------------
    def shared_prefix(self, n: int, lr: str = "x"):
        """Append n base rows to SHARED on every layer plus every plane's LR rows.

        lr="x": rows X.A over one shared X (A_i per plane, or the shared A);
        lr="zero": adapter-off zero rows.
        """
        s = self.s
        for l in range(self.L):
            k, v = self._kv(n)
            self.events.append(AppendBase(l, SHARED, k, v))
            x = self.d.normal((n, s.hidden)) if lr == "x" else None
            for p in range(n_planes(s)):
                a = None if x is None else self.a_for(l, p)
                self.events.append(AppendLowrank(l, SHARED, p, n, x, a))
            self.P[l] += n

    def attach(self, agent: int, new_len: Optional[int] = None):
        new_len = min(self.P) if new_len is None else new_len
        self.events.append(Crop(agent, new_len))
        self._apply_crop(agent, new_len)

    def crop(self, seq: int, new_len: int):
        self.events.append(Crop(seq, new_len))
        self._apply_crop(seq, new_len)

    def _apply_crop(self, seq, new_len):
        if seq == SHARED:
            self.P = [new_len] * self.L
            return
        S = [self.S[l][seq] for l in range(self.L)]
        if all(x == 0 for x in S) and new_len >= self.b[seq]:
            self.b[seq] = new_len
        elif new_len < self.b[seq]:
            self.b[seq] = new_len
            for l in range(self.L):
                self.S[l][seq] = 0
        else:
            for l in range(self.L):
                self.S[l][seq] = new_len - self.b[seq]

    def own_rows(self, layer: int, agents: Sequence[int], counts: Sequence[int],
                 lr: str = "x", batched: bool = True):
        """Append counts[i] own rows to each agent at one layer (K/V and LR)."""
        s = self.s
        tot = int(sum(counts))
        k, v = self._kv(tot)
        x = self.d.normal((tot, s.hidden)) if lr == "x" else None
        if batched:
            a = None if x is None else self.A[layer]
            self.events.append(AppendAgents(layer, list(agents), list(counts), k, v, x, a))
        else:
            o = 0
            for ag, c in zip(agents, counts):
                self.events.append(AppendBase(layer, ag, k[o:o + c], v[o:o + c]))
                xa = None if x is None else x[o:o + c]
                aa = None if x is None else self.a_for(layer, ag)
                self.events.append(AppendLowrank(layer, ag, plane_of(s, ag), c, xa, aa))
                o += c
        for ag, c in zip(agents, counts):
            self.S[layer][ag] += c

    def decode_step(self, layer: int, agents: Sequence[int], lr: str = "x", tag=""):
        """Fused decode step: one new row per agent, then attention from it."""
        s = self.s
        n = len(agents)
        k, v = self._kv(n)
        x = self.d.normal((n, s.hidden)) if lr == "x" else None
        q = self._q(n)
        ev = DecodeStep(layer, list(agents), [self.b[a] for a in agents],
                        [self.S[layer][a] for a in agents], k, v, x,
                        None if x is None else self.A[layer], q, self.B[layer], tag)
        self.events.append(ev)
        for a in agents:
            self.S[layer][a] += 1
        return ev

    def set_lr_begin(self, agent: int, pos: int):
        self.events.append(SetLrBegin(agent, pos))

    def attend(self, kind: str, layer: int, agents: Sequence[int], n_q: Sequence[int], tag=""):
        q = self._q(int(sum(n_q)))
        ev = Attend(kind, layer, list(agents), [self.b[a] for a in agents],
                    [self.S[layer][a] for a in agents], list(n_q), q, self.B[layer], tag)
        self.events.append(ev)
        return ev


# ---------------------------------------------------------------------------
# The five workload schedules (layers and steps can be cut for parity runs).
# ---------------------------------------------------------------------------


def tiny_schedule(seed=1000, n_layers=None, decode_steps=16, prefill=32, fused=False, **kw) -> Schedule:
    """Tiny: shared prefix 1024, two agents, 32-token suffix prefill each, then decodes."""
    s = TINY
    sc = Schedule(s, seed, n_layers, **kw)
    sc.draw_adapters()
    sc.shared_prefix(s.prefix)
    for a in range(s.n_agents):
        sc.attach(a)
    for a in range(s.n_agents):
        for l in range(sc.L):
            sc.own_rows(l, [a], [prefill], batched=False)
            sc.attend("prefill", l, [a], [prefill], tag=f"prefill a{a}")
    agents = list(range(s.n_agents))
    for t in range(decode_steps):
        for l in range(sc.L):
            if fused:
                sc.decode_step(l, agents, tag=f"step t{t}")
            else:
                sc.own_rows(l, agents, [1] * len(agents))
                sc.attend("decode", l, agents, [1] * len(agents), tag=f"decode t{t}")
    return sc


def qwen25_schedule(prefix=1024, seed=1001, n_layers=1, turns=4, prefill=256, decode=128,
                    decode_sample=None, **kw) -> Schedule:
    """Two agents alternate turns; each turn ends with a handoff into the shared prefix."""
    s = QWEN25.with_(prefix=prefix)
    sc = Schedule(s, seed, n_layers, **kw)
    sc.draw_adapters()
    sc.shared_prefix(prefix)
    for a in range(s.n_agents):
        sc.attach(a)
    for t in range(turns):
        a = t % 2
        for l in range(sc.L):
            sc.own_rows(l, [a], [prefill])
            sc.attend("prefill", l, [a], [prefill], tag=f"turn{t} prefill")
        steps = range(decode) if decode_sample is None else decode_sample
        done = 0
        for st in range(decode):
            for l in range(sc.L):
                sc.own_rows(l, [a], [1])
                if st in steps:
                    sc.attend("decode", l, [a], [1], tag=f"turn{t} decode{st}")
            done += 1
        # handoff: drop the agent's own rows, recompute the turn with base weights
        # into the shared prefix, then every agent adds its LR rows and re-attaches.
        turn_len = prefill + decode
        sc.crop(a, sc.b[a])
        sc.shared_prefix(turn_len)
        for ag in range(s.n_agents):
            sc.attach(ag)
    return sc


def qwen3_schedule(takeover=160, seed=1002, n_layers=1, decode=64, **kw) -> Schedule:
    """Base prefix with adapters off; specialists re-take the last `takeover` tokens."""
    s = QWEN3
    sc = Schedule(s, seed, n_layers, **kw)
    sc.draw_adapters()
    sc.shared_prefix(s.prefix, lr="zero")
    agents = list(range(s.n_agents))
    for a in agents:
        sc.attach(a, s.prefix - takeover)
    if takeover > 0:
        for l in range(sc.L):
            sc.own_rows(l, agents, [takeover] * len(agents))
            sc.attend("prefill", l, agents, [takeover] * len(agents), tag=f"takeover{takeover}")
    for t in range(decode):
        for l in range(sc.L):
            sc.own_rows(l, agents, [1] * len(agents))
            sc.attend("decode", l, agents, [1] * len(agents), tag=f"decode t{t}")
    return sc


def llama3_schedule(prefix=33792, seed=1003, n_layers=1, decode=256, fused=False, prefill=0,
                    **kw) -> Schedule:
    """Shared-A agents decode one token each per step over a long shared trajectory;
    with prefill > 0 each agent first appends that many own tokens and they are
    prefilled together (the suffix-prefill shape of the throughput run)."""
    s = LLAMA3.with_(prefix=prefix)
    sc = Schedule(s, seed, n_layers, **kw)
    sc.draw_adapters()
    sc.shared_prefix(prefix)
    agents = list(range(s.n_agents))
    for a in agents:
        sc.attach(a)
    if prefill:
        for l in range(sc.L):
            sc.own_rows(l, agents, [prefill] * len(agents))
            sc.attend("prefill", l, agents, [prefill] * len(agents), tag="suffix prefill")
    for t in range(decode):
        for l in range(sc.L):
            if fused:
                sc.decode_step(l, agents, tag=f"step t{t}")
            else:
                sc.own_rows(l, agents, [1] * len(agents))
                sc.attend("decode", l, agents, [1] * len(agents), tag=f"decode t{t}")
    return sc


def many_schedule(seed=1004, n_layers=1, turns=6, prefill=512, handoff=256, **kw) -> Schedule:
    """Eight agents: one half prefills while the other half decodes; handoff each turn."""
    s = MANY
    sc = Schedule(s, seed, n_layers, **kw)
    sc.draw_adapters()
    sc.shared_prefix(s.prefix)
    for a in range(s.n_agents):
        sc.attach(a)
    for t in range(turns):
        pre = [0, 1, 2, 3] if t % 2 == 0 else [4, 5, 6, 7]
        dec = [4, 5, 6, 7] if t % 2 == 0 else [0, 1, 2, 3]
        for l in range(sc.L):
            sc.own_rows(l, pre, [prefill] * 4)
            sc.own_rows(l, dec, [1] * 4)
            sc.attend("prefill", l, pre, [prefill] * 4, tag=f"turn{t} mixed prefill")
            sc.attend("decode", l, dec, [1] * 4, tag=f"turn{t} mixed decode")
        lead = pre[0]
        L_lead = sc.b[lead] + sc.S[0][lead]
        sc.crop(lead, L_lead - handoff)
        for l in range(sc.L):
            sc.own_rows(l, [lead], [handoff], lr="zero", batched=False)
    return sc
