"""Thin ctypes binding of the C ABI in include/skv.h (argument marshalling only).

Every function has the name of the C entry point it wraps. Device tensors are
torch tensors on the GPU (bf16, contiguous); their data pointers go straight
to the library, which enqueues the work on the context's stream. Nothing here
computes any part of the method, and there is no fallback: if the native
library is missing, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))

SKV_SHARED = -1
SKV_BASE_SHARED = 0
SKV_BASE_LR_SHARED = 1
SKV_MAX_AGENTS = 16
KERNEL_KINDS = ("append_kv", "append_lowrank", "decode_split", "decode_merge", "prefill", "project")

_CODES = {0: "OK", -1: "ARG", -2: "STATE", -3: "OOM", -4: "UNSUPPORTED", -5: "HIP"}

_I = ctypes.c_int
_P = ctypes.c_void_p
_IP = ctypes.POINTER(ctypes.c_int)


class skv_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "n_q_heads", "n_kv_heads", "head_dim", "hidden", "rank", "n_agents", "mode",
        "page_size", "max_pages")]


class skv_pools(ctypes.Structure):
    _fields_ = [("k_off", ctypes.c_uint64), ("vt_off", ctypes.c_uint64), ("lrt_off", ctypes.c_uint64),
                ("tables_off", ctypes.c_uint64), ("scratch_off", ctypes.c_uint64),
                ("scratch_bytes", ctypes.c_uint64), ("arena_bytes", ctypes.c_uint64),
                ("planes", ctypes.c_int32)]


class skv_counters(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "base_rows_shared", "base_rows_own", "lr_rows", "lr_zero_rows", "rows_cropped",
        "pages_alloc", "pages_freed", "launches")]


class skv_kernel_times(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * 6), ("launches", ctypes.c_int64 * 6)]


EXPORTS = {
    "skv_arena_bytes": (ctypes.c_size_t, [ctypes.POINTER(skv_config)]),
    "skv_create": (_I, [ctypes.POINTER(skv_config), _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)]),
    "skv_destroy": (None, [_P]),
    "skv_append_base": (_I, [_P, _I, _I, _I, _P, _P]),
    "skv_append_lowrank": (_I, [_P, _I, _I, _I, _I, _P, _P]),
    "skv_append_agents": (_I, [_P, _I, _I, _IP, _IP, _P, _P, _P, _P]),
    "skv_attn_prefill": (_I, [_P, _I, _I, _IP, _IP, _IP, _IP, _P, _P, _P]),
    "skv_attn_decode": (_I, [_P, _I, _I, _IP, _IP, _IP, _P, _P, _P]),
    "skv_decode_step": (_I, [_P, _I, _I, _IP, _IP, _IP, _P, _P, _P, _P, _P, _P, _P]),
    "skv_decode_step_static": (_I, [_P, _I, _I, _IP, _IP, _IP, _P, _P, _P, _P, _P, _P, _P]),
    "skv_crop": (_I, [_P, _I, _I]),
    "skv_set_lr_begin": (_I, [_P, _I, _I]),
    "skv_project_append": (_I, [_P, _I, _I, _IP, _IP, _P, _P, _P, ctypes.c_float, _P]),
    "skv_pack_qkv": (_I, [_P, _P, _P]),
    "skv_get_lens": (_I, [_P, _I, _IP, _IP, _IP, _IP, _IP]),
    "skv_get_pages": (_I, [_P, _I, _I, ctypes.POINTER(ctypes.c_int32), _I]),
    "skv_get_pools": (_I, [_P, ctypes.POINTER(skv_pools)]),
    "skv_get_counters": (_I, [_P, ctypes.POINTER(skv_counters)]),
    "skv_set_timing": (_I, [_P, _I]),
    "skv_collect_timing": (_I, [_P, ctypes.POINTER(skv_kernel_times)]),
    "skv_sync": (_I, [_P]),
    "skv_last_error": (ctypes.c_char_p, [_P]),
    "skv_probe_stream_read": (_I, [_P, ctypes.c_uint64, _I, _P, ctypes.POINTER(ctypes.c_double)]),
    "skv_probe_mfma_bf16": (_I, [_P, ctypes.POINTER(ctypes.c_double)]),
    "skv_probe_mfma_bf16_data": (_I, [_P, ctypes.c_uint64, _P, ctypes.POINTER(ctypes.c_double)]),
    "skv_probe_launch_pattern": (_I, [_P, ctypes.c_uint64, _I, _I, _I, _P, ctypes.POINTER(ctypes.c_double),
                                      ctypes.POINTER(ctypes.c_double)]),
}

_LIBS = {}


def library_path(kind: str = "gpu") -> str:
    return os.path.join(_PKG, "libskv.so" if kind == "gpu" else "libskv_host.so")


def load_library(kind: str = "gpu"):
    """kind="gpu": libskv.so (HIP kernels). kind="host": the null-device build for metadata tests."""
    if kind in _LIBS:
        return _LIBS[kind]
    path = library_path(kind)
    if not os.path.exists(path):
        raise RuntimeError(f"native library {path} is not built; run `python -m lora_shared_kv_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in EXPORTS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIBS[kind] = lib
    return lib


class SkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        self.code = _CODES.get(code, str(code))
        super().__init__(f"skv error {self.code}: {msg}")


_torch = None
_bf16 = None


def _ints(xs):
    """A C int array for a host int list; a ctypes array passes through unchanged."""
    if isinstance(xs, ctypes.Array):
        return xs, len(xs)
    xs = [int(x) for x in xs]
    return (ctypes.c_int * max(1, len(xs)))(*xs), len(xs)


def int_array(xs):
    """Build a reusable C int array (for calls repeated in a loop)."""
    return (ctypes.c_int * max(1, len(xs)))(*[int(x) for x in xs])


def _ptr(t, shape=None, name="tensor"):
    """Device pointer of a tensor (checked) or an int address; None -> NULL."""
    global _torch, _bf16
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if _torch is None:
        import torch
        _torch, _bf16 = torch, torch.bfloat16
    if t.dtype is not _bf16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    if shape is not None and t.shape != shape:
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


class Ctx:
    """An skv_ctx* with the library it came from and the arena it lives in."""

    def __init__(self, lib, handle, cfg: dict, arena=None, kind="gpu"):
        self.lib, self.handle, self.cfg, self.arena, self.kind = lib, handle, dict(cfg), arena, kind
        c = self.cfg
        self.G = c["n_q_heads"] // c["n_kv_heads"]
        self.planes = c["n_agents"] if c["mode"] == SKV_BASE_SHARED else 1
        self.Hq, self.Hkv, self.d = c["n_q_heads"], c["n_kv_heads"], c["head_dim"]
        self.hidden, self.r, self.N = c["hidden"], c["rank"], c["n_agents"]
        self.b_shape = (self.N, self.r, self.Hkv * self.d)
        self.a_shape = ((self.N, self.hidden, self.r) if c["mode"] == SKV_BASE_SHARED
                        else (self.hidden, self.r))

    def _check(self, rc):
        if rc != 0:
            raise SkvError(rc, self.lib.skv_last_error(self.handle).decode())

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            self.lib.skv_destroy(h)
            self.handle = None


def _cfg(cfg: dict) -> skv_config:
    c = skv_config()
    defaults = dict(page_size=64, mode=SKV_BASE_SHARED)
    for name, _ in skv_config._fields_:
        setattr(c, name, int(cfg.get(name, defaults.get(name, 0))))
    return c


def skv_arena_bytes(cfg: dict, kind: str = "gpu") -> int:
    return int(load_library(kind).skv_arena_bytes(ctypes.byref(_cfg(cfg))))


def skv_create(cfg: dict, arena, stream=None, kind: str = "gpu") -> Ctx:
    """arena: a torch uint8 GPU tensor, or (address, bytes) for the host build.
    stream: a torch.cuda.Stream, a raw hipStream_t int, or None (current stream)."""
    lib = load_library(kind)
    if isinstance(arena, tuple):
        addr, nbytes = arena
    else:
        addr, nbytes = arena.data_ptr(), arena.numel() * arena.element_size()
    if stream is None and kind == "gpu":
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif stream is not None and not isinstance(stream, int):
        stream = stream.cuda_stream
    h = _P()
    rc = lib.skv_create(ctypes.byref(_cfg(cfg)), addr, nbytes, stream, ctypes.byref(h))
    if rc != 0:
        raise SkvError(rc, "skv_create")
    return Ctx(lib, h, cfg, arena, kind)


def skv_destroy(ctx: Ctx):
    if ctx.handle:
        ctx.lib.skv_destroy(ctx.handle)
        ctx.handle = None


def skv_append_base(ctx: Ctx, layer: int, seq: int, k, v, n: Optional[int] = None):
    c = ctx.cfg
    if n is None:
        n = k.shape[0]
    shp = (n, c["n_kv_heads"], c["head_dim"])
    ctx._check(ctx.lib.skv_append_base(ctx.handle, layer, seq, n, _ptr(k, shape=shp, name="k"),
                                       _ptr(v, shape=shp, name="v")))


def skv_append_lowrank(ctx: Ctx, layer: int, seq: int, plane: int, n: int, x=None, A=None):
    c = ctx.cfg
    ctx._check(ctx.lib.skv_append_lowrank(
        ctx.handle, layer, seq, plane, n, _ptr(x, shape=(n, c["hidden"]), name="x"),
        _ptr(A, shape=(c["hidden"], c["rank"]), name="A")))


def skv_append_agents(ctx: Ctx, layer: int, agents, counts, k, v, x=None, A=None):
    ag, n = _ints(agents)
    cn, _ = _ints(counts)
    tot = sum(cn[:n])
    shp = (tot, ctx.Hkv, ctx.d)
    ctx._check(ctx.lib.skv_append_agents(
        ctx.handle, layer, n, ag, cn, _ptr(k, shp, "k"), _ptr(v, shp, "v"),
        _ptr(x, (tot, ctx.hidden), "x"), _ptr(A, ctx.a_shape, "A")))


def skv_pack_qkv(ctx: Ctx, w_qkv, w_packed):
    shp = ((ctx.Hq + 2 * ctx.Hkv) * ctx.d, ctx.hidden)
    ctx._check(ctx.lib.skv_pack_qkv(ctx.handle, _ptr(w_qkv, shp, "w_qkv"), _ptr(w_packed, None, "w_packed")))


def skv_project_append(ctx: Ctx, layer: int, agents, counts, x, w_packed, A, rope_theta: float, q_out):
    """w_packed: the output of skv_pack_qkv (any shape holding (Hq + 2 Hkv) d hidden elements)."""
    ag, n = _ints(agents)
    cn, _ = _ints(counts)
    tot = sum(cn[:n])
    if w_packed is not None and not isinstance(w_packed, int):
        if w_packed.numel() != (ctx.Hq + 2 * ctx.Hkv) * ctx.d * ctx.hidden:
            raise ValueError("w_packed has the wrong number of elements")
    ctx._check(ctx.lib.skv_project_append(
        ctx.handle, layer, n, ag, cn, _ptr(x, (tot, ctx.hidden), "x"), _ptr(w_packed, None, "w_packed"),
        _ptr(A, ctx.a_shape, "A"), float(rope_theta), _ptr(q_out, (tot, ctx.Hq, ctx.d), "q_out")))


def skv_attn_prefill(ctx: Ctx, layer: int, agents, base_len, suffix_len, n_q, q, B, o):
    ag, n = _ints(agents)
    bl, _ = _ints(base_len)
    sl, _ = _ints(suffix_len)
    nq, _ = _ints(n_q)
    qs = (sum(nq[:n]), ctx.Hq, ctx.d)
    ctx._check(ctx.lib.skv_attn_prefill(ctx.handle, layer, n, ag, bl, sl, nq, _ptr(q, qs, "q"),
                                        _ptr(B, ctx.b_shape, "B"), _ptr(o, qs, "o")))


def skv_attn_decode(ctx: Ctx, layer: int, agents, base_len, suffix_len, q, B, o):
    ag, n = _ints(agents)
    bl, _ = _ints(base_len)
    sl, _ = _ints(suffix_len)
    qs = (n, ctx.Hq, ctx.d)
    ctx._check(ctx.lib.skv_attn_decode(ctx.handle, layer, n, ag, bl, sl, _ptr(q, qs, "q"),
                                       _ptr(B, ctx.b_shape, "B"), _ptr(o, qs, "o")))


def skv_decode_step(ctx: Ctx, layer: int, agents, base_len, suffix_len, k, v, x, A, q, B, o):
    ag, n = _ints(agents)
    bl, _ = _ints(base_len)
    sl, _ = _ints(suffix_len)
    kv = (n, ctx.Hkv, ctx.d)
    qs = (n, ctx.Hq, ctx.d)
    ctx._check(ctx.lib.skv_decode_step(
        ctx.handle, layer, n, ag, bl, sl, _ptr(k, kv, "k"), _ptr(v, kv, "v"),
        _ptr(x, (n, ctx.hidden), "x"), _ptr(A, ctx.a_shape, "A"), _ptr(q, qs, "q"),
        _ptr(B, ctx.b_shape, "B"), _ptr(o, qs, "o")))


def skv_decode_step_static(ctx: Ctx, layer: int, agents, base_len, suffix_len, k, v, x, A, q, B, o):
    """skv_decode_step with the partial rows in the library's static device scratch."""
    ag, n = _ints(agents)
    bl, _ = _ints(base_len)
    sl, _ = _ints(suffix_len)
    kv = (n, ctx.Hkv, ctx.d)
    qs = (n, ctx.Hq, ctx.d)
    ctx._check(ctx.lib.skv_decode_step_static(
        ctx.handle, layer, n, ag, bl, sl, _ptr(k, kv, "k"), _ptr(v, kv, "v"),
        _ptr(x, (n, ctx.hidden), "x"), _ptr(A, ctx.a_shape, "A"), _ptr(q, qs, "q"),
        _ptr(B, ctx.b_shape, "B"), _ptr(o, qs, "o")))


def skv_crop(ctx: Ctx, seq: int, new_len: int):
    ctx._check(ctx.lib.skv_crop(ctx.handle, seq, new_len))


def skv_set_lr_begin(ctx: Ctx, agent: int, pos: int):
    ctx._check(ctx.lib.skv_set_lr_begin(ctx.handle, agent, pos))


def skv_get_lens(ctx: Ctx, layer: int) -> dict:
    N, planes = ctx.cfg["n_agents"], ctx.planes
    P = ctypes.c_int()
    b = (ctypes.c_int * N)()
    S = (ctypes.c_int * N)()
    ls = (ctypes.c_int * planes)()
    lo = (ctypes.c_int * N)()
    ctx._check(ctx.lib.skv_get_lens(ctx.handle, layer, ctypes.byref(P), b, S, ls, lo))
    return dict(P=P.value, b=list(b), S=list(S), lr_shared=list(ls), lr_own=list(lo))


def skv_get_pages(ctx: Ctx, layer: int, seq: int) -> list:
    n = ctx.lib.skv_get_pages(ctx.handle, layer, seq, None, 0)
    if n < 0:
        raise SkvError(n, "skv_get_pages")
    buf = (ctypes.c_int32 * max(1, n))()
    ctx.lib.skv_get_pages(ctx.handle, layer, seq, buf, n)
    return list(buf)[:n]


def skv_get_pools(ctx: Ctx) -> dict:
    p = skv_pools()
    ctx._check(ctx.lib.skv_get_pools(ctx.handle, ctypes.byref(p)))
    return {name: getattr(p, name) for name, _ in skv_pools._fields_}


def skv_get_counters(ctx: Ctx) -> dict:
    p = skv_counters()
    ctx._check(ctx.lib.skv_get_counters(ctx.handle, ctypes.byref(p)))
    return {name: getattr(p, name) for name, _ in skv_counters._fields_}


def skv_set_timing(ctx: Ctx, enable, kinds=None):
    """Record HIP events around launches of the given kernel kinds (names from
    KERNEL_KINDS; default all) while enabled."""
    mask = 0
    if enable:
        kinds = KERNEL_KINDS if kinds is None else kinds
        for k in kinds:
            mask |= 1 << KERNEL_KINDS.index(k)
    ctx._check(ctx.lib.skv_set_timing(ctx.handle, mask))


def skv_collect_timing(ctx: Ctx) -> dict:
    t = skv_kernel_times()
    ctx._check(ctx.lib.skv_collect_timing(ctx.handle, ctypes.byref(t)))
    return {k: (t.ms[i], t.launches[i]) for i, k in enumerate(KERNEL_KINDS)}


def skv_sync(ctx: Ctx):
    ctx._check(ctx.lib.skv_sync(ctx.handle))


def skv_last_error(ctx: Ctx) -> str:
    return ctx.lib.skv_last_error(ctx.handle).decode()


def _stream_handle(stream):
    """hipStream_t of a torch.cuda.Stream, a raw int, or None (torch's current stream)."""
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)


def skv_probe_stream_read(buf, reps: int = 5, stream=None) -> float:
    """Streaming-read bandwidth (GB/s) over a device buffer (a CUDA tensor)."""
    lib = load_library("gpu")
    out = ctypes.c_double()
    nbytes = buf.numel() * buf.element_size()
    rc = lib.skv_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes - nbytes % 16, int(reps),
                                   _stream_handle(stream), ctypes.byref(out))
    if rc != 0:
        raise RuntimeError(f"skv_probe_stream_read failed: {_CODES.get(rc, rc)}")
    return out.value


def skv_probe_mfma_bf16(stream=None) -> float:
    """Dense bf16 MFMA rate (TFLOP/s) of a back-to-back issue loop."""
    lib = load_library("gpu")
    out = ctypes.c_double()
    rc = lib.skv_probe_mfma_bf16(_stream_handle(stream), ctypes.byref(out))
    if rc != 0:
        raise RuntimeError(f"skv_probe_mfma_bf16 failed: {_CODES.get(rc, rc)}")
    return out.value


def skv_probe_mfma_bf16_data(buf, stream=None, kind: str = "gpu") -> float:
    """Dense bf16 MFMA rate (TFLOP/s) of the issue loop on operand data taken
    from a device buffer (a CUDA tensor of at least 16 KiB, or a raw address
    with kind="host" for argument checks)."""
    lib = load_library(kind)
    if isinstance(buf, int):
        addr, nbytes = buf, 16 << 10
    else:
        addr, nbytes = buf.data_ptr(), buf.numel() * buf.element_size()
    out = ctypes.c_double()
    rc = lib.skv_probe_mfma_bf16_data(ctypes.c_void_p(addr), int(nbytes),
                                      _stream_handle(stream) if kind == "gpu" else None, ctypes.byref(out))
    if rc != 0:
        raise SkvError(rc, "skv_probe_mfma_bf16_data failed")
    return out.value


def skv_probe_launch_pattern(buf, layer_bytes: int, layers: int, steps: int = 20, tail_blocks: int = 128,
                             stream=None, kind: str = "gpu"):
    """(ms per step with a small dependent launch after every layer's streaming
    read, ms per step of the streaming reads alone) over `layers` consecutive
    layer_bytes slices of a device buffer (a CUDA tensor, or a raw address
    with kind="host" for argument checks)."""
    lib = load_library(kind)
    if isinstance(buf, int):
        addr, nbytes = buf, layer_bytes * layers
    else:
        addr, nbytes = buf.data_ptr(), buf.numel() * buf.element_size()
    if layer_bytes * layers > nbytes:
        raise SkvError(-1, "buffer smaller than layers * layer_bytes")
    pat, st = ctypes.c_double(), ctypes.c_double()
    rc = lib.skv_probe_launch_pattern(ctypes.c_void_p(addr), int(layer_bytes), int(layers), int(steps),
                                      int(tail_blocks), _stream_handle(stream) if kind == "gpu" else None,
                                      ctypes.byref(pat), ctypes.byref(st))
    if rc != 0:
        raise SkvError(rc, "skv_probe_launch_pattern failed")
    return pat.value, st.value
