"""ctypes binding of libmoe_routed.so (the C ABI in include/moe_routed.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch supplies device memory and the stream. The functions named
like the C entry points take torch tensors (and plain ints) in the C order
and raise MoeError on a non-OK status; the short-named helpers below them
allocate outputs with torch and call those.

There is no fallback: if the library is missing or no GPU tensor is given,
the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# a different build of the same sources may be named here (the tests load a
# build whose host code carries AddressSanitizer this way)
LIB_PATH = os.environ.get("MOE_ROUTED_LIB_OVERRIDE") or os.path.join(HERE, "libmoe_routed.so")

MOE_F32, MOE_F16, MOE_BF16 = 0, 1, 2
MOE_W_GATE_UP, MOE_W_DOWN = 0, 1
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP runtime error",
          4: "larger than the allocation-free call's fixed buffer"}
NOALLOC_WORKSPACE_BYTES = 64 << 20  # MOE_NOALLOC_WORKSPACE_BYTES
META_FIELDS = ("nent", "nblk", "nr", "nt", "nactive", "maxcnt", "nskip", "nbad", "tm", "E", "K")
META_N = 11
STAGES = ("hist", "scan", "place", "gather", "worklist", "gateup", "down", "combine")
TORCH_DTYPE = {MOE_F32: torch.float32, MOE_F16: torch.float16, MOE_BF16: torch.bfloat16}
DTYPE_OF = {torch.float32: MOE_F32, torch.float16: MOE_F16, torch.bfloat16: MOE_BF16}
DTYPE_NAME = {"f32": MOE_F32, "f16": MOE_F16, "bf16": MOE_BF16}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {STATUS.get(status, status)} (status {status})")
        self.status = status


class PlanSizes(ctypes.Structure):
    _fields_ = [("nent", ctypes.c_int64), ("nblk", ctypes.c_int64), ("max_rows", ctypes.c_int64),
                ("max_tiles", ctypes.c_int64), ("scratch_bytes", ctypes.c_size_t)]


class ForwardLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("cnt", "eoff", "tiles", "stok", "sw", "pos", "boff", "meta", "plan_scratch", "xs",
                 "h", "y", "ffn_scratch", "total")]


_lib = None
P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t

_SIGS = {
    "moe_route_topk": [P, I32, I32, I32, P, P, P],
    "moe_plan_sizes": [I32, I32, I32, I32, ctypes.POINTER(PlanSizes)],
    "moe_plan": [P, P, I32, I32, I32, I32, P, P, P, P, P, P, P, P, P, SZ, P],
    "moe_gather": [P, I32, I32, I32, P, P, I64, P, P],
    "moe_ffn_scratch_bytes": [I32, I32, I32, I32, I64, I32, ctypes.POINTER(ctypes.c_size_t)],
    "moe_ffn_splits": [I32, I32, I32, I32, I64, I32, ctypes.POINTER(ctypes.c_int),
                       ctypes.POINTER(ctypes.c_int)],
    "moe_ffn_big_cells": [I32, I32, I32, I32, I64, I32, ctypes.POINTER(ctypes.c_int)],
    "moe_expert_ffn": [P, P, P, P, I32, I32, I32, I32, I32, P, P, P, P, I64, P, P, P, SZ, P],
    "moe_combine": [P, I64, P, I32, I32, I32, P, P],
    "moe_forward_workspace": [I32, I32, I32, I32, I32, I32, I32, ctypes.POINTER(ctypes.c_size_t)],
    "moe_forward_layout": [I32, I32, I32, I32, I32, I32, I32, ctypes.POINTER(ForwardLayout)],
    "moe_forward": [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, P, SZ, P, P],
    "moe_forward_timed": [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, P, SZ, P, P, P],
    "moe_timer_create": [ctypes.POINTER(P), I32, ctypes.c_uint],
    "moe_timer_destroy": [P],
    "moe_timer_read": [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)],
    "moe_packed_weight_bytes": [I32, I32, I32, I32, I32, ctypes.POINTER(ctypes.c_size_t)],
    "moe_pack_weights": [P, I32, I32, I32, I32, I32, P, SZ, P],
    "moe_expert_ffn_packed": [P, P, P, P, I32, I32, I32, I32, I32, P, P, P, P, I64, P, P, P, SZ,
                              P],
    "moe_forward_packed": [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, P, SZ, P, P],
    "moe_host_cache_bytes": [I32, I32, I32, I32, I32, I32, I32, I32,
                             ctypes.POINTER(ctypes.c_size_t)],
    "moe_host_cache_init": [P, SZ, I32, I32, I32, I32, I32, I32, P],
    "moe_forward_host_weights": [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, I32, P,
                                 SZ, P, SZ, P, P],
    "moe_forward_packed_timed": [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, P, SZ, P, P,
                                 P],
    "moe_forward_packed_noalloc": [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, P, P],
}

EXPORTS = tuple(_SIGS) + ("moe_status_str",)


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeError("load", 3) from FileNotFoundError(
                f"{LIB_PATH} is missing: build it with mixture_experts_routed_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = I32
        L.moe_status_str.argtypes = [I32]
        L.moe_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise MoeError(fn, rc)


def _dev(t, name):
    """device address of a CUDA tensor (or None)"""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


def _host(t, name):
    """address of a host tensor (the library checks that it is pinned)"""
    if not isinstance(t, torch.Tensor) or t.is_cuda:
        raise TypeError(f"{name}: expected a host tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


# --------------------------------------------------------- host-only sizes --

def moe_plan_sizes(T: int, K: int, E: int, tm: int) -> PlanSizes:
    z = PlanSizes()
    _check("moe_plan_sizes", lib().moe_plan_sizes(T, K, E, tm, ctypes.byref(z)))
    return z


def moe_ffn_scratch_bytes(E: int, d: int, f: int, tm: int, max_rows: int, dtype: int) -> int:
    v = ctypes.c_size_t()
    _check("moe_ffn_scratch_bytes",
           lib().moe_ffn_scratch_bytes(E, d, f, tm, max_rows, dtype, ctypes.byref(v)))
    return v.value


def moe_ffn_splits(E: int, d: int, f: int, tm: int, max_rows: int, dtype: int):
    """(gate/up splits, down splits) of the reduction for these sizes."""
    a, b = ctypes.c_int(), ctypes.c_int()
    _check("moe_ffn_splits",
           lib().moe_ffn_splits(E, d, f, tm, max_rows, dtype, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def moe_ffn_big_cells(E: int, d: int, f: int, tm: int, max_rows: int, dtype: int) -> int:
    """which packed 16-bit projections run their runs of 4 items on the 8-wavefront
    kernel: bit 0 gate/up, bit 1 down"""
    on = ctypes.c_int()
    _check("moe_ffn_big_cells",
           lib().moe_ffn_big_cells(E, d, f, tm, max_rows, dtype, ctypes.byref(on)))
    return on.value


def moe_forward_workspace(T, K, E, d, f, tm, dtype: int) -> int:
    v = ctypes.c_size_t()
    _check("moe_forward_workspace", lib().moe_forward_workspace(T, K, E, d, f, tm, dtype,
                                                                ctypes.byref(v)))
    return v.value


def moe_forward_layout(T, K, E, d, f, tm, dtype: int) -> ForwardLayout:
    L = ForwardLayout()
    _check("moe_forward_layout", lib().moe_forward_layout(T, K, E, d, f, tm, dtype, ctypes.byref(L)))
    return L


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


# ------------------------------------------------ entry points (same names) --

def moe_route_topk(logits, T, E, K, ids, w, stream=None):
    _check("moe_route_topk", lib().moe_route_topk(_dev(logits, "logits"), T, E, K, _dev(ids, "ids"),
                                                  _dev(w, "w"), _stream(stream)))


def moe_plan(ids, w, T, K, E, tm, cnt, eoff, tiles, stok, sw, pos, boff, meta, scratch,
             stream=None):
    _check("moe_plan", lib().moe_plan(
        _dev(ids, "ids"), _dev(w, "w"), T, K, E, tm, _dev(cnt, "cnt"), _dev(eoff, "eoff"),
        _dev(tiles, "tiles"), _dev(stok, "stok"), _dev(sw, "sw"), _dev(pos, "pos"),
        _dev(boff, "boff"), _dev(meta, "meta"), _dev(scratch, "scratch"),
        scratch.numel() * scratch.element_size(), _stream(stream)))


def moe_gather(x, dtype, T, d, stok, meta, max_rows, xs, stream=None):
    _check("moe_gather", lib().moe_gather(_dev(x, "x"), dtype, T, d, _dev(stok, "stok"),
                                          _dev(meta, "meta"), max_rows, _dev(xs, "xs"),
                                          _stream(stream)))


def moe_packed_weight_bytes(E: int, d: int, f: int, dtype: int, kind: int) -> int:
    v = ctypes.c_size_t()
    _check("moe_packed_weight_bytes",
           lib().moe_packed_weight_bytes(E, d, f, dtype, kind, ctypes.byref(v)))
    return v.value


def moe_pack_weights(w, kind: int, packed=None, stream=None):
    """Pack one set of expert matrices (W_gate/W_up [E, d, f] with kind
    MOE_W_GATE_UP, W_down [E, f, d] with MOE_W_DOWN); returns the packed bytes."""
    E = w.shape[0]
    d, f = (w.shape[1], w.shape[2]) if kind == MOE_W_GATE_UP else (w.shape[2], w.shape[1])
    dtype = DTYPE_OF[w.dtype]
    need = moe_packed_weight_bytes(E, d, f, dtype, kind)
    if packed is None:
        packed = torch.empty(need, dtype=torch.uint8, device=w.device)
    _check("moe_pack_weights", lib().moe_pack_weights(
        _dev(w, "w"), dtype, E, d, f, kind, _dev(packed, "packed"),
        packed.numel() * packed.element_size(), _stream(stream)))
    return packed


def pack(w_gate, w_up, w_down, stream=None) -> dict:
    """The three packed matrix sets of a layer, keyed gate / up / down."""
    return {"gate": moe_pack_weights(w_gate, MOE_W_GATE_UP, stream=stream),
            "up": moe_pack_weights(w_up, MOE_W_GATE_UP, stream=stream),
            "down": moe_pack_weights(w_down, MOE_W_DOWN, stream=stream)}


def moe_expert_ffn_packed(xs, pw_gate, pw_up, pw_down, dtype, E, d, f, tm, eoff, stok, sw, meta,
                          max_rows, h, y, scratch, stream=None):
    _check("moe_expert_ffn_packed", lib().moe_expert_ffn_packed(
        _dev(xs, "xs"), _dev(pw_gate, "pw_gate"), _dev(pw_up, "pw_up"), _dev(pw_down, "pw_down"),
        dtype, E, d, f, tm, _dev(eoff, "eoff"), _dev(stok, "stok"), _dev(sw, "sw"),
        _dev(meta, "meta"), max_rows, _dev(h, "h"), _dev(y, "y"), _dev(scratch, "scratch"),
        scratch.numel() * scratch.element_size(), _stream(stream)))


def moe_expert_ffn(xs, w_gate, w_up, w_down, dtype, E, d, f, tm, eoff, stok, sw, meta, max_rows,
                   h, y, scratch, stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        _dev(xs, "xs"), _dev(w_gate, "w_gate"), _dev(w_up, "w_up"), _dev(w_down, "w_down"), dtype,
        E, d, f, tm, _dev(eoff, "eoff"), _dev(stok, "stok"), _dev(sw, "sw"), _dev(meta, "meta"),
        max_rows, _dev(h, "h"), _dev(y, "y"), _dev(scratch, "scratch"),
        scratch.numel() * scratch.element_size(), _stream(stream)))


def moe_combine(y, max_rows, pos, T, K, d, out, stream=None):
    _check("moe_combine", lib().moe_combine(_dev(y, "y"), max_rows, _dev(pos, "pos"), T, K, d,
                                            _dev(out, "out"), _stream(stream)))


def moe_forward(x, ids, w, w_gate, w_up, w_down, dtype, T, K, E, d, f, tm, workspace, out,
                stream=None, timer=None, packed: bool = False):
    """packed=True: w_gate / w_up / w_down are packed matrix sets (moe_pack_weights)."""
    args = (_dev(x, "x"), _dev(ids, "ids"), _dev(w, "w"), _dev(w_gate, "w_gate"),
            _dev(w_up, "w_up"), _dev(w_down, "w_down"), dtype, T, K, E, d, f, tm,
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _dev(out, "out"), _stream(stream))
    name = "moe_forward_packed" if packed else "moe_forward"
    if timer is None:
        _check(name, getattr(lib(), name)(*args))
    else:
        _check(name + "_timed", getattr(lib(), name + "_timed")(*args, timer.handle))


def moe_forward_packed_noalloc(x, ids, w, pw_gate, pw_up, pw_down, dtype, T, K, E, d, f, tm, out,
                               stream=None):
    """moe_forward_packed with the library's fixed workspace (no workspace argument)."""
    _check("moe_forward_packed_noalloc", lib().moe_forward_packed_noalloc(
        _dev(x, "x"), _dev(ids, "ids"), _dev(w, "w"), _dev(pw_gate, "pw_gate"),
        _dev(pw_up, "pw_up"), _dev(pw_down, "pw_down"), dtype, T, K, E, d, f, tm,
        _dev(out, "out"), _stream(stream)))


def moe_host_cache_bytes(T: int, K: int, E: int, d: int, f: int, dtype: int, packed: bool,
                         slots: int = 0) -> int:
    n = ctypes.c_size_t()
    _check("moe_host_cache_bytes", lib().moe_host_cache_bytes(T, K, E, d, f, dtype, int(packed),
                                                              slots, ctypes.byref(n)))
    return n.value


def moe_host_cache_init(cache, E, d, f, dtype, packed: bool, slots: int, stream=None):
    _check("moe_host_cache_init", lib().moe_host_cache_init(
        _dev(cache, "cache"), cache.numel() * cache.element_size(), E, d, f, dtype, int(packed),
        slots, _stream(stream)))


def moe_forward_host_weights(x, ids, w, hw_gate, hw_up, hw_down, packed: bool, dtype, T, K, E, d,
                             f, tm, slots, cache, workspace, out, stream=None):
    """moe_forward / moe_forward_packed with the expert weights in pinned host tensors."""
    _check("moe_forward_host_weights", lib().moe_forward_host_weights(
        _dev(x, "x"), _dev(ids, "ids"), _dev(w, "w"), _host(hw_gate, "hw_gate"),
        _host(hw_up, "hw_up"), _host(hw_down, "hw_down"), int(packed), dtype, T, K, E, d, f, tm,
        slots, _dev(cache, "cache"), cache.numel() * cache.element_size(),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _dev(out, "out"), _stream(stream)))


class Timer:
    """Per-kernel HIP-event timer of moe_forward_timed."""

    def __init__(self, capacity: int = 256, stages=STAGES):
        h = ctypes.c_void_p()
        mask = 0
        for s in stages:
            mask |= 1 << STAGES.index(s)
        _check("moe_timer_create", lib().moe_timer_create(ctypes.byref(h), capacity, mask))
        self.handle = h
        self.total_ms = (ctypes.c_double * len(STAGES))()
        self.launches = (ctypes.c_int64 * len(STAGES))()

    def read(self) -> dict:
        """Wait for the recorded events and accumulate; returns {stage: (ms_total, launches)}."""
        _check("moe_timer_read", lib().moe_timer_read(self.handle, self.total_ms, self.launches))
        return {s: (self.total_ms[i], self.launches[i]) for i, s in enumerate(STAGES)}

    def reset(self):
        for i in range(len(STAGES)):
            self.total_ms[i] = 0.0
            self.launches[i] = 0

    def close(self):
        if self.handle:
            lib().moe_timer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------ allocating helpers --

def _empty(n, dtype, device):
    return torch.empty(int(max(n, 1)), dtype=dtype, device=device)


def route(logits, K: int, stream=None):
    """Router on GPU logits [T, E] fp32: returns (ids [T, K] int32, w [T, K] fp32)."""
    T, E = logits.shape
    ids = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    moe_route_topk(logits, T, E, K, ids, w, stream)
    return ids, w


def plan(ids, w, E: int, tm: int = 16, stream=None) -> dict:
    """Run moe_plan on ids/w ([T, K] int32 / fp32 GPU tensors); returns the outputs."""
    T, K = ids.shape
    z = moe_plan_sizes(T, K, E, tm)
    dev = ids.device
    o = dict(cnt=_empty(E, torch.int32, dev), eoff=_empty(E + 1, torch.int32, dev),
             tiles=_empty(z.max_tiles, torch.int32, dev), stok=_empty(z.max_rows, torch.int32, dev),
             sw=_empty(z.max_rows, torch.float32, dev), pos=_empty(T * K, torch.int32, dev),
             boff=_empty(z.nblk * E, torch.int32, dev), meta=_empty(META_N, torch.int32, dev),
             scratch=_empty(z.scratch_bytes, torch.uint8, dev))
    moe_plan(ids, w, T, K, E, tm, o["cnt"], o["eoff"], o["tiles"], o["stok"], o["sw"], o["pos"],
             o["boff"], o["meta"], o["scratch"], stream)
    o["sizes"] = z
    return o


def forward(x, ids, w, w_gate, w_up, w_down, tm: int = 16, workspace=None, out=None, stream=None,
            timer=None, packed=None):
    """One routed MoE layer on GPU tensors; returns (out [T, d] fp32, workspace).
    packed: optional dict of packed matrix sets (see pack()); the layer then reads
    those instead of w_gate / w_up / w_down, which still give the shapes."""
    T, d = x.shape
    K = ids.shape[1]
    E, _, f = w_gate.shape
    dtype = DTYPE_OF[x.dtype]
    need = moe_forward_workspace(T, K, E, d, f, tm, dtype)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=x.device)
    if packed is not None:
        moe_forward(x, ids, w, packed["gate"], packed["up"], packed["down"], dtype, T, K, E, d, f,
                    tm, workspace, out, stream, timer, packed=True)
    else:
        moe_forward(x, ids, w, w_gate, w_up, w_down, dtype, T, K, E, d, f, tm, workspace, out,
                    stream, timer)
    return out, workspace


def forward_host(x, ids, w, hw_gate, hw_up, hw_down, tm: int = 16, packed: bool = False,
                 shapes=None, slots: int = 0, cache=None, workspace=None, out=None, stream=None):
    """One routed MoE layer whose expert weights are pinned host tensors (row-major
    [E, d, f] / [E, f, d], or packed arrays with shapes=(E, d, f)), through a device
    cache of `slots` experts (0: the fewest for T tokens); a new cache is made and
    cleared here, a given one must have been made for the same sizes and slots.
    Returns (out, cache, workspace)."""
    T, d = x.shape
    K = ids.shape[1]
    E, _, f = shapes if shapes is not None else hw_gate.shape
    dtype = DTYPE_OF[x.dtype]
    slots = slots or min(E, T * K)
    need = moe_forward_workspace(T, K, E, d, f, tm, dtype)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if cache is None:
        cache = torch.empty(moe_host_cache_bytes(T, K, E, d, f, dtype, packed, slots),
                            dtype=torch.uint8, device=x.device)
        moe_host_cache_init(cache, E, d, f, dtype, packed, slots, stream)
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=x.device)
    moe_forward_host_weights(x, ids, w, hw_gate, hw_up, hw_down, packed, dtype, T, K, E, d, f, tm,
                             slots, cache, workspace, out, stream)
    return out, cache, workspace
