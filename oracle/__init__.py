"""CPU oracle of the routed MoE layer (numpy front end of ``oracle.c``).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package. The product path
(``mixture_experts_routed_amd``) never imports it, and the two share no code.

Every function returns plain numpy arrays. Floating-point element types are
passed as raw storage: float32 for "f32", uint16 bit patterns for "f16" and
"bf16" (the same storage the synthetic-input module produces).

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (closed forms, a textbook stable sort, brute force,
numpy/torch number formats, a dense SwiGLU MLP in torch fp64, metamorphic
relations and the pages' printed statistics). None is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
# a different build of oracle.c (used only by the mutation test, which plants
# mistakes in a copy of the source to show the pins catch them)
_LIB_OVERRIDE = os.environ.get("MOE_ORACLE_LIB_OVERRIDE")

DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
META_FIELDS = ("nent", "nblk", "nr", "nt", "nactive", "maxcnt", "nskip", "nbad", "tm", "E", "K")


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc (OpenMP over tokens; no fp contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(LIB):
                build()
            L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        for n in ("oracle_f16_to_f64_n", "oracle_bf16_to_f64_n", "oracle_f64_to_f16_n",
                  "oracle_f64_to_bf16_n"):
            getattr(L, n).restype = None
            getattr(L, n).argtypes = [P, P, i64]
        L.oracle_plan.restype = i32
        L.oracle_plan.argtypes = [P, P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P, P]
        L.oracle_gather.restype = None
        L.oracle_gather.argtypes = [P, i32, i64, i32, P, i64, P]
        L.oracle_ffn.restype = i32
        L.oracle_ffn.argtypes = [P, P, P, P, P, P, i32, i64, i32, i32, i32, i32, i32, P, i64, P, i32]
        L.oracle_ffn_entries.restype = i32
        L.oracle_ffn_entries.argtypes = [P, P, P, P, P, P, i32, i64, i32, i32, i32, i32, i32, P, i64,
                                         P, P, i32]
        L.oracle_dense_masked.restype = i32
        L.oracle_dense_masked.argtypes = [P, P, P, P, P, P, i32, i64, i32, i32, i32, i32, i32, P]
        L.oracle_route_topk.restype = i32
        L.oracle_route_topk.argtypes = [P, i64, i32, i32, P, P]
        L.oracle_combine_f32.restype = None
        L.oracle_combine_f32.argtypes = [P, P, i64, i32, i32, P]
        L.oracle_y16_exponent.restype = i32
        L.oracle_y16_exponent.argtypes = [ctypes.c_float]
        for n in ("oracle_y16_encode", "oracle_y16_decode"):
            getattr(L, n).restype = None
        L.oracle_y16_encode.argtypes = [P, i64, i32, P, P]
        L.oracle_y16_decode.argtypes = [P, P, i64, i32, P]
        L.oracle_combine_y16.restype = None
        L.oracle_combine_y16.argtypes = [P, P, P, i64, i32, i32, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.c_void_p)


def nthreads_default() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 1


# ---------------------------------------------------------------- formats --

def f16_to_f64(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().oracle_f16_to_f64_n(_p(h), _p(out), h.size)
    return out


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    out = np.empty(b.shape, np.float64)
    lib().oracle_bf16_to_f64_n(_p(b), _p(out), b.size)
    return out


def f64_to_f16(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f64_to_f16_n(_p(v), _p(out), v.size)
    return out


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f64_to_bf16_n(_p(v), _p(out), v.size)
    return out


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage of the element type -> float64 values."""
    if dtype == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    return f16_to_f64(a) if dtype == "f16" else bf16_to_f64(a)


# ------------------------------------------------------------------- plan --

def plan(ids: np.ndarray, w: np.ndarray, E: int, tm: int, B: int = 1024):
    """Counting-sort routing plan. Returns a dict of numpy arrays:
    cnt[E], eoff[E+1], tiles[nt], stok[nr], sw[nr], pos[T*K], meta[11], boff[nblk*E]."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, K = ids.shape
    nent = T * K
    valid = int(((ids >= 0) & (ids < E)).sum())
    max_rows = valid + min(E, max(valid, 0)) * (tm - 1) + tm
    nblk = (nent + B - 1) // B
    cnt = np.empty(E, np.int32)
    eoff = np.empty(E + 1, np.int32)
    tiles = np.empty(max_rows // tm + 1, np.int32)
    stok = np.empty(max_rows, np.int32)
    sw = np.empty(max_rows, np.float32)
    pos = np.empty(nent, np.int32)
    meta = np.empty(11, np.int32)
    boff = np.empty(max(nblk, 1) * E, np.int32)
    rc = lib().oracle_plan(_p(ids), _p(w), T, K, E, tm, B, _p(cnt), _p(eoff), _p(tiles), _p(stok),
                           _p(sw), _p(pos), _p(meta), _p(boff))
    if rc != 0:
        raise ValueError("oracle_plan: bad arguments")
    nr, nt = int(meta[2]), int(meta[3])
    return dict(cnt=cnt, eoff=eoff, tiles=tiles[:nt].copy(), stok=stok[:nr].copy(),
                sw=sw[:nr].copy(), pos=pos, meta=meta, boff=boff[: nblk * E].copy())


def meta_dict(meta: np.ndarray) -> dict:
    return {k: int(v) for k, v in zip(META_FIELDS, meta)}


# ----------------------------------------------------------------- gather --

def gather(x: np.ndarray, stok: np.ndarray) -> np.ndarray:
    """XS[r] = x[stok[r]] bit for bit; all-zero bits where stok[r] < 0."""
    x = np.ascontiguousarray(x)
    stok = np.ascontiguousarray(stok, dtype=np.int32)
    T, d = x.shape
    xs = np.empty((len(stok), d), dtype=x.dtype)
    lib().oracle_gather(_p(x), x.itemsize, T, d, _p(stok), len(stok), _p(xs))
    return xs


# -------------------------------------------------------------------- ffn --

def ffn(x, ids, w, wg, wu, wd, dtype: str, round_h: bool, tokens=None, nthreads=None):
    """Layer output in float64 for the listed tokens (all by default): [len(tokens), d]."""
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, d = x.shape
    K = ids.shape[1]
    E, _, f = wg.shape
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, np.int32)
    out = np.empty((len(tok), d), np.float64)
    rc = lib().oracle_ffn(_p(x), _p(ids), _p(w), _p(wg), _p(wu), _p(wd), DTYPE_CODE[dtype], T, K, E,
                          d, f, int(round_h), _p(tok), len(tok), _p(out),
                          nthreads or nthreads_default())
    if rc != 0:
        raise RuntimeError("oracle_ffn failed")
    return out


def ffn_entries(x, ids, w, wg, wu, wd, dtype: str, round_h: bool, entries, nthreads=None):
    """Per-entry weighted expert output y [n, d] and the down-projection input h [n, f]."""
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, d = x.shape
    K = ids.shape[1]
    E, _, f = wg.shape
    ent = np.ascontiguousarray(entries, np.int32)
    y = np.empty((len(ent), d), np.float64)
    h = np.empty((len(ent), f), np.float64)
    rc = lib().oracle_ffn_entries(_p(x), _p(ids), _p(w), _p(wg), _p(wu), _p(wd), DTYPE_CODE[dtype], T,
                                  K, E, d, f, int(round_h), _p(ent), len(ent), _p(y), _p(h),
                                  nthreads or nthreads_default())
    if rc != 0:
        raise RuntimeError("oracle_ffn_entries failed")
    return y, h


def dense_masked(x, ids, w, wg, wu, wd, dtype: str, round_h: bool):
    """Every expert on every token, masked by the router's choice (tiny inputs only)."""
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, d = x.shape
    K = ids.shape[1]
    E, _, f = wg.shape
    out = np.empty((T, d), np.float64)
    rc = lib().oracle_dense_masked(_p(x), _p(ids), _p(w), _p(wg), _p(wu), _p(wd), DTYPE_CODE[dtype],
                                   T, K, E, d, f, int(round_h), _p(out))
    if rc != 0:
        raise RuntimeError("oracle_dense_masked failed")
    return out


# ---------------------------------------------------------------- combine --

def combine_f32(Y: np.ndarray, pos: np.ndarray, T: int, K: int) -> np.ndarray:
    """out[t] = fp32 sum of Y[pos[t*K+k]] over k ascending from +0.0f (pos < 0 skipped)."""
    Y = np.ascontiguousarray(Y, dtype=np.float32)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    d = Y.shape[1]
    out = np.empty((T, d), np.float32)
    lib().oracle_combine_f32(_p(Y), _p(pos), T, K, d, _p(out))
    return out


# --------------------------------------------------- compact expert outputs --

Y16_BLOCK = 128  # columns per exponent


def y16_exponent(M: float) -> int:
    """The exponent e of a block whose largest magnitude is M (see oracle.c)."""
    return int(lib().oracle_y16_exponent(float(M)))


def y16_encode(y: np.ndarray):
    """fp32 rows [n, d] -> (binary16 bit patterns uint16 [n, d], exponents int8 [n, nb])."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    n, d = y.shape
    s = np.empty((n, d), np.uint16)
    e = np.empty((n, (d + Y16_BLOCK - 1) // Y16_BLOCK), np.int8)
    lib().oracle_y16_encode(_p(y), n, d, _p(s), _p(e))
    return s, e


def y16_decode(s: np.ndarray, e: np.ndarray) -> np.ndarray:
    """Exact fp32 values s * 2^-e of compact rows."""
    s = np.ascontiguousarray(s, dtype=np.uint16)
    e = np.ascontiguousarray(e, dtype=np.int8)
    n, d = s.shape
    y = np.empty((n, d), np.float32)
    lib().oracle_y16_decode(_p(s), _p(e), n, d, _p(y))
    return y


def combine_y16(s: np.ndarray, e: np.ndarray, pos: np.ndarray, T: int, K: int) -> np.ndarray:
    """out[t] = fp32 sum over k ascending from +0.0f of the decoded compact rows pos[t*K+k]."""
    s = np.ascontiguousarray(s, dtype=np.uint16)
    e = np.ascontiguousarray(e, dtype=np.int8)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    d = s.shape[1]
    out = np.empty((T, d), np.float32)
    lib().oracle_combine_y16(_p(s), _p(e), _p(pos), T, K, d, _p(out))
    return out


# ----------------------------------------------------------------- router --

def route_topk(logits: np.ndarray, K: int):
    """ids int32 [T, K] (descending logit, ties to the lower id, NaN never picked, -1 if
    fewer than K finite picks) and renormalised softmax weights float64 [T, K]."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    ids = np.empty((T, K), np.int32)
    w = np.empty((T, K), np.float64)
    if lib().oracle_route_topk(_p(logits), T, E, K, _p(ids), _p(w)) != 0:
        raise ValueError("oracle_route_topk: bad arguments")
    return ids, w
