"""GPU parity of moe_gather (bit copy) and moe_combine (fp32, fixed k order):
both bit-exact against the oracle on the oracle's own plan arrays."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import POLLUTE, abi, dev, host, make_case, polluted, say, synth

pytestmark = pytest.mark.gpu


def gpu_gather(x: np.ndarray, dtype: str, p: dict, max_rows: int):
    T, d = x.shape
    stok = np.full(max_rows, POLLUTE, np.int32)
    stok[: len(p["stok"])] = p["stok"]
    es = synth.ELEM_BYTES[dtype]
    xs = polluted(max_rows * d * es // 4)
    abi.moe_gather(dev(x, dtype), abi.DTYPE_NAME[dtype], T, d, dev(stok), dev(p["meta"]), max_rows,
                   xs)
    torch.cuda.synchronize()
    return host(xs).view(np.uint8).reshape(max_rows, d * es)


@pytest.mark.parametrize("name", ["tiny_fp32", "prefill_fp16", "decode_bf16", "ubatch_bf16",
                                  "long_skewed_fp16"])
def test_gather_bit_exact(name):
    cfg = synth.CONFIGS[name]
    ids, w = synth.routing(cfg)
    x = synth.activations(cfg)
    Tc = cfg.tokens_per_call
    for c in sorted({0, cfg.ncalls - 1}):
        sl = slice(c * Tc, (c + 1) * Tc)
        say(f"[gather] {name} call {c}")
        p = oracle.plan(ids[sl], w[sl], cfg.E, cfg.tm)
        z = abi.moe_plan_sizes(Tc, cfg.K, cfg.E, cfg.tm)
        got = gpu_gather(x[sl], cfg.dtype, p, z.max_rows)
        ref = oracle.gather(x[sl], p["stok"])
        nr = len(p["stok"])
        assert np.array_equal(got[:nr], ref.view(np.uint8).reshape(nr, -1))
        assert np.all(got[nr:].view(np.int32) == POLLUTE)  # rows past nr untouched


def test_gather_odd_width_and_single_row():
    for d, dtype in ((8, "f16"), (24, "bf16"), (4, None), (1000, "f32")):
        if dtype is None:
            continue
        g = np.random.default_rng(d)
        T = 7
        x = synth.to_dtype(g.standard_normal((T, d)).astype(np.float32), dtype)
        ids = g.integers(-1, 3, size=(T, 2)).astype(np.int32)
        w = g.random((T, 2)).astype(np.float32)
        p = oracle.plan(ids, w, 3, 4)
        z = abi.moe_plan_sizes(T, 2, 3, 4)
        say(f"[gather] d={d} {dtype}")
        got = gpu_gather(x, dtype, p, z.max_rows)
        nr = len(p["stok"])
        assert np.array_equal(got[:nr], oracle.gather(x, p["stok"]).view(np.uint8).reshape(nr, -1))


def gpu_combine(Y: np.ndarray, pos: np.ndarray, T: int, K: int):
    d = Y.shape[1]
    out = polluted(T * d, torch.float32)
    abi.moe_combine(dev(Y), Y.shape[0], dev(pos), T, K, d, out)
    torch.cuda.synchronize()
    return host(out).reshape(T, d)


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_combine_bit_exact(name):
    cfg = synth.CONFIGS[name]
    ids, w = synth.routing(cfg)
    Tc = cfg.tokens_per_call
    p = oracle.plan(ids[:Tc], w[:Tc], cfg.E, cfg.tm)
    nr = len(p["stok"])
    Y = synth.random_rows(cfg.seed, nr, cfg.d)  # synthetic expert outputs
    say(f"[combine] {name}")
    got = gpu_combine(Y, p["pos"], Tc, cfg.K)
    ref = oracle.combine_f32(Y, p["pos"], Tc, cfg.K)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_combine_order_cancellation_and_skips():
    d = 16
    Y = np.zeros((4, d), np.float32)
    Y[0], Y[1], Y[2], Y[3] = 1e8, 1.0, -1e8, -0.0
    # token 0: ((1e8 + 1) - 1e8) + -0 = 0 ; token 1: skip, then (1e8 - 1e8) + 1 = 1
    pos = np.array([0, 1, 2, 3, -1, 0, 2, 1], np.int32)
    got = gpu_combine(Y, pos, 2, 4)
    ref = oracle.combine_f32(Y, pos, 2, 4)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert got[0, 0] == 0.0 and not np.signbit(got[0, 0])
    assert got[1, 0] == 1.0


def test_combine_ragged_width():
    g = np.random.default_rng(3)
    for d in (8, 1032, 2056, 4104):  # vectors per row not a multiple of the 256-wide chunk
        T, K, nr = 9, 3, 20
        Y = g.standard_normal((nr, d)).astype(np.float32)
        pos = g.integers(-1, nr, size=T * K).astype(np.int32)
        say(f"[combine] d={d}")
        got = gpu_combine(Y, pos, T, K)
        assert np.array_equal(got.view(np.uint32), oracle.combine_f32(Y, pos, T, K).view(np.uint32))


def random_gc(n=30, seed=5151):
    """seeded random shapes: widths up to 8,192, top-k up to 40 (every group size
    the combine is instantiated for -- 2, 4, 8, 10, 12, 16 -- and more than one
    group of 16), tiles 1-32, skipped ids"""
    g = np.random.default_rng(seed)
    out = []
    for k in range(n):
        E = int(g.choice([1, 3, 16, 64, 300, 1024]))
        K = int(g.choice([1, 2, 4, 7, 10, 12, 16, 17, 33, 40]))
        T = int(g.choice([1, 3, 64, 500, 2049]))
        d = 8 * int(g.integers(1, 1025))
        d = max(8, min(d, (1 << 25) // (T * K) // 8 * 8))  # expert outputs <= 128 MB
        out.append((T, K, E, d, int(g.choice([1, 4, 16, 32])), ("f32", "f16", "bf16")[k % 3],
                    float(g.choice([0.0, 0.2])), 200 + k))
    return out


@pytest.mark.parametrize("T,K,E,d,tm,dtype,ps,seed", random_gc())
def test_gather_combine_random_shapes(T, K, E, d, tm, dtype, ps, seed):
    ids = synth.random_ids(seed, T, K, E, p_skip=ps, p_bad=0.0)
    w = synth.random_rows(seed, T, K)
    g = np.random.default_rng(seed)
    x = synth.to_dtype(g.standard_normal((T, d)).astype(np.float32), dtype)
    p = oracle.plan(ids, w, E, tm)
    z = abi.moe_plan_sizes(T, K, E, tm)
    nr = len(p["stok"])
    say(f"[gather/combine] T={T} K={K} E={E} d={d} tm={tm} {dtype}")
    got = gpu_gather(x, dtype, p, z.max_rows)
    ref = oracle.gather(x, p["stok"]).view(np.uint8).reshape(nr, d * synth.ELEM_BYTES[dtype])
    assert np.array_equal(got[:nr], ref)
    Y = g.standard_normal((max(nr, 1), d)).astype(np.float32)
    out = gpu_combine(Y, p["pos"], T, K)
    assert np.array_equal(out.view(np.uint32), oracle.combine_f32(Y, p["pos"], T, K).view(np.uint32))
