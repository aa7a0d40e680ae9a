"""Pins for the oracle's gather (bit copy) and fp32 fixed-order combine."""
import numpy as np

import oracle
from mixture_experts_routed_amd import synth


def test_gather_bitwise_against_entries():
    cfg = synth.CONFIGS["tiny_fp32"]
    ids, w = synth.routing(cfg)
    x = synth.activations(cfg)
    p = oracle.plan(ids, w, cfg.E, cfg.tm)
    xs = oracle.gather(x, p["stok"])
    flat = ids.reshape(-1)
    for i in range(len(flat)):
        assert np.array_equal(xs[p["pos"][i]].view(np.uint32), x[i // cfg.K].view(np.uint32))
    pad = p["stok"] < 0
    assert pad.any() and np.all(xs[pad].view(np.uint32) == 0)


def test_gather_equals_fancy_indexing_u16():
    g = np.random.default_rng(2)
    x = g.integers(0, 65536, size=(50, 24)).astype(np.uint16)
    stok = g.integers(-1, 50, size=300).astype(np.int32)
    ref = x[np.maximum(stok, 0)].copy()
    ref[stok < 0] = 0
    assert np.array_equal(oracle.gather(x, stok), ref)


def test_combine_order_matters_cancellation():
    # rows: 1e8, 1, -1e8 ; fp32 summed in k order: (0 + 1e8) + 1 = 1e8 ; - 1e8 = 0
    Y = np.array([[1e8], [1.0], [-1e8]], np.float32)
    out = oracle.combine_f32(Y, np.array([0, 1, 2], np.int32), 1, 3)
    assert out[0, 0] == 0.0
    # another order gives 1 -- so the test can see a reordering
    out = oracle.combine_f32(Y, np.array([0, 2, 1], np.int32), 1, 3)
    assert out[0, 0] == 1.0


def test_combine_exact_on_integers_and_skips():
    g = np.random.default_rng(4)
    T, K, d, nr = 30, 5, 12, 200
    Y = g.integers(-1000, 1000, size=(nr, d)).astype(np.float32)  # sums exact in fp32
    pos = g.integers(-1, nr, size=T * K).astype(np.int32)
    out = oracle.combine_f32(Y, pos, T, K)
    ref = np.zeros((T, d), np.int64)
    for i, r in enumerate(pos):
        if r >= 0:
            ref[i // K] += Y[r].astype(np.int64)
    assert np.array_equal(out.astype(np.int64), ref)


def test_combine_k1_is_a_copy_and_zero_is_positive():
    Y = np.array([[-0.0, 2.5], [7.0, -3.0]], np.float32)
    out = oracle.combine_f32(Y, np.array([1, 0], np.int32), 2, 1)
    assert np.array_equal(out, Y[[1, 0]] + np.float32(0.0))
    assert not np.signbit(out[1, 0])  # +0.0f + -0.0f = +0.0f
    out = oracle.combine_f32(Y, np.array([-1, -1], np.int32), 2, 1)
    assert np.all(out == 0) and not np.any(np.signbit(out))
