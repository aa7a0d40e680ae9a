"""Pins for the oracle's fp16 / bf16 codecs: exhaustive against numpy's float16
and torch-CPU bfloat16, round trips, ties-to-even and gradual underflow."""
import numpy as np
import torch

import oracle

ALL16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def _same(a, b):
    """equal values, NaN == NaN, and the sign of zero must match"""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


def test_f16_decode_exhaustive_vs_numpy():
    assert _same(oracle.f16_to_f64(ALL16), ALL16.view(np.float16).astype(np.float64))


def test_bf16_decode_exhaustive_vs_torch():
    ref = torch.from_numpy(ALL16.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(oracle.bf16_to_f64(ALL16), ref)


def test_f16_round_trip_exhaustive():
    v = oracle.f16_to_f64(ALL16)
    fin = ~np.isnan(v)
    assert np.array_equal(oracle.f64_to_f16(v[fin]), ALL16[fin])


def test_bf16_round_trip_exhaustive():
    v = oracle.bf16_to_f64(ALL16)
    fin = ~np.isnan(v)
    assert np.array_equal(oracle.f64_to_bf16(v[fin]), ALL16[fin])


def _neighbours_and_midpoints(decoded):
    """finite positive values in order, their midpoints, and points just off the midpoints"""
    v = np.unique(decoded[np.isfinite(decoded) & (decoded >= 0)])
    mid = (v[:-1] + v[1:]) / 2  # exact in double
    return v, mid, np.nextafter(mid, np.inf), np.nextafter(mid, -np.inf)


def test_f16_ties_to_even_and_near_ties_vs_numpy():
    v, mid, up, dn = _neighbours_and_midpoints(oracle.f16_to_f64(ALL16))
    for pts in (mid, up, dn, -mid, -up):
        ref = pts.astype(np.float16).view(np.uint16)  # numpy rounds double -> half correctly
        assert np.array_equal(oracle.f64_to_f16(pts), ref)
    # ties go to the even neighbour: the encoded result of every midpoint is even
    assert np.all(oracle.f64_to_f16(mid) % 2 == 0)


def test_f16_random_doubles_vs_numpy():
    g = np.random.default_rng(0)
    x = g.standard_normal(200000) * np.exp(g.uniform(-20, 12, 200000))
    assert np.array_equal(oracle.f64_to_f16(x), x.astype(np.float16).view(np.uint16))


def test_f16_subnormals_and_overflow():
    assert oracle.f64_to_f16(np.array([2.0 ** -24]))[0] == 0x0001
    assert oracle.f64_to_f16(np.array([2.0 ** -25]))[0] == 0x0000      # tie -> even (zero)
    assert oracle.f64_to_f16(np.array([3 * 2.0 ** -25]))[0] == 0x0002  # tie 1.5 ulp -> 2
    assert oracle.f64_to_f16(np.array([2.0 ** -14 - 2.0 ** -26]))[0] == 0x0400  # rounds up to min normal
    assert oracle.f64_to_f16(np.array([65504.0]))[0] == 0x7BFF
    assert oracle.f64_to_f16(np.array([65519.99]))[0] == 0x7BFF
    assert oracle.f64_to_f16(np.array([65520.0]))[0] == 0x7C00
    assert oracle.f64_to_f16(np.array([-0.0]))[0] == 0x8000


def test_bf16_vs_torch_on_fp32_midpoints():
    # bf16 midpoints are representable in fp32, where torch's float -> bfloat16 is exact RNE
    v, mid, _, _ = _neighbours_and_midpoints(oracle.bf16_to_f64(ALL16))
    mid = mid[mid < 3.0e38].astype(np.float32)
    mid = np.concatenate([mid, -mid, np.nextafter(mid, np.float32(np.inf)),
                          np.nextafter(mid, np.float32(-np.inf))])
    ref = torch.from_numpy(mid).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16(mid.astype(np.float64)), ref)
    assert np.all(oracle.f64_to_bf16(mid[: len(mid) // 4].astype(np.float64)) % 2 == 0)


def test_bf16_random_fp32_vs_torch():
    g = np.random.default_rng(1)
    x = (g.standard_normal(200000) * np.exp(g.uniform(-80, 80, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16(x.astype(np.float64)), ref)
