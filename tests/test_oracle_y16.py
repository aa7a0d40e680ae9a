"""Pins of the oracle's compact expert-output format (binary16 values with one
power-of-two exponent per row block of 128 columns) and of the combine over it:
  * the exponent puts the block's largest magnitude in [2^14, 2^15) (closed form,
    checked with numpy's frexp/ldexp), 0 for an all-zero or non-finite block,
    clamped to [-112, 100];
  * encoding equals numpy's own float64 -> float16 rounding of v * 2^e, and
    decoding equals numpy's float16 -> float64 conversion times 2^-e, exactly;
  * the round trip keeps every value within half a binary16 ulp (relative
    2^-11) of the block maximum's scale;
  * the combine over compact rows equals the fp32 combine (itself pinned) of the
    decoded rows, bit for bit, and shows its fixed order on a cancellation case."""
import numpy as np

import oracle

rng = np.random.default_rng(77)


def np_exponent(M):
    if not (M > 0) or not np.isfinite(M):
        return 0
    _, k = np.frexp(np.float64(M))
    return int(np.clip(15 - k, -112, 100))


def test_exponent_places_the_block_max_below_2_15():
    Ms = np.concatenate([np.float32(2.0) ** np.arange(-149, 128, dtype=np.float64),
                         rng.standard_normal(2000) ** 2 * 10.0 ** rng.integers(-30, 30, 2000),
                         [np.finfo(np.float32).max, np.finfo(np.float32).tiny, 1e-45]])
    Ms = Ms.astype(np.float32)
    Ms = Ms[np.isfinite(Ms) & (Ms > 0)]
    for M in Ms:
        e = oracle.y16_exponent(M)
        assert -112 <= e <= 100
        scaled = np.ldexp(np.float64(M), e)
        if -112 < e < 100:
            assert 2.0 ** 14 <= scaled < 2.0 ** 15, (M, e)
        elif e == 100:
            assert scaled < 2.0 ** 15  # tiny blocks: clamped, never overflow
        else:
            assert scaled < 2.0 ** 16
    for M in (0.0, -0.0, np.inf, np.nan):
        assert oracle.y16_exponent(M) == 0


def block_rows(n, d, spread=True):
    """rows whose 128-column blocks have very different magnitudes"""
    y = rng.standard_normal((n, d)).astype(np.float32)
    nb = (d + 127) // 128
    scale = 10.0 ** rng.integers(-12, 6, (n, nb)) if spread else np.ones((n, nb))
    return (y * np.repeat(scale, 128, axis=1)[:, :d]).astype(np.float32)


def test_encode_and_decode_match_numpy_binary16():
    for d in (8, 128, 200, 384, 2560):
        y = block_rows(40, d)
        y[3, :5] = 0.0
        y[5] = 0.0  # an all-zero row
        s, e = oracle.y16_encode(y)
        nb = (d + 127) // 128
        assert e.shape == (40, nb)
        for r in range(40):
            for b in range(nb):
                blk = y[r, b * 128:(b + 1) * 128]
                assert e[r, b] == np_exponent(np.max(np.abs(blk)))
        ee = np.repeat(e.astype(np.int64), 128, axis=1)[:, :d]
        want = np.ldexp(y.astype(np.float64), ee).astype(np.float16).view(np.uint16)
        assert np.array_equal(s, want)
        dec = oracle.y16_decode(s, e)
        ref = np.ldexp(s.view(np.float16).astype(np.float64), -ee)
        assert np.array_equal(dec.astype(np.float64), ref)  # exact in fp32


def test_round_trip_error_is_half_a_binary16_ulp_of_the_block():
    y = block_rows(64, 640)
    s, e = oracle.y16_encode(y)
    dec = oracle.y16_decode(s, e).astype(np.float64)
    nb = 5
    M = np.abs(y).reshape(64, nb, 128).max(axis=2)
    err = np.abs(dec - y).reshape(64, nb, 128).max(axis=2)
    # |v| >= M / 2 keeps 11 bits: relative error <= 2^-11 of its binade; below,
    # binary16's absolute step at the block's scale bounds it
    assert np.all(err <= M * 2.0 ** -11)
    big = np.abs(y) >= 2.0 ** -14 * M.repeat(128, axis=1)
    rel = np.abs(dec - y)[big] / np.abs(y)[big]
    assert rel.max() <= 2.0 ** -11


def test_special_values_survive():
    y = np.zeros((2, 256), np.float32)
    y[0, 0], y[0, 1], y[0, 2] = np.nan, 1.5, -3.0
    y[1, 130], y[1, 131] = np.inf, 2.0
    s, e = oracle.y16_encode(y)
    dec = oracle.y16_decode(s, e)
    assert np.isnan(dec[0, 0]) and dec[0, 1] == 1.5 and dec[0, 2] == -3.0
    assert e[1, 1] == 0 and np.isinf(dec[1, 130]) and dec[1, 131] == 2.0
    assert not np.any(np.signbit(dec[0, 3:]))  # +0 stays +0


def test_combine_over_compact_rows_equals_fp32_combine_of_decoded_rows():
    T, K, d = 33, 5, 328
    nrows = T * K + 20
    y = block_rows(nrows, d)
    s, e = oracle.y16_encode(y)
    pos = rng.permutation(nrows)[: T * K].astype(np.int32)
    pos[rng.random(T * K) < 0.2] = -1
    got = oracle.combine_y16(s, e, pos, T, K)
    want = oracle.combine_f32(oracle.y16_decode(s, e), pos, T, K)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_combine_over_compact_rows_keeps_the_k_order():
    # (2^27 + 1 - 2^27) in fp32 from +0: 2^27 + 1 rounds to 2^27, so the sum is 0;
    # the order (2^27, -2^27, 1) gives 1
    y = np.zeros((3, 128), np.float32)
    y[0, 0], y[1, 0], y[2, 0] = 2.0 ** 27, 1.0, -(2.0 ** 27)
    y[:, 1] = 1.0
    s, e = oracle.y16_encode(y)
    out = oracle.combine_y16(s, e, np.array([0, 1, 2], np.int32), 1, 3)
    assert out[0, 0] == 0.0 and out[0, 1] == 3.0
    out = oracle.combine_y16(s, e, np.array([0, 2, 1], np.int32), 1, 3)
    assert out[0, 0] == 1.0
