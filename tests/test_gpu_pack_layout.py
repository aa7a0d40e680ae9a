"""moe_pack_weights writes exactly the tile layout the header documents (the
packed path's equality with the row-major path is checked elsewhere; this pins
the format itself, for callers that pack offline): per expert, column group g
of 4 slices of 64*M columns (M = 1 stream for gate/up, 2 for down), K-step s,
slice w and stream m, one 4 KB tile at ((((e*gs + g)*nst + s)*4 + w)*M + m) *
4096 bytes, holding 4 x 64 words of 16 bytes, word [c][lane] at (64*c + lane)
* 16: for 16-bit types the 8 K-values 32s + 8*(lane >> 4) + i (i = 0..7) of
column (4g + w)*64M + 64m + 4*(lane & 15) + c; for fp32 the 4 columns
(4g + w)*64M + 64m + 4*(lane & 15) + j (j = 0..3) of K-row 16s + 4*(lane >> 4) + c.
Positions outside [0, Kd) x [0, N) hold zeros. A numpy model of that
description, byte for byte against the GPU's packing."""
import numpy as np
import pytest

from gpu_util import abi, dev, host, say, synth

pytestmark = pytest.mark.gpu


def pack_model(W: np.ndarray, gateup: bool, es: int) -> np.ndarray:
    """W [E][Kd][N] raw storage (uint16 or float32) -> packed bytes"""
    E, Kd, N = W.shape
    M = 1 if gateup else 2
    ks = 32 if es == 2 else 16
    gs, nst = -(-N // (256 * M)), -(-Kd // ks)
    lane = np.arange(64)
    per = 8 if es == 2 else 4  # values per 16-byte word
    out = np.zeros((E, gs, nst, 4, M, 4, 64, per), W.dtype)
    q = np.arange(per)
    for g in range(gs):
        for s in range(nst):
            for w in range(4):
                for m in range(M):
                    c = np.arange(4)[:, None, None]
                    base = (4 * g + w) * 64 * M + 64 * m + 4 * (lane[None, :, None] & 15)
                    if es == 2:
                        k = 32 * s + 8 * (lane[None, :, None] >> 4) + q[None, None, :]
                        col = base + c
                    else:
                        k = 16 * s + 4 * (lane[None, :, None] >> 4) + c
                        col = base + q[None, None, :]
                    k, col = np.broadcast_arrays(k, col)
                    ok = (k < Kd) & (col < N)
                    vals = W[:, np.minimum(k, Kd - 1), np.minimum(col, N - 1)]
                    out[:, g, s, w, m] = np.where(ok[None], vals, 0)
    return out.reshape(-1).view(np.uint8)


CASES = [
    ("f16", 2, 72, 200),    # ragged N and K
    ("bf16", 3, 328, 136),
    ("f32", 2, 40, 24),
    ("f16", 1, 32, 512),    # whole groups and steps
    ("bf16", 2, 8, 8),      # smallest
]


@pytest.mark.parametrize("dtype,E,d,f", CASES, ids=[f"{c[0]}_E{c[1]}_d{c[2]}_f{c[3]}" for c in CASES])
def test_pack_layout_matches_the_documented_format(dtype, E, d, f):
    g = np.random.default_rng(E * 1000 + d + f)
    es = synth.ELEM_BYTES[dtype]
    mats = {k: synth.to_dtype(g.standard_normal(shape).astype(np.float32), dtype)
            for k, shape in (("gate", (E, d, f)), ("up", (E, d, f)), ("down", (E, f, d)))}
    say(f"[pack layout] {dtype} E={E} d={d} f={f}")
    pk = abi.pack(dev(mats["gate"], dtype), dev(mats["up"], dtype), dev(mats["down"], dtype))
    for k in ("gate", "up", "down"):
        got = host(pk[k]).view(np.uint8).reshape(-1)
        ref = pack_model(mats[k], k != "down", es)
        assert got.size == ref.size, (k, got.size, ref.size)
        assert np.array_equal(got, ref), k
