"""A seeded sweep of random layer shapes beside the hand-picked cases: experts
1..1024, top-k 1..12, 1..3300 tokens (past the one-launch plan's 32,768
entries), hidden and intermediate sizes any multiple of 8 up to 1024, row
tiles 1..32, fp32 / fp16 / bf16, uniform or skewed routing. moe_forward
against the oracle (every token when T <= 64, else a seeded sample), and for
16-bit types moe_forward_packed equal to moe_forward bit for bit."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, abi, custom, dev, host, make_case, rel_err, say

pytestmark = pytest.mark.gpu


def random_shapes(n=64, seed=2024):
    """the sweep's configurations (host memory of the weights <= ~0.8 GB each)"""
    g = np.random.default_rng(seed)
    out = []
    for k in range(n):
        dtype = ("f32", "f16", "bf16")[k % 3]
        E = int(g.choice([1, 2, 3, 7, 16, 33, 64, 100, 128, 257, 512, 1000, 1024]))
        K = int(g.integers(1, min(E, 12) + 1))
        T = int(g.choice([1, 2, 5, 17, 64, 130, 333, 700, 1500, 3300]))
        d = 8 * int(g.integers(1, 129))
        f = 8 * int(g.integers(1, 129))
        while E * d * f > 64 * 2**20:  # bound the expert matrices
            if d >= f:
                d = max(8, d // 16 * 8)
            else:
                f = max(8, f // 16 * 8)
        tm = int(g.choice([1, 3, 8, 16, 16, 32]))
        bias = str(g.choice(["none", "normal0.5", "zipf1.1"]))
        x_std = float(g.choice([0.02, 1.0]))
        out.append(custom(f"rand{k:02d}_{dtype}_T{T}_E{E}_K{K}_d{d}_f{f}_tm{tm}_{bias}", T=T,
                          d=d, E=E, K=K, f=f, dtype=dtype, tm=tm, bias=bias, seed=3000 + k,
                          x_std=x_std))
    return out


SHAPES = random_shapes() + [
    # past 32,768 entries (the three-launch plan), skewed
    custom("rand_plan3_f16", T=3300, d=136, E=64, K=12, f=200, dtype="f16", bias="zipf1.1",
           seed=3100),
    # big cells with a 3-row tile and ragged sizes
    custom("rand_big_bf16_tm3", T=3300, d=264, E=8, K=4, f=392, dtype="bf16", tm=3,
           bias="normal0.5", seed=3101, x_std=1.0),
]


@pytest.mark.parametrize("cfg", SHAPES, ids=[c.name for c in SHAPES])
def test_random_shape_forward(cfg):
    case = make_case(cfg)
    say(f"[random] {cfg.name}")
    x, ids, w = dev(case.x, cfg.dtype), dev(case.ids), dev(case.w)
    wg, wu, wd = case.d("wg"), case.d("wu"), case.d("wd")
    out, ws = abi.forward(x, ids, w, wg, wu, wd, tm=cfg.tm)
    got = host(out).copy()
    if cfg.dtype != "f32":
        pk = abi.pack(wg, wu, wd)
        out2, _ = abi.forward(x, ids, w, wg, wu, wd, tm=cfg.tm, workspace=ws, packed=pk)
        assert np.array_equal(host(out2).view(np.uint32), got.view(np.uint32))
        del pk
    if cfg.T <= 64:
        toks = np.arange(cfg.T, dtype=np.int32)
    else:
        g = np.random.default_rng(cfg.seed)
        toks = np.unique(np.concatenate([[0, cfg.T - 1], g.choice(cfg.T, 40, replace=False)]))
        toks = toks.astype(np.int32)
    ref = oracle.ffn(case.x, case.ids, case.w, case.wg, case.wu, case.wd, cfg.dtype, True,
                     tokens=toks)
    assert rel_err(got[toks], ref.astype(np.float32)) <= TOL[cfg.dtype]
    case.drop_device()
