"""GPU parity of moe_expert_ffn alone, fed the oracle's plan and gathered rows:
the SwiGLU output h and the weighted expert output y of every (sampled) entry
against the oracle's per-entry loop, max|d|/max|ref| within the tolerance of
the element type (1e-5 fp32, 5e-3 fp16/bf16). Pad rows of y stay untouched."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (POLLUTE, TOL, abi, custom, dev, host, make_case, polluted, rel_err, say,
                      synth)

pytestmark = pytest.mark.gpu


def run_ffn(case, ids, w, x, entries=None):
    cfg = case.cfg
    T, K = ids.shape
    p = oracle.plan(ids, w, cfg.E, cfg.tm)
    z = abi.moe_plan_sizes(T, K, cfg.E, cfg.tm)
    R = z.max_rows
    nr = len(p["stok"])
    xs = np.zeros((R, cfg.d), x.dtype)
    xs[:nr] = oracle.gather(x, p["stok"])
    stok = np.full(R, -1, np.int32)
    stok[:nr] = p["stok"]
    sw = np.zeros(R, np.float32)
    sw[:nr] = p["sw"]
    es = synth.ELEM_BYTES[cfg.dtype]
    h = polluted(R * cfg.f * es // 4)
    y = polluted(R * cfg.d, torch.float32)
    scratch = torch.empty(abi.moe_ffn_scratch_bytes(cfg.E, cfg.tm, R), dtype=torch.uint8,
                          device="cuda")
    say(f"[ffn] {cfg.name}: T={T} d={cfg.d} E={cfg.E} K={K} f={cfg.f} {cfg.dtype} tm={cfg.tm} "
        f"nr={nr}")
    abi.moe_expert_ffn(dev(xs, cfg.dtype), case.d("wg"), case.d("wu"), case.d("wd"),
                       abi.DTYPE_NAME[cfg.dtype], cfg.E, cfg.d, cfg.f, cfg.tm, dev(p["eoff"]),
                       dev(stok), dev(sw), dev(p["meta"]), R, h, y, scratch)
    torch.cuda.synchronize()
    hh = host(h).view(np.uint16 if es == 2 else np.float32).reshape(R, cfg.f)
    yy = host(y).reshape(R, cfg.d)
    flat = ids.reshape(-1)
    valid = np.nonzero((flat >= 0) & (flat < cfg.E))[0]
    if entries is None:
        entries = valid
    ry, rh = oracle.ffn_entries(x, ids, w, case.wg, case.wu, case.wd, cfg.dtype, True, entries)
    rows = p["pos"][entries]
    got_h = oracle.decode(hh[rows], cfg.dtype)
    assert rel_err(got_h, rh) <= TOL[cfg.dtype], rel_err(got_h, rh)
    assert rel_err(yy[rows], ry) <= TOL[cfg.dtype], rel_err(yy[rows], ry)
    # y is not written on pad rows
    pad = np.nonzero(stok[:nr] < 0)[0]
    assert np.all(yy[pad].view(np.int32) == POLLUTE)
    return rel_err(yy[rows], ry)


SMALL = [
    custom("ragged_tails_f16", T=96, d=328, E=12, K=3, f=200, dtype="f16"),
    custom("ragged_tails_bf16", T=96, d=328, E=12, K=3, f=200, dtype="bf16", x_std=1.0),
    custom("ragged_tails_f32", T=96, d=328, E=12, K=3, f=200, dtype="f32"),
    custom("tm1_partial_tiles", T=150, d=256, E=10, K=2, f=128, dtype="f16", tm=1),
    custom("tm8_skew", T=300, d=192, E=20, K=2, f=96, dtype="bf16", tm=8, bias="zipf1.1"),
    custom("one_expert_many_items", T=300, d=64, E=1, K=1, f=64, dtype="f16"),
    custom("unit_scale_swiglu", T=64, d=512, E=8, K=2, f=256, dtype="f16", x_std=1.0),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_ffn_small_all_entries(cfg):
    case = make_case(cfg)
    run_ffn(case, case.ids, case.w, case.x)


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_ffn_configs_sampled(name):
    cfg = synth.CONFIGS[name]
    case = make_case(cfg)
    Tc = cfg.tokens_per_call
    ids, w, x = case.ids[:Tc], case.w[:Tc], case.x[:Tc]
    flat = ids.reshape(-1)
    valid = np.nonzero((flat >= 0) & (flat < cfg.E))[0]
    g = np.random.default_rng(cfg.seed)
    n = min(len(valid), 96)
    ent = np.unique(np.concatenate([valid[:4], valid[-4:], g.choice(valid, n, replace=False)]))
    if name == "long_skewed_fp16":  # include entries of the heaviest expert (several work items)
        top = np.bincount(flat[valid], minlength=cfg.E).argmax()
        heavy = valid[flat[valid] == top]
        ent = np.unique(np.concatenate([ent, heavy[:: max(1, len(heavy) // 24)]]))
    run_ffn(case, ids, w, x, ent.astype(np.int32))
    case.drop_device()
