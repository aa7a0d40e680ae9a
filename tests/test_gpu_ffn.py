"""GPU parity of moe_expert_ffn alone, fed the oracle's plan and gathered rows:
the SwiGLU output h and the weighted expert output y of every entry (a large
sample at the 32K-token one-call shape) against the oracle's per-entry loop, max|d|/max|ref| within the tolerance of
the element type (1e-5 fp32, 5e-3 fp16/bf16). Pad rows of y stay untouched.
Shapes are chosen to take every launch path: K split into ranges (few work
items) in either projection, and runs of 2 or 4 work items of one expert that
share the weight tile (experts with more than 64 rows)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (POLLUTE, TOL, TORCH16, abi, custom, dev, host, make_case, polluted,
                      rel_err, say, synth)

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
    # scratch starts as garbage (the call must not rely on its contents: the
    # work list and the split-K partial sums are rewritten on every call), and
    # the second call on the same scratch must give the same bits
    scratch = polluted(abi.moe_ffn_scratch_bytes(cfg.E, cfg.d, cfg.f, cfg.tm, R,
                                                 abi.DTYPE_NAME[cfg.dtype]) // 4 + 1)
    say(f"[ffn] {cfg.name}: T={T} d={cfg.d} E={cfg.E} K={K} f={cfg.f} {cfg.dtype} tm={cfg.tm} "
        f"nr={nr}")
    outs = []
    for _ in range(2):
        h = polluted(R * cfg.f * es // 4)
        y = polluted(R * cfg.d, torch.float32)
        abi.moe_expert_ffn(dev(xs, cfg.dtype), case.d("wg"), case.d("wu"), case.d("wd"),
                           abi.DTYPE_NAME[cfg.dtype], cfg.E, cfg.d, cfg.f, cfg.tm, dev(p["eoff"]),
                           dev(stok), dev(sw), dev(p["meta"]), R, h, y, scratch)
        torch.cuda.synchronize()
        outs.append((host(h), host(y)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    hh = outs[0][0].view(np.uint16 if es == 2 else np.float32).reshape(R, cfg.f)
    yy = outs[0][1].reshape(R, cfg.d)
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
def test_ffn_configs_every_entry(name):
    """h and y of every entry of the workload's first layer call against the
    oracle; the long prompt planned as one call (327,680 entries) compares 8,192:
    its first and last, every 16th of the heaviest expert's and a seeded sample"""
    cfg = synth.CONFIGS[name]
    case = make_case(cfg)
    Tc = cfg.tokens_per_call
    ids, w, x = case.ids[:Tc], case.w[:Tc], case.x[:Tc]
    flat = ids.reshape(-1)
    valid = np.nonzero((flat >= 0) & (flat < cfg.E))[0]
    ent = valid
    if len(valid) > 32768:
        g = np.random.default_rng(cfg.seed)
        top = np.bincount(flat[valid], minlength=cfg.E).argmax()
        heavy = valid[flat[valid] == top]
        ent = np.unique(np.concatenate([valid[:64], valid[-64:], heavy[::16]]))
        ent = np.unique(np.concatenate([ent, g.choice(valid, 8192 - len(ent), replace=False)]))
    say(f"[ffn] {name}: {len(ent)} of {len(valid)} entries")
    run_ffn(case, ids, w, x, ent.astype(np.int32))
    case.drop_device()


def item_runs(cfg, ids):
    """run lengths (1, 2, 4) of the work items the plan of `ids` yields: items of
    64 rows per expert, grouped 4 by 4, then a pair, then singles"""
    cnt = np.bincount(ids[(ids >= 0) & (ids < cfg.E)].ravel(), minlength=cfg.E)
    rows = (cnt + cfg.tm - 1) // cfg.tm * cfg.tm
    runs = {1: 0, 2: 0, 4: 0}
    for n in (rows + 63) // 64:
        runs[4] += n // 4
        rest = n % 4
        runs[2] += 1 if rest >= 2 else 0
        runs[1] += rest % 2
    return runs


# (config, expect gate/up split, expect down split, expect runs of 4 or 2)
PATHS = [
    (custom("split_gateup_f32", T=8, d=1024, E=16, K=2, f=128, dtype="f32"), True, False, False),
    (custom("split_both_bf16", T=6, d=1536, E=64, K=4, f=1024, dtype="bf16"), True, True, False),
    (custom("tall4_split_f16", T=600, d=2048, E=2, K=1, f=256, dtype="f16"), True, False, True),
    (custom("tall4_split_bf16_tm1", T=700, d=1024, E=3, K=1, f=512, dtype="bf16", tm=1), True,
     True, True),
    (custom("tall_mix_f32", T=400, d=256, E=4, K=2, f=192, dtype="f32", bias="zipf1.1"), True,
     False, True),
    (custom("tall_split_unit_f16", T=1024, d=512, E=8, K=2, f=1024, dtype="f16", bias="zipf1.1",
            x_std=1.0), True, True, True),
]


@pytest.mark.parametrize("cfg,sgu,sdn,tall", PATHS, ids=[c[0].name for c in PATHS])
def test_ffn_launch_paths(cfg, sgu, sdn, tall):
    case = make_case(cfg)
    z = abi.moe_plan_sizes(cfg.T, cfg.K, cfg.E, cfg.tm)
    splits = abi.moe_ffn_splits(cfg.E, cfg.d, cfg.f, cfg.tm, z.max_rows, abi.DTYPE_NAME[cfg.dtype])
    assert (splits[0] > 1, splits[1] > 1) == (sgu, sdn), splits
    runs = item_runs(cfg, case.ids)
    assert (runs[4] + runs[2] > 0) == tall, runs
    say(f"[ffn paths] {cfg.name}: splits={splits} runs={runs}")
    run_ffn(case, case.ids, case.w, case.x)


def worklist_model(eoff, E, max_rows, runs_first=True):
    """The grouped FFN's work list as the header describes it: each expert's
    rows cut into items of 64; per expert runs of 4 items first, then a run of
    2 if at least 2 items remain, then single items; the items in runs of 4 of
    all experts come first (ascending expert), then the others (ascending
    expert), or, without runs_first, each expert's items together by expert;
    run = length | index << 8. Returns (items [n, 4], items in runs of 4 when
    they come first, else 0, items in runs of 2 or 4)."""
    quad, rest = [], []
    for e in range(E):
        a = min(max(int(eoff[e]), 0), max_rows)
        b = min(max(int(eoff[e + 1]), a), max_rows)
        n = (b - a + 63) // 64
        n4 = n & ~3
        for q in range(n):
            if q < n4:
                run = 4 | ((q & 3) << 8)
            elif n - n4 >= 2 and q - n4 < 2:
                run = 2 | ((q - n4) << 8)
            else:
                run = 1
            (quad if q < n4 or not runs_first else rest).append(
                (e, a + 64 * q, min(64, b - a - 64 * q), run))
    items = np.array(quad + rest, np.int32).reshape(-1, 4)
    return items, len(quad) if runs_first else 0, int(np.sum((items[:, 3] & 0xFF) > 1))


WL = [synth.CONFIGS["prefill_fp16"], custom("wl_skewed", T=3000, d=64, E=24, K=3, f=64,
                                            dtype="f16", bias="zipf1.1"),
      # at most 64 entries (the one-wavefront plan): decode, and one expert whose 64
      # rows pad to 96 (a run of 2 items)
      synth.CONFIGS["decode_bf16"],
      custom("wl_one_wavefront", T=64, d=64, E=1, K=1, f=64, dtype="f16", tm=48)]


@pytest.mark.parametrize("cfg", WL, ids=[c.name for c in WL])
@pytest.mark.parametrize("fused", [False, True], ids=["moe_expert_ffn", "moe_forward"])
@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
def test_worklist_layout(cfg, fused, packed):
    """the work list the FFN kernels consume (written by the worklist kernel
    for moe_expert_ffn, by the one-launch plan for moe_forward) equals the
    model above, with its counts (items, leading items in runs of 4, items in
    runs); the runs of 4 come first only where the big-cell kernels take them"""
    ids, w = synth.routing(cfg)
    T, K = ids.shape
    p = oracle.plan(ids, w, cfg.E, cfg.tm)
    z = abi.moe_plan_sizes(T, K, cfg.E, cfg.tm)
    R = z.max_rows
    dt = abi.DTYPE_NAME[cfg.dtype]
    first = packed and abi.moe_ffn_big_cells(cfg.E, cfg.d, cfg.f, cfg.tm, R, dt) != 0
    want, nfour, nruns = worklist_model(p["eoff"], cfg.E, R, first)
    say(f"[worklist] {cfg.name} {'forward' if fused else 'expert_ffn'} packed={packed}")
    wts = [torch.zeros((cfg.E, a, b), dtype=TORCH16[cfg.dtype], device="cuda")
           for a, b in ((cfg.d, cfg.f), (cfg.d, cfg.f), (cfg.f, cfg.d))]
    pk = abi.pack(*wts) if packed else None
    if fused:
        x = torch.zeros((T, cfg.d), dtype=TORCH16[cfg.dtype], device="cuda")
        _, ws = abi.forward(x, dev(ids), dev(w), *wts, tm=cfg.tm, packed=pk)
        L = abi.moe_forward_layout(T, K, cfg.E, cfg.d, cfg.f, cfg.tm, dt)
        scratch = ws[L.ffn_scratch:]
    else:
        nr = len(p["stok"])
        stok = np.full(R, -1, np.int32)
        stok[:nr] = p["stok"]
        sw = np.zeros(R, np.float32)
        sw[:nr] = p["sw"]
        scratch = torch.empty(abi.moe_ffn_scratch_bytes(cfg.E, cfg.d, cfg.f, cfg.tm, R, dt),
                              dtype=torch.uint8, device="cuda")
        xs = torch.zeros((R, cfg.d), dtype=TORCH16[cfg.dtype], device="cuda")
        h = torch.empty((R, cfg.f), dtype=TORCH16[cfg.dtype], device="cuda")
        y = torch.empty((R, cfg.d), dtype=torch.float32, device="cuda")
        args = (dt, cfg.E, cfg.d, cfg.f, cfg.tm, dev(p["eoff"]), dev(stok), dev(sw),
                dev(p["meta"]), R, h, y, scratch)
        if packed:
            abi.moe_expert_ffn_packed(xs, pk["gate"], pk["up"], pk["down"], *args)
        else:
            abi.moe_expert_ffn(xs, *wts, *args)
    torch.cuda.synchronize()
    raw = scratch[: 256 + 16 * len(want)].cpu().numpy().view(np.int32)
    assert raw[0] == len(want) and raw[1] == nfour and raw[2] == nruns
    assert np.array_equal(raw[64:].reshape(-1, 4), want)
