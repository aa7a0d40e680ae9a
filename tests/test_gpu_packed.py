"""Packed expert weights (moe_pack_weights): the packed layer feeds the matrix
cores the same operand bits in the same order as the row-major one, so
moe_forward_packed must equal moe_forward and moe_expert_ffn_packed must equal
moe_expert_ffn bit for bit, on every launch path (wide and tall cells, K split
or not, fp32 / fp16 / bf16, ragged d and f). The row-major path is itself
checked against the oracle in test_gpu_forward / test_gpu_ffn; the prefill
workload is also checked against the oracle here, through the packed path."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, abi, custom, dev, host, make_case, rel_err, say, synth
from test_gpu_ffn import PATHS as FFN_PATHS

pytestmark = pytest.mark.gpu

CASES = [
    synth.CONFIGS["tiny_fp32"],
    custom("ragged_tails_f16", T=96, d=328, E=12, K=3, f=200, dtype="f16"),
    custom("ragged_tails_bf16", T=96, d=328, E=12, K=3, f=200, dtype="bf16", x_std=1.0),
    custom("ragged_tails_f32", T=80, d=136, E=6, K=2, f=72, dtype="f32", x_std=1.0),
    custom("tm1_no_padding", T=150, d=256, E=10, K=2, f=128, dtype="f16", tm=1),
    custom("max_experts_f16", T=300, d=64, E=1024, K=8, f=64, dtype="f16"),
    custom("min_dims_bf16", T=50, d=8, E=4, K=2, f=8, dtype="bf16", x_std=1.0, w_std=0.5),
    custom("k_equals_e_f32", T=20, d=40, E=6, K=6, f=24, dtype="f32", x_std=1.0),
    custom("tm48_f16", T=200, d=96, E=16, K=3, f=80, dtype="f16", tm=48),
    # few work items, skewed: split K on both paths, items of 1 to 4 m-tiles,
    # ragged d and f
    custom("few_items_skewed_bf16", T=96, d=328, E=48, K=2, f=200, dtype="bf16",
           bias="zipf1.1", x_std=1.0),
    custom("few_items_skewed_f16", T=130, d=256, E=64, K=3, f=136, dtype="f16", bias="zipf1.1"),
] + [c[0] for c in FFN_PATHS]

# shapes whose packed 16-bit gate/up runs each expert's runs of 4 items on the
# 8-wavefront kernel (plan bound >= 64 rows per expert, no K split): h columns
# not a multiple of 128 (f = 320, 136), an odd number of 32-wide K-steps
# (d = 328), a run whose last item is partial, tm = 1, runs followed by items
# left to the 4-wavefront kernel, down projection split
BIG = [
    custom("big_cells_f16", T=2048, d=328, E=4, K=2, f=320, dtype="f16", bias="zipf1.1"),
    custom("big_cells_bf16_tm1", T=1500, d=360, E=3, K=2, f=256, dtype="bf16", tm=1,
           bias="zipf1.1", x_std=1.0),
    custom("big_cells_f16_16e", T=4096, d=256, E=16, K=4, f=512, dtype="f16", bias="zipf1.1"),
    custom("big_cells_bf16_24e", T=3000, d=264, E=24, K=3, f=136, dtype="bf16",
           bias="normal0.5"),
    # fewer 32-wide K-steps than the kernel keeps in flight (gate/up 3, down 2)
    custom("big_cells_short_k_f16", T=2048, d=96, E=4, K=2, f=40, dtype="f16", bias="zipf1.1",
           x_std=1.0),
    # big gate/up cells next to a down projection split along f (few down cells)
    custom("big_cells_split_down_f16", T=2048, d=256, E=4, K=2, f=2048, dtype="f16",
           bias="zipf1.1"),
]
CASES += BIG


def packed_of(case):
    return abi.pack(case.d("wg"), case.d("wu"), case.d("wd"))


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_forward_packed_equals_rowmajor(cfg):
    case = make_case(cfg)
    say(f"[packed forward] {cfg.name}")
    x, ids, w = dev(case.x, cfg.dtype), dev(case.ids), dev(case.w)
    a, ws = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm)
    pk = packed_of(case)
    b, _ = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm,
                       workspace=ws, packed=pk)
    torch.cuda.synchronize()
    assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32))
    case.drop_device()


@pytest.mark.parametrize("cfg", BIG, ids=[c.name for c in BIG])
def test_big_cells_forward_vs_oracle(cfg):
    """the packed layer on the shapes that take the 8-wavefront kernels (gate/up
    always, down unless it is split), every token against the oracle"""
    z = abi.moe_plan_sizes(cfg.T, cfg.K, cfg.E, cfg.tm)
    big = abi.moe_ffn_big_cells(cfg.E, cfg.d, cfg.f, cfg.tm, z.max_rows, abi.DTYPE_NAME[cfg.dtype])
    splits = abi.moe_ffn_splits(cfg.E, cfg.d, cfg.f, cfg.tm, z.max_rows, abi.DTYPE_NAME[cfg.dtype])
    assert big & 1  # gate/up
    assert bool(big & 2) == (splits[1] == 1)  # down, unless split along f
    case = make_case(cfg)
    say(f"[packed forward, big cells {big}] {cfg.name}")
    x, ids, w = dev(case.x, cfg.dtype), dev(case.ids), dev(case.w)
    out, _ = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm,
                         packed=packed_of(case))
    torch.cuda.synchronize()
    got = host(out)
    for round_h in (True, False):
        ref = oracle.ffn(case.x, case.ids, case.w, case.wg, case.wu, case.wd, cfg.dtype, round_h)
        assert rel_err(got, ref.astype(np.float32)) <= TOL[cfg.dtype], round_h
    case.drop_device()


FFN_CASES = CASES[:5] + BIG


@pytest.mark.parametrize("cfg", FFN_CASES, ids=[c.name for c in FFN_CASES])
def test_expert_ffn_packed_equals_rowmajor(cfg):
    case = make_case(cfg)
    T, K = case.ids.shape
    p = oracle.plan(case.ids, case.w, cfg.E, cfg.tm)
    z = abi.moe_plan_sizes(T, K, cfg.E, cfg.tm)
    R, nr = z.max_rows, len(p["stok"])
    xs = np.zeros((R, cfg.d), case.x.dtype)
    xs[:nr] = oracle.gather(case.x, p["stok"])
    stok = np.full(R, -1, np.int32)
    stok[:nr] = p["stok"]
    sw = np.zeros(R, np.float32)
    sw[:nr] = p["sw"]
    dt = abi.DTYPE_NAME[cfg.dtype]
    tdt = abi.TORCH_DTYPE[dt]
    scratch = torch.empty(abi.moe_ffn_scratch_bytes(cfg.E, cfg.d, cfg.f, cfg.tm, R, dt),
                          dtype=torch.uint8, device="cuda")
    args = (dev(p["eoff"]), dev(stok), dev(sw), dev(p["meta"]), R)
    outs = []
    pk = packed_of(case)
    for packed in (False, True):
        h = torch.zeros((R, cfg.f), dtype=tdt, device="cuda")
        y = torch.zeros((R, cfg.d), dtype=torch.float32, device="cuda")
        if packed:
            abi.moe_expert_ffn_packed(dev(xs, cfg.dtype), pk["gate"], pk["up"], pk["down"], dt,
                                      cfg.E, cfg.d, cfg.f, cfg.tm, *args, h, y, scratch)
        else:
            abi.moe_expert_ffn(dev(xs, cfg.dtype), case.d("wg"), case.d("wu"), case.d("wd"), dt,
                               cfg.E, cfg.d, cfg.f, cfg.tm, *args, h, y, scratch)
        torch.cuda.synchronize()
        outs.append((host(h), host(y)))
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    case.drop_device()


@pytest.mark.parametrize("name", ["prefill_fp16", "decode_bf16", "ubatch_bf16",
                                  "long_onepass_fp16"])
def test_forward_packed_full_size(name):
    """full-size workloads: packed == row-major bitwise, and packed vs the oracle
    on a sample of tokens"""
    cfg = synth.CONFIGS[name]
    case = make_case(cfg)
    say(f"[packed forward] {name} full size")
    x, ids, w = dev(case.x, cfg.dtype), dev(case.ids), dev(case.w)
    a, ws = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm)
    got_a = host(a)
    pk = packed_of(case)
    b, _ = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm,
                       workspace=ws, packed=pk)
    got = host(b)
    assert np.array_equal(got_a.view(np.uint32), got.view(np.uint32))
    g = np.random.default_rng(cfg.seed)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], g.choice(cfg.T, min(16, cfg.T),
                                                              replace=False)])).astype(np.int32)
    ref = oracle.ffn(case.x, case.ids, case.w, case.wg, case.wu, case.wd, cfg.dtype, True,
                     tokens=toks)
    assert rel_err(got[toks], ref.astype(np.float32)) <= TOL[cfg.dtype]
    del pk
    case.drop_device()
