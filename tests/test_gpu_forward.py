"""GPU parity of moe_forward (the whole layer, the launch configuration the
benchmark times) against the oracle's naive per-(token, expert) loop, with the
SwiGLU output rounded like the GPU's operand (REF-R) and exact (REF-X):
max|d|/max|ref| <= 1e-5 for fp32 inputs, <= 5e-3 for fp16/bf16. Full-size
workloads compare every token against REF-R, with row-major and with packed
weights (the benchmark's layout), and a seeded sample of 256 tokens against
REF-X; the long prompt runs all 16 chunks. Also: bitwise run-to-run
determinism and the degenerate cases."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TOL, abi, chunk_of, custom, dev, host, make_case, polluted, rel_err, say,
                      synth)

pytestmark = pytest.mark.gpu


def gpu_forward(case, ids, w, x, ws=None):
    cfg = case.cfg
    out, ws = abi.forward(dev(x, cfg.dtype), dev(ids), dev(w), case.d("wg"), case.d("wu"),
                          case.d("wd"), tm=cfg.tm, workspace=ws)
    torch.cuda.synchronize()
    return host(out), ws


def compare(case, ids, w, x, got, tokens):
    cfg = case.cfg
    for round_h in (True, False):
        ref = oracle.ffn(x, ids, w, case.wg, case.wu, case.wd, cfg.dtype, round_h, tokens=tokens)
        err = rel_err(got[tokens], ref.astype(np.float32))
        say(f"  {'REF-R' if round_h else 'REF-X'} max|d|/max|ref| = {err:.3e}")
        assert err <= TOL[cfg.dtype], (round_h, err)


SMALL = [
    synth.CONFIGS["tiny_fp32"],
    custom("ragged_tails_f16", T=96, d=328, E=12, K=3, f=200, dtype="f16"),
    custom("ragged_tails_bf16_unit", T=96, d=328, E=12, K=3, f=200, dtype="bf16", x_std=1.0),
    custom("ragged_tails_f32", T=80, d=136, E=6, K=2, f=72, dtype="f32", x_std=1.0),
    custom("tm1_no_padding", T=150, d=256, E=10, K=2, f=128, dtype="f16", tm=1),
    custom("skewed_small_bf16", T=400, d=192, E=32, K=4, f=96, dtype="bf16", bias="zipf1.1"),
    custom("single_expert", T=200, d=64, E=1, K=1, f=64, dtype="f32"),
    custom("single_token", T=1, d=512, E=64, K=6, f=256, dtype="f16"),
    custom("max_experts_f16", T=300, d=64, E=1024, K=8, f=64, dtype="f16"),
    custom("min_dims_bf16", T=50, d=8, E=4, K=2, f=8, dtype="bf16", x_std=1.0, w_std=0.5),
    custom("k_equals_e_f32", T=20, d=40, E=6, K=6, f=24, dtype="f32", x_std=1.0),
    custom("tm48_f16", T=200, d=96, E=16, K=3, f=80, dtype="f16", tm=48),
]


# shapes that split K (few work items) and that run several work items of one
# expert against a shared weight tile, with the gather fused into the loads
PATHS = [
    custom("split_both_bf16", T=6, d=1536, E=64, K=4, f=1024, dtype="bf16"),
    custom("tall4_split_f16", T=600, d=2048, E=2, K=1, f=256, dtype="f16"),
    custom("tall_mix_f32", T=400, d=256, E=4, K=2, f=192, dtype="f32", bias="zipf1.1"),
    custom("tall_split_unit_bf16", T=1024, d=512, E=8, K=2, f=1024, dtype="bf16",
           bias="zipf1.1", x_std=1.0),
    # T*K = 40,960 > 32,768: the plan runs as three launches and the work list
    # is written by its own kernel
    custom("three_launch_plan_f16", T=4096, d=128, E=48, K=10, f=64, dtype="f16",
           bias="normal0.5"),
]


@pytest.mark.parametrize("cfg", SMALL + PATHS, ids=[c.name for c in SMALL + PATHS])
def test_forward_small_all_tokens(cfg):
    case = make_case(cfg)
    say(f"[forward] {cfg.name}")
    got, _ = gpu_forward(case, case.ids, case.w, case.x)
    compare(case, case.ids, case.w, case.x, got, np.arange(cfg.T, dtype=np.int32))


def split_cases():
    """one small layer per (dtype, projection, split count 2..8): the K range
    of the split projection is 8 steps per split (32 K-values per step for
    16-bit types, 16 for fp32), the other projection too short to split"""
    out = []
    for dtype, kstep in (("f32", 16), ("f16", 32), ("bf16", 32)):
        for ns in range(2, 9):
            kd = 8 * kstep * ns
            out.append((custom(f"split_gateup_{ns}_{dtype}", T=8, d=kd, E=4, K=2, f=64,
                               dtype=dtype, x_std=1.0, seed=700 + ns), (ns, 1)))
            out.append((custom(f"split_down_{ns}_{dtype}", T=8, d=64, E=4, K=2, f=kd,
                               dtype=dtype, x_std=1.0, seed=800 + ns), (1, ns)))
    return out


SPLITS = split_cases()


@pytest.mark.parametrize("cfg,splits", SPLITS, ids=[c[0].name for c in SPLITS])
def test_forward_every_split_count(cfg, splits):
    """each split count's reduction (gate/up per dtype, down) against the oracle"""
    z = abi.moe_plan_sizes(cfg.T, cfg.K, cfg.E, cfg.tm)
    assert abi.moe_ffn_splits(cfg.E, cfg.d, cfg.f, cfg.tm, z.max_rows,
                              abi.DTYPE_NAME[cfg.dtype]) == splits
    case = make_case(cfg)
    say(f"[forward] {cfg.name}")
    got, _ = gpu_forward(case, case.ids, case.w, case.x)
    compare(case, case.ids, case.w, case.x, got, np.arange(cfg.T, dtype=np.int32))


def sample_tokens(T, seed, n=24):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], g.choice(T, min(n, T), replace=False)])).astype(
        np.int32)


_REF = {}


def ref_all_tokens(case):
    """REF-R of every token of a workload, from the oracle's per-token loop, in
    pieces of 4096 tokens (progress shows between them). A token's output does not
    depend on how the tokens are cut into layer calls, so the long prompt's chunked
    and one-call forms (same seed and inputs) share one reference."""
    cfg = case.cfg
    key = (cfg.seed, cfg.T, cfg.d, cfg.E, cfg.K, cfg.f, cfg.dtype, cfg.bias, cfg.tail_skip,
           cfg.x_std, cfg.w_std)
    if key not in _REF:
        ref = np.empty((cfg.T, cfg.d), np.float32)
        for t0 in range(0, cfg.T, 4096):
            tok = np.arange(t0, min(cfg.T, t0 + 4096), dtype=np.int32)
            ref[tok] = oracle.ffn(case.x, case.ids, case.w, case.wg, case.wu, case.wd, cfg.dtype,
                                  True, tokens=tok)
            say(f"  oracle REF-R: tokens {t0}..{tok[-1]} of {cfg.T}")
        _REF.clear()  # one workload's reference at a time (the long prompt's is 335 MB)
        _REF[key] = ref
    return _REF[key]


def compare_all(case, ids, w, x, got, t0, ref_r, nx=256, seed=0):
    """every token against REF-R (got[i] is token t0 + i), and a seeded sample of nx
    tokens (all of them when fewer) against REF-X"""
    cfg = case.cfg
    T = got.shape[0]
    err = rel_err(got, ref_r[t0:t0 + T])
    say(f"  REF-R all {T} tokens: max|d|/max|ref| = {err:.3e}")
    assert err <= TOL[cfg.dtype], err
    toks = (np.arange(T, dtype=np.int32) if T <= nx else
            np.sort(np.random.default_rng(seed).choice(T, nx, replace=False)).astype(np.int32))
    ref_x = oracle.ffn(x, ids, w, case.wg, case.wu, case.wd, cfg.dtype, False, tokens=toks)
    err = rel_err(got[toks], ref_x.astype(np.float32))
    say(f"  REF-X {len(toks)} tokens: max|d|/max|ref| = {err:.3e}")
    assert err <= TOL[cfg.dtype], err


@pytest.mark.parametrize("name", ["prefill_fp16", "decode_bf16", "ubatch_bf16",
                                  "prefill_tailskip_fp16", "long_onepass_fp16"])
def test_forward_full_size_every_token(name):
    """row-major weights (moe_forward) and packed weights (moe_forward_packed, as
    the benchmark runs the layer): every token's output against the oracle"""
    cfg = synth.CONFIGS[name]
    case = make_case(cfg)
    ref_r = ref_all_tokens(case)
    pk = abi.pack(case.d("wg"), case.d("wu"), case.d("wd"))
    x, ids, w = dev(case.x, cfg.dtype), dev(case.ids), dev(case.w)
    ws = None
    for packed in (None, pk):
        say(f"[forward] {name} full size, {'packed' if packed else 'row-major'} weights")
        out, ws = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm,
                              workspace=ws, packed=packed)
        torch.cuda.synchronize()
        compare_all(case, case.ids, case.w, case.x, host(out), 0, ref_r, seed=cfg.seed)
    del pk, out, ws
    case.drop_device()


def test_forward_long_prompt_all_chunks_every_token():
    """the long prompt as 16 layer calls of 2,048 tokens (packed weights, as the
    benchmark runs it; row-major on the first, last and most skewed chunk):
    every token of every chunk against REF-R, 64 tokens per chunk against REF-X"""
    cfg = synth.CONFIGS["long_skewed_fp16"]
    case = make_case(cfg)
    ref_r = ref_all_tokens(case)
    pk = abi.pack(case.d("wg"), case.d("wu"), case.d("wd"))
    Tc = cfg.tokens_per_call
    top_rows = [np.bincount(chunk_of(case, c)[0].reshape(-1), minlength=cfg.E).max()
                for c in range(cfg.ncalls)]
    skewed = int(np.argmax(top_rows))
    ws = None
    for c in range(cfg.ncalls):
        ids, w, x = chunk_of(case, c)
        for packed in ((pk, None) if c in (0, cfg.ncalls - 1, skewed) else (pk,)):
            say(f"[forward] long_skewed_fp16 chunk {c} (top expert {top_rows[c]} rows), "
                f"{'packed' if packed else 'row-major'}")
            out, ws = abi.forward(dev(x, cfg.dtype), dev(ids), dev(w), case.d("wg"),
                                  case.d("wu"), case.d("wd"), tm=cfg.tm, workspace=ws,
                                  packed=packed)
            torch.cuda.synchronize()
            compare_all(case, ids, w, x, host(out), c * Tc, ref_r, nx=64, seed=cfg.seed + c)
    del pk, out, ws
    case.drop_device()


@pytest.mark.parametrize("cfg", [synth.CONFIGS["prefill_fp16"], synth.CONFIGS["decode_bf16"],
                                 PATHS[-1]], ids=["prefill_fp16", "decode_bf16_split",
                                                  "tall_split_unit_bf16"])
def test_forward_deterministic(cfg):
    """bitwise equal on a second call (split-K partials are added in a fixed
    order), the first call on a workspace full of garbage (the plan rewrites the
    FFN's work list), and the result against the oracle"""
    case = make_case(cfg)
    say(f"[forward determinism] {cfg.name}")
    need = abi.moe_forward_workspace(cfg.T, cfg.K, cfg.E, cfg.d, cfg.f, cfg.tm,
                                     abi.DTYPE_NAME[cfg.dtype])
    a, ws = gpu_forward(case, case.ids, case.w, case.x, polluted(need // 4 + 1).view(torch.uint8))
    b, _ = gpu_forward(case, case.ids, case.w, case.x, ws)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    toks = np.unique(np.linspace(0, cfg.T - 1, min(cfg.T, 24)).astype(np.int32))
    ref = oracle.ffn(case.x, case.ids, case.w, case.wg, case.wu, case.wd, cfg.dtype, True,
                     tokens=toks)
    assert rel_err(a[toks], ref.astype(np.float32)) <= TOL[cfg.dtype]
    case.drop_device()


def test_forward_skipped_entries():
    cfg = custom("tail_skipping", T=128, d=256, E=16, K=4, f=128, dtype="f16")
    case = make_case(cfg)
    ids = case.ids.copy()
    g = np.random.default_rng(0)
    ids[g.random(ids.shape) < 0.3] = -1  # skipped experts
    ids[5, :] = -1                       # a token with no expert at all
    got, _ = gpu_forward(case, ids, case.w, case.x)
    compare(case, ids, case.w, case.x, got, np.arange(cfg.T, dtype=np.int32))
    assert np.all(got[5] == 0) and not np.any(np.signbit(got[5]))


def compact_outputs(ws, cfg, T, K):
    """moe_forward's expert outputs in the compact format, read from its workspace:
    binary16 rows [R, d] (uint16 bits), their block exponents as [R, nb] (int8;
    stored block-major, [nb][R]), the entry rows pos and the plan's nr"""
    dt = abi.DTYPE_NAME[cfg.dtype]
    L = abi.moe_forward_layout(T, K, cfg.E, cfg.d, cfg.f, cfg.tm, dt)
    R = abi.moe_plan_sizes(T, K, cfg.E, cfg.tm).max_rows
    nb = (cfg.d + 127) // 128
    raw = ws.cpu().numpy()
    s16 = raw[L.y: L.y + R * cfg.d * 2].view(np.uint16).reshape(R, cfg.d)
    ex = raw[L.y + R * cfg.d * 2: L.y + R * cfg.d * 2 + R * nb].view(np.int8).reshape(nb, R).T
    ex = np.ascontiguousarray(ex)
    pos = raw[L.pos: L.pos + 4 * T * K].view(np.int32)
    stok = raw[L.stok: L.stok + 4 * R].view(np.int32)
    nr = int(raw[L.meta: L.meta + 44].view(np.int32)[2])
    return s16, ex, pos, stok, nr


FOUR = [synth.CONFIGS["decode_bf16"], synth.CONFIGS["tiny_fp32"], PATHS[0],
        custom("no_split_f16", T=2048, d=2048, E=64, K=4, f=1024, dtype="f16"),
        custom("ragged_d_bf16", T=300, d=328, E=12, K=3, f=200, dtype="bf16", x_std=1.0)]


@pytest.mark.parametrize("cfg", FOUR, ids=["decode_bf16_split_gateup", "tiny_fp32_split_down",
                                           "split_both_bf16", "no_split_f16", "ragged_d_bf16"])
@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
def test_forward_equals_the_four_calls(cfg, packed):
    """moe_forward (one-launch plan, gather fused into gate/up) against moe_plan,
    moe_gather, moe_expert_ffn and moe_combine called one by one. fp32 layers: the
    same bits. fp16/bf16 layers keep the expert outputs in the compact format: its
    rows equal the oracle's encoding of the four calls' fp32 rows bit for bit, and
    its output equals the oracle's fixed-order combine over them bit for bit"""
    case = make_case(cfg)
    say(f"[forward vs four calls] {cfg.name} packed={packed}")
    T, K = case.ids.shape
    dt = abi.DTYPE_NAME[cfg.dtype]
    x, ids, w = dev(case.x, cfg.dtype), dev(case.ids), dev(case.w)
    pk = abi.pack(case.d("wg"), case.d("wu"), case.d("wd")) if packed else None
    wts = (pk["gate"], pk["up"], pk["down"]) if packed else (case.d("wg"), case.d("wu"),
                                                              case.d("wd"))
    a, ws = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm,
                        packed=pk)
    p = abi.plan(ids, w, cfg.E, cfg.tm)
    R = p["sizes"].max_rows
    xs = torch.empty((R, cfg.d), dtype=x.dtype, device="cuda")
    abi.moe_gather(x, dt, T, cfg.d, p["stok"], p["meta"], R, xs)
    h = torch.empty((R, cfg.f), dtype=x.dtype, device="cuda")
    y = torch.empty((R, cfg.d), dtype=torch.float32, device="cuda")
    scratch = torch.empty(abi.moe_ffn_scratch_bytes(cfg.E, cfg.d, cfg.f, cfg.tm, R, dt),
                          dtype=torch.uint8, device="cuda")
    ffn = abi.moe_expert_ffn_packed if packed else abi.moe_expert_ffn
    ffn(xs, *wts, dt, cfg.E, cfg.d, cfg.f, cfg.tm, p["eoff"], p["stok"], p["sw"], p["meta"], R,
        h, y, scratch)
    b = torch.empty((T, cfg.d), dtype=torch.float32, device="cuda")
    abi.moe_combine(y, R, p["pos"], T, K, cfg.d, b)
    torch.cuda.synchronize()
    if cfg.dtype == "f32":
        assert np.array_equal(host(a).view(np.uint32), host(b).view(np.uint32))
    else:
        s16, ex, pos, stok, nr = compact_outputs(ws, cfg, T, K)
        real = np.nonzero(stok[:nr] >= 0)[0]
        want_s, want_e = oracle.y16_encode(host(y)[real])
        assert np.array_equal(s16[real], want_s)
        assert np.array_equal(ex[real], want_e)
        out = oracle.combine_y16(s16, ex, pos, T, K)
        assert np.array_equal(host(a).view(np.uint32), out.view(np.uint32))
    case.drop_device()


@pytest.mark.parametrize("name", ["prefill_fp16", "ubatch_bf16", "prefill_tailskip_fp16"])
def test_forward_combine_over_compact_outputs_full_size(name):
    """at full size (packed weights, as the benchmark runs it), every token's output
    is the oracle's fixed-order combine over the layer's own compact expert
    outputs, bit for bit"""
    cfg = synth.CONFIGS[name]
    case = make_case(cfg)
    say(f"[forward compact combine] {name}")
    pk = abi.pack(case.d("wg"), case.d("wu"), case.d("wd"))
    out, ws = abi.forward(dev(case.x, cfg.dtype), dev(case.ids), dev(case.w), case.d("wg"),
                          case.d("wu"), case.d("wd"), tm=cfg.tm, packed=pk)
    torch.cuda.synchronize()
    T, K = case.ids.shape
    s16, ex, pos, _, _ = compact_outputs(ws, cfg, T, K)
    want = oracle.combine_y16(s16, ex, pos, T, K)
    assert np.array_equal(host(out).view(np.uint32), want.view(np.uint32))
    del pk, ws
    case.drop_device()


def test_forward_activation_of_2gib_gathers_first():
    """x of 2 GiB (T=131072, d=8192, fp16) is past what one buffer descriptor
    addresses, so moe_forward gathers the rows first (moe_gather's kernel,
    64-bit row offsets) and the gate/up projection reads them row-major. A
    token's output depends only on its own row: sampled tokens get seeded random
    rows (checked against the oracle), all others zero rows, whose output must
    be exactly zero."""
    from gpu_util import Case
    cfg = custom("x_2gib_f16", T=131072, d=8192, E=4, K=1, f=64, dtype="f16")
    assert cfg.T * cfg.d * 2 >= 1 << 31
    ids, w = synth.routing(cfg)
    toks = sample_tokens(cfg.T, cfg.seed, n=12)
    x = np.zeros((cfg.T, cfg.d), np.uint16)
    x[toks] = synth.to_dtype(synth.random_rows(cfg.seed, len(toks), cfg.d, std=0.02), "f16")
    case = Case(cfg, ids, w, x, synth.expert_weights(cfg, "gate"), synth.expert_weights(cfg, "up"),
                synth.expert_weights(cfg, "down"))
    say(f"[forward] {cfg.name}")
    got, _ = gpu_forward(case, case.ids, case.w, case.x)
    compare(case, case.ids, case.w, case.x, got, toks)
    got[toks] = 0.0
    assert not np.any(got.view(np.uint32))  # +0.0 on every other token
    case.drop_device()
