"""Expert weights in host memory (moe_forward_host_weights): the routed experts
are given slots of a device cache (a ring over the slots: resident experts
keep theirs, new ones take the next free slots from the hand, in ascending
expert order), the new ones' matrices are copied from pinned host memory, and
the work list is renumbered to slots. So the layer must give the same bits as
moe_forward / moe_forward_packed on device copies of the same weights (that
path is itself checked against the oracle in test_gpu_forward /
test_gpu_packed), whatever the cache held. Also: the cache state after every
call of a sequence against a model of the ring, a cache reused by calls with
other routing, and pageable host memory refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import abi, custom, dev, host, make_case, replace, say, synth

pytestmark = pytest.mark.gpu

CASES = [
    synth.CONFIGS["tiny_fp32"],
    synth.CONFIGS["decode_bf16"],
    custom("few_items_skewed_f16", T=130, d=256, E=64, K=3, f=136, dtype="f16", bias="zipf1.1"),
    custom("ragged_tails_bf16", T=96, d=328, E=12, K=3, f=200, dtype="bf16", x_std=1.0),
    custom("tm48_f16", T=200, d=96, E=16, K=3, f=80, dtype="f16", tm=48),
    custom("max_experts_f16", T=300, d=64, E=1024, K=8, f=64, dtype="f16"),
    custom("ragged_tails_f32", T=80, d=136, E=6, K=2, f=72, dtype="f32", x_std=1.0),
    # skipped slots (id -1): their experts need no slot unless another entry routes there
    replace(custom("tail_skip_f16", T=96, d=256, E=32, K=4, f=128, dtype="f16"), tail_skip=0.75),
]


def pinned(t):
    """a new pinned host tensor holding t (allocated pinned, then filled)"""
    out = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    out.copy_(t)
    return out


def host_sets(case, packed):
    """(device sets, pinned host sets) of the layer's three matrices"""
    wg, wu, wd = case.d("wg"), case.d("wu"), case.d("wd")
    if packed:
        pk = abi.pack(wg, wu, wd)
        devs = (pk["gate"], pk["up"], pk["down"])
    else:
        devs = (wg, wu, wd)
    torch.cuda.synchronize()
    return devs, tuple(pinned(t.cpu()) for t in devs)


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_host_weights_equal_device_weights(cfg, packed):
    case = make_case(cfg)
    T = cfg.tokens_per_call
    say(f"[host weights] {cfg.name} packed={packed}")
    x, ids, w = dev(case.x[:T], cfg.dtype), dev(case.ids[:T]), dev(case.w[:T])
    devs, hosts = host_sets(case, packed)
    ref, _ = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm,
                         packed=dict(zip(("gate", "up", "down"), devs)) if packed else None)
    got, cache, _ = abi.forward_host(x, ids, w, *hosts, tm=cfg.tm, packed=packed,
                                     shapes=(cfg.E, cfg.d, cfg.f))
    torch.cuda.synchronize()
    assert np.array_equal(host(got).view(np.uint32), host(ref).view(np.uint32))
    # the slot table: slot s = the s-th expert with entries, ascending; -1 otherwise
    p = oracle.plan(case.ids[:T], case.w[:T], cfg.E, cfg.tm)
    cnt = np.asarray(p["cnt"])
    want = np.full(cfg.E, -1, np.int32)
    act = np.nonzero(cnt > 0)[0]
    want[act] = np.arange(len(act), dtype=np.int32)
    table = host(cache[256: 256 + 4 * cfg.E]).view(np.int32)
    assert np.array_equal(table, want)
    del devs, hosts, cache
    case.drop_device()


def r256(v):
    return (v + 255) // 256 * 256


def ring_model(slot_of, exp_of, hand, routed, S):
    """one call of the cache ring: routed experts (ascending) without a slot take
    the free slots (those not holding an expert this call routes to) in ring
    order from the hand, evicting what they held; returns (hand, copies)"""
    rset = set(routed)
    new = [e for e in routed if slot_of[e] < 0]
    free = [(hand + q) % S for q in range(S)
            if not (exp_of[(hand + q) % S] >= 0 and exp_of[(hand + q) % S] in rset)]
    copies = []
    for r, e in enumerate(new):
        sl = free[r]
        if exp_of[sl] >= 0:
            slot_of[exp_of[sl]] = -1
        slot_of[e] = sl
        exp_of[sl] = e
        copies.append((sl, e))
    if new:
        hand = (free[len(new) - 1] + 1) % S
    return hand, copies


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("slots", [32, 48, 128])
def test_cache_ring_state_and_outputs_over_a_sequence(slots, packed):
    """eight decode calls (4 tokens, top-8 of 128 experts) with different routing
    through one cache of `slots` slots: after every call the hand, the number of
    experts copied, slot_of and exp_of equal the ring model, and the output equals
    the device-weight layer bit for bit"""
    cfg = replace(synth.CONFIGS["decode_bf16"], T=32, chunk=4)
    case = make_case(cfg)
    T, E = cfg.tokens_per_call, cfg.E
    devs, hosts = host_sets(case, packed)
    pk = dict(zip(("gate", "up", "down"), devs)) if packed else None
    slot_of, exp_of, hand = [-1] * E, [-1] * slots, 0
    cache = ws = None
    off_exp = r256(256 + 4 * E)
    copied = 0
    for c in range(cfg.ncalls):
        sl = slice(c * T, (c + 1) * T)
        x, ids, w = dev(case.x[sl], cfg.dtype), dev(case.ids[sl]), dev(case.w[sl])
        ref, _ = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm,
                             packed=pk)
        got, cache, ws = abi.forward_host(x, ids, w, *hosts, tm=cfg.tm, packed=packed,
                                          shapes=(E, cfg.d, cfg.f), slots=slots, cache=cache,
                                          workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(got).view(np.uint32), host(ref).view(np.uint32)), c
        cid = case.ids[sl]
        routed = sorted(set(int(e) for e in cid.ravel() if 0 <= e < E))
        hand, copies = ring_model(slot_of, exp_of, hand, routed, slots)
        copied += len(copies)
        hdr = host(cache[:8]).view(np.int32)
        assert (int(hdr[0]), int(hdr[1])) == (hand, len(copies)), c
        assert np.array_equal(host(cache[256: 256 + 4 * E]).view(np.int32), np.array(slot_of))
        assert np.array_equal(host(cache[off_exp: off_exp + 4 * slots]).view(np.int32),
                              np.array(exp_of))
    # a cache of every expert copies each routed expert once; smaller ones may
    # copy some again after evicting them
    nrouted = len(set(int(e) for e in case.ids.ravel() if 0 <= e < E))
    assert copied >= nrouted and (slots < E or copied == nrouted)
    del devs, hosts, pk, cache
    case.drop_device()


def test_one_cache_serves_calls_with_other_routing():
    """the cache is rewritten by every call: three calls with different routing
    (the skewed long prompt's first chunks) share one cache and one workspace,
    each equal to the device-weight layer"""
    cfg = synth.CONFIGS["long_skewed_fp16"]
    case = make_case(cfg)
    T = cfg.tokens_per_call
    devs, hosts = host_sets(case, True)
    pk = dict(zip(("gate", "up", "down"), devs))
    cache = ws = None
    for c in range(3):
        sl = slice(c * T, (c + 1) * T)
        say(f"[host weights] long_skewed chunk {c}")
        x, ids, w = dev(case.x[sl], cfg.dtype), dev(case.ids[sl]), dev(case.w[sl])
        ref, _ = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm,
                             packed=pk)
        got, cache, ws = abi.forward_host(x, ids, w, *hosts, tm=cfg.tm, packed=True,
                                          shapes=(cfg.E, cfg.d, cfg.f), cache=cache, workspace=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(got).view(np.uint32), host(ref).view(np.uint32)), c
    del devs, hosts, pk, cache
    case.drop_device()


def test_pageable_host_memory_is_refused():
    """weights in ordinary (pageable) host memory are refused with MOE_EINVAL
    before any launch; the output is left untouched"""
    cfg = synth.CONFIGS["tiny_fp32"]
    case = make_case(cfg)
    T = cfg.tokens_per_call
    x, ids, w = dev(case.x[:T], cfg.dtype), dev(case.ids[:T]), dev(case.w[:T])
    pageable = tuple(torch.from_numpy(np.ascontiguousarray(a)) for a in (case.wg, case.wu, case.wd))
    out = torch.full((T, cfg.d), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(abi.MoeError) as e:
        abi.forward_host(x, ids, w, *pageable, tm=cfg.tm, out=out)
    assert e.value.status == 1
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
    case.drop_device()


def test_host_weights_layer_in_a_graph():
    """moe_forward_host_weights captured in a HIP graph and replayed: the cache
    ring is driven by the GPU alone (no memset, no host wait), so three replays
    with eager work between them equal the device-weight layer, and a replay
    after new routing is copied into the captured inputs copies the newly
    routed experts in and equals the device-weight layer on that routing"""
    cfg = synth.CONFIGS["decode_bf16"]
    case = make_case(cfg)
    T, E = cfg.tokens_per_call, cfg.E
    x, ids, w = dev(case.x[:T], cfg.dtype), dev(case.ids[:T]), dev(case.w[:T])
    devs, hosts = host_sets(case, True)
    pk = dict(zip(("gate", "up", "down"), devs))
    ref, _ = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm, packed=pk)
    torch.cuda.synchronize()
    ref_bits = host(ref).view(np.uint32).copy()
    shapes = (E, cfg.d, cfg.f)
    _, cache, ws = abi.forward_host(x, ids, w, *hosts, tm=cfg.tm, packed=True, shapes=shapes)
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        abi.forward_host(x, ids, w, *hosts, tm=cfg.tm, packed=True, shapes=shapes, cache=cache,
                         workspace=ws, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        ws[: ws.numel() // 2].fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), ref_bits), f"replay {rep}"
    # new routing: experts the cache does not hold are copied in by the replay
    g = np.random.default_rng(99)
    ids2 = np.stack([g.permutation(E)[:cfg.K] for _ in range(T)]).astype(np.int32)
    ids.copy_(torch.from_numpy(ids2))
    ref2, _ = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm,
                          packed=pk)
    torch.cuda.synchronize()
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint32), host(ref2).view(np.uint32))
    assert int(host(cache[4:8]).view(np.int32)[0]) > 0  # the replay copied experts in
    del graph, devs, hosts, pk, cache
    case.drop_device()
