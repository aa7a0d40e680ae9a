"""moe_forward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: the
layer allocates nothing, clears nothing with memset and never waits on the
host, so a serving loop can capture it once. Every replay must give the same
bits as an eager call on the same inputs, with eager work and synchronisation
between replays, and a replay after new routing is copied into the captured
input tensors must give the eager result for the new inputs (nothing about
the routing is baked into the graph). Eager moe_forward itself is checked
against the oracle in test_gpu_forward / test_gpu_packed."""
import numpy as np
import pytest
import torch

from gpu_util import abi, custom, dev, host, make_case, say, synth

pytestmark = pytest.mark.gpu

CASES = [
    synth.CONFIGS["decode_bf16"],    # split-K with its reduction kernels
    synth.CONFIGS["prefill_fp16"],   # one-launch plan, gather fused into gate/up
    custom("graph_big_cells_f16", T=2048, d=328, E=4, K=2, f=320, dtype="f16", bias="zipf1.1"),
    custom("graph_three_launch_plan_f16", T=4096, d=128, E=48, K=10, f=64, dtype="f16",
           bias="normal0.5"),        # T*K > 32,768: hist, scan, place and a work-list launch
]


def other_routing(cfg, T):
    """a second routing of the same shape (another seed)"""
    g = np.random.default_rng(cfg.seed + 7777)
    ids = np.stack([g.permutation(cfg.E)[:cfg.K] for _ in range(T)]).astype(np.int32)
    w = g.random((T, cfg.K)).astype(np.float32)
    return ids, w / w.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_forward_graph_replays(cfg):
    case = make_case(cfg)
    T = cfg.tokens_per_call
    say(f"[graph] {cfg.name}: T={T}")
    x = dev(case.x[:T], cfg.dtype)
    ids, w = dev(case.ids[:T]), dev(case.w[:T])
    wg, wu, wd = case.d("wg"), case.d("wu"), case.d("wd")
    pk = abi.pack(wg, wu, wd) if cfg.dtype != "f32" else None

    ref, ws_ref = abi.forward(x, ids, w, wg, wu, wd, tm=cfg.tm, packed=pk)
    torch.cuda.synchronize()
    ref_bits = host(ref).view(np.uint32).copy()

    _, ws = abi.forward(x, ids, w, wg, wu, wd, tm=cfg.tm, packed=pk)
    out = torch.empty_like(ref)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        abi.forward(x, ids, w, wg, wu, wd, tm=cfg.tm, workspace=ws, out=out, packed=pk)
    torch.cuda.synchronize()

    for rep in range(3):
        out.fill_(float("nan"))  # eager work between replays
        ws[: ws.numel() // 2].fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), ref_bits), f"replay {rep}"

    # new routing into the captured tensors: the replay follows it
    ids2, w2 = other_routing(cfg, T)
    ids.copy_(torch.from_numpy(ids2))
    w.copy_(torch.from_numpy(w2))
    ref2, _ = abi.forward(x, ids, w, wg, wu, wd, tm=cfg.tm, workspace=ws_ref, packed=pk)
    torch.cuda.synchronize()
    out.fill_(float("nan"))
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint32), host(ref2).view(np.uint32))
    assert not np.array_equal(host(ref2).view(np.uint32), ref_bits)
    del graph, pk
    case.drop_device()
