"""The library keeps no state between calls and enqueues every kernel on the
caller's stream: two different layers issued alternately on two streams (each
with its own workspace, so they may overlap on the GPU) give the same bits as
each layer run alone on the default stream."""
import numpy as np
import pytest
import torch

from gpu_util import abi, custom, dev, host, make_case, say

pytestmark = pytest.mark.gpu


def layer(cfg):
    case = make_case(cfg)
    x, ids, w = dev(case.x, cfg.dtype), dev(case.ids), dev(case.w)
    wg, wu, wd = case.d("wg"), case.d("wu"), case.d("wd")
    pk = abi.pack(wg, wu, wd)
    return case, (x, ids, w, wg, wu, wd), pk


def test_two_layers_on_two_streams():
    cfg_a = custom("streams_a_f16", T=1024, d=512, E=64, K=6, f=256, dtype="f16", bias="zipf1.1")
    cfg_b = custom("streams_b_bf16", T=6, d=1536, E=64, K=4, f=1024, dtype="bf16")  # split-K
    (case_a, args_a, pk_a), (case_b, args_b, pk_b) = layer(cfg_a), layer(cfg_b)
    ref_a, ws_a = abi.forward(*args_a, tm=cfg_a.tm, packed=pk_a)
    ref_b, ws_b = abi.forward(*args_b, tm=cfg_b.tm, packed=pk_b)
    torch.cuda.synchronize()
    bits_a, bits_b = host(ref_a).view(np.uint32).copy(), host(ref_b).view(np.uint32).copy()

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    out_a, out_b = torch.empty_like(ref_a), torch.empty_like(ref_b)
    say("[streams] alternating calls on two streams")
    for rep in range(4):
        out_a.fill_(float("nan"))
        out_b.fill_(float("nan"))
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        for _ in range(3):
            with torch.cuda.stream(s1):
                abi.forward(*args_a, tm=cfg_a.tm, workspace=ws_a, out=out_a, packed=pk_a)
            with torch.cuda.stream(s2):
                abi.forward(*args_b, tm=cfg_b.tm, workspace=ws_b, out=out_b, packed=pk_b)
        torch.cuda.synchronize()
        assert np.array_equal(host(out_a).view(np.uint32), bits_a), rep
        assert np.array_equal(host(out_b).view(np.uint32), bits_b), rep
    case_a.drop_device()
    case_b.drop_device()
