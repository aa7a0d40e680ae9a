"""moe_forward_packed_noalloc (the layer with its workspace in the library's
fixed per-GPU buffer, for callers that cannot allocate) against
moe_forward_packed with a caller workspace: the same bits, on two calls in a
row, the second with a smaller input (the buffer keeps the first call's
contents), and a request beyond the buffer refused. Collected last, so that it
also runs after every other GPU test in the same process."""
import numpy as np
import pytest
import torch

from gpu_util import abi, custom, dev, host, make_case, say, synth

pytestmark = pytest.mark.gpu


def reference(case, pk, x, ids, w):
    """moe_forward_packed with its own (torch) workspace"""
    cfg = case.cfg
    out, _ = abi.forward(x, ids, w, case.d("wg"), case.d("wu"), case.d("wd"), tm=cfg.tm,
                         packed=pk)
    torch.cuda.synchronize()
    return host(out)


def noalloc(case, pk, x, ids, w):
    cfg = case.cfg
    T, K = ids.shape
    out = torch.full((T, cfg.d), float("nan"), dtype=torch.float32, device="cuda")
    abi.moe_forward_packed_noalloc(x, ids, w, pk["gate"], pk["up"], pk["down"],
                                   abi.DTYPE_NAME[cfg.dtype], T, K, cfg.E, cfg.d, cfg.f, cfg.tm,
                                   out)
    torch.cuda.synchronize()
    return host(out)


CASES = [
    # the decode workload (split-K gate/up: partial sums in the fixed buffer), then
    # its first two tokens
    (synth.CONFIGS["decode_bf16"], 2),
    # a small fp16 prefill-like layer, then a third of its tokens
    (custom("noalloc_f16", T=384, d=512, E=32, K=4, f=256, dtype="f16"), 128),
]


@pytest.mark.parametrize("cfg,t2", CASES, ids=[c[0].name for c in CASES])
def test_noalloc_equals_forward_packed_on_two_calls(cfg, t2):
    case = make_case(cfg)
    pk = abi.pack(case.d("wg"), case.d("wu"), case.d("wd"))
    x, ids, w = dev(case.x, cfg.dtype), dev(case.ids), dev(case.w)
    need = abi.moe_forward_workspace(cfg.T, cfg.K, cfg.E, cfg.d, cfg.f, cfg.tm,
                                     abi.DTYPE_NAME[cfg.dtype])
    assert need <= abi.NOALLOC_WORKSPACE_BYTES
    for T in (cfg.T, t2):  # the second call is smaller
        say(f"[noalloc] {cfg.name} T={T}")
        xs, idss, ws = x[:T].contiguous(), ids[:T].contiguous(), w[:T].contiguous()
        want = reference(case, pk, xs, idss, ws)
        got = noalloc(case, pk, xs, idss, ws)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (cfg.name, T)
    case.drop_device()


def test_noalloc_refuses_a_request_beyond_its_buffer():
    cfg = synth.CONFIGS["prefill_fp16"]
    assert abi.moe_forward_workspace(cfg.T, cfg.K, cfg.E, cfg.d, cfg.f, cfg.tm,
                                     abi.MOE_F16) > abi.NOALLOC_WORKSPACE_BYTES
    x = torch.zeros((cfg.T, cfg.d), dtype=torch.float16, device="cuda")
    ids = torch.zeros((cfg.T, cfg.K), dtype=torch.int32, device="cuda")
    w = torch.zeros((cfg.T, cfg.K), dtype=torch.float32, device="cuda")
    wt = torch.zeros(16, dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.T, cfg.d), dtype=torch.float32, device="cuda")
    with pytest.raises(abi.MoeError) as e:
        abi.moe_forward_packed_noalloc(x, ids, w, wt, wt, wt, abi.MOE_F16, cfg.T, cfg.K, cfg.E,
                                       cfg.d, cfg.f, cfg.tm, out)
    assert e.value.status == 4
