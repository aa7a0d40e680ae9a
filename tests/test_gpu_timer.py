"""moe_forward_timed / moe_forward_packed_timed (the per-kernel HIP events the
benchmark reads): a timed call returns the same bits as an untimed one; every
stage the call launches is counted once per call (the one-launch plan counts
as the placement; above 32,768 entries the plan is three launches and the work
list its own); only the stages in the mask are recorded; a full timer is
refused; the recorded times are positive and fit inside the calls' wall time."""
import time

import numpy as np
import pytest
import torch

from gpu_util import abi, custom, dev, host, make_case, say, synth

pytestmark = pytest.mark.gpu

CASES = [
    # (config, stages launched per call)
    (synth.CONFIGS["prefill_fp16"], {"place", "gateup", "down", "combine"}),
    (custom("timer_three_launch_f16", T=4096, d=128, E=48, K=10, f=64, dtype="f16",
            bias="normal0.5"), {"hist", "scan", "place", "worklist", "gateup", "down", "combine"}),
]


@pytest.mark.parametrize("cfg,stages", CASES, ids=[c[0].name for c in CASES])
@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
def test_timed_forward(cfg, stages, packed):
    case = make_case(cfg)
    T = cfg.tokens_per_call
    say(f"[timer] {cfg.name} packed={packed}")
    x, ids, w = dev(case.x[:T], cfg.dtype), dev(case.ids[:T]), dev(case.w[:T])
    wg, wu, wd = case.d("wg"), case.d("wu"), case.d("wd")
    pk = abi.pack(wg, wu, wd) if packed else None
    ref, ws = abi.forward(x, ids, w, wg, wu, wd, tm=cfg.tm, packed=pk)
    torch.cuda.synchronize()
    ref_bits = host(ref).view(np.uint32).copy()

    calls = 3
    timer = abi.Timer(capacity=calls)
    out = torch.empty_like(ref)
    t0 = time.perf_counter()
    for _ in range(calls):
        abi.forward(x, ids, w, wg, wu, wd, tm=cfg.tm, workspace=ws, out=out, timer=timer,
                    packed=pk)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    assert np.array_equal(host(out).view(np.uint32), ref_bits)
    st = timer.read()
    for s in abi.STAGES:
        ms, n = st[s]
        if s in stages:
            assert n == calls, (s, n)
            assert ms > 0, s
        else:
            assert n == 0 and ms == 0.0, (s, n, ms)
    assert sum(ms for ms, _ in st.values()) <= wall_ms

    # full: a fourth call is refused, and nothing is launched
    with pytest.raises(abi.MoeError):
        for _ in range(calls + 1):
            abi.forward(x, ids, w, wg, wu, wd, tm=cfg.tm, workspace=ws, out=out, timer=timer,
                        packed=pk)
    torch.cuda.synchronize()
    timer.close()

    # a mask: the gate/up kernel only
    only = abi.Timer(capacity=calls, stages=("gateup",))
    for _ in range(calls):
        abi.forward(x, ids, w, wg, wu, wd, tm=cfg.tm, workspace=ws, out=out, timer=only,
                    packed=pk)
    torch.cuda.synchronize()
    st = only.read()
    assert st["gateup"][1] == calls and st["gateup"][0] > 0
    assert all(n == 0 for s, (ms, n) in st.items() if s != "gateup")
    only.close()
    assert np.array_equal(host(out).view(np.uint32), ref_bits)
    case.drop_device()
