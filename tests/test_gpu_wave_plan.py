"""A call of at most 64 (token, expert) entries whose experts each get one work
item (tm divides 64) is planned inside moe_forward's gate/up launch: the
launch's first workgroup writes the plan and the work list, and every other
workgroup finds its work item from the ids alone. The plan it leaves in the
workspace must equal moe_plan's outputs bit for bit, and its work list must be
the routed experts in ascending order, one single item each, starting at the
expert's padded row offset (the layer's outputs are checked against the oracle
and against the four separate calls in test_gpu_forward.py)."""
import numpy as np
import pytest
import torch

from gpu_util import abi, dev, host, say, synth

pytestmark = pytest.mark.gpu

# T, K, E, tm, p_skip, p_bad, dtype, seed
CASES = [
    (4, 8, 128, 16, 0.0, 0.0, "bf16", 1),     # decode-shaped
    (1, 1, 1, 16, 0.0, 0.0, "f16", 2),        # one entry
    (8, 8, 1024, 16, 0.1, 0.05, "f32", 3),    # 64 entries, 1024 experts, skipped and bad ids
    (16, 4, 4, 1, 0.0, 0.0, "bf16", 4),       # tm 1, four experts shared by many entries
    (2, 32, 100, 64, 0.5, 0.0, "f16", 5),     # half skipped, tm 64
    (64, 1, 1, 64, 0.0, 0.0, "f32", 6),       # one expert with all 64 entries: one full item
    (3, 16, 16, 8, 0.2, 0.2, "f16", 7),       # K = E (duplicates), ragged
    (5, 2, 8, 32, 1.0, 0.0, "bf16", 8),       # every entry skipped: no items
]


def ws_view(ws, off, n, dtype=torch.int32):
    n = max(int(n), 0)
    return ws[off: off + 4 * n].view(dtype)


@pytest.mark.parametrize("T,K,E,tm,ps,pb,dtype,seed", CASES)
def test_in_launch_plan_equals_moe_plan(T, K, E, tm, ps, pb, dtype, seed):
    say(f"[in-launch plan] T={T} K={K} E={E} tm={tm} skip={ps} bad={pb} {dtype}")
    d = f = 64
    ids_h = synth.random_ids(seed, T, K, E, p_skip=ps, p_bad=pb)
    w_h = synth.random_rows(seed, T, K)
    g = np.random.default_rng(seed)
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    x = torch.from_numpy(g.standard_normal((T, d), dtype=np.float32)).to("cuda", tdt)
    wts = [torch.from_numpy(0.05 * g.standard_normal(s, dtype=np.float32)).to("cuda", tdt)
           for s in ((E, d, f), (E, d, f), (E, f, d))]
    ids, w = dev(ids_h), dev(w_h)
    out, ws = abi.forward(x, ids, w, *wts, tm=tm)
    p = abi.plan(ids, w, E, tm)
    torch.cuda.synchronize()
    L = abi.moe_forward_layout(T, K, E, d, f, tm, abi.DTYPE_OF[tdt])
    meta = host(p["meta"])
    assert np.array_equal(host(ws_view(ws, L.meta, abi.META_N)), meta)
    nr, nt = int(meta[2]), int(meta[3])
    for name, n, dt in (("cnt", E, torch.int32), ("eoff", E + 1, torch.int32),
                        ("stok", nr, torch.int32), ("sw", nr, torch.float32),
                        ("pos", T * K, torch.int32), ("tiles", nt, torch.int32)):
        got = host(ws_view(ws, getattr(L, name), n, dt))
        want = host(p[name])[:n]
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), name
    # the work list: the routed experts ascending, one single item each
    cnt, eoff = host(p["cnt"]), host(p["eoff"])
    routed = np.nonzero(cnt > 0)[0]
    ctl = host(ws_view(ws, L.ffn_scratch, 3))
    assert ctl[0] == len(routed) and ctl[1] == 0 and ctl[2] == 0
    items = host(ws_view(ws, L.ffn_scratch + 256, 4 * len(routed))).reshape(-1, 4)
    want = np.stack([routed, eoff[routed], np.minimum(64, eoff[routed + 1] - eoff[routed]),
                     np.ones_like(routed)], axis=1) if len(routed) else np.zeros((0, 4))
    assert np.array_equal(items, want.astype(np.int32))
    assert torch.isfinite(out).all()
