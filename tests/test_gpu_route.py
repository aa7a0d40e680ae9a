"""GPU parity of moe_route_topk against the oracle router: ids bit-exact,
weights within the fp32 bar (max|d|/max|ref| <= 1e-5)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import abi, rel_err, say, synth

pytestmark = pytest.mark.gpu


def gpu_route(logits, K):
    ids, w = abi.route(torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda(), K)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def check(logits, K, label):
    say(f"[route] {label}: T={logits.shape[0]} E={logits.shape[1]} K={K}")
    gi, gw = gpu_route(logits, K)
    ri, rw = oracle.route_topk(logits, K)
    assert np.array_equal(gi, ri), label
    assert rel_err(gw, rw) <= 1e-5, rel_err(gw, rw)
    return gi, gw


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_route_configs(name):
    cfg = synth.CONFIGS[name]
    T = min(cfg.T, 4096)
    check(synth.router_logits(cfg, T), cfg.K, name)


# E spans the kernel's logits-per-lane variants (2, 4, 8, 16 per lane) and
# each one's first size past the previous (129, 257, 513)
@pytest.mark.parametrize("T,E,K,seed", [(1, 1, 1, 0), (5, 3, 3, 1), (100, 64, 64, 2),
                                        (257, 1024, 16, 3), (33, 1000, 1, 4), (2048, 512, 10, 5),
                                        (40, 129, 8, 6), (40, 257, 4, 8), (40, 513, 8, 9)])
def test_route_shapes(T, E, K, seed):
    g = np.random.default_rng(seed)
    check(g.standard_normal((T, E)).astype(np.float32) * 3, K, f"seed {seed}")


def test_route_ties_nan_and_short_rows():
    g = np.random.default_rng(7)
    rough = np.round(g.standard_normal((300, 128)), 1).astype(np.float32)  # many equal logits
    check(rough, 12, "ties")
    nanny = g.standard_normal((64, 40)).astype(np.float32)
    nanny[g.random(nanny.shape) < 0.3] = np.nan
    nanny[3, :] = np.nan          # no finite logit
    nanny[4, 2:] = np.nan         # two finite logits, K = 6
    ids, w = check(nanny, 6, "nan")
    assert np.all(ids[3] == -1) and np.all(w[3] == 0)
    assert np.all(ids[4, 2:] == -1)
    neg = np.full((4, 16), -np.inf, np.float32)
    neg[:, 5] = 0.0
    check(neg, 3, "-inf")


def test_route_feeds_the_layer():
    """router -> forward on GPU equals oracle router -> oracle layer"""
    cfg = synth.CONFIGS["tiny_fp32"]
    logits = synth.router_logits(cfg)
    x = synth.activations(cfg)
    wg, wu, wd = (synth.expert_weights(cfg, k) for k in ("gate", "up", "down"))
    ids_d, w_d = abi.route(torch.from_numpy(logits).cuda(), cfg.K)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    out, _ = abi.forward(t(x), ids_d, w_d, t(wg), t(wu), t(wd), tm=cfg.tm)
    torch.cuda.synchronize()
    ri, rw = oracle.route_topk(logits, cfg.K)
    ref = oracle.ffn(x, ri, rw.astype(np.float32), wg, wu, wd, cfg.dtype, True)
    assert rel_err(out.cpu().numpy(), ref) <= 1e-5
