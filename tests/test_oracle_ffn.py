"""Pins for the oracle's expert FFN: brute force (every expert on every token,
then masked), the reduction to a dense SwiGLU MLP in torch fp64, metamorphic
relations, and the per-entry outputs against the per-token sum."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_routed_amd import synth


def tiny(dtype, T=6, d=16, E=5, K=2, f=24, seed=3, x_std=0.5, w_std=0.3):
    g = np.random.default_rng(seed)
    x = synth.to_dtype(g.standard_normal((T, d)).astype(np.float32) * x_std, dtype)
    wg = synth.to_dtype(g.standard_normal((E, d, f)).astype(np.float32) * w_std, dtype)
    wu = synth.to_dtype(g.standard_normal((E, d, f)).astype(np.float32) * w_std, dtype)
    wd = synth.to_dtype(g.standard_normal((E, f, d)).astype(np.float32) * w_std, dtype)
    ids = np.stack([g.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    w = g.random((T, K)).astype(np.float32)
    return x, ids, w, wg, wu, wd


def rel(a, b):
    return np.max(np.abs(a - b)) / np.max(np.abs(b))


@pytest.mark.parametrize("dtype", synth.DTYPES)
@pytest.mark.parametrize("round_h", [False, True])
def test_naive_loop_equals_dense_masked(dtype, round_h):
    x, ids, w, wg, wu, wd = tiny(dtype)
    a = oracle.ffn(x, ids, w, wg, wu, wd, dtype, round_h)
    b = oracle.dense_masked(x, ids, w, wg, wu, wd, dtype, round_h)
    assert rel(a, b) <= 1e-12


def test_dense_masked_with_duplicates_and_skips():
    x, ids, w, wg, wu, wd = tiny("f32", K=3)
    ids[0, 1] = ids[0, 0]  # same expert twice: both weights count
    ids[1, 2] = -1         # skipped entry
    ids[2, 0] = 99         # out of range entry
    a = oracle.ffn(x, ids, w, wg, wu, wd, "f32", False)
    b = oracle.dense_masked(x, ids, w, wg, wu, wd, "f32", False)
    assert rel(a, b) <= 1e-12


def _torch_mlp(x, wg, wu, wd, round_h_dtype=None):
    """out = (silu(x Wg) * (x Wu)) Wd in torch fp64 (one expert, weight 1)."""
    X = torch.from_numpy(x)
    h = torch.nn.functional.silu(X @ torch.from_numpy(wg)) * (X @ torch.from_numpy(wu))
    if round_h_dtype == "f16":
        h = h.to(torch.float16).to(torch.float64)
    elif round_h_dtype == "bf16":
        h = h.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    elif round_h_dtype == "f32":
        h = h.to(torch.float32).to(torch.float64)
    return (h @ torch.from_numpy(wd)).numpy(), h.numpy()


@pytest.mark.parametrize("dtype", synth.DTYPES)
def test_single_expert_reduces_to_dense_swiglu_mlp(dtype):
    T, d, f = 9, 32, 48
    x, ids, w, wg, wu, wd = tiny(dtype, T=T, d=d, E=1, K=1, f=f, seed=11)
    w[:] = 1.0
    xd, wgd, wud, wdd = (oracle.decode(a, dtype) for a in (x, wg[0], wu[0], wd[0]))
    ref, href = _torch_mlp(xd, wgd, wud, wdd)
    out = oracle.ffn(x, ids, w, wg, wu, wd, dtype, round_h=False)
    assert rel(out, ref) <= 1e-12
    y, h = oracle.ffn_entries(x, ids, w, wg, wu, wd, dtype, False, np.arange(T))
    assert rel(h, href) <= 1e-12 and rel(y, ref) <= 1e-12


def test_single_expert_rounded_h_matches_torch_rounding():
    # f16: torch rounds the fp64 h straight to half; the oracle does the same
    T, d, f = 9, 32, 48
    x, ids, w, wg, wu, wd = tiny("f16", T=T, d=d, E=1, K=1, f=f, seed=12)
    w[:] = 1.0
    xd, wgd, wud, wdd = (oracle.decode(a, "f16") for a in (x, wg[0], wu[0], wd[0]))
    ref, href = _torch_mlp(xd, wgd, wud, wdd, round_h_dtype="f16")
    y, h = oracle.ffn_entries(x, ids, w, wg, wu, wd, "f16", True, np.arange(T))
    assert np.array_equal(h, href)
    assert rel(y, ref) <= 1e-12


def test_silu_values():
    # E=1, d=1, f=1, identity-like weights: out = silu(x) * x * 1 with x exactly representable
    xs = np.array([[-30.0], [-2.0], [-0.5], [0.0], [0.25], [1.0], [3.0], [40.0]], np.float32)
    one = np.ones((1, 1, 1), np.float32)
    ids = np.zeros((len(xs), 1), np.int32)
    w = np.ones((len(xs), 1), np.float32)
    out = oracle.ffn(xs, ids, w, one, one, one, "f32", False)[:, 0]
    z = xs[:, 0].astype(np.float64)
    assert np.allclose(out, z * z / (1 + np.exp(-z)), rtol=1e-15, atol=0)
    assert out[3] == 0.0


def test_metamorphic_relabel_permute_scale_zero():
    dtype = "bf16"
    x, ids, w, wg, wu, wd = tiny(dtype, T=7, E=6, K=3, seed=21)
    base = oracle.ffn(x, ids, w, wg, wu, wd, dtype, True)
    # relabel experts: permute weight stacks and ids together
    perm = np.random.default_rng(0).permutation(6)
    inv = np.argsort(perm)
    out = oracle.ffn(x, inv[ids].astype(np.int32), w, wg[perm], wu[perm], wd[perm], dtype, True)
    assert np.array_equal(out, base)
    # permuting tokens permutes the output rows
    tp = np.random.default_rng(1).permutation(7)
    out = oracle.ffn(x[tp], ids[tp], w[tp], wg, wu, wd, dtype, True)
    assert np.array_equal(out, base[tp])
    # scaling every router weight by 2 scales the output exactly by 2
    out = oracle.ffn(x, ids, (w * 2).astype(np.float32), wg, wu, wd, dtype, True)
    assert np.array_equal(out, 2 * base)
    # a zero weight removes that term, the same as skipping the entry
    w0 = w.copy()
    w0[2, 1] = 0.0
    ids0 = ids.copy()
    ids0[2, 1] = -1
    a = oracle.ffn(x, ids, w0, wg, wu, wd, dtype, True)
    b = oracle.ffn(x, ids0, w, wg, wu, wd, dtype, True)
    assert np.array_equal(a, b)
    assert not np.array_equal(a[2], base[2])


def test_entries_sum_to_token_output_in_k_order():
    dtype = "f16"
    x, ids, w, wg, wu, wd = tiny(dtype, T=5, E=7, K=4, seed=31)
    out = oracle.ffn(x, ids, w, wg, wu, wd, dtype, True)
    y, _ = oracle.ffn_entries(x, ids, w, wg, wu, wd, dtype, True, np.arange(5 * 4))
    acc = np.zeros_like(out)
    for k in range(4):  # the same additions in the same order -> identical doubles
        acc = acc + y[k::4]
    assert np.array_equal(acc, out)


def test_token_subset_matches_full_run():
    dtype = "f32"
    x, ids, w, wg, wu, wd = tiny(dtype, T=12, E=4, K=2, seed=41)
    full = oracle.ffn(x, ids, w, wg, wu, wd, dtype, False)
    sub = oracle.ffn(x, ids, w, wg, wu, wd, dtype, False, tokens=[11, 0, 5])
    assert np.array_equal(sub, full[[11, 0, 5]])
