"""Pins for the oracle's router (top-K of the logits, renormalised softmax):
numpy's stable argsort and an fp64 softmax, ties, NaN, K = E, and the
generator's own routing on the same logits."""
import numpy as np
import pytest

import oracle
from mixture_experts_routed_amd import synth


def ref_route(logits, K):
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :K]
    sel = np.take_along_axis(logits.astype(np.float64), order, axis=1)
    p = np.exp(logits.astype(np.float64) - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)  # full softmax, then top-K renormalised
    pk = np.take_along_axis(p, order, axis=1)
    return order.astype(np.int32), pk / pk.sum(axis=1, keepdims=True), sel


@pytest.mark.parametrize("T,E,K", [(50, 8, 2), (200, 512, 10), (7, 128, 8), (3, 5, 5), (9, 1, 1),
                                   (20, 1024, 64)])
def test_route_matches_stable_argsort_and_softmax(T, E, K):
    g = np.random.default_rng(T * E + K)
    logits = g.standard_normal((T, E)).astype(np.float32)
    ids, w = oracle.route_topk(logits, K)
    rid, rw, _ = ref_route(logits, K)
    assert np.array_equal(ids, rid)
    assert np.max(np.abs(w - rw)) <= 1e-13
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)  # descending


def test_route_ties_go_to_lower_id():
    logits = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, -1.0]], np.float32)
    ids, w = oracle.route_topk(logits, 4)
    assert ids.tolist() == [[1, 2, 4, 3]]
    assert np.allclose(w[0, :3], w[0, 0]) and w[0, 3] < w[0, 0]
    g = np.random.default_rng(1)
    rough = np.round(g.standard_normal((300, 64)), 1).astype(np.float32)  # many ties
    ids, _ = oracle.route_topk(rough, 8)
    assert np.array_equal(ids, ref_route(rough, 8)[0])


def test_route_nan_never_picked_and_short_rows():
    logits = np.array([[np.nan, 0.5, np.nan, 0.25], [np.nan, np.nan, np.nan, 1.0]], np.float32)
    ids, w = oracle.route_topk(logits, 3)
    assert ids.tolist() == [[1, 3, -1], [3, -1, -1]]
    assert w[1].tolist() == [1.0, 0.0, 0.0]
    assert abs(w[0, :2].sum() - 1.0) < 1e-15 and w[0, 2] == 0.0


def test_route_shift_invariance_and_two_experts():
    g = np.random.default_rng(3)
    logits = g.standard_normal((40, 16)).astype(np.float32)
    ids, w = oracle.route_topk(logits, 2)
    # K = 2 closed form: w0 = sigmoid(l0 - l1)
    l0 = np.take_along_axis(logits, ids[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(logits, ids[:, 1:], 1)[:, 0].astype(np.float64)
    assert np.allclose(w[:, 0], 1 / (1 + np.exp(l1 - l0)), rtol=1e-14, atol=0)
    ids2, w2 = oracle.route_topk((logits + np.float32(8.0)).astype(np.float32), 2)
    assert np.array_equal(ids2[np.abs(logits).max(axis=1) < 4], ids[np.abs(logits).max(axis=1) < 4])


def test_route_agrees_with_generator_routing():
    cfg = synth.CONFIGS["prefill_fp16"]
    ids_gen, w_gen = synth.routing(cfg)
    ids, w = oracle.route_topk(synth.router_logits(cfg), cfg.K)
    # fp32 rounding of the logits may swap picks that are nearly tied in fp64
    same = (ids == ids_gen).all(axis=1)
    assert same.mean() > 0.999
    assert np.max(np.abs(w[same] - w_gen[same])) < 1e-5
