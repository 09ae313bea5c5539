"""Pins of the oracle's router (CPU only).

Page fact: the Part 2 blog, "Quantisation alone leaves a sparse execution
problem": a router scores the experts per token, the token picks 8 of 128,
and the chosen experts' outputs are weighted. The reading (the oracle's
header): the topk largest logits, largest first, ties to the lower id; the
weights are the softmax over the chosen logits.

Pinned against numpy's stable argsort (an independent selection routine),
scipy's softmax, closed forms (uniform logits, one dominant logit) and the
defining property that the weights are the renormalised full-softmax
probabilities.
"""
import numpy as np
import pytest
import scipy.special

import oracle
from synth import CONFIGS, router_logits


@pytest.mark.parametrize("T,E,topk", [(1, 1, 1), (7, 5, 3), (64, 8, 2), (256, 128, 8), (33, 1024, 16)])
def test_ids_are_stable_descending_argsort(T, E, topk):
    rng = np.random.default_rng(T * 1000 + E)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, ::5] = np.round(lg[:, ::5], 1)                 # plenty of exact ties
    ids, w = oracle.router(lg, topk)
    want = np.argsort(-lg, axis=1, kind="stable")[:, :topk]
    assert np.array_equal(ids, want)


def test_weights_are_softmax_of_chosen_and_renormalised_probabilities():
    rng = np.random.default_rng(3)
    lg = (rng.standard_normal((50, 128)) * 2).astype(np.float32)
    ids, w = oracle.router(lg, 8)
    sel = np.take_along_axis(lg.astype(np.float64), ids, axis=1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-14, atol=0)
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    pk = np.take_along_axis(p, ids, axis=1)
    assert np.allclose(w, pk / pk.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)               # largest first


def test_closed_forms():
    ids, w = oracle.router(np.zeros((3, 16), np.float32), 4)
    assert np.array_equal(ids, np.tile(np.arange(4), (3, 1)))   # all tied: lowest ids
    assert np.all(w == 0.25)
    lg = np.zeros((1, 8), np.float32)
    lg[0, 5] = 200.0                                      # one dominant expert
    ids, w = oracle.router(lg, 2)
    assert list(ids[0]) == [5, 0] and w[0, 0] == 1.0 and w[0, 1] < 1e-80
    with pytest.raises(ValueError):
        oracle.router(np.zeros((2, 4), np.float32), 5)     # topk > E


def test_agrees_with_a_float32_softmax_ranking():
    # ranking the fp32 softmax probabilities (numpy, the textbook route) picks
    # the same experts in the same order on N(0, 1) logits of the full
    # workload, and gives the same renormalised weights to fp32 rounding
    shp = CONFIGS["full"]
    lg = router_logits(shp, 0)
    p = np.exp(lg - lg.max(axis=1, keepdims=True), dtype=np.float32)
    p /= p.sum(axis=1, keepdims=True, dtype=np.float32)
    want = np.argsort(-p, axis=1, kind="stable")[:, :shp.topk]
    pk = np.take_along_axis(p, want, axis=1).astype(np.float64)
    ids, w = oracle.router(lg, shp.topk)
    assert np.array_equal(ids, want)
    assert np.allclose(w, pk / pk.sum(axis=1, keepdims=True), rtol=1e-6, atol=0)
