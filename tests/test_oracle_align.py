"""Pins of the oracle's token->expert alignment (Part 2 blog, 'Quantisation
alone leaves a sparse execution problem': sort assignments by expert, pad into
regular blocks) against numpy's bincount and stable argsort."""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, router_logits


def _check(ids, E, bm):
    r = oracle.align(ids, E, bm)
    flat = ids.ravel()
    A = flat.size
    cap = A + E * (bm - 1)
    counts, offsets, sid = r["counts"], r["offsets"], r["sorted_ids"]
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    padded = -(-counts // bm) * bm
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(padded)]))
    assert r["num_padded"][0] == offsets[-1]
    # the unpadded sequence is the stable argsort of the ids
    valid = sid[sid < A]
    assert np.array_equal(valid, np.argsort(flat, kind="stable"))
    # each expert's rows sit at the head of its padded range, pads after
    for e in range(E):
        seg = sid[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg[: counts[e]]] == e)
        assert np.all(seg[counts[e]:] == A)
    assert np.all(sid[offsets[-1]:cap] == A)
    te = r["tile_expert"]
    assert te.size == cap // bm
    expect = np.full(cap // bm, -1)
    for e in range(E):
        expect[offsets[e] // bm: offsets[e + 1] // bm] = e
    assert np.array_equal(te, expect)
    return r


@pytest.mark.parametrize("bm", [16, 32, 64])
def test_random_ids(bm):
    rng = np.random.default_rng(bm)
    for T, topk, E in [(1, 1, 1), (7, 3, 5), (64, 2, 8), (256, 8, 128), (33, 8, 200)]:
        ids = rng.integers(0, E, (T, topk)).astype(np.int32)
        _check(ids, E, bm)


def test_duplicates_and_empty_experts():
    ids = np.array([[3, 3], [3, 0], [0, 0]], np.int32)
    r = _check(ids, 6, 16)
    assert list(r["counts"]) == [3, 0, 0, 3, 0, 0]
    assert list(r["sorted_ids"][:3]) == [3, 4, 5]          # expert 0, ascending flat id


def test_no_tokens():
    r = _check(np.zeros((0, 8), np.int32), 128, 32)
    assert r["num_padded"][0] == 0 and np.all(r["tile_expert"] == -1)


@pytest.mark.parametrize("name", ["tiny", "full", "skew"])
def test_workload_routing(name):
    shp = CONFIGS[name]
    ids, w = oracle.router(router_logits(shp), shp.topk)
    r = _check(ids, shp.E, 32)
    # each token's ids are distinct and its weights sum to ~1 in descending order
    assert all(len(set(row)) == shp.topk for row in ids)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    if name == "skew":
        assert np.sum(r["counts"] == 0) >= 20
        assert r["counts"].max() >= 200


def test_out_of_range_rejected():
    with pytest.raises(ValueError):
        oracle.align(np.array([[0, 9]], np.int32), 8, 32)
