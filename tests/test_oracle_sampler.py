"""Pins of the oracle's sampler (CPU only).

Page facts: the kernel card's "Sampler" section — fused_entropy returns
Categorical(logits).entropy() in nats; gumbel_argmax_sample returns a sample
of the same Categorical distribution by Gumbel-max, with Philox noise, and
the plain argmax.

Pinned here against things other than the oracle itself: the published
known-answer vectors of Philox4x32-10, scipy's entropy of numpy's softmax,
closed forms (uniform logits, two classes), numpy's argmax (first index on
ties), and the distribution of the samples (a chi-square test against the
softmax probabilities over many independent rows).
"""
import json
import math
import os

import numpy as np
import scipy.stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")


def test_philox_known_answers():
    cases = json.load(open(GOLDEN))["cases"]
    for c in cases:
        ctr = [int(x, 16) for x in c["ctr"]]
        key = [int(x, 16) for x in c["key"]]
        want = [int(x, 16) for x in c["out"]]
        assert list(oracle.philox4x32_10(ctr, key)) == want


def test_entropy_closed_forms():
    V = 1000
    h, _, _, _ = oracle.sample(np.zeros((1, V), np.float32), 0)
    assert abs(h[0] - math.log(V)) < 1e-12 * math.log(V)
    # two classes with p = (1/4, 3/4)
    two = np.array([[0.0, math.log(3.0)]], np.float32)
    h, _, _, _ = oracle.sample(two, 0)
    p = np.array([0.25, 0.75])
    l3 = float(np.float32(math.log(3.0)))              # the fp32 logit actually used
    q = np.exp([0.0, l3]) / np.exp([0.0, l3]).sum()
    assert abs(h[0] - float(-(q * np.log(q)).sum())) < 1e-12
    assert abs(h[0] - float(-(p * np.log(p)).sum())) < 1e-6


def test_entropy_matches_scipy():
    rng = np.random.default_rng(11)
    lg = (rng.standard_normal((6, 4096)) * rng.uniform(0.5, 6.0, (6, 1))).astype(np.float32)
    h, _, _, _ = oracle.sample(lg, 0)
    for r in range(lg.shape[0]):
        x = lg[r].astype(np.float64)
        p = np.exp(x - x.max())
        p /= p.sum()
        assert abs(h[r] - scipy.stats.entropy(p)) < 1e-9 * max(1.0, abs(h[r]))


def test_argmax_first_index():
    rng = np.random.default_rng(12)
    lg = rng.standard_normal((8, 999)).astype(np.float32)
    lg[3, 17] = lg[3, 500] = 50.0                       # a tie: the first index wins
    _, _, am, _ = oracle.sample(lg, 0)
    assert np.array_equal(am, np.argmax(lg, axis=1))
    assert am[3] == 17


def test_gumbel_sample_follows_softmax():
    # rows are independent draws (the row is part of the Philox counter)
    logits = np.log(np.array([0.05, 0.1, 0.15, 0.2, 0.22, 0.28])).astype(np.float32)
    R = 60000
    _, smp, _, _ = oracle.sample(np.tile(logits, (R, 1)), 2024)
    counts = np.bincount(smp, minlength=logits.size)
    p = np.exp(logits.astype(np.float64))
    p /= p.sum()
    chi2, pval = scipy.stats.chisquare(counts, R * p)
    assert pval > 1e-6, (counts, R * p, chi2)


def test_gumbel_sample_properties():
    rng = np.random.default_rng(13)
    lg = rng.standard_normal((16, 300)).astype(np.float32)
    lg[:, 123] += 100.0                                  # the noise is bounded far below 100
    _, smp, am, sc = oracle.sample(lg, 7)
    assert np.all(smp == 123) and np.all(am == 123)
    # the winning score is the largest score of the row, at the sample's index
    for r in range(3):
        scores = [oracle.gumbel_score(lg[r, v], r, v, 7) for v in range(lg.shape[1])]
        assert sc[r] == max(scores) and scores.index(max(scores)) == smp[r]
    # same seed, same draw; another seed, another draw (somewhere)
    lg2 = rng.standard_normal((64, 50)).astype(np.float32)
    a = oracle.sample(lg2, 1)[1]
    assert np.array_equal(a, oracle.sample(lg2, 1)[1])
    assert not np.array_equal(a, oracle.sample(lg2, 2)[1])


def test_masked_entropy_matches_scipy():
    # -inf logits are masked entries (probability 0): the entropy is that of
    # the softmax over the live entries only, and a row with one live entry
    # has entropy exactly 0
    rng = np.random.default_rng(14)
    V = 777
    lg = (rng.standard_normal((5, V)) * 3.0).astype(np.float32)
    lg[0, ::3] = -np.inf
    lg[1, : V - 2] = -np.inf                          # two live entries
    lg[2, :] = -np.inf
    lg[2, 400] = 1.25                                 # one live entry
    lg[3, rng.choice(V, V // 2, replace=False)] = -np.inf
    h, smp, am, sc = oracle.sample(lg, 5)
    for r in range(lg.shape[0]):
        live = np.isfinite(lg[r])
        x = lg[r, live].astype(np.float64)
        p = np.exp(x - x.max())
        p /= p.sum()
        assert abs(h[r] - scipy.stats.entropy(p)) < 1e-9 * max(1.0, abs(h[r])), r
        assert np.isfinite(lg[r, am[r]]) and am[r] == int(np.argmax(lg[r]))
        assert np.isfinite(lg[r, smp[r]]), "a masked entry was sampled"
        assert np.isfinite(sc[r])
    assert h[2] == 0.0 and am[2] == 400 and smp[2] == 400


def test_gumbel_uniform_is_exact_and_open():
    # U = (floor(w / 2^9) + 1/2) 2^-23 must be exact in fp32 and strictly
    # inside (0, 1) for every 32-bit word, including both extremes, so that
    # -log(-log U) is always finite
    words = [0, 1, 511, 512, 0x7FFFFFFF, 0x80000000, 0xFFFFFE00, 0xFFFFFFFF]
    rng = np.random.default_rng(15)
    words += [int(v) for v in rng.integers(0, 2**32, 2000, dtype=np.uint64)]
    for w in words:
        u = oracle.gumbel_uniform(w)
        want = ((w >> 9) + 0.5) / 2.0**23            # exact in float64
        assert u == want, hex(w)
        assert 0.0 < u < 1.0, hex(w)
        g = -np.log(-np.log(np.float32(u)))           # the variate, in fp32
        assert np.isfinite(g), hex(w)
    assert oracle.gumbel_uniform(0xFFFFFFFF) == 1.0 - 2.0**-24
    assert oracle.gumbel_uniform(0) == 2.0**-24


def test_gumbel_scores_finite_on_a_large_row():
    # every score of a long row is finite (no word maps to U = 0 or 1)
    V = 1 << 16
    lg = np.zeros((2, V), np.float32)
    _, _, _, sc = oracle.sample(lg, 123)
    assert np.all(np.isfinite(sc))
    for v in range(0, V, 4099):
        assert np.isfinite(oracle.gumbel_score(0.0, 1, v, 123))
