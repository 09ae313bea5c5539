"""Pins of the oracle's min/max RTN quantiser, nibble packing and dequant.

Page facts: the DiffusionGemma-26B-A4B W4A16 model card ('Checkpoint format':
asymmetric uint4, fp16 scale and zero point per group, byte j = q[2j] |
q[2j+1] << 4, groups 128 for gate_up and 64 for down along the contraction
dim); the Part 2 blog ('The first constraint was capacity': integer q, scale
and zero point per group; a dequantised reference rebuilds the floats).
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests import npref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _grid_group(qvals, g, step=0.0625, zero=6):
    """Weights that sit exactly on the quantisation grid: w = (q - zero)*step
    with min(q)=0 and max(q)=15, so lo=-zero*step, hi=(15-zero)*step."""
    q = np.array(qvals, np.int64)
    assert q.size == g and q.min() == 0 and q.max() == 15
    return ((q - zero) * step).astype(np.float32)


def test_packing_worked_example():
    ex = json.load(open(os.path.join(GOLD, "pack_example.json")))
    g = 64
    rng = np.random.default_rng(5)
    q = np.concatenate([ex["q"], rng.integers(0, 16, g - len(ex["q"]))])
    q[-1], q[-2] = 0, 15                      # make the range span the whole grid
    w = _grid_group(q, g)[None, None, :]
    qb, s, z = oracle.quantize_rtn(w, g)
    assert list(qb[0, 0, : len(ex["bytes"])]) == ex["bytes"]
    # grid weights come back bit-exactly: s = 0.0625 (fp16 0x2C00), z = 6
    assert s[0, 0, 0] == 0x2C00 and z[0, 0, 0] == np.float16(6).view(np.uint16)
    assert np.array_equal(npref.unpack_nibbles(qb)[0, 0], q)


@pytest.mark.parametrize("g", [64, 128])
def test_grid_idempotent(g):
    rng = np.random.default_rng(g)
    rows = []
    for _ in range(16):
        q = rng.integers(0, 16, g)
        q[rng.integers(g)] = 0
        q[(rng.integers(g - 1) + 1 + np.argmin(q)) % g] = 15
        rows.append(q)
    q = np.stack(rows)
    w = np.stack([_grid_group(r, g) for r in rows])[None]
    qb, s, z = oracle.quantize_rtn(w, g)
    assert np.array_equal(npref.unpack_nibbles(qb)[0], q)
    assert np.all(s == 0x2C00)
    assert np.array_equal(npref.dequant(qb, s, z, g), w.astype(np.float64))


def test_rounding_ties_half_even():
    # On the grid step s=0.0625 with z=6: w = 0.5 s -> rint(0.5)=0 -> q=6;
    # w = 1.5 s -> rint(1.5)=2 -> q=8; w = -0.5 s -> q=6; w = 2.5 s -> q=8.
    g = 64
    base = np.zeros(g, np.int64) + 6
    base[0], base[1] = 0, 15
    w = _grid_group(base, g)
    w[2:6] = np.array([0.5, 1.5, -0.5, 2.5], np.float32) * np.float32(0.0625)
    qb, s, z = oracle.quantize_rtn(w[None, None], g)
    assert list(npref.unpack_nibbles(qb)[0, 0, 2:6]) == [6, 8, 6, 8]
    # odd zero point (z=5) separates rint(w/s) + z from rint(w/s + z):
    # w = 0.5 s -> 0 + 5 = 5 (not rint(5.5) = 6); w = 1.5 s -> 2 + 5 = 7
    base = np.zeros(g, np.int64) + 5
    base[0], base[1] = 0, 15
    w = _grid_group(base, g, zero=5)
    w[2:4] = np.array([0.5, 1.5], np.float32) * np.float32(0.0625)
    qb, s, z = oracle.quantize_rtn(w[None, None], g)
    assert z.view(np.float16)[0, 0, 0] == 5
    assert list(npref.unpack_nibbles(qb)[0, 0, 2:4]) == [5, 7]


def test_unpack_all_byte_values():
    # every byte value; s = 1, z = 0 makes dequant equal to the nibble
    K, g = 512, 64
    qb = np.arange(256, dtype=np.uint8)[None, None, :]
    s = np.full((1, 1, K // g), 0x3C00, np.uint16)
    z = np.zeros((1, 1, K // g), np.uint16)
    d = oracle.dequant(qb, s, z, g)[0, 0]
    b = np.arange(256)
    expect = np.empty(K)
    expect[0::2] = b % 16
    expect[1::2] = b // 16
    assert np.array_equal(d, expect)


def _bound_ok(w, qb, s, z, g):
    """|w - (q-z)s| <= s/2 + max(0, (hi-lo) - 15 s) + 1e-6 s, in fp64."""
    deq = oracle.dequant(qb, s, z, g)
    wg = w.astype(np.float64).reshape(*w.shape[:-1], -1, g)
    sg = s.view(np.float16).astype(np.float64)[..., None]
    lo, hi = wg.min(-1, keepdims=True), wg.max(-1, keepdims=True)
    slack = np.maximum(0.0, (hi - lo) - 15 * sg)
    err = np.abs(wg - deq.reshape(wg.shape))
    return np.all(err <= sg / 2 + slack + 1e-6 * sg), err / sg


@pytest.mark.parametrize("g", [64, 128])
def test_error_bound_random(g):
    rng = np.random.default_rng(100 + g)
    cases = [
        rng.standard_normal((4, 32, 4 * g)).astype(np.float32) * 0.02,
        rng.uniform(-1, 1, (2, 16, 2 * g)).astype(np.float32),
        rng.uniform(0.5, 2.0, (2, 16, 2 * g)).astype(np.float32),      # one-signed
        -rng.uniform(0.5, 2.0, (2, 16, 2 * g)).astype(np.float32),
        (rng.standard_t(2, (2, 16, 2 * g)) * 1e-3).astype(np.float32),  # outliers
    ]
    for w in cases:
        qb, s, z = oracle.quantize_rtn(w, g)
        ok, rel = _bound_ok(w, qb, s, z, g)
        assert ok, rel.max()
        zf = z.view(np.float16).astype(np.float64)
        assert np.array_equal(zf, np.round(zf))          # integer zero points
        # fp16 scale close to (hi-lo)/15 (one fp16 rounding)
        wg = w.reshape(*w.shape[:-1], -1, g).astype(np.float64)
        s_exact = (wg.max(-1) - wg.min(-1)) / 15
        sf = s.view(np.float16).astype(np.float64)
        assert np.all(np.abs(sf - s_exact) <= s_exact * 2.0 ** -11 * 1.0001)


def test_degenerate_groups():
    g = 64
    w = np.zeros((1, 3, 2 * g), np.float32)
    w[0, 1, :g] = 0.75            # constant positive group
    w[0, 2, g:] = -3.0            # constant negative group
    qb, s, z = oracle.quantize_rtn(w, g)
    assert np.all(s == 0x3C00)                                    # s = 1
    d = npref.dequant(qb, s, z, g)
    assert np.array_equal(d[0, 0], np.zeros(2 * g))               # all-zero row exact
    assert np.all(np.abs(d - w) <= 0.5)
    assert np.array_equal(d[0, 2, g:], np.full(g, -3.0))          # integer constant exact
    # the zero point is an integer: a zero point of 0 is stored as +0, also
    # when the group minimum is +0.0 (so -lo/s is -0.0)
    assert np.all(z[0, 0] == 0x0000)
    w2 = np.zeros((1, 1, g), np.float32)
    w2[0, 0, 1:] = np.linspace(0.01, 1.0, g - 1, dtype=np.float32)
    _, _, z2 = oracle.quantize_rtn(w2, g)
    assert z2[0, 0, 0] == 0x0000


def test_saturated_zero_point():
    # a narrow group far from zero: -lo/s is huge, so z saturates at -2048
    g = 64
    w = (np.float32(1000.0) + np.arange(g, dtype=np.float32) * np.float32(1e-3))[None, None]
    qb, s, z = oracle.quantize_rtn(w, g)
    assert z.view(np.float16)[0, 0, 0] == -2048
    assert np.all(npref.unpack_nibbles(qb) == 15)


def test_invalid_shapes():
    with pytest.raises(ValueError):
        oracle.quantize_rtn(np.zeros((1, 2, 100), np.float32), 64)
    with pytest.raises(ValueError):
        oracle.quantize_rtn(np.zeros((1, 2, 63), np.float32), 63)
