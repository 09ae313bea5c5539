"""Pins the oracle's own fp16 conversions against numpy's IEEE binary16 type."""
import numpy as np

import oracle


def test_f16_to_f32_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _ref16(a):
    with np.errstate(over="ignore"):
        return a.astype(np.float16).view(np.uint16)


def test_f32_to_f16_random_scales():
    rng = np.random.default_rng(0)
    for scale in (1e-9, 1e-7, 6e-5, 1e-3, 0.02, 1.0, 300.0, 6e4, 1e5):
        a = (rng.standard_normal(200_000) * scale).astype(np.float32)
        assert np.array_equal(oracle.f32_to_f16(a), _ref16(a)), scale


def test_f32_to_f16_ties_and_edges():
    # every binary16 value, and the exact midpoints between neighbours
    # (ties -> even), including the subnormal range and the overflow edge
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float64)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)
    above = np.nextafter(mids, np.float32(np.inf))
    below = np.nextafter(mids, np.float32(0))
    edge = np.array([65504, 65519.99, 65520, 65536, 1e30, np.inf, -np.inf,
                     2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -24, 2.0 ** -26,
                     1e-40, -0.0, 0.0], np.float32)
    for arr in (v.astype(np.float32), mids, above, below, edge, -mids, -edge):
        assert np.array_equal(oracle.f32_to_f16(arr), _ref16(arr))
    n = oracle.f32_to_f16(np.array([np.nan], np.float32))[0]
    assert (n & 0x7C00) == 0x7C00 and (n & 0x3FF) != 0
