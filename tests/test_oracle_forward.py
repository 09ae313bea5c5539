"""Pins of the oracle's layer forward.

Page facts: the kernel card ('W4A16': w4a16_linear(x, ...) equals
F.linear(x, dequant(W)); 'Grouped MoE': one launch for all experts with the
activation in the first GEMM's epilogue and a fixed-order weighted combine)
and the Part 2 blog ('Quantisation alone leaves a sparse execution problem':
each token runs through its 8 routed experts, outputs weighted and added).
The pins: numpy matmul on independently dequantised weights, exact GELU via
erf, one-hot and zero-point special cases, top-1 == one expert, and a dense
brute force that runs every token through every expert.
"""
import math

import numpy as np
import pytest

import oracle
from synth import CONFIGS, activations, expert_weights, router_logits
from tests import npref


def test_gelu_tanh_is_gelu():
    import torch
    import torch.nn.functional as F

    assert oracle.gelu_tanh(0.0) == 0.0
    vs = np.linspace(-8, 8, 4001)
    # torch's own tanh-approximate GELU, evaluated in fp64 on the CPU: an
    # implementation of the same published formula that shares nothing with
    # the oracle's C code; a slip in either constant (sqrt(2/pi), 0.044715)
    # moves the value by far more than 1e-12
    ref = F.gelu(torch.from_numpy(vs), approximate="tanh").numpy()
    for v, r in zip(vs, ref):
        g = oracle.gelu_tanh(v)
        assert abs(g - r) <= 1e-12 * max(1.0, abs(v)), (v, g, r)
        # odd part of GELU is v/2: gelu(v) - gelu(-v) = v
        assert abs(g - oracle.gelu_tanh(-v) - v) <= 1e-12 * max(1.0, abs(v))
        # and the tanh form stays within its known distance of exact GELU
        assert abs(g - npref.gelu_exact(v)) < 5e-4
    # large |v|: identity / zero
    assert abs(oracle.gelu_tanh(12.0) - 12.0) < 1e-12
    assert abs(oracle.gelu_tanh(-12.0)) < 1e-12


def _pack(rng, E, N, K, g, std=0.02):
    w = (rng.standard_normal((E, N, K)) * std).astype(np.float32)
    return oracle.quantize_rtn(w, g)


@pytest.mark.parametrize("g", [64, 128])
def test_linear_matches_matmul_of_dequant(g):
    rng = np.random.default_rng(g)
    M, K, N = 37, 4 * g, 48
    q, s, z = _pack(rng, 1, N, K, g)
    x = rng.standard_normal((M, K)).astype(np.float16)
    ours = oracle.w4a16_linear(x, q[0], s[0], z[0], g)
    ref = x.astype(np.float64) @ npref.dequant(q[0], s[0], z[0], g).T
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-12)


def test_linear_one_hot_and_zero_point():
    g = 64
    rng = np.random.default_rng(1)
    K, N = 256, 16
    q, s, z = _pack(rng, 1, N, K, g)
    x = np.zeros((K, K), np.float16)
    x[np.arange(K), np.arange(K)] = 1.0
    out = oracle.w4a16_linear(x, q[0], s[0], z[0], g)     # row k = column k of deq(W)^T
    assert np.array_equal(out, npref.dequant(q[0], s[0], z[0], g).T)
    # every nibble equal to the zero point -> exact zeros
    q0 = np.full_like(q[0], 0x77)
    z0 = np.full_like(z[0], np.float16(7).view(np.uint16))
    xr = rng.standard_normal((5, K)).astype(np.float16)
    assert np.all(oracle.w4a16_linear(xr, q0, s[0], z0, g) == 0.0)


def _tiny_layer(rng, T=6, E=4, topk=2, d=128, m=64):
    gq, gs, gz = _pack(rng, E, 2 * m, d, 128)
    dq, ds, dz = _pack(rng, E, d, m, 64)
    x = rng.standard_normal((T, d)).astype(np.float16)
    ids = np.stack([rng.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (T, topk)).astype(np.float32)
    return x, ids, w, (gq, gs, gz, 128), (dq, ds, dz, 64)


def test_forward_matches_dense_bruteforce():
    rng = np.random.default_rng(11)
    E = 4
    x, ids, w, gu, dn = _tiny_layer(rng, E=E)
    ours = oracle.moe_forward(x, ids, w, gu, dn, E)
    Wgu = npref.dequant(*gu[:3], gu[3])
    Wdn = npref.dequant(*dn[:3], dn[3])
    ref = npref.moe_dense_bruteforce(x, ids, w, Wgu, Wdn)
    assert np.allclose(ours, ref, rtol=1e-10, atol=1e-12)


def test_forward_duplicate_ids_count_twice():
    rng = np.random.default_rng(12)
    E = 4
    x, ids, w, gu, dn = _tiny_layer(rng, E=E)
    ids[:, 1] = ids[:, 0]
    ours = oracle.moe_forward(x, ids, w, gu, dn, E)
    Wgu = npref.dequant(*gu[:3], gu[3])
    Wdn = npref.dequant(*dn[:3], dn[3])
    ref = npref.moe_dense_bruteforce(x, ids, w, Wgu, Wdn)
    assert np.allclose(ours, ref, rtol=1e-10, atol=1e-12)


def test_top1_weight1_is_single_expert():
    rng = np.random.default_rng(13)
    E, T, d, m = 4, 5, 128, 64
    x, _, _, gu, dn = _tiny_layer(rng, T=T, E=E, d=d, m=m)
    ids = np.full((T, 1), 2, np.int32)
    w = np.ones((T, 1), np.float32)
    ours = oracle.moe_forward(x, ids, w, gu, dn, E)
    G = oracle.w4a16_linear(x, gu[0][2], gu[1][2], gu[2][2], 128)
    H = np.array([[oracle.gelu_tanh(v) for v in row] for row in G[:, :m]]) * G[:, m:]
    # second projection through numpy on the independently dequantised down weights
    ref = H @ npref.dequant(dn[0][2], dn[1][2], dn[2][2], 64).T
    assert np.allclose(ours, ref, rtol=1e-12, atol=1e-14)


def test_weights_scale_linearly_and_token_subset():
    rng = np.random.default_rng(14)
    E = 4
    x, ids, w, gu, dn = _tiny_layer(rng, E=E)
    a = oracle.moe_forward(x, ids, w, gu, dn, E)
    b = oracle.moe_forward(x, ids, (w * 2).astype(np.float32), gu, dn, E)
    assert np.array_equal(b, 2 * a)
    sub = np.array([4, 0, 2], np.int32)
    c, y = oracle.moe_forward(x, ids, w, gu, dn, E, tokens=sub, want_y=True)
    assert np.array_equal(c, a[sub])
    assert np.allclose((w[sub][:, :, None] * y).sum(1), c, rtol=1e-12, atol=1e-15)


def test_tiny_workload_runs():
    shp = CONFIGS["tiny"]
    gw, dw = expert_weights(shp)
    gu = (*oracle.quantize_rtn(gw, shp.g_gu), shp.g_gu)
    dn = (*oracle.quantize_rtn(dw, shp.g_dn), shp.g_dn)
    x = activations(shp)
    ids, w = oracle.router(router_logits(shp), shp.topk)
    w = w.astype(np.float32)
    out = oracle.moe_forward(x, ids, w, gu, dn, shp.E)
    assert out.shape == (shp.T, shp.d) and np.all(np.isfinite(out))
    # outputs are O(0.1): weights 0.02 * sqrt(d) ... keeps fp16 far from overflow
    assert 1e-3 < np.abs(out).max() < 10
    ref = npref.moe_dense_bruteforce(x, ids, w, npref.dequant(*gu[:3], gu[3]),
                                     npref.dequant(*dn[:3], dn[3]))
    assert np.allclose(out, ref, rtol=1e-9, atol=1e-12)


def test_invalid_arguments():
    rng = np.random.default_rng(15)
    x, ids, w, gu, dn = _tiny_layer(rng)
    ids[0, 0] = 99
    with pytest.raises(ValueError):
        oracle.moe_forward(x, ids, w, gu, dn, 4)
