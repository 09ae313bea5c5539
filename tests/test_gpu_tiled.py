"""GPU: the tiled weight layout (include/dgw4.h, "Tiled weight layout").

dgw4_pack_tiled is compared byte for byte with the tests' description of the
layout (tests/tiled_layout.py); every GEMM entry point given tiled weights must give results
bit-identical to the same call on the canonical weights (the same arithmetic
in the same order, only the load addresses differ), and the layer output is
also checked against the oracle on the shapes each kernel family covers.
"""
import numpy as np
import pytest
import torch

import oracle
import w4a16_grouped_moe_amd as dg
from synth import CONFIGS
from synth.inputs import linear_inputs
from tests import layer_cases as lc
from tests.tiled_layout import pack_tiled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    dg.lib()


def _tiled(w):
    """Device pack -> tiled pack, checked against the layout's description."""
    t = dg.pack_tiled(w)
    torch.cuda.synchronize()
    want = pack_tiled(w[0].cpu().numpy(), w[3])
    assert np.array_equal(t[0].cpu().numpy(), want), "tiled bytes differ from the layout"
    return t


@pytest.mark.parametrize("g,E,N,K", [(64, 3, 48, 384), (128, 2, 32, 512), (64, 1, 16, 64),
                                     (128, 1, 16, 128), (128, 5, 1408, 2816)])
def test_pack_tiled_bitexact(g, E, N, K):
    lc.log(f"[tiled] pack g={g} E={E} N={N} K={K}")
    rng = np.random.default_rng(g + E + N + K)
    q = torch.from_numpy(rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)).cuda()
    _tiled((q, None, None, g))


def test_pack_tiled_empty_stack():
    q = torch.empty((0, 16, 64), dtype=torch.uint8, device="cuda")
    qt, _, _, g = dg.pack_tiled((q, None, None, 128))
    assert qt.numel() == 0 and g == 128 | dg.WEIGHTS_TILED


def _forward_pair(L, gu_t=True, dn_t=True, workspace=None):
    # both layouts on 32-row tiles, where they give bit-identical results (at
    # many rows per expert the library's choice for tiled weights is 128-row
    # chunks, which round differently; the chunk tests cover those)
    gu = _tiled(L.gu_dev) if gu_t else L.gu_dev
    dn = _tiled(L.dn_dev) if dn_t else L.dn_dev
    canon = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, L.gu_dev, L.dn_dev, workspace=workspace,
                           rows="tiles").clone()
    tiled = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, workspace=workspace, rows="tiles")
    torch.cuda.synchronize()
    assert torch.equal(tiled.view(torch.int16), canon.view(torch.int16)), "tiled != canonical"
    return tiled.cpu().numpy()


def test_forward_tiled_tiny_every_element():
    L = lc.build(CONFIGS["tiny"])
    lc.assert_close(_forward_pair(L), lc.oracle_forward(L), "tiled tiny")


@pytest.mark.parametrize("case", [
    dict(name="ragged", E=8, topk=2, T=333, d=640, m=320),
    dict(name="edge_n", E=6, topk=3, T=97, d=576, m=192, g_gu=64),
    dict(name="top1", E=1, topk=1, T=45, d=256, m=256, g_dn=128),
    dict(name="long_m", E=4, topk=2, T=50, d=384, m=1088),
])
def test_forward_tiled_shapes_every_element(case):
    L = lc.build(lc.custom_shape(**case))
    lc.assert_close(_forward_pair(L), lc.oracle_forward(L), "tiled " + case["name"])


@pytest.mark.parametrize("T", [1, 37])
def test_forward_tiled_layer_shape_small_T(T):
    L = lc.build(lc.custom_shape(f"tiled_T{T}", E=16, topk=8, T=T, d=2816, m=704, index=94))
    lc.assert_close(_forward_pair(L), lc.oracle_forward(L), f"tiled layer shape T={T}")


def test_forward_tiled_mixed_layouts():
    # one stack tiled, the other canonical: the pair runs as two launches (the
    # generic gate_up kernel, then the layer-shape down kernel), which round
    # differently from the one-launch pair; the two mixed orders run the same
    # kernels and must agree bit for bit
    L = lc.build(lc.custom_shape("tiled_mixed", E=16, topk=8, T=64, d=2816, m=704, index=95))
    ref = lc.oracle_forward(L)
    gu_t, dn_t = _tiled(L.gu_dev), _tiled(L.dn_dev)
    a = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu_t, L.dn_dev).clone()
    b = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, L.gu_dev, dn_t)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    lc.assert_close(a.cpu().numpy(), ref, "gate_up tiled, down canonical")


def test_forward_tiled_full_every_token():
    L = lc.cached("full")
    lc.assert_close(_forward_pair(L), lc.oracle_forward(L), "tiled full (all 256 tokens)")


def test_forward_tiled_full_deterministic_100():
    # the benchmarked configuration: tiled weights, the one-launch layer kernel
    L = lc.cached("full")
    sh = L.shape
    gu, dn = dg.pack_tiled(L.gu_dev), dg.pack_tiled(L.dn_dev)
    ws = torch.empty(dg.workspace_bytes(sh.T, sh.topk, sh.E, sh.d, sh.m, gu[3], dn[3]),
                     dtype=torch.uint8, device="cuda")
    first = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, workspace=ws).clone()
    bad = 0
    for i in range(100):
        if i % 10 == 0:
            ws.random_(0, 256)
        o = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, workspace=ws)
        bad += int(not torch.equal(o.view(torch.int16), first.view(torch.int16)))
    lc.log(f"[tiled] full: 100 runs, {bad} differing")
    assert bad == 0


def test_forward_tiled_unfused_layer_shape():
    shp = lc.custom_shape("tiled_unfused", E=32, topk=8, T=64, d=2816, m=704, g_gu=64, index=96)
    L = lc.build(shp)
    lc.assert_close(_forward_pair(L), lc.oracle_forward(L), "tiled unfused (all 64 tokens)")


@pytest.mark.parametrize("rows", ["tiles", "chunks"])
@pytest.mark.parametrize("g,T,K,N", [(128, 37, 2816, 1408), (64, 70, 704, 2816), (128, 1, 512, 48),
                                     (128, 300, 2816, 1408), (64, 256, 1024, 384)])
def test_linear_tiled_equals_canonical(g, T, K, N, rows):
    x, wf = linear_inputs(11, T, K, N)
    q, s, z = dg.quantize_rtn(torch.from_numpy(wf).cuda(), g)
    xd = torch.from_numpy(x).cuda()
    canon = dg.w4a16_linear(xd, (q, s, z, g), rows=rows).clone()
    tiled = dg.w4a16_linear(xd, _tiled((q, s, z, g)), rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(tiled.view(torch.int16), canon.view(torch.int16))


def test_forward_tiled_skew_every_token():
    # Zipf-skewed routing: hot experts span many tiles (their tiled weights
    # are read through the caches), cold ones one tile (read past them)
    L = lc.cached("skew")
    lc.assert_close(_forward_pair(L), lc.oracle_forward(L), "tiled skew (all 256 tokens)")


def test_forward_tiled_wide_every_token():
    L = lc.cached("wide")
    lc.assert_close(_forward_pair(L), lc.oracle_forward(L), "tiled wide (all 1024 tokens)")


@pytest.mark.parametrize("name", ["down_g64", "down_g128"])
def test_forward_tiled_down_group_variants_every_token(name):
    L = lc.build(CONFIGS[name])
    lc.assert_close(_forward_pair(L), lc.oracle_forward(L), f"tiled {name} (all 256 tokens)")
