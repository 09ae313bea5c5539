"""GPU: the router (dgw4_router) against the oracle's, and the routed forward.

The ids are compared bit for bit (the choice compares fp32 logits, so it is
exact on both sides), the weights within 2e-6 relative (fp32 exp and divide
against the oracle's fp64). The routed forward must equal the plain forward
given the router's own ids and weights, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import w4a16_grouped_moe_amd as dg
from synth import CONFIGS, router_logits
from tests import layer_cases as lc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    dg.lib()


def _check(lg, topk, what):
    ids, w = dg.router(torch.from_numpy(lg).cuda(), topk)
    torch.cuda.synchronize()
    rid, rw = oracle.router(lg, topk)
    assert np.array_equal(ids.cpu().numpy(), rid), f"{what}: ids differ"
    err = np.abs(w.cpu().numpy().astype(np.float64) - rw).max() / np.abs(rw).max()
    lc.log(f"[router] {what}: ids identical, weight max rel err {err:.2e}")
    assert err <= 2e-6


@pytest.mark.parametrize("T,E,topk", [(1, 1, 1), (7, 5, 3), (64, 8, 2), (256, 128, 8),
                                      (1000, 128, 8), (33, 1024, 16), (5, 70, 64), (3, 300, 1)])
def test_router_matches_oracle(T, E, topk):
    rng = np.random.default_rng(T + 7 * E + topk)
    lg = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    lg[:, ::3] = np.round(lg[:, ::3], 1)                  # exact ties
    if T > 2:
        lg[2, :] = 0.5                                     # a row of equal logits
    if T > 4:
        # +0 and -0 compare equal (ties to the lower id); negative values,
        # subnormals and the extremes of the fp32 range order as floats
        lg[3, :] = np.where(np.arange(E) % 2 == 0, np.float32(0.0), np.float32(-0.0))
        lg[3, ::5] = -1.0
        lg[4, :] = -np.abs(lg[4, :])
        lg[4, 1::4] = np.float32(1e-40)
        lg[4, 2::4] = np.float32(-1e-40)
        lg[4, 3::7] = np.float32(-3.4e38)
        lg[4, 0] = np.float32(3.4e38)
    _check(lg, topk, f"T={T} E={E} top-{topk}")


@pytest.mark.parametrize("name", ["full", "skew", "wide"])
def test_router_workloads(name):
    shp = CONFIGS[name]
    _check(router_logits(shp, 0), shp.topk, name)


def test_router_empty():
    ids, w = dg.router(torch.empty((0, 128), dtype=torch.float32, device="cuda"), 8)
    assert ids.shape == (0, 8) and w.shape == (0, 8)


@pytest.mark.parametrize("layer_shape", [False, True])
def test_routed_forward_equals_forward_on_router_output(layer_shape):
    if layer_shape:
        shp = lc.custom_shape("routed_layer", E=16, topk=8, T=37, d=2816, m=704, index=99)
    else:
        shp = lc.custom_shape("routed_generic", E=8, topk=2, T=50, d=512, m=192, index=99)
    L = lc.build(shp)
    lg = torch.from_numpy(router_logits(shp, 0)).cuda()
    ids, w = dg.router(lg, shp.topk)
    plain = dg.moe_forward(L.x_dev, ids, w, L.gu_dev, L.dn_dev).clone()
    routed = dg.moe_forward_routed(L.x_dev, lg, shp.topk, L.gu_dev, L.dn_dev)
    torch.cuda.synchronize()
    assert torch.equal(routed.view(torch.int16), plain.view(torch.int16))
    # and the oracle, routing the same logits itself
    lc.assert_close(routed.cpu().numpy(), lc.oracle_forward(L), f"routed {shp.name}")
