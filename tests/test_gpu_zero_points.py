"""GPU: forward parity when zero points leave the grid [0, 15].

Min/max RTN gives 0 <= z <= 15 whenever a group holds both signs. A
one-signed group whose spread is small against its offset gets a zero point
far outside: z = rint(-lo / s) with s = (hi - lo) / 15, saturated to
[-2048, 2048]. The kernels form (1024 + z), (64 + z) and q - z in fp16,
which is exact for -2033 <= z <= 1024 and off by at most one unit of s per
weight beyond (a relative error near 1/|z|, far inside the layer's
tolerance). These layers plant such groups on both sides of that range, in
gate_up and in down, check that the packing really holds the planted zero
points, and compare every output element with the oracle. The measured
ratios are printed.
"""
import zlib

import numpy as np
import pytest
import torch

import w4a16_grouped_moe_amd as dg
from synth import expert_weights
from tests import layer_cases as lc

pytestmark = pytest.mark.gpu

# zero points inside the exactly represented range, and outside it
INSIDE = [-2033, -2000, -1500, -1024, -300, -16, 16, 30, 300, 1000, 1024]
OUTSIDE = [-2048, -2047, -2040, -2034, 1025, 1031, 1500, 1999, 2047, 2048]


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    dg.lib()


def _plant(rng, w, g, targets, per_target, spread):
    """Overwrite `per_target` random groups of w [E, N, K] for each target z
    with a one-signed group of that zero point: values lo + spread * u with
    u in [0, 1] (both ends present) and lo = -z * spread / 15, so that
    -lo / s = z exactly when s = spread / 15 is an fp16 number. z = +-2048
    also gets groups past the saturation (|lo| / s > 2048). Returns the
    planted (e, n, group, z)."""
    E, N, K = w.shape
    s16 = float(np.float16(spread / 15))
    spread = s16 * 15
    planted = []
    used = set()
    for z in targets:
        for _ in range(per_target):
            while True:                      # a group not planted before
                e, n, gi = int(rng.integers(E)), int(rng.integers(N)), int(rng.integers(K // g))
                if (e, n, gi) not in used:
                    used.add((e, n, gi))
                    break
            u = rng.uniform(0, 1, g)
            i0, i1 = rng.choice(g, 2, replace=False)   # both ends present
            u[i0], u[i1] = 0.0, 1.0
            zz = z * 1.01 if abs(z) == 2048 else z
            lo = -zz * s16
            w[e, n, gi * g:(gi + 1) * g] = (lo + spread * u).astype(np.float32)
            planted.append((e, n, gi, z))
    return planted


def _check_planted(pack, planted):
    _, _, zb, _ = pack
    zf = zb.view(np.float16).astype(np.float64)
    for e, n, gi, z in planted:
        assert zf[e, n, gi] == z, (e, n, gi, z, zf[e, n, gi])


@pytest.mark.parametrize("where", ["gate_up", "down"])
@pytest.mark.parametrize("side", ["inside", "outside"])
@pytest.mark.parametrize("kind", ["generic", "layer_shape"])
def test_forward_far_zero_points(where, side, kind):
    if kind == "generic":
        shp = lc.custom_shape(f"zp_{kind}", E=4, topk=2, T=64, d=512, m=192, index=97)
    else:
        shp = lc.custom_shape(f"zp_{kind}", E=16, topk=8, T=37, d=2816, m=704, index=98)
    rng = np.random.default_rng(zlib.crc32(f"{where}/{side}/{kind}".encode()))
    gw, dw = expert_weights(shp)
    targets = INSIDE if side == "inside" else OUTSIDE
    if where == "gate_up":
        planted = _plant(rng, gw, shp.g_gu, targets, 6, 0.004)
    else:
        planted = _plant(rng, dw, shp.g_dn, targets, 6, 0.004)
    L = lc.build(shp, weights=(gw, dw))
    _check_planted(L.gu_host if where == "gate_up" else L.dn_host, planted)
    ref = lc.oracle_forward(L)
    gpu = lc.gpu_forward(L)
    tiled = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, dg.pack_tiled(L.gu_dev),
                           dg.pack_tiled(L.dn_dev))
    torch.cuda.synchronize()
    assert torch.equal(tiled.cpu().view(torch.int16), torch.from_numpy(gpu).view(torch.int16))
    lc.assert_close(gpu, ref, f"z {side} the exact range, planted in {where} ({kind})")
