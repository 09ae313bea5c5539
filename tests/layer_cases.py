"""Builds one routed-expert layer for a parity test (test helper).

Both sides receive the same seeded inputs from synth/. The oracle packs the
fp32 weights with its own quantiser; the HIP path packs the same fp32
weights on the device. The two packings are asserted bit-identical before
any forward pass compares outputs, and each forward then runs on its own
side's packing, so no oracle input comes from the HIP path.
"""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import oracle
import w4a16_grouped_moe_amd as dg
from synth import CONFIGS, LayerShape, activations, expert_weights, router_logits

# The layer's tolerance: max |gpu - ref| <= 1e-2 * max |ref| (fp32 accumulation,
# fp16 intermediate and output against the fp64 oracle).
REL_TOL = 1e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class Layer:
    shape: LayerShape
    x: np.ndarray            # fp16 [T, d]
    ids: np.ndarray          # int32 [T, topk]
    w: np.ndarray            # fp32 [T, topk]
    gu_host: tuple           # oracle packs (q, s, z, g)
    dn_host: tuple
    gu_dev: tuple            # device packs (q, s, z, g)
    dn_dev: tuple
    x_dev: torch.Tensor
    ids_dev: torch.Tensor
    w_dev: torch.Tensor


def _to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def route(shape: LayerShape, layer: int = 0):
    """The layer's routing inputs: the oracle's router on the seeded logits
    (ids int32, weights rounded once to fp32)."""
    ids, w = oracle.router(router_logits(shape, layer), shape.topk)
    return ids, w.astype(np.float32)


def pack_both(wf: np.ndarray, g: int):
    """Quantise fp32 [E, N, K] on the host (oracle) and on the device; assert
    the two are bit-identical; return (host pack, device pack)."""
    hq, hs, hz = oracle.quantize_rtn(wf, g)
    wd = _to_dev(wf)
    dq, ds, dz = dg.quantize_rtn(wd, g)
    torch.cuda.synchronize()
    del wd
    assert np.array_equal(dq.cpu().numpy(), hq), "packed nibbles differ"
    assert np.array_equal(ds.cpu().numpy().view(np.uint16), hs), "scales differ"
    assert np.array_equal(dz.cpu().numpy().view(np.uint16), hz), "zero points differ"
    return (hq, hs, hz, g), (dq, ds, dz, g)


def build(shape: LayerShape, layer: int = 0, ids=None, w=None, weights=None) -> Layer:
    """weights: optional fp32 masters (gate_up [E, 2m, d], down [E, d, m]) in
    place of the seeded ones."""
    log(f"[layer] building {shape.name} T={shape.T} E={shape.E} topk={shape.topk} "
        f"d={shape.d} m={shape.m} layer={layer}")
    gw, dw = expert_weights(shape, layer) if weights is None else weights
    gu_h, gu_d = pack_both(gw, shape.g_gu)
    del gw
    dn_h, dn_d = pack_both(dw, shape.g_dn)
    del dw
    x = activations(shape, layer)
    if ids is None:
        ids, w = route(shape, layer)
    return Layer(shape, x, ids, w, gu_h, dn_h, gu_d, dn_d,
                 _to_dev(x), _to_dev(ids.astype(np.int32)), _to_dev(w.astype(np.float32)))


_CACHE: dict = {}


def cached(name: str) -> Layer:
    """The named workload's layer 0, built once per test process (the
    full-size layers take seconds to draw and pack on the host)."""
    if name not in _CACHE:
        _CACHE[name] = build(CONFIGS[name])
    return _CACHE[name]


def custom_shape(name, E, topk, T, d, m, g_gu=128, g_dn=64, zipf=None, index=90):
    return LayerShape(name, index, E=E, topk=topk, T=T, d=d, m=m, g_gu=g_gu, g_dn=g_dn,
                      zipf=zipf)


def gpu_forward(L: Layer, workspace=None, rows: str = "auto") -> np.ndarray:
    out = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, L.gu_dev, L.dn_dev, workspace=workspace,
                         rows=rows)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def oracle_forward(L: Layer, tokens=None) -> np.ndarray:
    return oracle.moe_forward(L.x, L.ids, L.w, L.gu_host, L.dn_host, L.shape.E, tokens=tokens)


def assert_close(gpu16: np.ndarray, ref: np.ndarray, what: str) -> float:
    g = gpu16.astype(np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    scale = np.abs(ref).max()
    err = np.abs(g - ref).max()
    ratio = err / scale
    log(f"[parity] {what}: max|err|={err:.3e} max|ref|={scale:.3e} ratio={ratio:.3e}")
    assert ratio <= REL_TOL, f"{what}: max|err|/max|ref| = {ratio:.3e} > {REL_TOL}"
    return ratio
