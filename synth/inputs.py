"""Seeded input generators (numpy PCG64 on the host, torch Philox on a device).

Workloads follow the routed-expert layer the DiffusionGemma-26B-A4B W4A16
model card describes (section "What the model is": 128 experts, top-8, a
256-token canvas) at the hidden/intermediate sizes d=2816, m=704 (the down
projection's contraction width 704 is the one the card's "Checkpoint format"
section names). Values:

* expert weights  ~ N(0, 0.02) in fp32, layout [E, N, K] (K = contraction);
* activations     ~ N(0, 1) rounded once to fp16 (numpy's IEEE RN cast);
* router logits   ~ N(0, 1) in fp32 (plus ln p_rank for the Zipf-skewed
  workload). The routing itself (top-k and weights) is a step of the method:
  the oracle's router and the library's router compute it from these logits.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Streams within one (config, layer): gate_up weights, down weights,
# activations, router logits, Zipf permutation.
STREAM_GU, STREAM_DN, STREAM_X, STREAM_ROUTER, STREAM_PERM = range(5)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    index: int          # workload index used in the seed
    E: int              # experts
    topk: int           # experts per token
    T: int              # tokens (canvas rows)
    d: int              # hidden width (gate_up contraction, down output)
    m: int              # intermediate width (down contraction)
    g_gu: int = 128     # gate_up group size along d
    g_dn: int = 64      # down group size along m
    zipf: float | None = None   # Zipf exponent of the router prior, None = uniform
    layers: int = 1     # distinct weight sets (rotated stack)

    @property
    def A(self) -> int:
        return self.T * self.topk


CONFIGS = {
    "tiny": LayerShape("tiny", 0, E=8, topk=2, T=64, d=512, m=192),
    "full": LayerShape("full", 1, E=128, topk=8, T=256, d=2816, m=704),
    "skew": LayerShape("skew", 2, E=128, topk=8, T=256, d=2816, m=704, zipf=1.2),
    "stack": LayerShape("stack", 3, E=128, topk=8, T=256, d=2816, m=704, layers=30),
    "wide": LayerShape("wide", 4, E=128, topk=8, T=1024, d=2816, m=704),
    # the down projection with g = 64 at K = 704 (gate_up at g = 64, so the
    # two GEMMs run as separate launches) against the pages' variant with
    # g = 128 and K padded to 768: timing cases for the down stage
    "down_g64": LayerShape("down_g64", 5, E=128, topk=8, T=256, d=2816, m=704, g_gu=64),
    "down_g128": LayerShape("down_g128", 6, E=128, topk=8, T=256, d=2816, m=768, g_gu=64, g_dn=128),
}


def seed_for(cfg_index: int, layer: int, stream: int) -> int:
    return 1_000_000 * cfg_index + 1000 * layer + stream


def _normal_rows(seed: int, rows: int, cols: int, std: float, threads: int) -> np.ndarray:
    """[rows, cols] fp32 N(0, std); row r draws from its own child stream
    ``default_rng([seed, r])`` so the values do not depend on thread count."""
    out = np.empty((rows, cols), dtype=np.float32)

    def fill(r: int) -> None:
        rng = np.random.default_rng([seed, r])
        rng.standard_normal(cols, dtype=np.float32, out=out[r])
        out[r] *= np.float32(std)

    if threads <= 1 or rows == 1:
        for r in range(rows):
            fill(r)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(rows)))
    return out


def expert_weights(shape: LayerShape, layer: int = 0, std: float = 0.02,
                   threads: int = 8) -> tuple[np.ndarray, np.ndarray]:
    """fp32 master weights: gate_up [E, 2m, d] (rows 0..m-1 gate, m..2m-1 up)
    and down [E, d, m]. One child stream per expert."""
    E, d, m = shape.E, shape.d, shape.m
    gu = _normal_rows(seed_for(shape.index, layer, STREAM_GU), E, 2 * m * d, std, threads)
    dn = _normal_rows(seed_for(shape.index, layer, STREAM_DN), E, d * m, std, threads)
    return gu.reshape(E, 2 * m, d), dn.reshape(E, d, m)


def expert_weights_device(shape: LayerShape, layer: int, device, std: float = 0.02):
    """Same distribution drawn on a device with torch's seeded generator
    (different values from the host path). For the rotated benchmark stack,
    where 30 host-drawn layers would take minutes."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(shape.index, layer, STREAM_GU))
    gu = torch.randn((shape.E, 2 * shape.m, shape.d), generator=g, device=device,
                     dtype=torch.float32).mul_(std)
    g.manual_seed(seed_for(shape.index, layer, STREAM_DN))
    dn = torch.randn((shape.E, shape.d, shape.m), generator=g, device=device,
                     dtype=torch.float32).mul_(std)
    return gu, dn


def activations(shape: LayerShape, layer: int = 0) -> np.ndarray:
    """x [T, d] as np.float16 (N(0,1) in fp32, then numpy's RN cast)."""
    rng = np.random.default_rng(seed_for(shape.index, layer, STREAM_X))
    return rng.standard_normal((shape.T, shape.d), dtype=np.float32).astype(np.float16)


def zipf_prior(E: int, s: float, seed: int) -> np.ndarray:
    """ln p_rank(e) per expert: p_r proportional to r^-s over ranks r=1..E,
    ranks assigned by a seeded permutation of expert ids."""
    r = np.arange(1, E + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    perm = np.random.default_rng(seed).permutation(E)   # perm[rank-1] = expert
    lnp = np.empty(E, dtype=np.float32)
    lnp[perm] = np.log(p).astype(np.float32)
    return lnp


def router_logits(shape: LayerShape, layer: int = 0) -> np.ndarray:
    """Router logits fp32 [T, E]: N(0, 1), plus ln p_rank(e) for the
    Zipf-skewed workload."""
    rng = np.random.default_rng(seed_for(shape.index, layer, STREAM_ROUTER))
    logits = rng.standard_normal((shape.T, shape.E), dtype=np.float32)
    if shape.zipf is not None:
        logits += zipf_prior(shape.E, shape.zipf,
                             seed_for(shape.index, layer, STREAM_PERM))[None, :]
    return logits


def linear_inputs(seed: int, T: int, K: int, N: int, std: float = 0.02,
                  threads: int = 8) -> tuple[np.ndarray, np.ndarray]:
    """A dense layer's inputs: x fp16 [T, K] ~ N(0, 1) (rounded to nearest) and
    the fp32 master weight [N, K] ~ N(0, std), each from its own child stream
    of ``seed``."""
    x = _normal_rows(seed * 2 + 1, T, K, 1.0, threads).astype(np.float16)
    w = _normal_rows(seed * 2, N, K, std, threads)
    return x, w


def sampler_logits(seed: int, R: int, V: int, std: float = 2.0, threads: int = 8) -> np.ndarray:
    """fp32 logits [R, V] ~ N(0, std), one child stream per row."""
    return _normal_rows(seed, R, V, std, threads)

