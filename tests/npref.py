"""Independent numpy helpers the oracle pins compare against (test code).

Nothing here is imported by the oracle or by the HIP path. The unpack uses
numpy bit operations and numpy's own fp16 type, so it shares no routine with
oracle.c.
"""
import math

import numpy as np


def unpack_nibbles(q: np.ndarray) -> np.ndarray:
    """u8 [..., K/2] -> int [..., K]: even k = low nibble, odd k = high nibble."""
    lo = (q & 0x0F).astype(np.int64)
    hi = (q >> 4).astype(np.int64)
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.int64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant(q, s_bits, z_bits, g):
    nib = unpack_nibbles(q).astype(np.float64)
    s = np.asarray(s_bits, np.uint16).view(np.float16).astype(np.float64)
    z = np.asarray(z_bits, np.uint16).view(np.float16).astype(np.float64)
    s = np.repeat(s, g, axis=-1)
    z = np.repeat(z, g, axis=-1)
    return (nib - z) * s


def gelu_tanh(v):
    v = np.asarray(v, np.float64)
    return 0.5 * v * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (v + 0.044715 * v ** 3)))


def gelu_exact(v: float) -> float:
    return 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))


def moe_dense_bruteforce(x16, ids, w, Wgu, Wdn):
    """Every token through every expert (numpy matmul), then select + combine.

    x16 fp16 [T, d]; Wgu fp64 [E, 2m, d]; Wdn fp64 [E, d, m]."""
    X = x16.astype(np.float64)
    E = Wgu.shape[0]
    m = Wdn.shape[2]
    Y = []
    for e in range(E):
        G = X @ Wgu[e].T
        H = gelu_tanh(G[:, :m]) * G[:, m:]
        Y.append(H @ Wdn[e].T)
    Y = np.stack(Y)                     # [E, T, d]
    T, topk = ids.shape
    out = np.zeros_like(X)
    for t in range(T):
        for k in range(topk):
            out[t] += float(w[t, k]) * Y[ids[t, k], t]
    return out
