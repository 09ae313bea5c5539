"""ctypes marshalling for liboracle.so (see the package docstring: test
infrastructure only)."""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fexcess-precision=standard", "-fPIC", "-shared", "-Wall"]


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so (next to the source)."""
    global _lib
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L = ctypes.c_long
        lib.orc_f32_to_f16.restype = ctypes.c_uint16
        lib.orc_f32_to_f16.argtypes = [ctypes.c_float]
        lib.orc_f32_to_f16_array.argtypes = [P, L, P]
        lib.orc_f16_to_f32_array.argtypes = [P, L, P]
        lib.orc_quantize_rtn.argtypes = [P, I, I, I, I, P, P, P]
        lib.orc_dequant.argtypes = [P, P, P, I, I, I, I, P]
        lib.orc_align.argtypes = [P, I, I, I, I, P, P, P, P, P]
        lib.orc_gelu_tanh.restype = ctypes.c_double
        lib.orc_gelu_tanh.argtypes = [ctypes.c_double]
        lib.orc_w4a16_linear.argtypes = [P, I, I, I, P, P, P, I, P]
        lib.orc_moe_forward.argtypes = [P, P, P, I, I, I, I, I,
                                        P, P, P, I, P, P, P, I, P, I, P, P]
        lib.orc_philox4x32_10.argtypes = [P, P, P]
        lib.orc_router.restype = I
        lib.orc_router.argtypes = [P, I, I, I, P, P]
        lib.orc_set_threads.restype = I
        lib.orc_set_threads.argtypes = [I]
        lib.orc_gumbel_uniform.restype = ctypes.c_float
        lib.orc_gumbel_uniform.argtypes = [ctypes.c_uint32]
        lib.orc_gumbel_score.restype = ctypes.c_float
        lib.orc_gumbel_score.argtypes = [ctypes.c_float, I, I, ctypes.c_uint64]
        lib.orc_sample.argtypes = [P, I, I, ctypes.c_uint64, P, P, P, P]
        for f in ("orc_quantize_rtn", "orc_dequant", "orc_align",
                  "orc_w4a16_linear", "orc_moe_forward", "orc_sample"):
            getattr(lib, f).restype = I
        _lib = lib
    return _lib


def threads() -> int:
    """Threads the oracle's OpenMP loops use now."""
    return int(load().orc_set_threads(0))


def set_threads(n: int) -> int:
    """Set the threads of the oracle's OpenMP loops; returns the count in force."""
    return int(load().orc_set_threads(int(n)))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def f32_to_f16(a) -> np.ndarray:
    """fp32 -> fp16 bit patterns (uint16), the oracle's own RN-even routine."""
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    load().orc_f32_to_f16_array(_p(a), a.size, _p(out))
    return out


def f16_to_f32(bits) -> np.ndarray:
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float32)
    load().orc_f16_to_f32_array(_p(bits), bits.size, _p(out))
    return out


def _bits16(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.float16:
        return np.ascontiguousarray(a).view(np.uint16)
    return _c(a, np.uint16)


def quantize_rtn(w, g: int):
    """w fp32 [..., N, K] -> (q u8 [..., N, K/2], s u16 [..., N, K/g], z u16)."""
    w = _c(w, np.float32)
    *lead, N, K = w.shape
    E = int(np.prod(lead)) if lead else 1
    q = np.zeros((*lead, N, K // 2), np.uint8)
    s = np.zeros((*lead, N, K // g), np.uint16)
    z = np.zeros((*lead, N, K // g), np.uint16)
    rc = load().orc_quantize_rtn(_p(w), E, N, K, g, _p(q), _p(s), _p(z))
    if rc != 0:
        raise ValueError("orc_quantize_rtn: invalid shape")
    return q, s, z


def dequant(q, s, z, g: int) -> np.ndarray:
    q, s, z = _c(q, np.uint8), _bits16(s), _bits16(z)
    *lead, N, Kh = q.shape
    E = int(np.prod(lead)) if lead else 1
    K = 2 * Kh
    out = np.empty((*lead, N, K), np.float64)
    rc = load().orc_dequant(_p(q), _p(s), _p(z), E, N, K, g, _p(out))
    if rc != 0:
        raise ValueError("orc_dequant: invalid shape")
    return out


def align(ids, E: int, block_m: int) -> dict:
    ids = _c(ids, np.int32)
    T, topk = ids.shape
    A = T * topk
    cap = A + E * (block_m - 1)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_ids = np.empty(cap, np.int32)
    tile_expert = np.empty(cap // block_m, np.int32)
    num_padded = np.empty(1, np.int32)
    rc = load().orc_align(_p(ids), T, topk, E, block_m, _p(counts), _p(offsets),
                          _p(sorted_ids), _p(tile_expert), _p(num_padded))
    if rc != 0:
        raise ValueError("orc_align: invalid arguments")
    return dict(counts=counts, offsets=offsets, sorted_ids=sorted_ids,
                tile_expert=tile_expert, num_padded=num_padded)


def router(logits, topk: int):
    """fp32 logits [T, E] -> (ids int32 [T, topk], weights fp64 [T, topk])."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, topk), np.int32)
    w = np.empty((T, topk), np.float64)
    rc = load().orc_router(_p(lg), T, E, topk, _p(ids), _p(w))
    if rc != 0:
        raise ValueError("orc_router: invalid arguments")
    return ids, w


def gelu_tanh(v: float) -> float:
    return load().orc_gelu_tanh(float(v))


def w4a16_linear(x, q, s, z, g: int) -> np.ndarray:
    """x fp16 [M, K]; q [N, K/2]; s, z [N, K/g] -> fp64 [M, N]."""
    x = _bits16(x)
    q, s, z = _c(q, np.uint8), _bits16(s), _bits16(z)
    M, K = x.shape
    N = q.shape[0]
    out = np.empty((M, N), np.float64)
    rc = load().orc_w4a16_linear(_p(x), M, K, N, _p(q), _p(s), _p(z), g, _p(out))
    if rc != 0:
        raise ValueError("orc_w4a16_linear: invalid shape")
    return out


def moe_forward(x, ids, w, gu, dn, E: int, tokens=None, want_y: bool = False):
    """x fp16 [T, d]; ids int32 [T, topk]; w fp32 [T, topk];
    gu = (q [E, 2m, d/2], s, z, g); dn = (q [E, d, m/2], s, z, g).
    Returns fp64 out [n_tok, d] (and y [n_tok, topk, d] if want_y)."""
    x = _bits16(x)
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    gq, gs, gz, gg = gu
    dq, ds, dz, dg = dn
    gq, gs, gz = _c(gq, np.uint8), _bits16(gs), _bits16(gz)
    dq, ds, dz = _c(dq, np.uint8), _bits16(ds), _bits16(dz)
    T, d = x.shape
    topk = ids.shape[1]
    m = dq.shape[2] * 2
    if tokens is None:
        tok = None
        n_tok = T
    else:
        tok = _c(tokens, np.int32)
        n_tok = tok.size
    out = np.empty((n_tok, d), np.float64)
    y = np.empty((n_tok, topk, d), np.float64) if want_y else None
    rc = load().orc_moe_forward(
        _p(x), _p(ids), _p(w), T, topk, E, d, m,
        _p(gq), _p(gs), _p(gz), gg, _p(dq), _p(ds), _p(dz), dg,
        _p(tok) if tok is not None else None, n_tok, _p(out),
        _p(y) if y is not None else None)
    if rc != 0:
        raise ValueError("orc_moe_forward: invalid arguments")
    return (out, y) if want_y else out


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 block: ctr 4 x uint32, key 2 x uint32 -> 4 x uint32."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.empty(4, np.uint32)
    load().orc_philox4x32_10(_p(c), _p(k), _p(out))
    return out


def gumbel_uniform(w: int) -> float:
    """The uniform in (0, 1) the sampler derives from one 32-bit Philox word."""
    return float(load().orc_gumbel_uniform(int(w) & 0xFFFFFFFF))


def gumbel_score(l: float, r: int, v: int, seed: int) -> float:
    return float(load().orc_gumbel_score(float(l), int(r), int(v), int(seed)))


def sample(logits, seed: int):
    """logits fp32 [R, V] -> (entropy fp64 [R], sample int32 [R], argmax int32 [R],
    winning Gumbel score fp32 [R])."""
    lg = _c(logits, np.float32)
    R, V = lg.shape
    h = np.empty(R, np.float64)
    smp = np.empty(R, np.int32)
    am = np.empty(R, np.int32)
    sc = np.empty(R, np.float32)
    rc = load().orc_sample(_p(lg), R, V, int(seed), _p(h), _p(smp), _p(am), _p(sc))
    if rc != 0:
        raise ValueError("orc_sample: invalid shape")
    return h, smp, am, sc

