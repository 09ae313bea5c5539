"""Python binding of libdgw4 (include/dgw4.h): argument marshalling only.

Functions take torch tensors that live on a ROCm device, check dtypes,
shapes and contiguity, and pass raw device pointers plus the current HIP
stream to the C ABI. Every step of the layer runs in the library's HIP
kernels; there is no fallback: if the library is missing or a call fails,
an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdgw4.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "dgw4.h")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
BLOCK_M = 32          # rows per tile used inside dgw4_moe_forward

_lib = None


class Dgw4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = f"{fn} returned {status_string(status)}"
        if status == ERR_HIP:
            msg += f" ({lib().dgw4_last_error().decode()})"
        super().__init__(msg)
        self.status = status


def lib():
    """Load libdgw4.so (built in-tree). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python -m w4a16_grouped_moe_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.dgw4_status_string.restype = ctypes.c_char_p
        L.dgw4_status_string.argtypes = [I]
        L.dgw4_version.restype = I
        L.dgw4_version.argtypes = []
        L.dgw4_last_error.restype = ctypes.c_char_p
        L.dgw4_last_error.argtypes = []
        L.dgw4_quantize_rtn.restype = I
        L.dgw4_quantize_rtn.argtypes = [P, I, I, I, I, P, P, P, P]
        L.dgw4_align_capacity.restype = S
        L.dgw4_align_capacity.argtypes = [I, I, I, I]
        L.dgw4_align.restype = I
        L.dgw4_align.argtypes = [P, I, I, I, I, P, P, P, P, P, P]
        L.dgw4_moe_row_block.restype = I
        L.dgw4_moe_row_block.argtypes = [I, I, I, I, I, I, I]
        L.dgw4_moe_forward.restype = I
        L.dgw4_moe_forward.argtypes = [P, P, P, I, I, I, I, I,
                                       P, P, P, I, P, P, P, I,
                                       P, ctypes.POINTER(S), P, P]
        L.dgw4_moe_forward_timed.restype = I
        L.dgw4_moe_forward_timed.argtypes = [P, P, P, I, I, I, I, I,
                                             P, P, P, I, P, P, P, I,
                                             P, ctypes.POINTER(S), P, P,
                                             ctypes.POINTER(P), I]
        L.dgw4_w4a16_linear.restype = I
        L.dgw4_w4a16_linear.argtypes = [P, I, I, I, P, P, P, I, P, P]
        L.dgw4_linear_row_block.restype = I
        L.dgw4_linear_row_block.argtypes = [I, I, I, I]
        L.dgw4_moe_experts.restype = I
        L.dgw4_moe_experts.argtypes = [P, P, I, I, I, I, I, P, P, P, I, P, P, P, I,
                                       P, ctypes.POINTER(S), P]
        L.dgw4_sample.restype = I
        L.dgw4_sample.argtypes = [P, I, I, ctypes.c_uint64, P, P, P, P, ctypes.POINTER(S), P]
        L.dgw4_moe_forward_routed.restype = I
        L.dgw4_moe_forward_routed.argtypes = [P, P, I, I, I, I, I, P, P, P, I, P, P, P, I,
                                              P, ctypes.POINTER(S), P, P]
        L.dgw4_router.restype = I
        L.dgw4_router.argtypes = [P, I, I, I, P, P, P]
        L.dgw4_sample_noalloc.restype = I
        L.dgw4_sample_noalloc.argtypes = [P, I, I, ctypes.c_uint64, P, P, P, P]
        L.dgw4_pack_tiled.restype = I
        L.dgw4_pack_tiled.argtypes = [P, I, I, I, I, P, P]
        L.dgw4_hbm_read_probe.restype = I
        L.dgw4_hbm_read_probe.argtypes = [P, S, P, P]
        L.dgw4_mfma_probe.restype = I
        L.dgw4_mfma_probe.argtypes = [I, P, ctypes.POINTER(ctypes.c_double), P]
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/dgw4.h declares."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"DGW4_API\s+[\w\s\*]*?\b(dgw4_\w+)\s*\(", text)))


def status_string(status: int) -> str:
    return lib().dgw4_status_string(int(status)).decode()


def version() -> int:
    return lib().dgw4_version()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise Dgw4Error(fn, status)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtypes) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_F16 = (torch.float16, torch.int16, torch.uint16)


def quantize_rtn(w: torch.Tensor, g: int):
    """w fp32 [..., N, K] (device) -> (q uint8 [..., N, K/2], s fp16 [..., N, K/g],
    z fp16 [..., N, K/g])."""
    pw = _dev(w, "w", (torch.float32,))
    *lead, N, K = w.shape
    E = 1
    for v in lead:
        E *= v
    q = torch.empty((*lead, N, K // 2), dtype=torch.uint8, device=w.device)
    s = torch.empty((*lead, N, K // g), dtype=torch.float16, device=w.device)
    z = torch.empty((*lead, N, K // g), dtype=torch.float16, device=w.device)
    _check("dgw4_quantize_rtn", lib().dgw4_quantize_rtn(
        pw, E, N, K, g, q.data_ptr(), s.data_ptr(), z.data_ptr(), _stream(w)))
    return q, s, z


# Or-ed into a weight tuple's group size: q is in the tiled layout of
# include/dgw4.h (DGW4_WEIGHTS_TILED).
WEIGHTS_TILED = 0x10000


# Or-ed into the layer's gate_up group size (include/dgw4.h): the expert
# GEMMs' row blocks, 32-row tiles or 128-row chunks.
ROWS_TILES = 0x20000
ROWS_CHUNKS = 0x40000
_ROWS = {"auto": 0, "tiles": ROWS_TILES, "chunks": ROWS_CHUNKS}


def _group(g: int) -> int:
    return g & 0xFFFF


def _rows_flag(rows: str) -> int:
    if rows not in _ROWS:
        raise ValueError(f"rows must be one of {sorted(_ROWS)}, not {rows!r}")
    return _ROWS[rows]


def pack_tiled(w: tuple) -> tuple:
    """(q, s, z, g) with q uint8 [..., N, K/2] in the canonical layout ->
    (qt, s, z, g | WEIGHTS_TILED), qt a new tensor of the same shape in the
    tiled layout (s and z are shared, not copied). The GEMM entry points take
    either tuple and give identical results."""
    q, s, z, g = w
    if g & WEIGHTS_TILED:
        raise ValueError("weights are already tiled")
    pq = _dev(q, "q", (torch.uint8,))
    *lead, N, K2 = q.shape
    E = 1
    for v in lead:
        E *= v
    qt = torch.empty_like(q)
    _check("dgw4_pack_tiled", lib().dgw4_pack_tiled(pq, E, N, 2 * K2, g, qt.data_ptr(), _stream(q)))
    return qt, s, z, g | WEIGHTS_TILED


def w4a16_linear(x: torch.Tensor, w: tuple, out: torch.Tensor | None = None,
                 rows: str = "auto") -> torch.Tensor:
    """Dense W4A16 linear: y = x * deq(W)^T.

    x fp16 [T, K]; w = (q uint8 [N, K/2], s fp16 [N, K/g], z fp16 [N, K/g], g),
    e.g. one matrix of quantize_rtn, or its pack_tiled form. Returns y fp16 [T, N].
    ``rows``: "auto", "tiles" (32-row tiles) or "chunks" (the many-row
    kernel, 256-row blocks), see dgw4_w4a16_linear in include/dgw4.h."""
    q, s, z, g = w
    g |= _rows_flag(rows)
    T, K = x.shape
    N = q.shape[0]
    if q.shape != (N, K // 2) or s.shape != (N, K // _group(g)) or z.shape != s.shape:
        raise ValueError(f"packed shapes {tuple(q.shape)}, {tuple(s.shape)} do not match x {tuple(x.shape)}")
    px = _dev(x, "x", _F16)
    pq = _dev(q, "q", (torch.uint8,))
    ps = _dev(s, "s", _F16)
    pz = _dev(z, "z", _F16)
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=x.device)
    if out.shape != (T, N):
        raise ValueError("out must be [T, N]")
    py = _dev(out, "out", _F16)
    _check("dgw4_w4a16_linear", lib().dgw4_w4a16_linear(px, T, K, N, pq, ps, pz, g, py, _stream(x)))
    return out


def linear_row_block(T: int, K: int, N: int, g: int = 128, rows: str = "auto") -> int:
    """The row block of the kernel w4a16_linear runs for these sizes and g
    (with its layout bit): 32 (tiles) or 256 (the many-row kernel)."""
    r = lib().dgw4_linear_row_block(T, K, N, g | _rows_flag(rows))
    if r < 0:
        _check("dgw4_linear_row_block", -r)
    return r


def sample(logits: torch.Tensor, seed: int = 0, entropy: bool = True, draw: bool = True,
           workspace: torch.Tensor | None = None):
    """The sampler in one pass over fp32 logits [R, V] (V a multiple of 4):
    returns (entropy fp32 [R] or None, sample int32 [R] or None, argmax int32 [R]).
    The sample is a Gumbel-max draw from Categorical(softmax(row)) with
    Philox4x32-10 noise keyed by ``seed`` (see dgw4_sample)."""
    if logits.dim() != 2:
        raise ValueError("logits must be [R, V]")
    R, V = logits.shape
    pl = _dev(logits, "logits", (torch.float32,))
    n = ctypes.c_size_t(0)
    _check("dgw4_sample", lib().dgw4_sample(None, R, V, int(seed) & (2**64 - 1), None, None, None,
                                            None, ctypes.byref(n), None))
    if workspace is None:
        workspace = torch.empty(max(n.value, 16), dtype=torch.uint8, device=logits.device)
    pws = _dev(workspace, "workspace", (torch.uint8,))
    n = ctypes.c_size_t(workspace.numel())
    dev = logits.device
    h = torch.empty(R, dtype=torch.float32, device=dev) if entropy else None
    smp = torch.empty(R, dtype=torch.int32, device=dev) if draw else None
    am = torch.empty(R, dtype=torch.int32, device=dev)
    _check("dgw4_sample", lib().dgw4_sample(
        pl, R, V, int(seed) & (2**64 - 1), h.data_ptr() if h is not None else None,
        smp.data_ptr() if smp is not None else None, am.data_ptr(), pws, ctypes.byref(n),
        _stream(logits)))
    return h, smp, am


def sample_noalloc(logits: torch.Tensor, seed: int = 0, out=None):
    """sample() through dgw4_sample_noalloc: the library's own partials, no
    workspace. ``out`` = (entropy fp32 [R] or None, sample int32 [R] or
    None, argmax int32 [R]) preallocated by the caller; returns it."""
    if logits.dim() != 2:
        raise ValueError("logits must be [R, V]")
    R, V = logits.shape
    pl = _dev(logits, "logits", (torch.float32,))
    if out is None:
        dev = logits.device
        out = (torch.empty(R, dtype=torch.float32, device=dev),
               torch.empty(R, dtype=torch.int32, device=dev),
               torch.empty(R, dtype=torch.int32, device=dev))
    h, smp, am = out
    ptrs = [_dev(t, n, d) if t is not None else None
            for t, n, d in ((h, "entropy", (torch.float32,)), (smp, "sample", (torch.int32,)),
                            (am, "argmax", (torch.int32,)))]
    _check("dgw4_sample_noalloc", lib().dgw4_sample_noalloc(
        pl, R, V, int(seed) & (2**64 - 1), ptrs[0], ptrs[1], ptrs[2], _stream(logits)))
    return out


def fused_entropy(logits: torch.Tensor) -> torch.Tensor:
    """Categorical(logits).entropy() in nats, one pass (no noise drawn)."""
    return sample(logits, 0, entropy=True, draw=False)[0]


def gumbel_argmax_sample(logits: torch.Tensor, seed: int):
    """(Gumbel-max sample, argmax) of each row, one pass."""
    _, smp, am = sample(logits, seed, entropy=False, draw=True)
    return smp, am


def router(logits: torch.Tensor, topk: int, ids: torch.Tensor | None = None,
           w: torch.Tensor | None = None):
    """Router logits fp32 [T, E] (device) -> (topk_ids int32 [T, topk],
    topk_w fp32 [T, topk]) as dgw4_router defines them."""
    if logits.dim() != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    pl = _dev(logits, "logits", (torch.float32,))
    if ids is None:
        ids = torch.empty((T, topk), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, topk), dtype=torch.float32, device=logits.device)
    if ids.shape != (T, topk) or w.shape != (T, topk):
        raise ValueError("ids / w must be [T, topk]")
    _check("dgw4_router", lib().dgw4_router(pl, T, E, topk, _dev(ids, "ids", (torch.int32,)),
                                            _dev(w, "w", (torch.float32,)), _stream(logits)))
    return ids, w


def align_capacity(T: int, topk: int, E: int, block_m: int) -> int:
    return int(lib().dgw4_align_capacity(T, topk, E, block_m))


def align(topk_ids: torch.Tensor, E: int, block_m: int = BLOCK_M) -> dict:
    """topk_ids int32 [T, topk] (device) -> dict of device int32 tensors
    counts [E], offsets [E+1], sorted_ids [cap], tile_expert [cap/block_m],
    num_padded [1]."""
    pid = _dev(topk_ids, "topk_ids", (torch.int32,))
    T, topk = topk_ids.shape
    cap = align_capacity(T, topk, E, block_m)
    if cap == 0:
        raise ValueError("invalid alignment shape")
    dev = topk_ids.device
    out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
               sorted_ids=torch.empty(cap, dtype=torch.int32, device=dev),
               tile_expert=torch.empty(cap // block_m, dtype=torch.int32, device=dev),
               num_padded=torch.empty(1, dtype=torch.int32, device=dev))
    _check("dgw4_align", lib().dgw4_align(
        pid, T, topk, E, block_m, out["counts"].data_ptr(), out["offsets"].data_ptr(),
        out["sorted_ids"].data_ptr(), out["tile_expert"].data_ptr(),
        out["num_padded"].data_ptr(), _stream(topk_ids)))
    return out


def workspace_bytes(T: int, topk: int, E: int, d: int, m: int, gu_g: int = 128,
                    dn_g: int = 64, rows: str = "auto") -> int:
    """Device workspace dgw4_moe_forward needs for this shape and row-block
    choice (host-only query)."""
    n = ctypes.c_size_t(0)
    _check("dgw4_moe_forward(query)", lib().dgw4_moe_forward(
        None, None, None, T, topk, E, d, m, None, None, None, gu_g | _rows_flag(rows), None,
        None, None, dn_g,
        None, ctypes.byref(n), None, None))
    return int(n.value)


def row_block(T: int, topk: int, E: int, d: int, m: int, gu_g: int = 128, dn_g: int = 64,
              rows: str = "auto") -> int:
    """The row blocks moe_forward runs its expert GEMMs on for these
    arguments (gu_g / dn_g with their layout bits): 32 (tiles) or 128
    (chunks). Host-only query."""
    r = lib().dgw4_moe_row_block(T, topk, E, d, m, gu_g | _rows_flag(rows), dn_g)
    if r < 0:
        _check("dgw4_moe_row_block", -r)
    return r


def hbm_read_probe(buf: torch.Tensor, sink: torch.Tensor) -> None:
    """Enqueue one whole-chip read of ``buf`` (a measurement aid: time it
    with events on the current stream). ``buf`` device uint8, size a multiple
    of 16; ``sink`` device int32 with at least one element."""
    pb = _dev(buf, "buf", (torch.uint8,))
    ps = _dev(sink, "sink", (torch.int32,))
    _check("dgw4_hbm_read_probe",
           lib().dgw4_hbm_read_probe(pb, buf.numel(), ps, _stream(buf)))


def mfma_probe(iters: int, sink: torch.Tensor) -> float:
    """Enqueue the whole-chip MFMA throughput probe (a measurement aid: time
    it with events on the current stream); returns the launch's
    floating-point operations. ``sink`` device int32, at least one element."""
    ps = _dev(sink, "sink", (torch.int32,))
    flops = ctypes.c_double(0.0)
    _check("dgw4_mfma_probe", lib().dgw4_mfma_probe(int(iters), ps, ctypes.byref(flops),
                                                    _stream(sink)))
    return flops.value


STAGES = ("align", "gate_up", "down", "combine")


def moe_forward(x: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor,
                gu: tuple, dn: tuple, workspace: torch.Tensor | None = None,
                out: torch.Tensor | None = None, events=None, rows: str = "auto") -> torch.Tensor:
    """One routed-expert layer.

    x fp16 [T, d]; topk_ids int32 [T, topk]; topk_w fp32 [T, topk];
    gu = (q uint8 [E, 2m, d/2], s fp16 [E, 2m, d/g], z fp16 [E, 2m, d/g], g);
    dn = (q uint8 [E, d, m/2], s, z, g). Either tuple may come from
    pack_tiled (g carries WEIGHTS_TILED). Returns out fp16 [T, d].
    ``workspace`` (uint8 device tensor of at least workspace_bytes(...)) is
    allocated here when not given; pass one to avoid allocation per call.
    ``events``: optional list of 5 torch.cuda.Event(enable_timing=True),
    recorded on the current stream before the alignment kernel and after each
    of the four kernels (see STAGES). ``rows``: "auto", "tiles" (32-row
    tiles) or "chunks" (128-row chunks), see DGW4_ROWS_TILES /
    DGW4_ROWS_CHUNKS in include/dgw4.h."""
    gq, gs, gz, gg = gu
    gg |= _rows_flag(rows)
    dq, ds, dz, dg = dn
    T, d = x.shape
    topk = topk_ids.shape[1]
    E = gq.shape[0]
    m = dq.shape[2] * 2
    if gq.shape != (E, 2 * m, d // 2) or dq.shape != (E, d, m // 2):
        raise ValueError(f"packed shapes {tuple(gq.shape)} / {tuple(dq.shape)} do not match "
                         f"x {tuple(x.shape)}")
    if gs.shape != (E, 2 * m, d // _group(gg)) or gz.shape != gs.shape:
        raise ValueError("gate_up scale/zero shape mismatch")
    if ds.shape != (E, d, m // _group(dg)) or dz.shape != ds.shape:
        raise ValueError("down scale/zero shape mismatch")
    if topk_ids.shape != (T, topk) or topk_w.shape != (T, topk):
        raise ValueError("topk_ids / topk_weights must be [T, topk]")
    ptrs = [_dev(x, "x", _F16), _dev(topk_ids, "topk_ids", (torch.int32,)),
            _dev(topk_w, "topk_w", (torch.float32,)),
            _dev(gq, "gu_q", (torch.uint8,)), _dev(gs, "gu_s", _F16), _dev(gz, "gu_z", _F16),
            _dev(dq, "dn_q", (torch.uint8,)), _dev(ds, "dn_s", _F16), _dev(dz, "dn_z", _F16)]
    need = workspace_bytes(T, topk, E, d, m, gg, dg)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    pws = _dev(workspace, "workspace", (torch.uint8,))
    if out is None:
        out = torch.empty((T, d), dtype=torch.float16, device=x.device)
    pout = _dev(out, "out", _F16)
    n = ctypes.c_size_t(workspace.numel())
    if events is None:
        _check("dgw4_moe_forward", lib().dgw4_moe_forward(
            ptrs[0], ptrs[1], ptrs[2], T, topk, E, d, m,
            ptrs[3], ptrs[4], ptrs[5], gg, ptrs[6], ptrs[7], ptrs[8], dg,
            pws, ctypes.byref(n), pout, _stream(x)))
    else:
        if len(events) != 5:
            raise ValueError("events: need 5 torch.cuda.Event")
        for e in events:
            if not e.cuda_event:          # torch creates the HIP event on first record
                e.record()
        ev = (ctypes.c_void_p * 5)(*[e.cuda_event for e in events])
        _check("dgw4_moe_forward_timed", lib().dgw4_moe_forward_timed(
            ptrs[0], ptrs[1], ptrs[2], T, topk, E, d, m,
            ptrs[3], ptrs[4], ptrs[5], gg, ptrs[6], ptrs[7], ptrs[8], dg,
            pws, ctypes.byref(n), pout, _stream(x), ev, 5))
    return out


def moe_experts(x: torch.Tensor, topk_ids: torch.Tensor, gu: tuple, dn: tuple,
                workspace: torch.Tensor, rows: str = "auto") -> None:
    """The expert stages of moe_forward alone (alignment, gate_up, down; no
    combine), leaving the expert outputs in ``workspace``: a measurement aid
    for timing those kernels back to back (see dgw4_moe_experts)."""
    gq, gs, gz, gg = gu
    gg |= _rows_flag(rows)
    dq, ds, dz, dg = dn
    T, d = x.shape
    topk = topk_ids.shape[1]
    E = gq.shape[0]
    m = dq.shape[2] * 2
    if gq.shape != (E, 2 * m, d // 2) or dq.shape != (E, d, m // 2) or topk_ids.shape != (T, topk):
        raise ValueError("shapes do not match")
    ptrs = [_dev(x, "x", _F16), _dev(topk_ids, "topk_ids", (torch.int32,)),
            _dev(gq, "gu_q", (torch.uint8,)), _dev(gs, "gu_s", _F16), _dev(gz, "gu_z", _F16),
            _dev(dq, "dn_q", (torch.uint8,)), _dev(ds, "dn_s", _F16), _dev(dz, "dn_z", _F16)]
    pws = _dev(workspace, "workspace", (torch.uint8,))
    n = ctypes.c_size_t(workspace.numel())
    _check("dgw4_moe_experts", lib().dgw4_moe_experts(
        ptrs[0], ptrs[1], T, topk, E, d, m, ptrs[2], ptrs[3], ptrs[4], gg,
        ptrs[5], ptrs[6], ptrs[7], dg, pws, ctypes.byref(n), _stream(x)))


def moe_forward_routed(x: torch.Tensor, router_logits: torch.Tensor, topk: int, gu: tuple,
                       dn: tuple, workspace: torch.Tensor | None = None,
                       out: torch.Tensor | None = None, rows: str = "auto") -> torch.Tensor:
    """One routed-expert layer from router logits fp32 [T, E]: the router
    (dgw4_router), then the layer, in one C-ABI call (dgw4_moe_forward_routed)."""
    gq, gs, gz, gg = gu
    gg |= _rows_flag(rows)
    dq, ds, dz, dg = dn
    T, d = x.shape
    E = gq.shape[0]
    m = dq.shape[2] * 2
    if router_logits.shape != (T, E):
        raise ValueError("router_logits must be [T, E]")
    if gq.shape != (E, 2 * m, d // 2) or dq.shape != (E, d, m // 2):
        raise ValueError("packed shapes do not match x")
    ptrs = [_dev(x, "x", _F16), _dev(router_logits, "router_logits", (torch.float32,)),
            _dev(gq, "gu_q", (torch.uint8,)), _dev(gs, "gu_s", _F16), _dev(gz, "gu_z", _F16),
            _dev(dq, "dn_q", (torch.uint8,)), _dev(ds, "dn_s", _F16), _dev(dz, "dn_z", _F16)]
    need = workspace_bytes(T, topk, E, d, m, gg, dg)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    pws = _dev(workspace, "workspace", (torch.uint8,))
    if out is None:
        out = torch.empty((T, d), dtype=torch.float16, device=x.device)
    pout = _dev(out, "out", _F16)
    n = ctypes.c_size_t(workspace.numel())
    _check("dgw4_moe_forward_routed", lib().dgw4_moe_forward_routed(
        ptrs[0], ptrs[1], T, topk, E, d, m, ptrs[2], ptrs[3], ptrs[4], gg, ptrs[5], ptrs[6],
        ptrs[7], dg, pws, ctypes.byref(n), pout, _stream(x)))
    return out

