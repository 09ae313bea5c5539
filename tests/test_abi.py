"""The C ABI (include/dgw4.h) on the host: the library loads, exports every
declared function, and rejects bad arguments before any HIP call. No kernel
is launched here."""
import ctypes

import pytest

import w4a16_grouped_moe_amd as dg
from w4a16_grouped_moe_amd import binding as B


def test_exports_every_declared_function():
    names = B.header_functions()
    assert set(names) >= {"dgw4_quantize_rtn", "dgw4_align", "dgw4_moe_forward",
                          "dgw4_align_capacity", "dgw4_status_string", "dgw4_version"}
    L = dg.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    assert dg.status_string(0) == "DGW4_OK"
    assert dg.status_string(3) == "DGW4_ERR_WORKSPACE"
    assert dg.status_string(99) == "DGW4_UNKNOWN_STATUS"
    assert dg.version() >= 100


def test_align_capacity():
    assert dg.align_capacity(256, 8, 128, 32) == 256 * 8 + 128 * 31
    assert dg.align_capacity(0, 8, 128, 32) == 128 * 31
    assert dg.align_capacity(-1, 8, 128, 32) == 0


def test_workspace_query():
    n = dg.workspace_bytes(256, 8, 128, 2816, 704)
    cap = 256 * 8 + 128 * 31
    # H fp16 [cap, m] + two fp16 partials of Y [2][A, d] + alignment buffers
    data = cap * 704 * 2 + 2 * 2048 * 2816 * 2
    assert data <= n < data + 64 * 1024
    assert n % 256 == 0


def _fwd(**kw):
    a = dict(x=1 << 12, ids=1 << 12, w=1 << 12, T=4, topk=2, E=8, d=512, m=192,
             gq=1 << 12, gs=1 << 12, gz=1 << 12, gg=128, dq=1 << 12, ds=1 << 12, dz=1 << 12,
             dg=64, ws=1 << 12, out=1 << 12, n=1 << 30)
    a.update(kw)
    n = ctypes.c_size_t(a["n"])
    return dg.lib().dgw4_moe_forward(a["x"], a["ids"], a["w"], a["T"], a["topk"], a["E"],
                                     a["d"], a["m"], a["gq"], a["gs"], a["gz"], a["gg"],
                                     a["dq"], a["ds"], a["dz"], a["dg"], a["ws"],
                                     ctypes.byref(n), a["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(gq=None), B.ERR_INVALID_ARG),
    (dict(x=None), B.ERR_INVALID_ARG),
    (dict(topk=9), B.ERR_INVALID_ARG),           # topk > E
    (dict(E=0), B.ERR_INVALID_ARG),
    (dict(E=2000, topk=2), B.ERR_INVALID_ARG),   # > 1024 experts
    (dict(d=500), B.ERR_INVALID_ARG),            # d % 128
    (dict(m=100), B.ERR_INVALID_ARG),            # m % 64
    (dict(gg=32), B.ERR_UNSUPPORTED),
    (dict(dg=96), B.ERR_UNSUPPORTED),
    (dict(ws=(1 << 12) + 4), B.ERR_INVALID_ARG),  # misaligned workspace
    (dict(x=(1 << 12) + 2), B.ERR_INVALID_ARG),   # misaligned x
    (dict(gs=(1 << 12) + 8), B.ERR_INVALID_ARG),  # scale/zero arrays are read 16 bytes at a time
    (dict(dz=(1 << 12) + 2), B.ERR_INVALID_ARG),
    (dict(n=16), B.ERR_WORKSPACE),
    (dict(T=-1), B.ERR_INVALID_ARG),
])
def test_forward_rejects(kw, code):
    assert _fwd(**kw) == code


def test_forward_t0_is_noop():
    assert _fwd(T=0, x=None, ids=None, w=None, out=None) == B.OK


def test_quantize_rejects():
    q = dg.lib().dgw4_quantize_rtn
    assert q(None, 1, 1, 128, 128, 1 << 12, 1 << 12, 1 << 12, None) == B.ERR_INVALID_ARG
    assert q(1 << 12, 1, 1, 127, 64, 1 << 12, 1 << 12, 1 << 12, None) == B.ERR_INVALID_ARG
    assert q(1 << 12, 1, 1, 192, 128, 1 << 12, 1 << 12, 1 << 12, None) == B.ERR_INVALID_ARG
    assert q(1 << 12, 1, 1, 96, 32, 1 << 12, 1 << 12, 1 << 12, None) == B.ERR_UNSUPPORTED
    assert q(1 << 12, 0, 1, 128, 64, 1 << 12, 1 << 12, 1 << 12, None) == B.ERR_INVALID_ARG


def test_align_rejects():
    a = dg.lib().dgw4_align
    p = 1 << 12
    assert a(p, 4, 2, 8, 24, p, p, p, p, p, None) == B.ERR_INVALID_ARG    # block_m
    assert a(p, 4, 2, 1025, 32, p, p, p, p, p, None) == B.ERR_INVALID_ARG
    assert a(None, 4, 2, 8, 32, p, p, p, p, p, None) == B.ERR_INVALID_ARG
    assert a(p, 4, 2, 8, 32, p, None, p, p, p, None) == B.ERR_INVALID_ARG
    assert a(p, -1, 2, 8, 32, p, p, p, p, p, None) == B.ERR_INVALID_ARG


def test_read_probe_rejects():
    # checked on the host before any launch: null pointers, sizes that are
    # not a positive multiple of 16, misaligned buffers
    r = dg.lib().dgw4_hbm_read_probe
    p = 1 << 12
    assert r(None, 16, p, None) == B.ERR_INVALID_ARG
    assert r(p, 16, None, None) == B.ERR_INVALID_ARG
    assert r(p, 0, p, None) == B.ERR_INVALID_ARG
    assert r(p, 24, p, None) == B.ERR_INVALID_ARG
    assert r(p + 8, 16, p, None) == B.ERR_INVALID_ARG


def test_mfma_probe_rejects():
    # checked on the host before any launch: no iterations, null sink or
    # FLOP count
    r = dg.lib().dgw4_mfma_probe
    p = 1 << 12
    f = ctypes.c_double(0.0)
    assert r(0, p, ctypes.byref(f), None) == B.ERR_INVALID_ARG
    assert r(-5, p, ctypes.byref(f), None) == B.ERR_INVALID_ARG
    assert r(10, None, ctypes.byref(f), None) == B.ERR_INVALID_ARG
    assert r(10, p, None, None) == B.ERR_INVALID_ARG


def test_linear_rejects():
    # host-side checks before any launch
    f = dg.lib().dgw4_w4a16_linear
    p = 1 << 12
    assert f(p, 4, 256, 64, p, p, p, 100, p, None) == B.ERR_UNSUPPORTED      # g
    assert f(p, 4, 255, 64, p, p, p, 64, p, None) == B.ERR_INVALID_ARG       # odd K
    assert f(p, 4, 320, 64, p, p, p, 128, p, None) == B.ERR_INVALID_ARG      # K % g
    assert f(p, 4, 256, 40, p, p, p, 64, p, None) == B.ERR_UNSUPPORTED       # N % 16
    assert f(p, 4, 64 * 65, 64, p, p, p, 64, p, None) == B.ERR_UNSUPPORTED   # > 64 groups
    assert f(None, 4, 256, 64, p, p, p, 64, p, None) == B.ERR_INVALID_ARG
    assert f(p, 4, 256, 64, p, p, p, 64, None, None) == B.ERR_INVALID_ARG
    assert f(p, -1, 256, 64, p, p, p, 64, p, None) == B.ERR_INVALID_ARG
    assert f(p + 8, 4, 256, 64, p, p, p, 64, p, None) == B.ERR_INVALID_ARG   # alignment
    assert f(None, 0, 256, 64, None, None, None, 64, None, None) == B.OK     # T = 0: no-op


def test_sample_workspace_and_rejects():
    import ctypes
    f = dg.lib().dgw4_sample
    n = ctypes.c_size_t(0)
    assert f(None, 256, 262144, 1, None, None, None, None, ctypes.byref(n), None) == B.OK
    assert n.value == 256 * 8 * 32                       # 8 splits per row, 32-byte partials
    assert f(None, 256, 262146, 1, None, None, None, None, ctypes.byref(n), None) == B.ERR_UNSUPPORTED
    assert f(None, -1, 1024, 1, None, None, None, None, ctypes.byref(n), None) == B.ERR_INVALID_ARG
    assert f(None, 4, 1024, 1, None, None, None, None, None, None) == B.ERR_INVALID_ARG
    p = 1 << 12
    small = ctypes.c_size_t(8)
    assert f(p, 4, 1024, 1, None, None, None, p, ctypes.byref(small), None) == B.ERR_WORKSPACE
    big = ctypes.c_size_t(1 << 20)
    assert f(p + 4, 4, 1024, 1, None, None, None, p, ctypes.byref(big), None) == B.ERR_INVALID_ARG
    assert f(None, 0, 1024, 1, None, None, None, p, ctypes.byref(big), None) == B.OK   # R = 0


def test_moe_experts_checks_like_forward():
    import ctypes
    f = dg.lib().dgw4_moe_experts
    n = ctypes.c_size_t(0)
    # workspace query: the forward's size
    assert f(None, None, 256, 8, 128, 2816, 704, None, None, None, 128, None, None, None, 64,
             None, ctypes.byref(n), None) == B.OK
    assert n.value == dg.workspace_bytes(256, 8, 128, 2816, 704)
    assert f(None, None, 256, 8, 128, 2816, 704, None, None, None, 96, None, None, None, 64,
             None, ctypes.byref(n), None) == B.ERR_UNSUPPORTED
    assert f(None, None, 256, 9, 8, 2816, 704, None, None, None, 128, None, None, None, 64,
             None, ctypes.byref(n), None) == B.ERR_INVALID_ARG           # topk > E
    p = 1 << 12
    big = ctypes.c_size_t(1 << 30)
    assert f(None, p, 4, 8, 128, 2816, 704, p, p, p, 128, p, p, p, 64,
             p, ctypes.byref(big), None) == B.ERR_INVALID_ARG            # x null


def test_pack_tiled_rejects():
    f = dg.lib().dgw4_pack_tiled
    p = 1 << 20
    assert f(p, 1, 16, 128, 32, p + (1 << 16), None) == B.ERR_UNSUPPORTED        # g
    assert f(p, 1, 24, 128, 64, p + (1 << 16), None) == B.ERR_INVALID_ARG        # N % 16
    assert f(p, 1, 16, 96, 64, p + (1 << 16), None) == B.ERR_INVALID_ARG         # K % g
    assert f(None, 1, 16, 128, 64, p, None) == B.ERR_INVALID_ARG
    assert f(p, 1, 16, 128, 64, None, None) == B.ERR_INVALID_ARG
    assert f(p + 4, 1, 16, 128, 64, p + (1 << 16), None) == B.ERR_INVALID_ARG    # alignment
    assert f(p, 1, 16, 128, 64, p + 512, None) == B.ERR_INVALID_ARG              # overlap (1 KiB)
    assert f(p, -1, 16, 128, 64, p + (1 << 16), None) == B.ERR_INVALID_ARG
    assert f(None, 0, 16, 128, 64, None, None) == B.OK                           # E = 0: no-op


def test_layout_flag_bits():
    tiled = B.WEIGHTS_TILED
    assert tiled == 0x10000
    # the flag is accepted on either stack; any other high bit is not
    assert _fwd(T=0, x=None, ids=None, w=None, out=None, gg=128 | tiled, dg=64 | tiled) == B.OK
    assert _fwd(gg=128 | 0x80000) == B.ERR_INVALID_ARG
    assert _fwd(dg=64 | (1 << 30)) == B.ERR_INVALID_ARG
    assert _fwd(gg=-128) == B.ERR_INVALID_ARG
    n = dg.workspace_bytes(256, 8, 128, 2816, 704, 128 | tiled, 64 | tiled)
    assert n == dg.workspace_bytes(256, 8, 128, 2816, 704)
    f = dg.lib().dgw4_w4a16_linear
    p = 1 << 12
    assert f(p, 4, 256, 64, p, p, p, 64 | 0x80000, p, None) == B.ERR_INVALID_ARG
    assert f(p, 4, 256, 64, p, p, p, 64 | B.ROWS_TILES | B.ROWS_CHUNKS, p, None) == B.ERR_INVALID_ARG
    assert f(None, 0, 256, 64, None, None, None, 64 | tiled, None, None) == B.OK


def test_rows_flags():
    # the row-block choice rides on gate_up's group argument; every call here
    # is a workspace query or fails validation, so nothing is launched
    assert (B.ROWS_TILES, B.ROWS_CHUNKS) == (0x20000, 0x40000)
    t = B.WEIGHTS_TILED
    both = B.ROWS_TILES | B.ROWS_CHUNKS
    layer = dict(ws=None, T=4, topk=2, E=8, d=2816, m=704)
    assert _fwd(ws=None, gg=128 | both) == B.ERR_INVALID_ARG
    assert _fwd(ws=None, dg=64 | B.ROWS_CHUNKS) == B.ERR_INVALID_ARG     # not on down's
    # chunks exist for d = 2816 at g = 128 and m = 704 at g = 64, both stacks
    # tiled
    assert _fwd(ws=None, gg=128 | t | B.ROWS_CHUNKS, dg=64 | t) == B.ERR_UNSUPPORTED
    assert _fwd(**layer, gg=64 | t | B.ROWS_CHUNKS, dg=64 | t) == B.ERR_UNSUPPORTED
    assert _fwd(**layer, gg=128 | B.ROWS_CHUNKS, dg=64) == B.ERR_UNSUPPORTED
    assert _fwd(**layer, gg=128 | t | B.ROWS_CHUNKS, dg=64) == B.ERR_UNSUPPORTED
    assert _fwd(ws=None, gg=128 | B.ROWS_TILES) == B.OK
    assert _fwd(**layer, gg=128 | t | B.ROWS_CHUNKS, dg=64 | t) == B.OK
    # workspace: tiles at the layer's shape keep two Y partials; chunks keep
    # H for 128-row padding and one Y
    for T in (256, 1024):
        A = T * 8
        tiles = dg.workspace_bytes(T, 8, 128, 2816, 704, 128 | t, 64 | t, rows="tiles")
        chunks = dg.workspace_bytes(T, 8, 128, 2816, 704, 128 | t, 64 | t, rows="chunks")
        t_data = (A + 128 * 31) * 704 * 2 + 2 * A * 2816 * 2
        c_data = (A + 128 * 127) * 704 * 2 + A * 2816 * 2
        assert t_data <= tiles < t_data + 256 * 1024
        assert c_data <= chunks < c_data + 256 * 1024
        # the library's choice: chunks from 22 assignments per expert on
        # average with tiled weights, tiles otherwise
        auto = dg.workspace_bytes(T, 8, 128, 2816, 704, 128 | t, 64 | t)
        assert auto == (chunks if A >= 22 * 128 else tiles)
        assert dg.workspace_bytes(T, 8, 128, 2816, 704) == tiles
    with pytest.raises(ValueError):
        dg.workspace_bytes(256, 8, 128, 2816, 704, rows="rows")
    # the row-block query agrees with the workspace sizes above
    assert dg.row_block(1024, 8, 128, 2816, 704, 128 | t, 64 | t) == 128
    assert dg.row_block(256, 8, 128, 2816, 704, 128 | t, 64 | t) == 32
    assert dg.row_block(1024, 8, 128, 2816, 704) == 32                  # canonical weights
    assert dg.row_block(256, 8, 128, 2816, 704, 128 | t, 64 | t, rows="chunks") == 128
    assert dg.row_block(1024, 8, 128, 2816, 704, 128 | t, 64 | t, rows="tiles") == 32
    assert dg.lib().dgw4_moe_row_block(4, 2, 8, 512, 192, 128 | B.ROWS_CHUNKS, 64) == -B.ERR_UNSUPPORTED
    assert dg.lib().dgw4_moe_row_block(4, 9, 8, 512, 192, 128, 64) == -B.ERR_INVALID_ARG


def test_largest_token_counts():
    # the layer's 32-bit offsets bound T: on tiles H (T * 8 + 31 E padded rows
    # x m x 2 bytes) stays under 2 GiB up to T = 190154 at E = 128; on chunks
    # Y (T * 8 x d x 2 bytes) up to T = 47662; one more token is refused
    t = dg.WEIGHTS_TILED
    for T, rows, ok in [(190154, "tiles", True), (190155, "tiles", False),
                        (47662, "chunks", True), (47663, "chunks", False)]:
        if ok:
            assert dg.workspace_bytes(T, 8, 128, 2816, 704, 128 | t, 64 | t, rows=rows) > 0
        else:
            with pytest.raises(dg.Dgw4Error, match="UNSUPPORTED"):
                dg.workspace_bytes(T, 8, 128, 2816, 704, 128 | t, 64 | t, rows=rows)
    # past the chunks' limit the library's choice is the tiles
    assert dg.row_block(47663, 8, 128, 2816, 704, 128 | t, 64 | t) == 32
    assert dg.row_block(47662, 8, 128, 2816, 704, 128 | t, 64 | t) == 128


def test_linear_row_block():
    # the dense linear's kernel: many-row (256) from 128 rows on once
    # T * N >= 2^23, else 32-row tiles; forced either way by the row flags
    t = dg.WEIGHTS_TILED
    for T, N, want in [(256, 16384, 32), (512, 16384, 256), (128, 32768, 32), (128, 65536, 256),
                       (1024, 8192, 256), (1024, 4096, 32), (127, 1 << 20, 32), (256, 262144, 256),
                       (0, 262144, 32)]:
        assert dg.linear_row_block(T, 2816, N, 128 | t) == want, (T, N)
        assert dg.linear_row_block(T, 2816, N, 128) == want, (T, N)
    assert dg.linear_row_block(256, 2816, 16384, rows="chunks") == 256
    assert dg.linear_row_block(1, 512, 48, rows="chunks") == 256
    assert dg.linear_row_block(256, 2816, 262144, rows="tiles") == 32
    f = dg.lib().dgw4_linear_row_block
    assert f(256, 2816, 16384, 128 | B.ROWS_TILES | B.ROWS_CHUNKS) == -B.ERR_INVALID_ARG
    assert f(256, 2816, 16384, 96) == -B.ERR_UNSUPPORTED
    assert f(256, 2816, 16390, 128) == -B.ERR_UNSUPPORTED
    assert f(-1, 2816, 16384, 128) == -B.ERR_INVALID_ARG
    # K too large for the many-row kernel's LDS staging: tiles by choice,
    # refused when asked for
    assert f(256, 64 * 128, 1 << 16, 128) == 32
    assert f(256, 64 * 128, 1 << 16, 128 | B.ROWS_CHUNKS) == -B.ERR_UNSUPPORTED


def test_sample_noalloc_rejects():
    f = dg.lib().dgw4_sample_noalloc
    p = 1 << 12
    # partials past the fixed 1 MiB array, checked before any HIP call
    assert f(p, 40000, 4, 0, None, None, p, None) == B.ERR_UNSUPPORTED
    assert f(p, 4, 6, 0, None, None, p, None) == B.ERR_UNSUPPORTED          # V % 4
    assert f(p, -1, 1024, 0, None, None, p, None) == B.ERR_INVALID_ARG
    assert f(p, 4, 2, 0, None, None, p, None) == B.ERR_INVALID_ARG          # V < 4
    assert f(None, 0, 1024, 0, None, None, None, None) == B.OK               # R = 0
    assert f(None, 4, 1024, 0, None, None, p, None) == B.ERR_INVALID_ARG     # null logits
    assert f(p + 4, 4, 1024, 0, None, None, p, None) == B.ERR_INVALID_ARG    # misaligned

