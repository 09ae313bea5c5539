"""Checks of the tests' description of the tiled weight layout (CPU only).

The layout is this library's own (include/dgw4.h, "Tiled weight layout"):
qt[b][j][p][r][i] = q[16 b + r][j g/2 + p g/8 + i]: per 16-row block b and
group j, lane (quarter p, row r) of a wave owns bytes p g/8 .. (p + 1) g/8 of
row 16 b + r's share of the group. The test helper writes it as a reshape
and transposition; here it is checked element by element against that index
formula (even and odd group counts), and against the property the GEMMs rely
on: one wave's load of a group of a 16-row block covers 8 g contiguous bytes,
lane (p, r) at offset (16 p + r) g/8.
"""
import numpy as np
import pytest

from tests.tiled_layout import pack_tiled


def _expected_order(N, K, g):
    """(row, byte) of each tiled byte of one [N, K/2] matrix, in order."""
    out = []
    for b in range(N // 16):
        for j in range(K // g):
            for p in range(4):
                for r in range(16):
                    out += [(16 * b + r, j * (g // 2) + p * (g // 8) + i) for i in range(g // 8)]
    return out


@pytest.mark.parametrize("g,K", [(64, 192), (64, 256), (64, 704), (128, 384), (128, 256)])
@pytest.mark.parametrize("lead", [(), (3,)])
def test_tiled_index_formula(g, K, lead):
    N = 32
    size = int(np.prod(lead, dtype=np.int64)) * N * (K // 2)
    q = np.arange(size, dtype=np.int64).reshape(*lead, N, K // 2)   # every byte its own id
    qt = pack_tiled(q, g)
    assert qt.shape == q.shape
    flat_q = q.reshape(-1, N, K // 2)
    flat_t = qt.reshape(-1, N * (K // 2))
    order = _expected_order(N, K, g)
    assert len(order) == N * (K // 2)
    rows = np.array([o[0] for o in order])
    cols = np.array([o[1] for o in order])
    for e in range(flat_q.shape[0]):
        assert np.array_equal(flat_t[e], flat_q[e, rows, cols])


@pytest.mark.parametrize("g,K", [(64, 256), (64, 704), (128, 512)])
def test_tiled_wave_loads(g, K):
    rng = np.random.default_rng(5)
    E, N = 2, 48
    q = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    qt = pack_tiled(q, g).reshape(E, -1)
    ng = K // g
    blk = 16 * (K // 2)                               # bytes per 16-row block
    share = g // 8
    for e in range(E):
        for b in range(N // 16):
            for j in range(ng):
                base = b * blk + j * 8 * g                # one wave's load, in bytes
                for lane in range(64):
                    p, r = lane // 16, lane % 16
                    got = qt[e, base + lane * share: base + (lane + 1) * share]
                    want = q[e, 16 * b + r, j * (g // 2) + p * share: j * (g // 2) + (p + 1) * share]
                    assert np.array_equal(got, want)
    # a permutation: same multiset of bytes, and not the identity
    assert np.array_equal(np.sort(qt.ravel()), np.sort(q.ravel()))
    assert not np.array_equal(qt.ravel(), q.ravel())
