"""Checks of the tests' description of the tiled weight layout (CPU only).

The layout is this library's own (include/dgw4.h, "Tiled weight layout"):
qt[b][j][p][r][i] = q[16 b + r][j g/2 + p g/8 + i]. The test helper writes it
as a reshape and transposition; here it is checked element by element against
that index formula on small stacks, and against the property the GEMMs rely
on: one wave's load of group j of a 16-row block (8 g contiguous bytes) holds
exactly those rows' bytes of that group, lane (p, r) at offset (16 p + r) g/8.
"""
import numpy as np
import pytest

from tests.tiled_layout import pack_tiled


@pytest.mark.parametrize("g", [64, 128])
@pytest.mark.parametrize("lead", [(), (3,)])
def test_tiled_index_formula(g, lead):
    N, K = 32, 3 * g
    size = int(np.prod(lead, dtype=np.int64)) * N * (K // 2)
    q = np.arange(size, dtype=np.int64).reshape(*lead, N, K // 2)   # every byte its own id
    qt = pack_tiled(q, g)
    assert qt.shape == q.shape
    flat_q = q.reshape(-1, N, K // 2)
    flat_t = qt.reshape(-1, N * (K // 2))
    for e in range(flat_q.shape[0]):
        pos = 0
        for b in range(N // 16):
            for j in range(K // g):
                for p in range(4):
                    for r in range(16):
                        for i in range(g // 8):
                            src = flat_q[e, 16 * b + r, j * (g // 2) + p * (g // 8) + i]
                            assert flat_t[e, pos] == src, (e, b, j, p, r, i)
                            pos += 1
        assert pos == N * (K // 2)


@pytest.mark.parametrize("g", [64, 128])
def test_tiled_wave_loads(g):
    rng = np.random.default_rng(5)
    E, N, K = 2, 48, 4 * g
    q = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    qt = pack_tiled(q, g).reshape(E, -1)
    share = g // 8
    for e in range(E):
        for b in range(N // 16):
            for j in range(K // g):
                base = (b * (K // g) + j) * 8 * g         # one wave's load, in bytes
                for lane in range(64):
                    p, r = lane // 16, lane % 16
                    got = qt[e, base + lane * share: base + (lane + 1) * share]
                    want = q[e, 16 * b + r, j * (g // 2) + p * share: j * (g // 2) + (p + 1) * share]
                    assert np.array_equal(got, want)
    # a permutation: same multiset of bytes, and not the identity
    assert np.array_equal(np.sort(qt.ravel()), np.sort(q.ravel()))
    assert not np.array_equal(qt.ravel(), q.ravel())
