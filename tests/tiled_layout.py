"""The library's tiled weight layout, written as a numpy reshape (test helper).

No page defines this layout: it is the order in which the gfx950 GEMMs load
packed weights (include/dgw4.h, "Tiled weight layout"), a byte permutation of
the canonical checkpoint layout done once at load time. It therefore lives
with the tests, not with the oracle: tests use it to check dgw4_pack_tiled
byte for byte, and the oracle never sees tiled bytes.
"""
from __future__ import annotations

import numpy as np


def pack_tiled(q, g: int) -> np.ndarray:
    """The bytes of q [..., N, K/2] reordered as [..., N/16, K/g, 4, 16, g/8]:
    blocks of 16 rows, then the groups along K, then the four quarters of a
    group's g/2 bytes, then the 16 rows, then the g/8 bytes of one quarter."""
    q = np.asarray(q)
    *lead, N, KB = q.shape
    assert N % 16 == 0 and (2 * KB) % g == 0
    v = q.reshape(*lead, N // 16, 16, KB // (g // 2), 4, g // 8)
    n = len(lead)
    axes = list(range(n)) + [n, n + 2, n + 3, n + 1, n + 4]
    return np.ascontiguousarray(v.transpose(axes)).reshape(q.shape)
