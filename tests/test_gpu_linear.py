"""GPU parity of the dense W4A16 linear (y = x * deq(W)^T) against the CPU
oracle, through the C ABI.

The kernel card's "W4A16" section states that w4a16_linear(x, qw, scale,
zero) equals F.linear(x, dequant(W)). Checked here: the device packing
against the oracle's bit for bit, the output element by element within
max|err| <= 1e-2 * max|ref| on shapes with ragged row tiles, idle column
tiles and both group sizes, and exactly on one-hot rows, where each output is
one dequantised weight rounded once to fp16. Both kernels run every check:
the 32-row tiles (rows="tiles") and the many-row kernel (rows="chunks": fp16
weights (q - z) * s formed in registers once per 256-row block, accumulated
in fp32); the library's own choice (from 128 rows on once T * N >= 2^23) is
checked on both sides of that line at K = 2816 on sampled columns.
"""
import numpy as np
import pytest
import torch

import oracle
import w4a16_grouped_moe_amd as dg
from synth import linear_inputs
from tests import layer_cases as lc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    dg.lib()


def _pack(w: np.ndarray, g: int):
    host, dev = lc.pack_both(w[None], g)
    hq, hs, hz, _ = host
    dq, ds, dz, _ = dev
    return (hq[0], hs[0], hz[0], g), (dq[0], ds[0], dz[0], g)


@pytest.mark.parametrize("rows", ["tiles", "chunks"])
@pytest.mark.parametrize("case", [
    dict(T=333, K=640, N=320, g=64),      # ragged last row tile / block, generic K loop
    dict(T=256, K=2816, N=1408, g=128),   # the layer's K (unrolled K loop), gate_up-sized N
    dict(T=1, K=2816, N=704, g=128),      # one row
    dict(T=70, K=512, N=48, g=128),       # last column block with idle waves
    dict(T=40, K=1536, N=96, g=64),       # 24 groups of 64 per row
    # several 256-row blocks with a ragged last one and a ragged last column
    # block, an idle second row half, the generic K loop at both group sizes
    dict(T=513, K=2816, N=2112, g=128),
    dict(T=128, K=1024, N=256, g=128),
    dict(T=200, K=2816, N=384, g=64),
    dict(T=300, K=768, N=144, g=128),
])
def test_linear_matches_oracle(case, rows):
    T, K, N, g = case["T"], case["K"], case["N"], case["g"]
    lc.log(f"[linear] T={T} K={K} N={N} g={g} rows={rows}")
    x, w = linear_inputs(100 + T + K + N, T, K, N)
    host, dev = _pack(w, g)
    y = dg.w4a16_linear(torch.from_numpy(x).cuda(), dev, rows=rows)
    torch.cuda.synchronize()
    ref = oracle.w4a16_linear(x, host[0], host[1], host[2], g)
    lc.assert_close(y.cpu().numpy(), ref, f"linear T={T} K={K} N={N} g={g} rows={rows}")


@pytest.mark.parametrize("T,N,want", [(256, 32768, 256), (256, 16384, 32), (128, 65536, 256)])
def test_linear_library_choice_sampled(T, N, want):
    # at K = 2816, g = 128 (tiled), around the T * N >= 2^23 line: the
    # library's choice runs the kernel linear_row_block names (bit for bit the
    # forced one's output) and 512 sampled columns match the oracle
    K, g = 2816, 128
    x, w = linear_inputs(50 + T + N // 1024, T, K, N)
    host, dev = _pack(w, g)
    dev = dg.pack_tiled(dev)
    assert dg.linear_row_block(T, K, N, dev[3]) == want
    xd = torch.from_numpy(x).cuda()
    auto = dg.w4a16_linear(xd, dev).clone()
    forced = dg.w4a16_linear(xd, dev, rows="chunks" if want == 256 else "tiles")
    torch.cuda.synchronize()
    assert torch.equal(auto.view(torch.int16), forced.view(torch.int16))
    cols = np.sort(np.random.default_rng(T + N).choice(N, 512, replace=False))
    ref = oracle.w4a16_linear(x, host[0][cols], host[1][cols], host[2][cols], g)
    lc.assert_close(auto.cpu().numpy()[:, cols], ref, f"linear T={T} N={N}, library's choice "
                    f"({want}-row blocks), 512 sampled columns")


@pytest.mark.parametrize("kernel", ["tiles", "chunks"])
@pytest.mark.parametrize("g,rows", [(64, 10), (128, 10), (64, 160), (128, 160)])
def test_linear_one_hot_rows_are_exact(g, rows, kernel):
    # row r of x is the unit vector e_{c_r}: y[r, n] = deq(W)[n, c_r], a small
    # integer times an fp16 scale (exact in fp32), rounded once to fp16, on
    # either kernel
    K, N = 1024, 160
    _, w = linear_inputs(7, 1, K, N)
    host, dev = _pack(w, g)
    base = np.array([0, 1, 7, 8, 63, 64, 127, 128, 500, 1023], dtype=np.int64)
    cols = np.resize(base, rows) if rows > base.size else base[:rows]
    x = np.zeros((cols.size, K), np.float16)
    x[np.arange(cols.size), cols] = 1.0
    y = dg.w4a16_linear(torch.from_numpy(x).cuda(), dev, rows=kernel)
    torch.cuda.synchronize()
    deq = oracle.dequant(host[0], host[1], host[2], g)          # fp64 [N, K], exact
    want = oracle.f32_to_f16(deq[:, cols].T.astype(np.float32)).view(np.float16)
    got = y.cpu().numpy()
    assert np.array_equal(got, want), f"{int((got != want).sum())} outputs differ"


@pytest.mark.parametrize("kernel", ["tiles", "chunks"])
def test_linear_zero_rows(kernel):
    # T = 0 is a no-op; all-zero rows give exact zeros
    K, N, g = 512, 64, 128
    x0, w = linear_inputs(9, 4, K, N)
    _, dev = _pack(w, g)
    y = dg.w4a16_linear(torch.zeros((4, K), dtype=torch.float16, device="cuda"), dev, rows=kernel)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    empty = dg.w4a16_linear(torch.zeros((0, K), dtype=torch.float16, device="cuda"), dev)
    assert empty.shape == (0, N)


@pytest.mark.parametrize("g", [64, 128])
def test_linear_many_rows_are_independent_and_deterministic(g):
    # the many-row kernel stages 256-row activation blocks shared by all its
    # waves: an output row depends on its own input row only (changing every
    # other row leaves it bit for bit the same), and a call repeated gives
    # the same bits
    T, K, N = 300, 2816, 512
    x, w = linear_inputs(31 + g, T, K, N)
    _, dev = _pack(w, g)
    xd = torch.from_numpy(x).cuda()
    y1 = dg.w4a16_linear(xd, dev, rows="chunks").clone()
    y2 = dg.w4a16_linear(xd, dev, rows="chunks").clone()
    x2 = xd.clone()
    x2[100:] = torch.flip(x2[100:], dims=[0])                # rows 100.. permuted
    x2[:100:3] = 0                                           # and some early rows zeroed
    y3 = dg.w4a16_linear(x2, dev, rows="chunks")
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    keep = torch.ones(100, dtype=torch.bool, device="cuda")
    keep[::3] = False
    assert torch.equal(y3[:100][keep].view(torch.int16), y1[:100][keep].view(torch.int16))
    assert torch.equal(y3[100:].view(torch.int16), torch.flip(y1[100:], dims=[0]).view(torch.int16))
    assert torch.count_nonzero(y3[:100:3]).item() == 0
