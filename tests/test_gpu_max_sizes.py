"""GPU parity at the largest token counts the library accepts for the
layer's widths (d = 2816, m = 704), where its 32-bit offsets come closest to
their bounds: on 32-row tiles the gated intermediate H (padded rows x m x 2
bytes) just under 2 GiB, on 128-row chunks the expert outputs Y (T * topk x
d x 2 bytes) just under 2 GiB. Eight experts, top-8: every token reaches
every expert, so the alignment's per-expert ranges are as long as they get.
The largest T is the library's own answer (its workspace query accepts it,
and refuses T + 1); 48 tokens spread over the whole range, the first and
last included, are compared with the CPU oracle, and every output is
checked finite.
"""
import numpy as np
import pytest
import torch

import w4a16_grouped_moe_amd as dg
from tests import layer_cases as lc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    dg.lib()


def _largest_T(gu_g, dn_g, rows):
    def ok(T):
        try:
            dg.workspace_bytes(T, 8, 8, 2816, 704, gu_g, dn_g, rows=rows)
            return True
        except dg.Dgw4Error as e:
            assert "UNSUPPORTED" in str(e)
            return False
    lo, hi = 1, 1 << 20
    while lo < hi:
        mid = (lo + hi + 1) // 2
        lo, hi = (mid, hi) if ok(mid) else (lo, mid - 1)
    assert ok(lo) and not ok(lo + 1)
    return lo


@pytest.mark.parametrize("rows", ["tiles", "chunks"])
def test_largest_T(rows):
    t = dg.WEIGHTS_TILED
    T = _largest_T(128 | t, 64 | t, rows)
    A = 8 * T
    if rows == "tiles":
        assert (A + 8 * 31) * 704 * 2 < 1 << 31 <= (A + 8 + 8 * 31) * 704 * 2
    else:
        assert A * 2816 * 2 < 1 << 31 <= (A + 8) * 2816 * 2
    lc.log(f"[max sizes] {rows}: T = {T}")
    L = lc.build(lc.custom_shape(f"max_{rows}", E=8, topk=8, T=T, d=2816, m=704, index=102))
    gu, dn = dg.pack_tiled(L.gu_dev), dg.pack_tiled(L.dn_dev)
    assert dg.row_block(T, 8, 8, 2816, 704, gu[3], dn[3], rows=rows) == (32 if rows == "tiles" else 128)
    out = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, rows=rows)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    tok = np.unique(np.concatenate([[0, T - 1], np.random.default_rng(T).choice(T, 46, replace=False)]))
    lc.assert_close(out[torch.as_tensor(tok, device="cuda")].cpu().numpy(), lc.oracle_forward(L, tokens=tok),
                    f"largest T on {rows} (T = {T}, {tok.size} sampled tokens)")
