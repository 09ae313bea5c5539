"""GPU: audit of the benchmarked workload against the oracle.

The benchmark times a rotated stack of 30 full-size layers whose fp32 master
weights are drawn on the device. Three of them (0, 17 and 29) are rebuilt
here exactly as bench.py builds them (bench.make_layer): the device masters
are copied to the host, the device packing is checked bit for bit against
the oracle's quantiser, the tiled copy byte for byte against the layout's
description, and the tiled forward (the launch the benchmark times) on all
256 tokens against the oracle forward on the oracle's own packing.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import w4a16_grouped_moe_amd as dg
from synth import CONFIGS
from tests import layer_cases as lc
from tests.tiled_layout import pack_tiled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    dg.lib()


@pytest.mark.parametrize("layer", [0, 17, 29])
def test_stack_layer_audit(layer):
    shape = CONFIGS["stack"]
    dev = torch.device("cuda:0")
    lc.log(f"[stack] layer {layer}: building as the benchmark does")
    ly = bench.make_layer(torch, dg, shape, layer, dev, "tiled", keep_masters=True)
    gw, dw = (t.cpu().numpy() for t in ly["masters"])
    ly["masters"] = None
    host = {}
    for name, wf, g, tiled, canon in (("gate_up", gw, shape.g_gu, ly["gu"], ly["gu_other"]),
                                      ("down", dw, shape.g_dn, ly["dn"], ly["dn_other"])):
        hq, hs, hz = oracle.quantize_rtn(wf, g)
        assert np.array_equal(canon[0].cpu().numpy(), hq), f"{name}: nibbles differ"
        assert np.array_equal(canon[1].cpu().numpy().view(np.uint16), hs), f"{name}: scales differ"
        assert np.array_equal(canon[2].cpu().numpy().view(np.uint16), hz), f"{name}: zeros differ"
        assert np.array_equal(tiled[0].cpu().numpy(), pack_tiled(hq, g)), f"{name}: tiled bytes differ"
        host[name] = (hq, hs, hz, g)
    del gw, dw
    sh = shape
    ws = torch.empty(dg.workspace_bytes(sh.T, sh.topk, sh.E, sh.d, sh.m, ly["gu"][3], ly["dn"][3]),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((sh.T, sh.d), dtype=torch.float16, device=dev)
    dg.moe_forward(ly["x"], ly["ids"], ly["w"], ly["gu"], ly["dn"], workspace=ws, out=out)
    torch.cuda.synchronize()
    # the oracle routes the same logits itself; the device router's choice
    # (which the forward above used) must be the same bit for bit
    ids, w = oracle.router(ly["logits_host"], sh.topk)
    assert np.array_equal(ly["ids"].cpu().numpy(), ids), "router ids differ"
    assert np.allclose(ly["w"].cpu().numpy(), w, rtol=2e-6, atol=0), "router weights differ"
    ref = oracle.moe_forward(ly["x_host"], ids, w.astype(np.float32), host["gate_up"],
                             host["down"], sh.E)
    lc.assert_close(out.cpu().numpy(), ref, f"stack layer {layer} (tiled, all 256 tokens)")
