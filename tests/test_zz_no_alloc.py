"""GPU: dgw4_sample_noalloc (the library's own partials, no workspace)
against dgw4_sample (a caller workspace), through the C ABI.

Two calls in a row on the same device, the second with a smaller input, each
compared bit for bit with the workspace call on the same logits and seed (the
same kernels: entropy, sample and argmax identical). Then a shape whose
partials exceed the fixed array is refused before any launch.
"""
import numpy as np
import pytest
import torch

import w4a16_grouped_moe_amd as dg
from synth import sampler_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    dg.lib()


def _same(a, b):
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_sample_noalloc_matches_workspace_call():
    print("[no_alloc] two calls, the second smaller", flush=True)
    for i, (R, V, seed) in enumerate([(64, 65536, 11), (5, 4100, 12)]):
        lg = torch.from_numpy(sampler_logits(40 + i, R, V, 2.0)).cuda()
        if i == 1:
            lg[1, ::7] = float("-inf")                   # masked entries too
        h0, s0, a0 = dg.sample(lg, seed)
        h1, s1, a1 = dg.sample_noalloc(lg, seed)
        torch.cuda.synchronize()
        assert _same(h0, h1), f"entropy differs (call {i})"
        assert torch.equal(s0, s1), f"sample differs (call {i})"
        assert torch.equal(a0, a1), f"argmax differs (call {i})"
        print(f"[no_alloc] call {i}: R={R} V={V} identical", flush=True)


def test_sample_noalloc_refuses_oversized():
    lg = torch.zeros((40000, 4), dtype=torch.float32, device="cuda")   # 40000 x 1 x 32 B > 1 MiB
    with pytest.raises(dg.Dgw4Error) as ei:
        dg.sample_noalloc(lg, 0)
    assert ei.value.status == dg.binding.ERR_UNSUPPORTED
