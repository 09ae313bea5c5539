"""GPU parity of the layer on 128-row chunks (DGW4_ROWS_CHUNKS): the
alignment with 128-row blocks, the chunk gate_up and the chunk down, against
the CPU oracle, element by element within max|err| <= 1e-2 * max|ref|.

The chunk GEMMs take tiled weights (dgw4_pack_tiled); the canonical layout
asked to run on chunks is refused. Covers nearly empty chunks (T = 1, 5,
37), experts whose rows end exactly at, one past and well past a chunk
boundary, empty experts, experts with three chunks and a ragged last one
(Zipf routing at T = 300 over 16 experts), duplicate and dropped ids, the
routed entry point, the full-size workloads (T = 256 uniform and skewed on
chunks; T = 1024, which takes chunks by default, also on 32-row tiles),
determinism over reruns with stale workspace contents, graph replay, and
1024 experts of which 7 hold rows (on chunks and on tiles).
"""
import numpy as np
import pytest
import torch

import w4a16_grouped_moe_amd as dg
from synth import CONFIGS
from tests import layer_cases as lc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    dg.lib()


def _layer_shape(name, T, E=16, topk=8, zipf=None, index=94):
    return lc.custom_shape(name, E=E, topk=topk, T=T, d=2816, m=704, zipf=zipf, index=index)


def _tiled(L):
    return dg.pack_tiled(L.gu_dev), dg.pack_tiled(L.dn_dev)


def _forward(L, rows="chunks", workspace=None, out=None, events=None):
    gu, dn = _tiled(L)
    o = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, workspace=workspace, out=out,
                       events=events, rows=rows)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("T", [1, 5, 37])
def test_chunks_small_T_every_element(T):
    # nearly empty chunks: one to a few rows of a 128-row chunk
    L = lc.build(_layer_shape(f"chunks_T{T}", T))
    lc.assert_close(_forward(L).cpu().numpy(), lc.oracle_forward(L), f"chunks T={T}")


@pytest.mark.parametrize("case", ["boundary_129", "boundary_128"])
def test_chunks_at_chunk_boundaries(case):
    # expert rows ending exactly at a chunk (128), one row past it (129), a
    # second chunk of 65 rows, and experts with no rows at all
    if case == "boundary_129":
        T = 193
        ids = np.zeros((T, 2), np.int32)
        ids[:129] = (0, 1)
        ids[129:] = (1, 2)                 # e0: 129, e1: 193, e2: 64, e3: none
    else:
        T = 128
        ids = np.tile(np.array([[0, 3]], np.int32), (T, 1))   # e0, e3: 128 each
    w = np.random.default_rng(11).uniform(0.1, 1, (T, 2)).astype(np.float32)
    L = lc.build(lc.custom_shape(case, E=4, topk=2, T=T, d=2816, m=704, index=95), ids=ids, w=w)
    lc.assert_close(_forward(L).cpu().numpy(), lc.oracle_forward(L), case)


def test_chunks_three_chunk_experts_skewed():
    # Zipf routing over 16 experts at T = 300: hot experts hold up to 300
    # rows (three chunks, the last ragged), cold ones a few
    L = lc.build(_layer_shape("chunks_zipf", 300, zipf=1.2, index=96))
    counts = np.bincount(L.ids.ravel(), minlength=16)
    lc.log(f"[chunks] expert rows {sorted(counts.tolist())}")
    assert counts.max() > 256
    lc.assert_close(_forward(L).cpu().numpy(), lc.oracle_forward(L), "chunks zipf T=300")


def test_chunks_duplicate_and_dropped_ids():
    shp = _layer_shape("chunks_dups", 24, index=97)
    rng = np.random.default_rng(8)
    ids = rng.integers(0, 16, (24, 8)).astype(np.int32)
    ids[:, 1] = ids[:, 0]                                   # duplicates are independent
    w = rng.uniform(0.1, 1, (24, 8)).astype(np.float32)
    bad = ids.copy()
    bad[::3, 2] = -1                                        # dropped by the GPU path
    bad[1::5, 7] = 16
    L = lc.build(shp, ids=bad, w=w)
    gpu = _forward(L).cpu().numpy()
    keep = (bad >= 0) & (bad < 16)
    L.ids = np.where(keep, bad, 0).astype(np.int32)
    L.w = np.where(keep, w, 0).astype(np.float32)
    lc.assert_close(gpu, lc.oracle_forward(L), "chunks dups/dropped")


def test_chunks_routed_and_canonical_refused():
    # the routed entry point (router in the same call) on chunks; the
    # canonical layout on chunks is refused, on the library's choice it runs
    # (on tiles)
    L = lc.build(_layer_shape("chunks_routed", 64, index=98))
    ref = lc.oracle_forward(L)
    from synth import router_logits
    logits = torch.from_numpy(router_logits(L.shape, 0)).cuda()
    gu, dn = _tiled(L)
    routed = dg.moe_forward_routed(L.x_dev, logits, L.shape.topk, gu, dn, rows="chunks")
    torch.cuda.synchronize()
    lc.assert_close(routed.cpu().numpy(), ref, "chunks routed")
    with pytest.raises(dg.Dgw4Error, match="UNSUPPORTED"):
        dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, L.gu_dev, L.dn_dev, rows="chunks")
    lc.assert_close(lc.gpu_forward(L), ref, "canonical, library's choice")


@pytest.mark.parametrize("name", ["full", "skew"])
def test_chunks_full_size_every_token(name):
    L = lc.cached(name)
    lc.assert_close(_forward(L).cpu().numpy(), lc.oracle_forward(L),
                    f"{name} on chunks (all {L.shape.T} tokens)")


def test_wide_on_tiles_every_token():
    # T = 1024 runs on chunks by default; the 32-row tiles stay correct there
    L = lc.cached("wide")
    lc.assert_close(lc.gpu_forward(L, rows="tiles"), lc.oracle_forward(L),
                    "wide on tiles (all 1024 tokens)")


def test_chunks_deterministic_with_stale_workspace():
    # T = 1024 with tiled weights: chunks by the library's choice
    L = lc.cached("wide")
    s = L.shape
    gu, dn = _tiled(L)
    ws = torch.empty(dg.workspace_bytes(s.T, s.topk, s.E, s.d, s.m, gu[3], dn[3]),
                     dtype=torch.uint8, device="cuda")
    assert ws.numel() == dg.workspace_bytes(s.T, s.topk, s.E, s.d, s.m, gu[3], dn[3], rows="chunks")
    first = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, workspace=ws).clone()
    lc.assert_close(first.cpu().numpy(), lc.oracle_forward(L), "wide, library's choice (chunks)")
    bad = 0
    for i in range(30):
        if i % 10 == 0:
            ws.random_(0, 256)
        o = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, workspace=ws)
        bad += int(not torch.equal(o.view(torch.int16), first.view(torch.int16)))
    torch.cuda.synchronize()
    lc.log(f"[chunks determinism] 30 runs, {bad} differing")
    assert bad == 0


def test_chunks_timed_and_graph_replay():
    L = lc.cached("full")
    s = L.shape
    gu, dn = _tiled(L)
    ws = torch.empty(dg.workspace_bytes(s.T, s.topk, s.E, s.d, s.m, gu[3], dn[3], rows="chunks"),
                     dtype=torch.uint8, device="cuda")
    ref = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, workspace=ws, rows="chunks").clone()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    timed = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, workspace=ws, events=evs,
                           rows="chunks")
    torch.cuda.synchronize()
    assert torch.equal(timed.view(torch.int16), ref.view(torch.int16))
    stages = [evs[i].elapsed_time(evs[i + 1]) for i in range(4)]
    lc.log(f"[chunks timed] stage ms {stages}")
    assert all(t > 0.0 for t in stages)
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, workspace=ws, out=out, rows="chunks")
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, workspace=ws, out=out, rows="chunks")
    for r in range(3):
        out.zero_()
        ws.random_(0, 256)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        lc.log(f"[chunks graph] replay {r}")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r} differs"
    del g


def test_chunks_many_chunks_per_expert_sampled():
    # 32 experts at T = 2048, top-8: ~512 rows (four chunks) per expert, a
    # grid of several rounds; 64 sampled tokens against the oracle, the rest
    # checked for finiteness, and a rerun bitwise equal
    L = lc.build(lc.custom_shape("chunks_T2048", E=32, topk=8, T=2048, d=2816, m=704, index=99))
    gu, dn = _tiled(L)
    s = L.shape
    assert dg.row_block(s.T, s.topk, s.E, s.d, s.m, gu[3], dn[3]) == 128
    out = _forward(L, rows="auto")
    again = _forward(L, rows="auto")
    assert torch.equal(out.view(torch.int16), again.view(torch.int16))
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got.astype(np.float32)))
    tok = np.random.default_rng(5).choice(s.T, 64, replace=False)
    tok.sort()
    lc.assert_close(got[tok], lc.oracle_forward(L, tokens=tok), "chunks T=2048, 64 sampled tokens")


def test_chunks_top4_every_token():
    # E = 64, top-4 at T = 1024: 64 rows per expert, chunks by the library's
    # choice
    L = lc.build(lc.custom_shape("chunks_top4", E=64, topk=4, T=1024, d=2816, m=704, index=100))
    gu, dn = _tiled(L)
    s = L.shape
    assert dg.row_block(s.T, s.topk, s.E, s.d, s.m, gu[3], dn[3]) == 128
    lc.assert_close(_forward(L, rows="auto").cpu().numpy(), lc.oracle_forward(L),
                    "chunks E=64 top-4 T=1024 (every token)")


def _scatter_experts(pack, slots, E):
    # a device pack of E experts whose experts slots[i] hold pack's expert i
    # (the rest zero, never routed to)
    q, s, z, g = pack
    out = []
    for a in (q, s, z):
        big = torch.zeros((E,) + tuple(a.shape[1:]), dtype=a.dtype, device=a.device)
        big[torch.as_tensor(slots, device=a.device)] = a
        out.append(big)
    return (*out, g)


@pytest.mark.parametrize("rows", ["chunks", "tiles"])
def test_many_experts_few_live(rows):
    # E = 1024 (the largest expert count) with 7 live experts spread over it
    # (0 .. 1023), the others empty: the alignment's per-expert workgroups and
    # offsets over 1024 experts; on tiles the layer kernel does not take so
    # many experts, so the separate alignment and GEMMs run
    E = 1024
    slots = [0, 63, 64, 130, 511, 700, 1023]
    T, topk = 200, 4
    rng = np.random.default_rng(13)
    small = np.stack([rng.choice(len(slots), topk, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.uniform(0.1, 1, (T, topk)).astype(np.float32)
    L = lc.build(lc.custom_shape(f"many_experts_{rows}", E=len(slots), topk=topk, T=T, d=2816, m=704,
                                 index=101), ids=small, w=w)
    ref = lc.oracle_forward(L)
    gu, dn = _tiled(L)
    gu_big, dn_big = _scatter_experts(gu, slots, E), _scatter_experts(dn, slots, E)
    big_ids = torch.as_tensor(np.asarray(slots, np.int32)[small], device="cuda")
    lc.log(f"[many experts] live expert rows {np.bincount(small.ravel()).tolist()}")
    o = dg.moe_forward(L.x_dev, big_ids, L.w_dev, gu_big, dn_big, rows=rows)
    torch.cuda.synchronize()
    lc.assert_close(o.cpu().numpy(), ref, f"E={E} on {rows}, 7 live experts")
