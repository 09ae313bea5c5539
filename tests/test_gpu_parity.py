"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer work (packing, alignment) is compared bit for bit; the layer output
element by element within max|err| <= 1e-2 * max|ref|, on every output
element of every workload: the tiny one, shapes with several tiles and
ragged tails, and the full-size workloads (T = 256 uniform and Zipf-skewed,
T = 1024) in the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import w4a16_grouped_moe_amd as dg
from synth import CONFIGS
from tests import layer_cases as lc

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no ROCm device")
    dg.lib()


# ------------------------------------------------------------- quantiser ----

@pytest.mark.parametrize("g", [64, 128])
def test_quantize_edge_groups(g):
    lc.log(f"[quant] edge groups g={g}")
    rng = np.random.default_rng(g)
    rows = []
    rows.append(np.zeros(4 * g, np.float32))                                # all zero
    rows.append(np.full(4 * g, 0.75, np.float32))                           # constant
    r = np.zeros(4 * g, np.float32); r[1:g] = np.linspace(0.01, 1, g - 1); rows.append(r)  # min +0
    r = -np.zeros(4 * g, np.float32); r[g:] = rng.standard_normal(3 * g); rows.append(r)   # -0s
    rows.append((1000 + np.arange(4 * g) * 1e-3).astype(np.float32))       # saturated z
    rows.append((rng.standard_normal(4 * g) * 1e-6).astype(np.float32))    # subnormal-ish s
    rows.append((rng.standard_t(2, 4 * g) * 1e-2).astype(np.float32))      # outliers
    rows.append(rng.uniform(0.5, 2, 4 * g).astype(np.float32))             # one-signed
    rows.append(-rng.uniform(0.5, 2, 4 * g).astype(np.float32))
    base = np.zeros(4 * g, np.int64) + 5
    base[0], base[1] = 0, 15
    r = ((base - 5) * 0.0625).astype(np.float32); r[2:6] = np.array([0.5, 1.5, -0.5, 2.5]) * 0.0625
    rows.append(r)                                                          # exact ties
    w = np.stack(rows)[None]
    lc.pack_both(w, g)


@pytest.mark.parametrize("name", ["tiny", "full"])
def test_quantize_workload_bitexact(name):
    shp = CONFIGS[name]
    lc.log(f"[quant] workload {name}")
    from synth import expert_weights
    gw, dw = expert_weights(shp)
    lc.pack_both(gw, shp.g_gu)
    lc.pack_both(dw, shp.g_dn)


# ------------------------------------------------------------- alignment ----

def _align_case(ids, E, bm):
    ref = oracle.align(ids, E, bm)
    # garbage in the output buffers must not matter
    got = dg.align(torch.from_numpy(ids).cuda(), E, bm)
    torch.cuda.synchronize()
    for k in ref:
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k


@pytest.mark.parametrize("bm", [16, 32, 64])
def test_align_random(bm):
    lc.log(f"[align] random bm={bm}")
    rng = np.random.default_rng(bm)
    for T, topk, E in [(1, 1, 1), (7, 3, 5), (64, 2, 8), (256, 8, 128), (1024, 8, 128),
                       (333, 4, 1024), (5, 8, 8)]:
        _align_case(rng.integers(0, E, (T, topk)).astype(np.int32), E, bm)


@pytest.mark.parametrize("name", ["tiny", "full", "skew", "wide"])
def test_align_workloads(name):
    shp = CONFIGS[name]
    lc.log(f"[align] workload {name}")
    ids, _ = lc.route(shp)
    _align_case(ids, shp.E, 32)


def test_align_degenerate():
    lc.log("[align] degenerate")
    _align_case(np.zeros((300, 8), np.int32), 128, 32)                 # one expert takes all
    _align_case(np.full((3, 2), 7, np.int32), 8, 16)
    _align_case(np.zeros((0, 8), np.int32), 128, 32)                    # no tokens


def test_align_skips_out_of_range_ids():
    lc.log("[align] out-of-range ids")
    ids = np.array([[0, 9], [-1, 3], [3, 3]], np.int32)
    got = dg.align(torch.from_numpy(ids).cuda(), 8, 16)
    torch.cuda.synchronize()
    assert list(got["counts"].cpu().numpy()) == [1, 0, 0, 3, 0, 0, 0, 0]
    sid = got["sorted_ids"].cpu().numpy()
    assert list(sid[:1]) == [0] and list(sid[16:19]) == [3, 4, 5]


# --------------------------------------------------------------- forward ----

def test_forward_tiny_every_element():
    L = lc.build(CONFIGS["tiny"])
    lc.assert_close(lc.gpu_forward(L), lc.oracle_forward(L), "tiny")


@pytest.mark.parametrize("case", [
    # several 32-row tiles per expert with a ragged last tile; ragged last K chunk
    dict(name="ragged", E=8, topk=2, T=333, d=640, m=320),
    # down N-blocks with idle waves (576 = 4.5 x 128), g=64 for gate_up too
    dict(name="edge_n", E=6, topk=3, T=97, d=576, m=192, g_gu=64),
    # g=128 on the down projection, single expert, top-1
    dict(name="top1", E=1, topk=1, T=45, d=256, m=256, g_dn=128),
    # one token
    dict(name="one_token", E=16, topk=4, T=1, d=512, m=192),
    # m > 768: down streams K = m in chunks (odd chunk count, odd group count);
    # gate_up's last N-block has idle waves (1088 = 8.5 x 128)
    dict(name="long_m", E=4, topk=2, T=50, d=384, m=1088),
])
def test_forward_shapes_every_element(case):
    shp = lc.custom_shape(**case)
    L = lc.build(shp)
    lc.assert_close(lc.gpu_forward(L), lc.oracle_forward(L), case["name"])


@pytest.mark.parametrize("T", [1, 5, 37])
def test_forward_layer_shape_small_T_every_element(T):
    # the one-launch gate_up + down path with nearly empty, ragged tiles
    shp = lc.custom_shape(f"fused_T{T}", E=16, topk=8, T=T, d=2816, m=704, index=92)
    L = lc.build(shp)
    lc.assert_close(lc.gpu_forward(L), lc.oracle_forward(L), f"layer shape T={T}")


def test_forward_layer_shape_duplicate_and_dropped_ids():
    shp = lc.custom_shape("fused_dups", E=16, topk=8, T=24, d=2816, m=704, index=93)
    rng = np.random.default_rng(8)
    ids = rng.integers(0, 16, (24, 8)).astype(np.int32)
    ids[:, 1] = ids[:, 0]                                   # duplicates are independent
    w = rng.uniform(0.1, 1, (24, 8)).astype(np.float32)
    bad = ids.copy()
    bad[::3, 2] = -1                                        # dropped by the GPU path
    bad[1::5, 7] = 16
    L = lc.build(shp, ids=bad, w=w)
    gpu = lc.gpu_forward(L)
    keep = (bad >= 0) & (bad < 16)
    L.ids = np.where(keep, bad, 0).astype(np.int32)
    L.w = np.where(keep, w, 0).astype(np.float32)
    lc.assert_close(gpu, lc.oracle_forward(L), "layer shape dups/dropped")


def test_forward_duplicate_and_dropped_ids():
    shp = lc.custom_shape("dups", E=8, topk=4, T=40, d=512, m=192)
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 8, (40, 4)).astype(np.int32)
    ids[:, 1] = ids[:, 0]                                   # duplicates are independent
    w = rng.uniform(0.1, 1, (40, 4)).astype(np.float32)
    bad = ids.copy()
    bad[::3, 2] = -1                                        # dropped by the GPU path
    bad[1::5, 3] = 8
    L = lc.build(shp, ids=bad, w=w)
    gpu = lc.gpu_forward(L)
    keep = (bad >= 0) & (bad < 8)
    L.ids = np.where(keep, bad, 0).astype(np.int32)         # oracle: same layer without them
    L.w = np.where(keep, w, 0).astype(np.float32)
    lc.assert_close(gpu, lc.oracle_forward(L), "dups/dropped")


def _every_token(L, what):
    gpu = lc.gpu_forward(L)
    lc.assert_close(gpu, lc.oracle_forward(L), what)
    return gpu


@pytest.fixture(scope="module")
def full_layer():
    return lc.cached("full")


def test_forward_full_every_token(full_layer):
    _every_token(full_layer, "full (all 256 tokens)")


def test_forward_full_deterministic_100(full_layer):
    L = full_layer
    ws = torch.empty(dg.workspace_bytes(L.shape.T, L.shape.topk, L.shape.E, L.shape.d,
                                        L.shape.m), dtype=torch.uint8, device="cuda")
    first = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, L.gu_dev, L.dn_dev, workspace=ws).clone()
    bad = 0
    for i in range(100):
        if i % 10 == 0:                          # stale workspace contents must not matter
            ws.random_(0, 256)
        o = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, L.gu_dev, L.dn_dev, workspace=ws)
        bad += int(not torch.equal(o.view(torch.int16), first.view(torch.int16)))
    torch.cuda.synchronize()
    lc.log(f"[determinism] 100 runs, {bad} differing")
    assert bad == 0


@pytest.mark.parametrize("rows", ["tiles", "chunks"])
def test_forward_out_8_byte_aligned(full_layer, rows):
    # an output at the API's minimum alignment (8 bytes, not 16) gets the same
    # bits as a fresh tensor and nothing outside it is written, on the two Y
    # layouts (two partials on tiles, one array on chunks)
    L = full_layer
    T, d = L.shape.T, L.shape.d
    gu, dn = (dg.pack_tiled(L.gu_dev), dg.pack_tiled(L.dn_dev)) if rows == "chunks" else (L.gu_dev, L.dn_dev)
    ref = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, rows=rows)
    buf = torch.full((T * d + 4,), float("nan"), dtype=torch.float16, device="cuda")
    out = buf[4:].view(T, d)
    assert out.data_ptr() % 16 == 8
    dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, gu, dn, out=out, rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert torch.isnan(buf[:4]).all()


def test_forward_layer_shape_unfused_every_token():
    # gate_up with g=64 at the layer's shape: the generic gate_up kernel, then
    # the layer-shape down kernel as a launch of its own
    shp = lc.custom_shape("unfused", E=128, topk=8, T=256, d=2816, m=704, g_gu=64, index=91)
    L = lc.build(shp)
    _every_token(L, "layer shape, gate_up g=64 (all 256 tokens)")


def test_forward_graph_replay_matches_eager(full_layer):
    # the forward enqueues kernels only (no host sync, no memset), so it can be
    # captured; every replay re-aligns and clears its tile counters on the
    # device, so replays after scribbling on the workspace stay bitwise equal
    L = full_layer
    ws = torch.empty(dg.workspace_bytes(L.shape.T, L.shape.topk, L.shape.E, L.shape.d,
                                        L.shape.m), dtype=torch.uint8, device="cuda")
    ref = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, L.gu_dev, L.dn_dev, workspace=ws).clone()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, L.gu_dev, L.dn_dev, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, L.gu_dev, L.dn_dev, workspace=ws, out=out)
    for r in range(4):
        out.zero_()
        ws.random_(0, 256)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        lc.log(f"[graph] replay {r}")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {r} differs"
    del g


def test_forward_skew_every_token():
    _every_token(lc.cached("skew"), "skew (all 256 tokens)")


def test_forward_wide_every_token():
    _every_token(lc.cached("wide"), "wide (all 1024 tokens)")


def test_forward_timed_equals_forward(full_layer):
    # the benchmark's stage split calls the timed entry point; it must run the
    # same kernels with the same results
    L = full_layer
    plain = lc.gpu_forward(L)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    out = dg.moe_forward(L.x_dev, L.ids_dev, L.w_dev, L.gu_dev, L.dn_dev, events=evs)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.int16), plain.view(np.int16))
    stages = [evs[i].elapsed_time(evs[i + 1]) for i in range(4)]
    lc.log(f"[timed] stage ms {stages}")
    assert all(t >= 0.0 for t in stages) and stages[1] > 0.0


def test_read_probe_runs():
    n = 64 << 20
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    dg.hbm_read_probe(buf, sink)
    e0.record()
    dg.hbm_read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbps = n / (e0.elapsed_time(e1) * 1e-3) / 1e9
    lc.log(f"[probe] 64 MiB read at {gbps:.0f} GB/s")
    assert sink.item() == 0 and gbps > 100.0


def test_mfma_probe_runs():
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    dg.mfma_probe(200, sink)
    e0.record()
    flops = dg.mfma_probe(2000, sink)
    e1.record()
    torch.cuda.synchronize()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops == cus * 2 * 8 * 2000 * 8 * 2 * 16 * 16 * 32
    tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    lc.log(f"[probe] MFMA f16 at {tflops:.0f} TFLOP/s")
    assert sink.item() == 0 and tflops > 100.0


@pytest.mark.parametrize("name", ["down_g64", "down_g128"])
def test_forward_down_group_variants_every_token(name):
    # the layer's shape with separate gate_up and down launches: down at
    # g = 64 (K = 704) and the g = 128 variant with K padded to 768
    L = lc.build(CONFIGS[name])
    _every_token(L, f"{name} (all 256 tokens)")
