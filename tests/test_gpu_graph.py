"""The two layer paths that use workspace memory (act order above 32 rows: x gathered
into stored order; skinny batches with K split over workgroups: fp32 partial tiles)
captured into a HIP graph and replayed: every replay bit-identical to the eager call,
with other eager work and synchronisations between replays, and parity with the oracle
on sampled rows.  A call that would have to grow the workspace during capture is
refused with an error instead of allocating."""

import pytest

import oracle
import w4a16_gemm_amd as w4
import workloads as wl
from gpu_common import device, note, oracle_layer, product_layer, sample_rows

pytestmark = pytest.mark.gpu
TOL = 1e-2

CASES = [
    # name, config, M: act order at M = 512 (the act-order configuration), and a
    # skinny batch whose K is split over workgroup slices
    ("act-order c5 M=512", wl.CONFIGS["c5"], 512),
    ("skinny split-K M=4", wl.custom_config("splitk", 61, K=16384, N=4096, group_size=128, M_list=(4,)), 4),
]


@pytest.mark.parametrize("name,cfg,M", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, cfg, M):
    import torch
    dev = device()
    note(f"graph capture: {name} N={cfg.N} K={cfg.K} g={cfg.group_size}")
    layer = product_layer(cfg, M)
    args = (layer["qweight"], layer["scales"], layer["qzeros"], layer["g_idx"], cfg.group_size)
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        y_eager = w4.w4a16_gemm(layer["x"], *args)       # sizes the stream's workspace
    s.synchronize()
    y_graph = torch.empty_like(y_eager)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        w4.w4a16_gemm(layer["x"], *args, y=y_graph)
    other = torch.randn(layer["x"].shape, device=dev).to(torch.float16)
    for rep in range(3):
        y_graph.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int16), y_eager.view(torch.int16)), f"replay {rep}"
        # eager work on the same stream between replays (same workspace, other inputs)
        with torch.cuda.stream(s):
            w4.w4a16_gemm(other, *args)
        torch.cuda.synchronize()
    rows = sample_rows(cfg.N, 24)
    ref = oracle_layer(cfg, M, rows)
    err = oracle.rel_err(y_graph.cpu().numpy()[:, rows], ref["y_ref"])
    assert err <= TOL, err


# the refused call records nothing, so the captured graph is empty by design
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_capture_refuses_to_grow_the_workspace():
    import torch
    dev = device()
    # act order at 4096 rows: 32 MB of gathered activations, more than any earlier test
    # reserves on a stream (torch hands out pooled streams, so the stream may have been
    # used before)
    cfg = wl.custom_config("act-cap", 62, K=4096, N=256, group_size=128, M_list=(4096,), act_order=True)
    M = 4096
    note("graph capture that needs a larger workspace than its stream holds (expects an error, no launch)")
    layer = product_layer(cfg, M)
    args = (layer["qweight"], layer["scales"], layer["qzeros"], layer["g_idx"], cfg.group_size)
    s = torch.cuda.Stream(device=dev)
    y = torch.empty((M, cfg.N), dtype=torch.float16, device=dev)
    graph = torch.cuda.CUDAGraph()
    caught = None
    with torch.cuda.graph(graph, stream=s):
        try:
            w4.w4a16_gemm(layer["x"], *args, y=y)
        except w4.W4A16Error as e:
            caught = e
    assert caught is not None and caught.status == w4.ERR_UNSUPPORTED
    assert "capture" in str(caught)
    # the same call eagerly on that stream then works, and so does its capture
    with torch.cuda.stream(s):
        y_eager = w4.w4a16_gemm(layer["x"], *args)
    s.synchronize()
    graph2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph2, stream=s):
        w4.w4a16_gemm(layer["x"], *args, y=y)
    graph2.replay()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16))
    rows = sample_rows(cfg.N, 16)
    ref = oracle_layer(cfg, 64, rows, x=wl.activations(cfg, M)[:64])
    err = oracle.rel_err(y_eager.cpu().numpy()[:64][:, rows], ref["y_ref"])
    assert err <= TOL, err
