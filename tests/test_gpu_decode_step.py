"""The decode step of the 1.5B example on the GPU (needs an MI355X): every linear
shape of the step against the oracle, and the step's launches captured in a HIP
graph and replayed, each replay bit-identical to the eager calls.

Shapes: "AWQ + GPTQ Quantization, in depth", Worked example: where the bytes go in a
1.5B model (28 layers of qkv 1536 -> 2048, o 1536 -> 1536, gate+up 1536 -> 17920 and
down 8960 -> 1536 at group size 128).
"""

import numpy as np
import pytest

import oracle
import w4a16_gemm_amd as w4
import workloads as wl
from gpu_common import device, note, oracle_layer, product_layer, run_gemm, sample_rows

pytestmark = pytest.mark.gpu

TOL = 1e-2
CONFIGS = wl.decode_step_configs()


@pytest.mark.parametrize("lin", range(len(CONFIGS)))
def test_decode_step_linears_match_oracle(lin):
    cfg = CONFIGS[lin]
    rows = np.unique(np.concatenate([sample_rows(cfg.N, 64), np.arange(cfg.N - 8, cfg.N)]))
    note(f"decode-step linear {cfg.name} (K={cfg.K} N={cfg.N})")
    prod = product_layer(cfg, 1)
    ref = oracle_layer(cfg, 1, rows)
    assert np.array_equal(prod["codes"][rows], ref["codes"])
    y = run_gemm(prod).cpu().numpy()[:, rows]
    assert oracle.rel_err(y, ref["y_ref"]) <= TOL
    y2 = run_gemm(prod).cpu().numpy()[:, rows]
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


def test_decode_step_graph_replays_match_eager():
    """One layer's four launches captured once and replayed three times, with eager
    library calls and host synchronisation between the replays."""
    import torch
    layers = [product_layer(cfg, 1) for cfg in CONFIGS]
    outs = [torch.empty((1, cfg.N), dtype=torch.float16, device=device()) for cfg in CONFIGS]

    def step():
        for L, cfg, y in zip(layers, CONFIGS, outs):
            w4.w4a16_gemm(L["x"][:1], L["qweight"], L["scales"], L["qzeros"], None, cfg.group_size, y=y)

    note("decode step: eager reference")
    step()
    torch.cuda.synchronize()
    eager = [y.clone() for y in outs]
    note("decode step: capture")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for y in outs:
            y.fill_(float("nan"))
        note(f"decode step: replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        for y, e in zip(outs, eager):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16))
        # eager work between replays
        other = run_gemm(layers[1])
        assert not bool(torch.isnan(other).any())
        torch.cuda.synchronize()
