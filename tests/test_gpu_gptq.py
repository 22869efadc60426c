"""GPU parity of the GPTQ quantiser against the oracle (needs an MI355X).

GPTQ: "AWQ + GPTQ Quantization, in depth", The two algorithms, compactly.  Both
sides work in binary64; the device factorises H and applies the error feedback in
blocks, so its weights before rounding differ from the oracle's by a few units in the
last place, and a rounding decision could differ only for a value within that
distance of a rounding boundary.  The bar is therefore exact: codes, scales, zeros
and g_idx identical (a mismatch would be reported with its count).  The output error
on the calibration rows is compared with round-to-nearest, and the codes run through
the layer's GEMM.
"""

import numpy as np
import pytest

import oracle
import w4a16_gemm_amd as w4
import workloads as wl
from gpu_common import device, note, sample_rows

pytestmark = pytest.mark.gpu

CASES = [
    # name, N, K, group, act_order
    ("q1", 64, 256, 32, False),
    ("q2", 40, 512, 128, True),
    ("q3", 24, 160, 32, False),      # K not a multiple of the 64-wide Hessian tiles
    ("q4", 16, 96, 96, True),        # per-channel, act order
    ("q5", 136, 1024, 64, True),     # more channels than calibration tokens
]


def _same(a, b, what):
    a = np.asarray(a)
    b = np.asarray(b)
    bad = int(np.count_nonzero(a != b))
    assert bad == 0, f"{what}: {bad} of {a.size} differ"


@pytest.mark.parametrize("case", range(len(CASES)))
def test_gptq_matches_oracle(case):
    name, N, K, g, act = CASES[case]
    cfg = wl.custom_config(name, 700 + case, K=K, N=N, group_size=g, M_list=(1,))
    note(f"GPTQ {name} N={N} K={K} g={g} act={act}")
    w = wl.weights(cfg)
    x = wl.calibration(cfg)
    codes, S, Z, g_idx = w4.w4a16_gptq(w, x, g, act)
    rc, rs, rz, rg = oracle.gptq_quantize(w, x, g, act)
    if act:
        _same(g_idx, rg, "g_idx")
    _same(codes, rc, "codes")
    _same(S.view(np.uint16), rs.view(np.uint16), "scales")
    _same(Z, rz, "zeros")
    # the error feedback lowers the layer's output error on the calibration rows
    qc, qs, qz = oracle.rtn_quantize(w, g, g_idx)
    e_gptq = oracle.output_error(w, codes, S, Z, g, g_idx, x)
    e_rtn = oracle.output_error(w, qc, qs, qz, g, g_idx, x)
    note(f"  output error GPTQ {e_gptq:.4g} vs RTN {e_rtn:.4g}")
    assert e_gptq < e_rtn


def test_gptq_codes_through_the_gemm():
    import torch
    N, K, g, M = 128, 512, 128, 4
    cfg = wl.custom_config("q6", 720, K=K, N=N, group_size=g, M_list=(M,))
    w = wl.weights(cfg)
    xcal = wl.calibration(cfg)
    codes, S, Z, g_idx = w4.w4a16_gptq(w, xcal, g, True)
    qweight = w4.w4a16_pack(codes, g_idx, g)
    qzeros = w4.w4a16_pack_zeros(Z)
    dev = device()
    x = wl.activations(cfg, M)
    y = w4.w4a16_gemm(torch.from_numpy(x).to(dev), torch.from_numpy(qweight).to(dev), torch.from_numpy(S).to(dev),
                      torch.from_numpy(qzeros).to(dev), torch.from_numpy(g_idx).to(dev), g)
    torch.cuda.synchronize()
    ref = oracle.linear(x, codes, S, Z, g, g_idx)
    assert oracle.rel_err(y.cpu().numpy(), ref) <= 1e-2


def test_gptq_prefill_layer_on_sampled_rows():
    """The 2048-token prefill layer (N = 14336, K = 4096, group 128) in act order at its
    full size on the device; sampled rows against the oracle, which quantises rows
    independently once H is fixed."""
    cfg = wl.config("c4")
    note(f"GPTQ full-size {cfg.name} N={cfg.N} K={cfg.K}")
    w = wl.weights(cfg)
    x = wl.calibration(cfg)
    codes, S, Z, g_idx = w4.w4a16_gptq(w, x, cfg.group_size, True)
    rows = np.unique(np.concatenate([sample_rows(cfg.N, 24), np.arange(cfg.N - 4, cfg.N)]))
    rc, rs, rz, rg = oracle.gptq_quantize(w[rows], x, cfg.group_size, True)
    _same(g_idx, rg, "g_idx")
    _same(codes[rows], rc, "codes")
    _same(S[:, rows].view(np.uint16), rs.view(np.uint16), "scales")
    _same(Z[:, rows], rz, "zeros")
