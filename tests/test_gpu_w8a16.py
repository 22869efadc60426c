"""GPU parity of the 8-bit weight path against the oracle (needs an MI355X).

8-bit weights: "AWQ + GPTQ Quantization, in depth", 4-bit bigger or 8-bit smaller; the
symmetric variant is the int8 absmax scheme of "LLM Quantization: INT8, GPTQ, and AWQ
Explained", What quantization actually does, per group.  Same bars as the 4-bit
parity tests: codes bit-exact, the device weight view bit-exact, unit-vector probes
bit-exact, outputs within max|y - y_ref| / rms(y_ref) <= 1e-2.
"""

import os

import numpy as np
import pytest

import oracle
import w4a16_gemm_amd as w4
import workloads as wl
from gpu_common import clear_knob, device, note, oracle_layer, product_layer, run_gemm, sample_rows, set_knob

pytestmark = pytest.mark.gpu

TOL = 1e-2

CASES = [
    # name, M, N, K, group, act_order, sym
    ("e1", 1, 264, 1536, 128, False, False),    # GEMV, exact split
    ("e2", 1, 520, 8192, 64, True, False),      # GEMV, rows split over two wavefronts, act order
    ("e3", 1, 136, 12288, 128, False, True),    # GEMV, four slices, symmetric
    ("e4", 1, 72, 1056, 32, False, False),      # GEMV, inexact split
    ("e5", 4, 392, 2048, 128, False, False),    # tiled MFMA, 16-row blocks
    ("e6", 20, 264, 1024, 64, True, True),      # tiled, 32-row blocks, act order, symmetric
    ("e7", 100, 136, 640, 128, False, False),   # tiled, 128-row blocks
    ("e8", 300, 264, 1536, 1536, False, False), # per-channel, three 128-row blocks
    ("e9", 1, 40, 96, 96, False, True),         # per-channel, tiny K, symmetric
]


@pytest.fixture(autouse=True)
def _clear_env():
    clear_knob("W4A16_FORCE_PATH")
    yield
    clear_knob("W4A16_FORCE_PATH")


@pytest.mark.parametrize("case", range(len(CASES)))
def test_w8a16_layers_match_oracle(case):
    import torch
    name, M, N, K, g, act, sym = CASES[case]
    cfg = wl.custom_config(name, 600 + case, K=K, N=N, group_size=g, M_list=(M,), act_order=act, sym=sym, bits=8)
    note(f"8-bit {name} M={M} N={N} K={K} g={g} act={act} sym={sym}")
    prod = product_layer(cfg, M)
    ref = oracle_layer(cfg, M, np.arange(N))
    assert np.array_equal(prod["codes"], ref["codes"])
    for path in (["gemv", "gemm"] if M == 1 else ["gemm"]):
        set_knob("W4A16_FORCE_PATH", path)
        note(f"  path={path}")
        y = run_gemm(prod).cpu().numpy()
        assert oracle.rel_err(y, ref["y_ref"]) <= TOL, path
    clear_knob("W4A16_FORCE_PATH")
    W16 = w4.w8a16_dequant(prod["qweight"], prod["scales"], prod["qzeros"], prod["g_idx"], g, K).cpu().numpy()
    assert np.array_equal(W16.view(np.uint16), ref["W16"].view(np.uint16))
    back = w4.w8a16_unpack(prod["qweight"].cpu().numpy(), prod["g_idx_np"], g, N, K)
    assert np.array_equal(back, ref["codes"])
    # unit-vector probes: x = e_k gives binary16(W^[:, k]) exactly, on both kernels
    ks = np.unique(np.concatenate([[0, K - 1], np.random.default_rng(case).integers(0, K, 6)]))
    E = torch.from_numpy(wl.unit_vectors(K, ks)).to(device())
    expect = ref["W16"][:, ks].T.copy()
    set_knob("W4A16_FORCE_PATH", "gemm")
    ye = run_gemm(prod, x=E).cpu().numpy()
    assert np.array_equal(ye.view(np.uint16), expect.view(np.uint16))
    set_knob("W4A16_FORCE_PATH", "gemv")
    for i in (0, len(ks) - 1):
        yi = run_gemm(prod, x=E[i:i + 1].contiguous()).cpu().numpy()
        assert np.array_equal(yi[0].view(np.uint16), expect[i].view(np.uint16))


@pytest.mark.parametrize("M", [1, 16])
def test_w8a16_full_size_layer_on_sampled_rows(M):
    import torch
    cfg = wl.config("c3w8")
    note(f"8-bit full-size {cfg.name} M={M} (N={cfg.N} K={cfg.K})")
    prod = product_layer(cfg, 16)
    rows = np.unique(np.concatenate([sample_rows(cfg.N, 96), np.arange(cfg.N - 8, cfg.N)]))
    ref = oracle_layer(cfg, M, rows)
    assert np.array_equal(prod["codes"][rows], ref["codes"])
    x = prod["x"][:M].contiguous()
    y = torch.full((M, cfg.N), float("nan"), dtype=torch.float16, device=x.device)
    run_gemm(prod, x=x, y=y)
    assert not bool(torch.isnan(y).any())
    assert oracle.rel_err(y.cpu().numpy()[:, rows], ref["y_ref"]) <= TOL


# skinny batches (2 <= M <= 32): the 8-bit skinny kernel, every shape family
SKINNY = [
    # name, M, N, K, group, act_order, sym
    ("f1", 4, 264, 2048, 128, False, False),    # one slice, subnormal path
    ("f2", 9, 136, 1024, 32, True, False),      # dequantised path, act order
    ("f3", 16, 392, 8192, 128, False, True),    # two K slices, symmetric
    ("f4", 20, 72, 4096, 64, False, False),     # two launches (16 + 4 rows)
    ("f5", 2, 40, 1536, 1536, False, False),    # per-channel
]


@pytest.mark.parametrize("case", range(len(SKINNY)))
def test_w8a16_skinny_batches_match_oracle(case):
    name, M, N, K, g, act, sym = SKINNY[case]
    cfg = wl.custom_config(name, 650 + case, K=K, N=N, group_size=g, M_list=(M,), act_order=act, sym=sym, bits=8)
    note(f"8-bit skinny {name} M={M} N={N} K={K} g={g} act={act} sym={sym}")
    prod = product_layer(cfg, M)
    ref = oracle_layer(cfg, M, np.arange(N))
    for tiled in ("1", "0"):
        set_knob("W4A16_TUNE_GEMM_SKINNY", tiled)
        y = run_gemm(prod).cpu().numpy()
        assert oracle.rel_err(y, ref["y_ref"]) <= TOL, tiled
    clear_knob("W4A16_TUNE_GEMM_SKINNY")


# larger batches (M >= 33): the 8-bit large-tile kernel at every tile height, the tiled
# kernel beside it, and the tiled kernel alone where N % 16 != 0
LARGE = [
    # name, M, N, K, group, act_order, sym
    ("h1", 40, 272, 1024, 128, False, False),     # 64-row tiles
    ("h2", 300, 528, 640, 64, True, True),        # 256-row tiles, act order, symmetric
    ("h3", 129, 1040, 1536, 1536, False, False),  # per-channel, ragged rows and columns
    ("h4", 100, 4112, 512, 32, False, False),     # 128-row tiles, many column tiles
    ("h5", 64, 264, 1024, 128, False, False),     # N % 16 != 0: tiled kernel only
]


@pytest.mark.parametrize("case", range(len(LARGE)))
def test_w8a16_large_batches_match_oracle(case):
    import torch
    name, M, N, K, g, act, sym = LARGE[case]
    cfg = wl.custom_config(name, 670 + case, K=K, N=N, group_size=g, M_list=(M,), act_order=act, sym=sym, bits=8)
    note(f"8-bit large {name} M={M} N={N} K={K} g={g} act={act} sym={sym}")
    prod = product_layer(cfg, M)
    ref = oracle_layer(cfg, M, np.arange(N))
    ks = np.unique(np.concatenate([[0, K - 1], np.random.default_rng(case).integers(0, K, 60)]))[:40]
    E = torch.from_numpy(wl.unit_vectors(K, ks)).to(device())
    expect = ref["W16"][:, ks].T.copy()
    try:
        for big, mb in (("1", None), ("1", "2"), ("1", "4"), ("1", "8"), ("0", None)):
            set_knob("W4A16_TUNE_GEMM_BIG", big)
            if mb is None:
                clear_knob("W4A16_TUNE_GEMM_BIG_MB")
            else:
                set_knob("W4A16_TUNE_GEMM_BIG_MB", mb)
            note(f"  big={big} mb={mb}")
            y = run_gemm(prod).cpu().numpy()
            assert oracle.rel_err(y, ref["y_ref"]) <= TOL, (big, mb)
            # unit-vector probes: x = e_k gives binary16(W^[:, k]) exactly
            ye = run_gemm(prod, x=E).cpu().numpy()
            assert np.array_equal(ye.view(np.uint16), expect.view(np.uint16)), (big, mb)
    finally:
        clear_knob("W4A16_TUNE_GEMM_BIG")
        clear_knob("W4A16_TUNE_GEMM_BIG_MB")


def test_w8a16_prefill_layer_on_sampled_rows():
    """The 2048-token prefill layer with 8-bit weights, at its full size, on the launch
    the timing runs use (one round of 256-column tiles and one of 192-column tiles)."""
    import torch
    cfg = wl.config("c4w8")
    M = cfg.M_list[0]
    note(f"8-bit full-size {cfg.name} M={M} (N={cfg.N} K={cfg.K})")
    prod = product_layer(cfg, M)
    rows = np.unique(np.concatenate([sample_rows(cfg.N, 96), np.arange(cfg.N - 8, cfg.N),
                                     np.arange(8192 - 4, 8192 + 4)]))
    ref = oracle_layer(cfg, M, rows)
    assert np.array_equal(prod["codes"][rows], ref["codes"])
    y = torch.full((M, cfg.N), float("nan"), dtype=torch.float16, device=prod["x"].device)
    run_gemm(prod, y=y)
    assert not bool(torch.isnan(y).any())
    assert oracle.rel_err(y.cpu().numpy()[:, rows], ref["y_ref"]) <= TOL


def test_w8a16_full_rounds_then_a_round_of_narrow_tiles():
    """8-bit weights on the tile plan with more than two rounds of full-width tiles (on 256
    compute units: two rounds of 256 x 256 tiles over columns [0, 32768), then one round of
    256 x 64 tiles): every output written and within the bar of the oracle."""
    import torch
    cfg = wl.custom_config("h9", 690, K=256, N=36864, group_size=128, M_list=(1024,), bits=8)
    note(f"8-bit full rounds then narrow tiles M=1024 N={cfg.N} K={cfg.K}")
    prod = product_layer(cfg, 1024)
    ref = oracle_layer(cfg, 1024, np.arange(cfg.N))
    y = torch.full((1024, cfg.N), float("nan"), dtype=torch.float16, device=prod["x"].device)
    run_gemm(prod, y=y)
    out = y.cpu().numpy()
    assert not np.isnan(out).any(), "outputs left unwritten"
    assert oracle.rel_err(out, ref["y_ref"]) <= TOL
