"""GPU parity of the HIP path against the oracle (needs an MI355X).

Bars: codes, zero points and the act-order mapping bit-exact; the device weight view
bit-exact against binary16((q - Z) * S); unit-vector probes bit-exact; outputs within
max|y - y_ref| / rms(y_ref) <= 1e-2 (float64 reference of the quantised layer).
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

# Small layers that span several tiles of every kernel and end on a ragged tail.
SMALL = [
    # name, M, N, K, group, act_order
    ("s1", 1, 264, 1536, 128, False),
    ("s2", 1, 520, 3072, 64, False),
    ("s3", 1, 136, 512, 32, False),
    ("s4", 1, 1032, 8192, 128, False),
    ("s5", 1, 328, 1024, 32, True),
    ("s6", 3, 264, 1536, 128, False),
    ("s7", 17, 520, 1024, 64, False),
    ("s8", 37, 264, 768, 128, True),
    ("s9", 130, 520, 1152, 32, False),
    ("s10", 257, 776, 640, 128, False),
    ("s11", 200, 264, 2048, 32, True),
    ("s12", 1, 8, 96, 32, False),
    # skinny batches: every (steps per wavefront, slab entries per thread) shape family
    ("s13", 5, 392, 8192, 32, True),
    ("s14", 16, 1048, 4096, 64, False),
    ("s15", 2, 200, 6144, 128, False),
    ("s16", 9, 72, 2048, 32, True),
    # largest K the decode kernel takes; smallest N; K not a multiple of 64 at M > 128;
    # a single K tile and a single group at M > 128 with act order
    ("s17", 1, 16, 16384, 128, False),
    ("s18", 129, 8, 96, 32, False),
    ("s19", 300, 40, 64, 64, True),
    # batches between the skinny and the prefill shapes: the skinny kernel twice (ragged
    # second launch) at M <= 32, the large-tile kernel with 64-row tiles (M = 33, 64 with
    # act order) and 128-row tiles (M = 100)
    ("s20", 33, 264, 2048, 128, False),
    ("s23", 27, 392, 2048, 128, False),
    ("s21", 64, 136, 1024, 32, True),
    ("s22", 100, 264, 512, 128, False),
    # long rows (K > 8192): the decode GEMV splits a row over 2 / 4 / 8 wavefronts;
    # exact slices, act order, ragged slices (K = 28672: 224 of 256 lane chunks), an odd
    # chunk count (uneven slices) and the longest row (K = 65536, 512 groups)
    ("s24", 1, 264, 16384, 128, False),
    ("s25", 1, 136, 12288, 64, True),
    ("s26", 1, 72, 28672, 128, False),
    ("s27", 1, 40, 10272, 32, False),
    ("s28", 1, 16, 65536, 128, False),
    # long rows at skinny batches: K split over 2 / 4 / 8 workgroup slices, fp32 partials
    # summed in a second kernel; act order, two launches of 16 + 4 rows, group size 32
    ("s29", 4, 264, 16384, 128, False),
    ("s30", 9, 136, 12288, 64, True),
    ("s31", 20, 72, 28672, 128, False),
    ("s32", 2, 40, 65536, 32, False),
    # act order at 17..32 rows: x gathered once, the skinny kernel twice over it (16 + 7)
    ("s33", 23, 264, 4096, 128, True),
]


def _small_cfg(name, M, N, K, g, act, idx):
    return wl.custom_config(name, 100 + idx, K=K, N=N, group_size=g, M_list=(M,), act_order=act)


@pytest.fixture(autouse=True)
def _clear_env():
    for v in ("W4A16_FORCE_PATH", "W4A16_TUNE_GEMM_SKINNY"):
        clear_knob(v)
    yield
    for v in ("W4A16_FORCE_PATH", "W4A16_TUNE_GEMM_SKINNY"):
        clear_knob(v)


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_layers_match_oracle(case):
    import torch
    name, M, N, K, g, act = SMALL[case]
    cfg = _small_cfg(name, M, N, K, g, act, case)
    note(f"small {name} M={M} N={N} K={K} g={g} act={act}")
    prod = product_layer(cfg, M)
    ref = oracle_layer(cfg, M, np.arange(N))
    assert np.array_equal(prod["codes"], ref["codes"])
    if act:
        assert np.array_equal(prod["g_idx_np"], ref["g_idx"])
    paths = ["gemv", "gemm"] if M == 1 else ["gemm"]
    if M <= 64:
        paths.append("gemm-tiled")      # the tiled MFMA kernel instead of the skinny one
    for path in paths:
        set_knob("W4A16_FORCE_PATH", path.split("-")[0])
        set_knob("W4A16_TUNE_GEMM_SKINNY", "0" if path == "gemm-tiled" else "1")
        note(f"  path={path}")
        y = run_gemm(prod).cpu().numpy()
        err = oracle.rel_err(y, ref["y_ref"])
        assert err <= TOL, (path, err)
    clear_knob("W4A16_TUNE_GEMM_SKINNY")
    # the device weight view is bit-exact
    W16 = w4.w4a16_dequant(prod["qweight"], prod["scales"], prod["qzeros"], prod["g_idx"], g, K).cpu().numpy()
    assert np.array_equal(W16.view(np.uint16), ref["W16"].view(np.uint16))
    # the device-resident packed buffer unpacks to the oracle's codes
    back = w4.w4a16_unpack(prod["qweight"].cpu().numpy(), prod["g_idx_np"], g, N, K)
    assert np.array_equal(back, ref["codes"])


@pytest.mark.parametrize("case,count", [(9, 300), (8, 140), (2, 40)])
def test_unit_vector_probes_bit_exact_many_rows(case, count):
    """The same probe with enough rows for the other kernels (M > 128: 256-row tiles;
    M = 40: 64-row tiles)."""
    import torch
    name, _, N, K, g, act = SMALL[case]
    cfg = _small_cfg(name, 1, N, K, g, act, case)
    ks = np.arange(min(K, count))
    E = wl.unit_vectors(K, ks)
    prod = product_layer(cfg, 1)
    ref = oracle_layer(cfg, 1, np.arange(N))
    expect = ref["W16"][:, ks].T.copy()
    note(f"probe {name} M={len(ks)}")
    y = run_gemm(prod, x=torch.from_numpy(E).to(device())).cpu().numpy()
    assert np.array_equal(y.view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("case", [0, 2, 4, 6, 7, 9, 23, 24, 25, 26])
def test_unit_vector_probes_bit_exact(case):
    """x = e_k selects column k of W^: y = binary16(W^[:, k]) exactly (one exact
    product, exact fp32 sums of zeros, one rounding)."""
    import torch
    name, _, N, K, g, act = SMALL[case]
    cfg = _small_cfg(name, 1, N, K, g, act, case)
    ks = np.unique(np.concatenate([[0, K - 1, K // 2], np.random.default_rng(case).integers(0, K, 13)]))
    E = wl.unit_vectors(K, ks)
    prod = product_layer(cfg, 1)
    ref = oracle_layer(cfg, 1, np.arange(N))
    expect = ref["W16"][:, ks].T.copy()                       # [len(ks)][N]
    xe = torch.from_numpy(E).to(device())
    note(f"probe {name} gemm M={len(ks)}")
    set_knob("W4A16_FORCE_PATH", "gemm")
    y = run_gemm(prod, x=xe).cpu().numpy()
    assert np.array_equal(y.view(np.uint16), expect.view(np.uint16))
    set_knob("W4A16_FORCE_PATH", "gemv")
    for i in range(len(ks)):
        note(f"probe {name} gemv k={ks[i]}")
        yi = run_gemm(prod, x=xe[i:i + 1].contiguous()).cpu().numpy()
        assert np.array_equal(yi[0].view(np.uint16), expect[i].view(np.uint16)), ks[i]


# The large-tile kernel's two MFMA tiles (16x16x32 and 32x32x16 blocks) at every tile
# height: forced row blocks per wavefront and tile kind on layers with several row and
# column tiles, ragged M and N, act order and symmetric weights.
LARGE_TILE_CASES = [
    # name, M, N, K, group, act_order, sym
    ("t1", 150, 520, 1024, 128, False, False),
    ("t2", 70, 776, 640, 64, True, False),
    ("t3", 300, 264, 512, 32, False, True),
]


@pytest.mark.parametrize("mb", [2, 4, 8])
@pytest.mark.parametrize("mfma32", [0, 1, 2])
def test_large_tile_kinds_match_oracle(mb, mfma32):
    import torch
    set_knob("W4A16_FORCE_PATH", "gemm")
    set_knob("W4A16_TUNE_GEMM_BIG_MB", str(mb))
    set_knob("W4A16_TUNE_GEMM_MFMA32", str(mfma32))
    try:
        for i, (name, M, N, K, g, act, sym) in enumerate(LARGE_TILE_CASES):
            cfg = wl.custom_config(name, 300 + i, K=K, N=N, group_size=g, M_list=(M,), act_order=act, sym=sym)
            note(f"large tile {name} M={M} N={N} K={K} g={g} act={act} sym={sym} mb={mb} mfma32={mfma32}")
            prod = product_layer(cfg, M)
            ref = oracle_layer(cfg, M, np.arange(N))
            y = run_gemm(prod).cpu().numpy()
            assert oracle.rel_err(y, ref["y_ref"]) <= TOL
            # wavefront priority changes only the schedule: bit-identical outputs without it
            set_knob("W4A16_TUNE_GEMM_PRIO", "0")
            y0 = run_gemm(prod).cpu().numpy()
            clear_knob("W4A16_TUNE_GEMM_PRIO")
            assert np.array_equal(y0.view(np.uint16), y.view(np.uint16))
            # x = e_k for 130 channels: every output exactly binary16(W^[n, k])
            ks = np.arange(0, K, max(1, K // 130))[:130]
            y = run_gemm(prod, x=torch.from_numpy(wl.unit_vectors(K, ks)).to(device())).cpu().numpy()
            assert np.array_equal(y.view(np.uint16), ref["W16"][:, ks].T.copy().view(np.uint16))
    finally:
        for v in ("W4A16_TUNE_GEMM_BIG_MB", "W4A16_TUNE_GEMM_MFMA32", "W4A16_TUNE_GEMM_PRIO"):
            clear_knob(v)


def test_large_tile_full_rounds_then_a_round_of_narrow_tiles():
    """More than two rounds of full-width tiles: on 256 compute units, 4 row panels x 144
    column tiles of 256 x 256 = 576 tiles run as two rounds of full tiles (columns
    [0, 32768)) and one round of 256 x 64 tiles (the last 4096 columns), every output
    written (NaN-filled y) and within the bar of the oracle."""
    import torch
    cfg = wl.custom_config("r1", 380, K=256, N=36864, group_size=128, M_list=(1024,))
    note(f"full rounds then narrow tiles M=1024 N={cfg.N} K={cfg.K}")
    prod = product_layer(cfg, 1024)
    ref = oracle_layer(cfg, 1024, np.arange(cfg.N))
    y = torch.full((1024, cfg.N), float("nan"), dtype=torch.float16, device=device())
    run_gemm(prod, y=y)
    out = y.cpu().numpy()
    assert not np.isnan(out).any(), "outputs left unwritten"
    assert oracle.rel_err(out, ref["y_ref"]) <= TOL


def test_kernel_switches_need_the_opt_in():
    """W4A16_FORCE_PATH (like every W4A16_TUNE_* switch) is ignored unless W4A16_TUNE=1:
    without the opt-in a batch of one runs the decode GEMV (bit-identical to the default),
    with it the MFMA GEMM (a different summation order: some outputs differ in their last
    bits, all within the bar)."""
    import os
    cfg = wl.custom_config("k1", 390, K=4096, N=1032, group_size=128, M_list=(1,))
    prod = product_layer(cfg, 1)
    ref = oracle_layer(cfg, 1, np.arange(cfg.N))
    try:
        clear_knob("W4A16_FORCE_PATH")
        y_default = run_gemm(prod).cpu().numpy()
        os.environ.pop("W4A16_TUNE", None)
        os.environ["W4A16_FORCE_PATH"] = "gemm"
        w4.w4a16_reload_env()
        y_ignored = run_gemm(prod).cpu().numpy()
        set_knob("W4A16_FORCE_PATH", "gemm")   # sets the opt-in as well
        y_forced = run_gemm(prod).cpu().numpy()
    finally:
        clear_knob("W4A16_FORCE_PATH")
    assert np.array_equal(y_ignored.view(np.uint16), y_default.view(np.uint16))
    assert not np.array_equal(y_forced.view(np.uint16), y_default.view(np.uint16))
    for y in (y_default, y_forced):
        assert oracle.rel_err(y, ref["y_ref"]) <= TOL


def test_dequantise_once_tile_matches_the_large_tile():
    # 256-row tiles whose codes are dequantised once per workgroup into a binary16 weight
    # tile in LDS (W4A16_TUNE_GEMM_LDSB=1): the same operands in the same MFMA order as the
    # large tile, so the same bits; with a 192-wide second round of tiles and ragged edges
    import torch
    # t6: more than one round of full tiles, so the launch also runs 256-column tiles
    cases = LARGE_TILE_CASES + [("t4", 520, 1400, 1024, 128, False, False), ("t5", 300, 776, 448, 32, True, False),
                                ("t6", 2048, 8448, 128, 128, False, False)]
    set_knob("W4A16_FORCE_PATH", "gemm")
    set_knob("W4A16_TUNE_GEMM_BIG_MB", "8")
    try:
        for i, (name, M, N, K, g, act, sym) in enumerate(cases):
            cfg = wl.custom_config(name, 340 + i, K=K, N=N, group_size=g, M_list=(M,), act_order=act, sym=sym)
            note(f"dequantise-once tile {name} M={M} N={N} K={K} g={g} act={act} sym={sym}")
            prod = product_layer(cfg, M)
            ref = oracle_layer(cfg, M, np.arange(N))
            set_knob("W4A16_TUNE_GEMM_LDSB", "0")
            y0 = run_gemm(prod).cpu().numpy()
            set_knob("W4A16_TUNE_GEMM_LDSB", "1")
            y1 = run_gemm(prod).cpu().numpy()
            assert oracle.rel_err(y1, ref["y_ref"]) <= TOL
            assert np.array_equal(y1.view(np.uint16), y0.view(np.uint16))
            ks = np.arange(0, K, max(1, K // 130))[:130]
            yk = run_gemm(prod, x=torch.from_numpy(wl.unit_vectors(K, ks)).to(device())).cpu().numpy()
            assert np.array_equal(yk.view(np.uint16), ref["W16"][:, ks].T.copy().view(np.uint16))
    finally:
        clear_knob("W4A16_TUNE_GEMM_BIG_MB", "W4A16_TUNE_GEMM_LDSB")


def test_all_ones_gives_row_sums():
    import torch
    cfg = _small_cfg("ones", 1, 520, 3072, 64, False, 50)
    prod = product_layer(cfg, 1)
    ref = oracle_layer(cfg, 1, np.arange(520), x=np.ones((1, 3072), np.float16))
    ones = torch.ones((4, 3072), dtype=torch.float16, device=device())
    for path, x in (("gemv", ones[:1]), ("gemm", ones)):
        set_knob("W4A16_FORCE_PATH", path)
        note(f"all-ones {path}")
        y = run_gemm(prod, x=x.contiguous()).cpu().numpy()
        for row in y:
            assert oracle.rel_err(row[None, :], ref["y_ref"]) <= TOL


def test_identity_gidx_equals_contiguous_and_runs_are_deterministic():
    import torch
    cfg = _small_cfg("ident", 64, 264, 1024, 32, False, 51)
    prod = product_layer(cfg, 64)
    ident = torch.from_numpy((np.arange(1024) // 32).astype(np.int32)).to(device())
    codes = prod["codes"]
    qw_id = torch.from_numpy(w4.w4a16_pack(codes, ident.cpu().numpy(), 32)).to(device())
    for M in (1, 64):
        x = prod["x"][:M].contiguous()
        note(f"identity g_idx M={M}")
        a = w4.w4a16_gemm(x, prod["qweight"], prod["scales"], prod["qzeros"], None, 32)
        b = w4.w4a16_gemm(x, qw_id, prod["scales"], prod["qzeros"], ident, 32)
        c = w4.w4a16_gemm(x, prod["qweight"], prod["scales"], prod["qzeros"], None, 32)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_device_errors_are_reported():
    import torch
    cfg = _small_cfg("err", 2, 264, 1024, 64, False, 52)
    prod = product_layer(cfg, 2)
    set_knob("W4A16_FORCE_PATH", "gemv")
    with pytest.raises(w4.W4A16Error) as e:
        run_gemm(prod)
    assert e.value.status == w4.ERR_UNSUPPORTED
    clear_knob("W4A16_FORCE_PATH")
    raw = torch.empty(1024 * 2 + 8, dtype=torch.float16, device=device())
    x_mis = raw[1:1 + 2 * 1024].view(2, 1024)
    lib = w4.lib()
    st = lib.w4a16_gemm(x_mis.data_ptr(), prod["qweight"].data_ptr(), prod["scales"].data_ptr(),
                        prod["qzeros"].data_ptr(), None, 64, 2, 264, 1024,
                        torch.empty(2, 264, dtype=torch.float16, device=device()).data_ptr(), None)
    assert st == w4.ERR_MISALIGNED


# --- symmetric weights (qzeros = NULL, every zero point 8) -----------------------------

SYM = [
    # name, M, N, K, group, act_order: every kernel family and its variants
    ("y1", 1, 264, 1536, 128, False),     # GEMV, one row per wavefront group
    ("y2", 1, 136, 16384, 64, True),      # GEMV, rows split over two wavefronts, act order
    ("y3", 4, 392, 2048, 128, False),     # skinny, subnormal path (group 128)
    ("y4", 9, 136, 1024, 32, True),       # skinny, dequantised path, act order
    ("y5", 5, 264, 12288, 128, False),    # skinny, K split over two workgroup slices
    ("y6", 40, 264, 1024, 64, False),     # large-tile kernel, 64-row tiles
    ("y7", 300, 520, 640, 128, True),     # large-tile kernel, 256-row tiles, act order
    ("y8", 3, 72, 96, 32, False),         # tiled fallback kernel (K not a multiple of 128)
]


# per-channel scales (group size = K: one scale and zero point per output row), with
# and without zero points
PERCH = [
    # name, M, N, K, act_order, sym
    ("p1", 1, 264, 1536, False, False),   # GEMV
    ("p2", 1, 136, 12288, False, True),   # GEMV, split rows, symmetric
    ("p3", 4, 392, 2048, False, False),   # skinny (dequantised path)
    ("p4", 5, 264, 12288, True, False),   # skinny, two K slices, act order (one group)
    ("p5", 40, 264, 1024, False, True),   # large-tile kernel, 64-row tiles, symmetric
    ("p6", 300, 520, 640, False, False),  # large-tile kernel, 256-row tiles
    ("p7", 3, 72, 96, False, False),      # tiled fallback kernel
]

VARIANT_CASES = ([(name, M, N, K, g, act, True) for name, M, N, K, g, act in SYM] +
                 [(name, M, N, K, K, act, sym) for name, M, N, K, act, sym in PERCH])


@pytest.mark.parametrize("case", range(len(VARIANT_CASES)))
def test_symmetric_and_per_channel_layers_match_oracle(case):
    import torch
    name, M, N, K, g, act, sym = VARIANT_CASES[case]
    cfg = wl.custom_config(name, 400 + case, K=K, N=N, group_size=g, M_list=(M,), act_order=act, sym=sym)
    note(f"variant {name} M={M} N={N} K={K} g={g} act={act} sym={sym}")
    prod = product_layer(cfg, M)
    assert (prod["qzeros"] is None) == sym
    ref = oracle_layer(cfg, M, np.arange(N))
    assert np.array_equal(prod["codes"], ref["codes"])
    paths = ["gemv", "gemm"] if M == 1 else ["gemm"]
    for path in paths:
        set_knob("W4A16_FORCE_PATH", path)
        note(f"  path={path}")
        y = run_gemm(prod).cpu().numpy()
        assert oracle.rel_err(y, ref["y_ref"]) <= TOL, path
    clear_knob("W4A16_FORCE_PATH")
    W16 = w4.w4a16_dequant(prod["qweight"], prod["scales"], prod["qzeros"], prod["g_idx"], g, K).cpu().numpy()
    assert np.array_equal(W16.view(np.uint16), ref["W16"].view(np.uint16))
    # unit-vector probes select binary16((code - 8) * S) exactly
    ks = np.unique(np.concatenate([[0, K - 1], np.random.default_rng(case).integers(0, K, 6)]))
    E = torch.from_numpy(wl.unit_vectors(K, ks)).to(device())
    set_knob("W4A16_FORCE_PATH", "gemm")
    ye = run_gemm(prod, x=E).cpu().numpy()
    clear_knob("W4A16_FORCE_PATH")
    assert np.array_equal(ye.view(np.uint16), ref["W16"][:, ks].T.copy().view(np.uint16))


# --- the configurations at full size (sampled outputs) -------------------------------

FULL = [("c1", 1), ("c2up", 1), ("c2down", 1), ("c3", 1), ("c3", 2), ("c3", 4), ("c3", 8), ("c3", 16),
        ("c3s", 1), ("c3s", 16), ("c4", 2048), ("c5", 1), ("c5", 512)]


@pytest.fixture(scope="module")
def full_layers():
    cache = {}

    def get(name):
        if name not in cache:
            cfg = wl.config(name)
            note(f"building {name} (N={cfg.N} K={cfg.K})")
            cache.clear()
            cache[name] = product_layer(cfg, max(cfg.M_list))
        return cache[name]
    return get


@pytest.mark.parametrize("name,M", FULL)
def test_configs_match_oracle_on_sampled_outputs(full_layers, name, M):
    import torch
    cfg = wl.config(name)
    prod = full_layers(name)
    rows = np.arange(cfg.N) if cfg.N <= 1024 else sample_rows(cfg.N, 96)
    ref = oracle_layer(cfg, M, rows)
    # codes of the sampled rows and the act-order mapping are bit-exact
    assert np.array_equal(prod["codes"][rows], ref["codes"])
    if cfg.act_order:
        assert np.array_equal(prod["g_idx_np"], ref["g_idx"])
    x = prod["x"][:M].contiguous()
    note(f"config {name} M={M}")
    # every output is written: start from NaN everywhere
    y_full = torch.full((M, cfg.N), float("nan"), dtype=torch.float16, device=x.device)
    run_gemm(prod, x=x, y=y_full)
    assert not bool(torch.isnan(y_full).any()), "outputs left unwritten"
    y = y_full.cpu().numpy()[:, rows]
    err = oracle.rel_err(y, ref["y_ref"])
    assert err <= TOL, err
    # and a second run is bit-identical (each output written once, fixed order)
    y2 = run_gemm(prod, x=x).cpu().numpy()[:, rows]
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


# M = 1 row shapes: with rows to spare the GEMV takes up to 4 chunks per lane (16 or 32
# lanes per row for K = 1024 .. 4096); every lanes-per-row value forced on one layer
GEMV_SHAPES = [
    # name, N, K, group, act_order, bits
    ("v1", 14344, 1024, 32, False, 4),    # 16 lanes per row, ragged last unit
    ("v2", 8200, 2048, 64, True, 4),      # 32 lanes, 2 chunks each, act order
    ("v3", 11008, 4096, 32, True, 4),     # 32 lanes, 4 chunks each (the act-order layer's shape)
    ("v4", 12296, 2048, 128, False, 8),   # 8-bit: 32 lanes, 4 chunks each
    ("v5", 10248, 8192, 32, False, 4),    # 64 lanes, 6 steps: all scales staged in two rounds
    ("v6", 4200, 16384, 128, False, 4),   # rows split over two wavefronts, 3 steps: staged once
    ("v7", 4104, 12288, 64, True, 4),     # split rows, act order, 3 steps: staged once
]


@pytest.mark.parametrize("case", range(len(GEMV_SHAPES)))
def test_gemv_row_shapes_match_oracle(case):
    name, N, K, g, act, bits = GEMV_SHAPES[case]
    cfg = wl.custom_config(name, 760 + case, K=K, N=N, group_size=g, M_list=(1,), act_order=act, bits=bits)
    note(f"GEMV shapes {name} N={N} K={K} g={g} act={act} bits={bits}")
    prod = product_layer(cfg, 1)
    ref = oracle_layer(cfg, 1, np.arange(N))
    C = K // (32 if bits == 4 else 16)
    try:
        for lpr in [None] + [l for l in (64, 32, 16, 8) if (C + l - 1) // l <= 4]:
            if lpr is None:
                clear_knob("W4A16_TUNE_GEMV_LPR")
            else:
                set_knob("W4A16_TUNE_GEMV_LPR", str(lpr))
            # scales staged once per launch (default where it fits) and per step: the
            # same pairs and the same order of every row's sums, so identical bits
            outs = []
            for pre in ("1", "0"):
                set_knob("W4A16_TUNE_GEMV_PRE", pre)
                note(f"  lanes per row {lpr or 'auto'}, staged once {pre}")
                y = run_gemm(prod).cpu().numpy()
                assert oracle.rel_err(y, ref["y_ref"]) <= TOL, (lpr, pre)
                outs.append(y)
            assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16)), lpr
    finally:
        clear_knob("W4A16_TUNE_GEMV_LPR", "W4A16_TUNE_GEMV_PRE")


def test_gemv_compact_table_matches_the_ring():
    """Group 32 on a layer whose staged-once table of float pairs would not fit in LDS
    (K = 8192, 16392 rows: 9 steps per workgroup): the compact table of binary16 scales and
    zero points gives the same pairs, so the same bits as the per-step ring, and sampled
    rows (the last ones included) within the bar of the oracle."""
    cfg = wl.custom_config("ct1", 790, K=8192, N=16392, group_size=32, M_list=(1,))
    note(f"compact table N={cfg.N} K={cfg.K} g=32")
    prod = product_layer(cfg, 1)
    rows = np.unique(np.concatenate([sample_rows(cfg.N, 48), np.arange(cfg.N - 16, cfg.N)]))
    ref = oracle_layer(cfg, 1, rows)
    try:
        outs = []
        for pre in ("1", "2"):   # compact table, then the ring (2: no compact table)
            set_knob("W4A16_TUNE_GEMV_PRE", pre)
            outs.append(run_gemm(prod).cpu().numpy())
    finally:
        clear_knob("W4A16_TUNE_GEMV_PRE")
    assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16))
    assert oracle.rel_err(outs[0][:, rows], ref["y_ref"]) <= TOL


def _runtime_libraries():
    """The HIP runtime libraries mapped into this process (torch's and the library's)."""
    import ctypes
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            p = line.split()[-1]
            if "libamdhip64.so" in p:
                paths.add(p)
    return [ctypes.CDLL(p) for p in sorted(paths)]


def test_an_earlier_failed_runtime_call_is_not_reported_as_a_launch_error():
    # hipGetLastError keeps the last failure of any runtime call on the thread until it
    # is read; a failed call made outside the library before a layer call (here
    # hipSetDevice on a device that does not exist: refused on the host) must not turn
    # into a launch error of the layer call
    cfg = _small_cfg(*SMALL[0], 0)
    prod = product_layer(cfg, 1)
    ref = oracle_layer(cfg, 1, np.arange(cfg.N))
    w4.lib()
    libs = _runtime_libraries()
    assert libs, "no HIP runtime mapped"
    for path in ("gemv", "gemm"):
        set_knob("W4A16_FORCE_PATH", path)
        for rt in libs:
            assert rt.hipSetDevice(9999) != 0
        y = run_gemm(prod).cpu().numpy()
        assert oracle.rel_err(y, ref["y_ref"]) <= TOL, path
