"""w4a16_gemm_noalloc (scratch from the library's fixed per-GPU array, no allocation)
against w4a16_gemm (its growing workspace) through the C ABI: bit-identical outputs on
two calls in a row, the second with a smaller input, for the paths that use scratch
memory (act order above one row, on the large-tile GEMM and on the skinny kernel; skinny
batches with K split over workgroups; both at once, the gathered activations and the
partial tiles in one request), a path without scratch, and the refusal of a call whose
scratch exceeds the array."""

import pytest

import w4a16_gemm_amd as w4
import workloads as wl
from gpu_common import device, note, product_layer

pytestmark = pytest.mark.gpu

CASES = [
    # name, config, (M of the first call, M of the second)
    ("act-order c5", wl.CONFIGS["c5"], (512, 96)),
    ("act-order skinny c5", wl.CONFIGS["c5"], (16, 3)),
    ("act-order skinny split-K", wl.custom_config("na-act-splitk", 73, K=16384, N=2048, group_size=128,
                                                   M_list=(16,), act_order=True), (16, 5)),
    ("skinny split-K", wl.custom_config("na-splitk", 71, K=16384, N=4096, group_size=128, M_list=(16,)), (16, 3)),
    ("decode GEMV (no scratch)", wl.CONFIGS["c3"], (1, 1)),
]


def _raw(fn, layer, x, y):
    import torch
    g = layer["cfg"].group_size
    M, K = x.shape
    N = y.shape[1]
    st = fn(x.data_ptr(), layer["qweight"].data_ptr(), layer["scales"].data_ptr(),
            None if layer["qzeros"] is None else layer["qzeros"].data_ptr(),
            None if layer["g_idx"] is None else layer["g_idx"].data_ptr(), g, M, N, K, y.data_ptr(),
            torch.cuda.current_stream().cuda_stream)
    return st


@pytest.mark.parametrize("name,cfg,ms", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_gemm(name, cfg, ms):
    import torch
    dev = device()
    lib = w4.lib()
    note(f"no-alloc entry point: {name} N={cfg.N} K={cfg.K} M={ms}")
    layer = product_layer(cfg, max(ms))
    for M in ms:
        x = layer["x"][:M].contiguous()
        # a different input for the second call, so stale scratch would show
        if M != ms[0]:
            x = (x.float() * -0.5).to(torch.float16)
        y_ref = torch.full((M, cfg.N), float("nan"), dtype=torch.float16, device=dev)
        y_na = torch.full((M, cfg.N), float("nan"), dtype=torch.float16, device=dev)
        assert _raw(lib.w4a16_gemm, layer, x, y_ref) == w4.OK
        st = _raw(lib.w4a16_gemm_noalloc, layer, x, y_na)
        assert st == w4.OK, lib.w4a16_last_error().decode()
        torch.cuda.synchronize()
        assert not bool(torch.isnan(y_na).any())
        assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16)), f"M={M}"


def test_noalloc_refuses_scratch_beyond_its_array():
    import torch
    dev = device()
    lib = w4.lib()
    cfg = wl.custom_config("na-big", 72, K=4096, N=256, group_size=128, M_list=(4096,), act_order=True)
    note("no-alloc entry point: act order at M=4096 needs 32 MiB of scratch (expects a refusal, no launch)")
    layer = product_layer(cfg, 4096)
    y = torch.zeros((4096, cfg.N), dtype=torch.float16, device=dev)
    st = _raw(lib.w4a16_gemm_noalloc, layer, layer["x"], y)
    assert st == w4.ERR_UNSUPPORTED
    assert "scratch" in lib.w4a16_last_error().decode()
    torch.cuda.synchronize()
    assert not bool(y.any())          # nothing was launched


def test_noalloc_binding_needs_y():
    layer_cfg = wl.CONFIGS["c1"]
    layer = product_layer(layer_cfg, 1)
    with pytest.raises(ValueError):
        w4.w4a16_gemm_noalloc(layer["x"], layer["qweight"], layer["scales"], layer["qzeros"], None, 128, None)
