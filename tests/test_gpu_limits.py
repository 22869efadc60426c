"""GPU parity at the largest layers: 2 GB of packed codes (needs an MI355X).

The decode GEMV and the skinny-batch kernel address the codes with 32-bit byte
offsets and take layers with N K / 2 < 2^31 bytes of codes; larger layers go to the
tiled MFMA kernels.  Both sides of that limit are checked against the oracle on
sampled output rows, including the last rows (the highest offsets).  The layers are
uniform random packed words (uniform 4-bit codes and zero points) with random
scales: quantising 4.3 G weights on the host would take far too long, and the
arithmetic under test does not depend on where the codes came from.
"""

import os

import numpy as np
import pytest

import oracle
import w4a16_gemm_amd as w4
import workloads as wl
from gpu_common import clear_knob, codes_of_library_words, device, note, sample_rows, set_knob

pytestmark = pytest.mark.gpu

TOL = 1e-2
K = 16384          # the largest K the decode GEMV takes
G128 = 128
N_BELOW = (1 << 31) // (K // 2) - 8     # 262136 rows: 2 GB - 64 KB of codes
N_ABOVE = (1 << 31) // (K // 2) + 8     # 262152 rows: 2 GB + 64 KB


@pytest.fixture(scope="module")
def big_layer():
    cache = {}

    def get(N):
        import torch
        if N not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            note(f"building random packed layer N={N} K={K} ({N * K // 2} bytes of codes)")
            qw = wl.random_words(N, K // 8, seed=N)
            S = wl.random_scales(K // G128, N, seed=N)
            qz = wl.random_words(K // G128, N // 8, seed=N + 1)
            dev = device()
            cache[N] = {"qw_np": qw, "S": S, "qz_np": qz,
                        "qweight": torch.from_numpy(qw).to(dev), "scales": torch.from_numpy(S).to(dev),
                        "qzeros": torch.from_numpy(qz).to(dev)}
        return cache[N]
    return get


def _rows(N):
    return np.unique(np.concatenate([sample_rows(N, 24), np.arange(N - 16, N)]))


@pytest.mark.parametrize("N,M,path", [(N_BELOW, 1, "gemv"), (N_BELOW, 2, "skinny"),
                                      (N_ABOVE, 1, "tiled"), (N_ABOVE, 2, "tiled"), (N_ABOVE, 33, "large")])
def test_two_gigabyte_layers_match_oracle(big_layer, N, M, path):
    import torch
    L = big_layer(N)
    rows = _rows(N)
    x_np = wl.random_activations(M, K, seed=M)
    codes = codes_of_library_words(L["qw_np"][rows])
    Z = oracle.unpack_zeros(L["qz_np"])[:, rows]
    y_ref = oracle.linear(x_np, codes, L["S"][:, rows], Z, G128)
    x = torch.from_numpy(x_np).to(device())
    note(f"2 GB layer N={N} M={M} ({path})")
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device=x.device)
    w4.w4a16_gemm(x, L["qweight"], L["scales"], L["qzeros"], None, G128, y=y)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(y).any()), "outputs left unwritten"
    err = oracle.rel_err(y.cpu().numpy()[:, rows], y_ref)
    assert err <= TOL, err


def test_gemv_refuses_layers_of_two_gigabytes(big_layer):
    import torch
    L = big_layer(N_ABOVE)
    x = torch.from_numpy(wl.random_activations(1, K, seed=1)).to(device())
    set_knob("W4A16_FORCE_PATH", "gemv")
    try:
        note("forced GEMV on a 2 GB + 64 KB layer (expects an error, no launch)")
        with pytest.raises(w4.W4A16Error) as e:
            w4.w4a16_gemm(x, L["qweight"], L["scales"], L["qzeros"], None, G128)
        assert e.value.status == w4.ERR_UNSUPPORTED
    finally:
        clear_knob("W4A16_FORCE_PATH")
