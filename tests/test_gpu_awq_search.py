"""The AWQ alpha search on the device against the oracle (needs an MI355X).

"AWQ + GPTQ Quantization, in depth", The two algorithms, compactly.  The device
loss is || y^_ref - y^ ||_F with both outputs rounded once to binary16 (fp32
accumulation); the oracle's is || y_ref - y ||_F in float64 on the same quantised
layer.  By the triangle inequality the two differ by at most || y^_ref - y_ref || +
|| y^ - y ||, each at most 2^-11 || y || from the output rounding plus the fp32
accumulation error; the bound used is 1.25 * 2^-10 * || y_ref ||.  The best alpha
must agree unless the oracle's losses of the two candidates are within twice that.
"""

import numpy as np
import pytest

import oracle
import w4a16_gemm_amd as w4
import workloads as wl
from gpu_common import note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,T,g", [(264, 1024, 128, 128), (136, 2048, 200, 64)])
def test_awq_search_matches_oracle(N, K, T, g):
    cfg = wl.custom_config("awqs", 800 + K, K=K, N=N, group_size=g, outlier_frac=0.01, outlier_mult=20.0)
    w = wl.weights(cfg)
    X = wl.calibration(cfg, T)
    alphas = np.linspace(0.0, 1.0, 11)
    note(f"AWQ search N={N} K={K} T={T} g={g}")
    lp, bp = w4.w4a16_awq_search(w, X, g, alphas)
    lo, bo = oracle.awq_search(w, X, g, alphas)
    y_norm = np.linalg.norm(X.astype(np.float64) @ w.astype(np.float64).T)
    tol = 1.25 * 2.0 ** -10 * y_norm
    assert np.all(np.abs(lp - lo) <= tol), np.max(np.abs(lp - lo)) / tol
    assert bp == bo or lo[bp] <= lo[bo] + 2 * tol
    assert bo > 0          # the outlier channels make some alpha > 0 beat plain rounding


def test_awq_search_rejects_bad_arguments():
    w = np.zeros((8, 64), np.float16)
    X = np.zeros((4, 64), np.float16)
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_awq_search(w, X, 32, [0.5, -1.0])
    assert e.value.status == w4.ERR_INVALID_ARG
    with pytest.raises(w4.W4A16Error) as e:
        w4.w4a16_awq_search(w, X, 48, [0.5])
    assert e.value.status == w4.ERR_UNSUPPORTED


@pytest.mark.parametrize("N,K,g,sym,scaled", [(264, 1024, 128, False, False), (136, 2048, 64, True, True),
                                              (72, 1536, 32, False, True), (40, 1536, 1536, True, False)])
def test_device_quantiser_is_bit_exact_with_the_host(N, K, g, sym, scaled):
    import torch
    cfg = wl.custom_config("qdev", 900 + K + g, K=K, N=N, group_size=g)
    w = wl.weights(cfg)
    w[3, :g] = 0                                          # an all-zero group
    s = oracle.awq_scales(wl.calibration(cfg, 64), 0.4) if scaled else None
    note(f"device quantiser N={N} K={K} g={g} sym={sym} scaled={scaled}")
    dev = torch.device("cuda:0")
    qw, S, qz = w4.w4a16_quantize_device(torch.from_numpy(w).to(dev), g,
                                         None if s is None else torch.from_numpy(s).to(dev), sym)
    torch.cuda.synchronize()
    if sym:
        codes, Sh = w4.w4a16_quantize_sym(w, g, None, s)
        assert qz is None
    else:
        codes, Sh, Zh = w4.w4a16_quantize(w, g, None, s)
        assert np.array_equal(qz.cpu().numpy(), w4.w4a16_pack_zeros(Zh))
    assert np.array_equal(qw.cpu().numpy(), w4.w4a16_pack(codes, None, g))
    assert np.array_equal(S.cpu().numpy().view(np.uint16), Sh.view(np.uint16))
