"""Pins of the oracle's GPTQ quantiser ("AWQ + GPTQ Quantization, in depth", The two
algorithms, compactly), against what the mathematics fixes, not against itself:

* the Hessian against exact rational arithmetic on a tiny input;
* a diagonal H (orthogonal calibration channels) gives no error feedback, so GPTQ
  reduces to the round-to-nearest quantiser exactly (codes, scales, zeros), in
  natural and in act order;
* least squares: the value every column has when it is rounded equals the optimal
  compensation of the columns already rounded, W_R + (W_F - Q_F) H_FR H_RR^-1 with
  np.linalg.solve, which checks the inverse, the Cholesky orientation, the sign and
  index of the update and the order of the visit;
* two columns by hand: w1' = w1 + (w0 - q0) H01 / H11;
* the error feedback lowers the layer's output error on the calibration rows below
  round-to-nearest on a synthetic layer of the workloads' distribution.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl
from oracle.gptq import group_params, gptq_hessian, gptq_quantize, output_error


def _layer(seed, N, K, T, w_std=0.02):
    rng = np.random.default_rng([900, seed])
    w = (rng.standard_normal((N, K)) * w_std).astype(np.float16)
    x = rng.standard_normal((T, K))
    x[:, rng.choice(K, max(1, K // 64), replace=False)] *= 8.0     # a few large channels
    return w, x.astype(np.float16)


def test_hessian_matches_exact_rationals():
    w, x = _layer(1, 8, 6, 5)
    damp = 0.01
    H = gptq_hessian(x, damp)
    X = [[Fraction(float(v)) for v in row] for row in x]
    K = x.shape[1]
    exact = [[2 * sum(X[t][i] * X[t][j] for t in range(len(X))) for j in range(K)] for i in range(K)]
    mean_diag = sum(exact[i][i] for i in range(K)) / K
    for i in range(K):
        exact[i][i] += Fraction(damp) * mean_diag
    for i in range(K):
        for j in range(K):
            assert H[i, j] == pytest.approx(float(exact[i][j]), rel=1e-14, abs=1e-300)
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("use_act_order", [False, True])
@pytest.mark.parametrize("g", [8, 32])
def test_diagonal_hessian_reduces_to_rtn(use_act_order, g):
    """Calibration rows that each excite one channel: H is diagonal, U is diagonal,
    U[j, j+1:] = 0, nothing is fed forward and GPTQ is round-to-nearest."""
    N, K = 24, 64
    w, _ = _layer(2, N, K, 1)
    rng = np.random.default_rng(3)
    x = np.zeros((K, K), dtype=np.float16)
    x[np.arange(K), np.arange(K)] = rng.uniform(0.5, 4.0, K).astype(np.float16)
    codes, S, Z, g_idx = gptq_quantize(w, x, g, use_act_order)
    if use_act_order:
        assert np.array_equal(g_idx, oracle.act_order(x, g)[0])
    rc, rs, rz = oracle.rtn_quantize(w, g, g_idx)
    assert np.array_equal(codes, rc)
    assert np.array_equal(S.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(Z, rz)


@pytest.mark.parametrize("use_act_order", [False, True])
@pytest.mark.parametrize("damp", [0.01, 0.1])
def test_every_column_is_the_least_squares_compensation(use_act_order, damp):
    N, K, T, g = 6, 24, 48, 8
    w, x = _layer(4, N, K, T)
    codes, S, Z, g_idx, pre, order = gptq_quantize(w, x, g, use_act_order, damp, return_trace=True)
    # the Hessian in the visiting order, built here from its definition
    Xd = x.astype(np.float64)
    H = 2.0 * Xd.T @ Xd
    H += damp * np.trace(H) / K * np.eye(K)
    H = H[np.ix_(order, order)]
    W = w.astype(np.float64)[:, order]
    Q = oracle.dequant(codes, S, Z, g, g_idx)[:, order]
    for i in range(K):
        F, R = np.arange(i), np.arange(i, K)
        if i == 0:
            expect = W[:, 0]
        else:
            comp = np.linalg.solve(H[np.ix_(R, R)], H[np.ix_(F, R)].T @ (W[:, F] - Q[:, F]).T).T
            expect = W[:, i] + comp[:, 0]
        np.testing.assert_allclose(pre[:, i], expect, rtol=1e-9, atol=1e-12)
    # each group's grid comes from its columns as they stand when its first column is
    # reached: the least-squares compensation of the earlier groups
    for i0 in range(0, K, g):
        F, R = np.arange(i0), np.arange(i0, K)
        vals = W[:, R]
        if i0 > 0:
            vals = vals + np.linalg.solve(H[np.ix_(R, R)], H[np.ix_(F, R)].T @ (W[:, F] - Q[:, F]).T).T
        S16, _, z = group_params(vals[:, :g])
        assert np.array_equal(S[i0 // g].view(np.uint16), S16.view(np.uint16))
        assert np.array_equal(Z[i0 // g], z.astype(np.uint8))
    # and every rounded value is on its group's grid at the nearest point
    for i in range(K):
        gam = i // g
        s = S[gam].astype(np.float64)
        q = np.clip(np.rint(pre[:, i] / s) + Z[gam], 0, 15)
        assert np.array_equal(q, codes[:, order[i]])


def test_two_columns_by_hand():
    """K = 2, one group: q0 from the group's grid, then w1' = w1 + (w0 - q0^) H01 / H11."""
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((16, 2)) * 0.1).astype(np.float16)
    x = rng.standard_normal((7, 2)).astype(np.float16)
    codes, S, Z, _ = gptq_quantize(w, x, 2, damp=0.05)
    H = gptq_hessian(x, 0.05)
    W = w.astype(np.float64)
    S16, s, z = group_params(W)
    assert np.array_equal(S[0].view(np.uint16), S16.view(np.uint16))
    q0 = np.clip(np.rint(W[:, 0] / s) + z, 0, 15)
    w1 = W[:, 1] + (W[:, 0] - (q0 - z) * s) * H[0, 1] / H[1, 1]
    q1 = np.clip(np.rint(w1 / s) + z, 0, 15)
    assert np.array_equal(codes[:, 0], q0)
    assert np.array_equal(codes[:, 1], q1)


@pytest.mark.parametrize("use_act_order", [False, True])
def test_output_error_below_rtn_on_synthetic_layer(use_act_order):
    cfg = wl.custom_config("gq", 910, K=256, N=64, group_size=32, M_list=(1,))
    w = wl.weights(cfg)
    x = wl.calibration(cfg)
    codes, S, Z, g_idx = gptq_quantize(w, x, 32, use_act_order)
    e_gptq = output_error(w, codes, S, Z, 32, g_idx, x)
    rc, rs, rz = oracle.rtn_quantize(w, 32, g_idx)
    e_rtn = output_error(w, rc, rs, rz, 32, g_idx, x)
    assert e_gptq < 0.9 * e_rtn, (e_gptq, e_rtn)


def test_act_order_is_the_natural_order_of_the_permuted_layer():
    w, x = _layer(6, 8, 32, 40)
    codes, S, Z, g_idx = gptq_quantize(w, x, 8, True)
    _, perm = oracle.act_order(x, 8)
    c2, S2, Z2, _ = gptq_quantize(np.ascontiguousarray(w[:, perm]), np.ascontiguousarray(x[:, perm]), 8, False)
    assert np.array_equal(codes[:, perm], c2)
    assert np.array_equal(S.view(np.uint16), S2.view(np.uint16))
    assert np.array_equal(Z, Z2)


# --- output error ----------------------------------------------------------------------
# ||(W - W^) X^T||_F / ||W X^T||_F ("AWQ + GPTQ Quantization, in depth", The two
# algorithms, compactly: GPTQ lowers the error of the layer's output on the calibration
# activations).  Pinned by closed forms on layers whose dequantised weights are known
# multiples of W, and by an exact rational recomputation.

def _exact_layer(seed, N=4, K=8, g=4, T=5):
    """A layer whose binary16 weights are exactly (q - Z) S with S a power of two, so
    that W^ = W (and 2W, W/2 are exact binary16 values too)."""
    rng = np.random.default_rng([901, seed])
    G = K // g
    codes = rng.integers(0, 16, (N, K)).astype(np.uint8)
    Z = rng.integers(1, 15, (G, N)).astype(np.uint8)
    S = np.full((G, N), 2.0 ** -6, np.float16)
    gid = np.arange(K) // g
    w = ((codes.astype(np.float64) - Z[gid].T) * S[gid].T.astype(np.float64)).astype(np.float16)
    x = rng.standard_normal((T, K)).astype(np.float16)
    return w, codes, S, Z, g, x


def _error_exact(w, codes, S, Z, g, g_idx, x):
    """The same ratio in Fractions (squared), with the group of channel k taken from
    g_idx or k // g."""
    N, K = w.shape
    gid = np.arange(K) // g if g_idx is None else np.asarray(g_idx)
    num = Fraction(0)
    den = Fraction(0)
    for n in range(N):
        for t in range(x.shape[0]):
            e = Fraction(0)
            v = Fraction(0)
            for k in range(K):
                wk = Fraction(float(w[n, k]))
                what = (int(codes[n, k]) - int(Z[gid[k], n])) * Fraction(float(S[gid[k], n]))
                xk = Fraction(float(x[t, k]))
                e += (wk - what) * xk
                v += wk * xk
            num += e * e
            den += v * v
    return num / den


def _output_error_pins_hold(err_fn) -> bool:
    w, codes, S, Z, g, x = _exact_layer(0)
    if abs(err_fn(w, codes, S, Z, g, None, x)) > 0.0:                    # W^ = W
        return False
    zc = np.repeat(Z.T, g, axis=1).astype(np.uint8)                      # q = Z: W^ = 0
    if abs(err_fn(w, zc, S, Z, g, None, x) - 1.0) > 1e-14:
        return False
    half = (w.astype(np.float64) / 2).astype(np.float16)                 # W^ = 2W
    if abs(err_fn(half, codes, S, Z, g, None, x) - 1.0) > 1e-14:
        return False
    double = (w.astype(np.float64) * 2).astype(np.float16)               # W^ = W/2
    if abs(err_fn(double, codes, S, Z, g, None, x) - 0.5) > 1e-14:
        return False
    # rational recomputation on a layer with a real quantisation error, contiguous and
    # with a permuted group map
    rng = np.random.default_rng(902)
    w2 = (rng.standard_normal((4, 8)) * 0.05).astype(np.float16)
    x2 = rng.standard_normal((6, 8)).astype(np.float16)
    for g_idx in (None, np.array([1, 0, 1, 0, 0, 1, 1, 0], np.int32)):
        c2, S2, Z2 = oracle.rtn_quantize(w2, 4, g_idx)
        ref = _error_exact(w2, c2, S2, Z2, 4, g_idx, x2)
        got = err_fn(w2, c2, S2, Z2, 4, g_idx, x2)
        if not (0.0 < got and abs(Fraction(got) ** 2 / ref - 1) < 1e-12):
            return False
    return True


def test_output_error_pinned():
    assert _output_error_pins_hold(output_error)


def test_output_error_pins_catch_mistakes():
    # planted mistakes (copies of the step, on the CPU): normalising by the quantised
    # layer's output, dropping the activations, transposing the group map
    def by_what(w, codes, S, Z, g, g_idx, x):
        W = w.astype(np.float64)
        Wh = oracle.dequant(codes, S, Z, g, g_idx)
        X = x.astype(np.float64)
        with np.errstate(divide="ignore", invalid="ignore"):
            return float(np.linalg.norm((W - Wh) @ X.T) / np.linalg.norm(Wh @ X.T))

    def no_x(w, codes, S, Z, g, g_idx, x):
        W = w.astype(np.float64)
        Wh = oracle.dequant(codes, S, Z, g, g_idx)
        return float(np.linalg.norm(W - Wh) / np.linalg.norm(W))

    def ignores_gidx(w, codes, S, Z, g, g_idx, x):
        return output_error(w, codes, S, Z, g, None, x)

    for bad in (by_what, no_x, ignores_gidx):
        assert not _output_error_pins_hold(bad), bad.__name__
