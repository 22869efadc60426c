"""Pins of the oracle's dequantisation and float64 matmul (no GPU)."""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact_ref import linear_exact


def _random_layer(seed, M, N, K, g, with_gidx):
    rng = np.random.default_rng([21, seed])
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    G = K // g
    scales = rng.uniform(0.001, 0.05, size=(G, N)).astype(np.float16)
    zeros = rng.integers(0, 16, size=(G, N), dtype=np.uint8)
    x = rng.standard_normal((M, K)).astype(np.float16)
    g_idx = None
    if with_gidx:
        perm = rng.permutation(K)
        g_idx = np.empty(K, dtype=np.int32)
        g_idx[perm] = np.arange(K) // g
    return x, codes, scales, zeros, g_idx


@pytest.mark.parametrize("with_gidx", [False, True])
@pytest.mark.parametrize("shape", [(3, 8, 16, 4), (2, 16, 8, 2), (1, 8, 8, 8)])
def test_linear_matches_exact_triple_loop(shape, with_gidx):
    M, N, K, g = shape
    x, codes, scales, zeros, g_idx = _random_layer(sum(shape), M, N, K, g, with_gidx)
    y = oracle.linear(x, codes, scales, zeros, g, g_idx)
    ye = linear_exact(x, codes, scales, zeros, g, g_idx)
    assert y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            # float64 matmul of exact products: relative error far below 1e-12
            assert abs(Fraction(y[m, n]) - ye[m][n]) <= Fraction(1, 10**12) * (1 + abs(ye[m][n]))


@pytest.mark.parametrize("with_gidx", [False, True])
def test_dequant_entries_exact(with_gidx):
    _, codes, scales, zeros, g_idx = _random_layer(5, 1, 16, 32, 8, with_gidx)
    W = oracle.dequant(codes, scales, zeros, 8, g_idx)
    gid = np.arange(32) // 8 if g_idx is None else g_idx
    for n in range(16):
        for k in range(32):
            gam = gid[k]
            exact = (int(codes[n, k]) - int(zeros[gam, n])) * Fraction(float(scales[gam, n]))
            assert Fraction(W[n, k]) == exact
    W16 = oracle.dequant_fp16(codes, scales, zeros, 8, g_idx)
    assert W16.dtype == np.float16 and np.array_equal(W16, W.astype(np.float16))


def test_unit_vector_probe_selects_a_column():
    x, codes, scales, zeros, g_idx = _random_layer(9, 1, 24, 64, 16, True)
    W = oracle.dequant(codes, scales, zeros, 16, g_idx)
    for k in [0, 1, 17, 63]:
        e = np.zeros((1, 64), dtype=np.float16)
        e[0, k] = 1
        assert np.array_equal(oracle.linear(e, codes, scales, zeros, 16, g_idx)[0], W[:, k])


def test_all_ones_gives_row_sums():
    _, codes, scales, zeros, _ = _random_layer(10, 1, 40, 128, 32, False)
    W = oracle.dequant(codes, scales, zeros, 32)
    y = oracle.linear(np.ones((1, 128), dtype=np.float16), codes, scales, zeros, 32)[0]
    assert np.allclose(y, W.sum(axis=1), rtol=1e-13, atol=1e-15)


def test_identity_gidx_equals_contiguous():
    x, codes, scales, zeros, _ = _random_layer(12, 2, 16, 64, 16, False)
    ident = (np.arange(64) // 16).astype(np.int32)
    assert np.array_equal(oracle.linear(x, codes, scales, zeros, 16),
                          oracle.linear(x, codes, scales, zeros, 16, ident))


def test_rel_err():
    y_ref = np.array([[3.0, -4.0]])
    assert oracle.rel_err(y_ref, y_ref) == 0.0
    rms = np.sqrt(12.5)
    assert oracle.rel_err(y_ref + [[0.0, 0.5]], y_ref) == pytest.approx(0.5 / rms)
