"""Pins of the oracle's AWQ alpha search (no GPU).

Each pin is something other than the search itself: alpha = 0 reduces it to plain
round-to-nearest (s = 1), an exact rational recomputation of the loss on a tiny
layer, and exact equivariance under power-of-two scaling of the weights.
"""

from fractions import Fraction

import numpy as np

import oracle
import workloads as wl


def _layer(seed, N=16, K=64, T=32):
    cfg = wl.custom_config("awq", 700 + seed, K=K, N=N, group_size=32)
    return wl.weights(cfg), wl.calibration(cfg, T)


def test_alpha_zero_is_plain_rtn():
    w, X = _layer(0)
    losses, _ = oracle.awq_search(w, X, 32, [0.0])
    codes, S, Z = oracle.rtn_quantize(w, 32)
    y_rtn = oracle.linear(X, codes, S, Z, 32)
    y_ref = X.astype(np.float64) @ w.astype(np.float64).T
    assert losses[0] == np.sqrt(np.sum((y_ref - y_rtn) ** 2))


def test_loss_matches_exact_rational_recomputation():
    w, X = _layer(1, N=8, K=32, T=4)
    alphas = [0.25, 0.5, 1.0]
    losses, best = oracle.awq_search(w, X, 32, alphas)
    for a, loss in zip(alphas, losses):
        s = oracle.awq_scales(X, a)
        codes, S, Z = oracle.rtn_quantize(w, 32, None, s)
        xs = oracle.awq_fold_activations(X, s)
        total = Fraction(0)
        for t in range(X.shape[0]):
            for n in range(w.shape[0]):
                ref = sum(Fraction(float(X[t, k])) * Fraction(float(w[n, k])) for k in range(32))
                got = sum(Fraction(float(xs[t, k])) * (int(codes[n, k]) - int(Z[0, n])) * Fraction(float(S[0, n]))
                          for k in range(32))
                total += (ref - got) ** 2
        assert abs(loss - np.sqrt(float(total))) <= 1e-12 * max(loss, 1e-30)
    assert best == int(np.argmin(losses))


def test_power_of_two_weight_scaling_scales_every_loss():
    w, X = _layer(2)
    alphas = [0.0, 0.3, 0.6, 0.9]
    l1, b1 = oracle.awq_search(w, X, 32, alphas)
    l2, b2 = oracle.awq_search((w.astype(np.float32) * 4).astype(np.float16), X, 32, alphas)
    assert np.array_equal(l2, 4 * l1) and b1 == b2


def test_salient_channels_prefer_a_positive_alpha():
    """Calibration activations with a few large channels (the pages' salient
    channels): some alpha > 0 beats plain rounding on the configuration-2 layer."""
    cfg = wl.CONFIGS["c2up"]
    rows = np.arange(64)
    w = wl.weights(cfg, rows)
    X = wl.calibration(cfg)[:128]
    alphas = np.linspace(0, 1, 11)
    losses, best = oracle.awq_search(w, X, cfg.group_size, alphas)
    assert best > 0 and losses[best] < losses[0]
