"""Pins of the oracle's quantiser, AWQ scale and act-order steps (no GPU).

Each pin is something other than the oracle itself: hand-worked groups
(tests/golden), an exact exhaustive-search reference (tests/exact_ref.py),
torch.round as the pages' rounding, and invariants that follow from "round to
the nearest grid point".
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from exact_ref import fp16_ceil_exact, fp16_round_exact, quantize_exact, quantize_exact_sym

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _tile(seed, N, K, scale=0.5):
    rng = np.random.default_rng([7, seed])
    return (rng.standard_normal((N, K)) * scale).astype(np.float16)


def _gidx_random(K, g, seed):
    perm = np.random.default_rng([8, seed]).permutation(K)
    g_idx = np.empty(K, dtype=np.int32)
    g_idx[perm] = np.arange(K) // g
    return g_idx


# --- hand-worked groups ------------------------------------------------------------

def test_worked_groups():
    data = json.load(open(os.path.join(GOLDEN, "rtn_worked_groups.json")))
    assert len(data["groups"]) >= 7
    for grp in data["groups"]:
        w = np.array(grp["w"], dtype=np.float16)[None, :]
        codes, S, Z = oracle.rtn_quantize(w, w.shape[1])
        assert codes[0].tolist() == grp["codes"], grp["name"]
        assert float(S[0, 0]) == grp["scale"], grp["name"]
        assert hex(int(S.view(np.uint16)[0, 0])) == grp["scale_bits"], grp["name"]
        assert int(Z[0, 0]) == grp["zero"], grp["name"]


def test_round_half_even_is_torch_round():
    v = np.array([-3.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5, 14.5, 15.5,
                  0.49999999, 0.50000001, -7.25, 7.75, 1e-300])
    assert np.array_equal(oracle.round_half_even(v), torch.round(torch.from_numpy(v)).numpy())


def test_fp16_ceil_matches_exact_scan():
    rng = np.random.default_rng(3)
    vals = list(rng.uniform(1e-7, 3e3, 400)) + list(10.0 ** rng.uniform(-7, 3.5, 400))
    exact16 = [float(v) for v in np.array([0x0001, 0x03FF, 0x0400, 0x2E66, 0x3C00, 0x7BFF],
                                           dtype=np.uint16).view(np.float16)]
    vals += exact16 + [np.nextafter(v, 0.0) for v in exact16] + [np.nextafter(v, 1e9) for v in exact16[:-1]]
    got = oracle.fp16_ceil(np.array(vals))
    for v, h in zip(vals, got):
        assert Fraction(float(h)) == fp16_ceil_exact(Fraction(v)), v


# --- exact exhaustive-search reference on 8x8 tiles ---------------------------------

def _plant_special_groups(w, g, g_idx):
    gid = (np.arange(w.shape[1]) // g) if g_idx is None else g_idx
    m0 = np.nonzero(gid == 0)[0]
    m1 = np.nonzero(gid == (1 % (w.shape[1] // g)))[0]
    w[0, m0] = np.abs(w[0, m0])          # one-signed positive group
    w[1, m0] = -np.abs(w[1, m0])         # one-signed negative group
    w[2, m0] = 0                         # all-zero group
    w[3, m1] = np.float16(0.25) * np.arange(m1.size, dtype=np.float16) - np.float16(0.75)  # ties
    return w


@pytest.mark.parametrize("g", [2, 4, 8])
@pytest.mark.parametrize("use_gidx", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rtn_matches_exact_search(g, use_gidx, seed):
    g_idx = _gidx_random(8, g, seed) if use_gidx else None
    w = _plant_special_groups(_tile(seed, 8, 8), g, g_idx)
    c, S, Z = oracle.rtn_quantize(w, g, g_idx)
    ce, Se, Ze = quantize_exact(w, g, g_idx)
    assert np.array_equal(c, ce)
    assert np.array_equal(Z, Ze)
    for gam in range(S.shape[0]):
        for n in range(S.shape[1]):
            assert Fraction(float(S[gam, n])) == Se[gam][n]


@pytest.mark.parametrize("seed", [0, 1])
def test_rtn_with_awq_scale_matches_exact_search(seed):
    w = _tile(seed, 8, 8, scale=0.05)
    s = np.random.default_rng([9, seed]).uniform(0.3, 3.0, 8)
    c, S, Z = oracle.rtn_quantize(w, 4, None, s)
    ce, Se, Ze = quantize_exact(w, 4, None, s)
    assert np.array_equal(c, ce) and np.array_equal(Z, Ze)
    assert all(Fraction(float(S[a, n])) == Se[a][n] for a in range(2) for n in range(8))


# --- invariants on every configuration (sampled rows; RTN is row-independent) -------

def _quantize_cfg_rows(cfg, rows):
    w = wl.weights(cfg, rows)
    g_idx = s = None
    if cfg.act_order:
        g_idx, _ = oracle.act_order(wl.calibration(cfg), cfg.group_size)
    if cfg.awq:
        s = oracle.awq_scales(wl.calibration(cfg))
    codes, S, Z = oracle.rtn_quantize(w, cfg.group_size, g_idx, s)
    return w, g_idx, s, codes, S, Z


@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_rtn_invariants_on_configs(name):
    cfg = wl.CONFIGS[name]
    rows = np.linspace(0, cfg.N - 1, 40).astype(np.int64)
    w, g_idx, s, codes, S, Z = _quantize_cfg_rows(cfg, rows)
    g = cfg.group_size
    W = w.astype(np.float64) * (1.0 if s is None else s[None, :])
    gid = oracle.group_index(cfg.K, g, g_idx)
    Sk = S.astype(np.float64)[gid, :].T
    Zk = Z.astype(np.float64)[gid, :].T
    What = oracle.dequant(codes, S, Z, g, g_idx)
    # every weight is within half a step of its grid point
    assert np.all(np.abs(W - What) <= Sk / 2)
    assert codes.max() <= 15 and Z.max() <= 15
    # re-quantising the reconstruction with the same S and Z returns the codes
    assert np.array_equal(np.clip(np.rint(What / Sk) + Zk, 0, 15), codes.astype(np.float64))
    for gam in range(cfg.G):
        members = np.nonzero(gid == gam)[0]
        Wg = W[:, members]
        lo = np.minimum(Wg.min(1), 0)
        hi = np.maximum(Wg.max(1), 0)
        # the scale is the smallest binary16 whose 15 steps cover the range
        prev = np.nextafter(S[gam], np.float16(0)).astype(np.float64)
        assert np.all(S[gam].astype(np.float64) * 15 >= hi - lo)
        assert np.all(prev * 15 < hi - lo)
        # the most negative weight lands on code 0
        neg = Wg.min(1) < 0
        qmin = codes[np.arange(len(rows)), members[np.argmin(Wg, axis=1)]]
        assert np.all(qmin[neg] == 0)


# --- symmetric quantiser --------------------------------------------------------------

def test_sym_worked_groups():
    data = json.load(open(os.path.join(GOLDEN, "rtn_sym_worked_groups.json")))
    for grp in data["groups"]:
        if "w_bits" in grp:
            w = np.array([int(b, 16) for b in grp["w_bits"]], dtype=np.uint16).view(np.float16)[None, :]
        else:
            w = np.array(grp["w"], dtype=np.float16)[None, :]
        codes, S = oracle.rtn_quantize_sym(w, w.shape[1])
        assert codes[0].tolist() == grp["codes"], grp["name"]
        assert float(S[0, 0]) == grp["scale"], grp["name"]
        assert hex(int(S.view(np.uint16)[0, 0])) == grp["scale_bits"], grp["name"]


@pytest.mark.parametrize("g", [2, 4, 8])
@pytest.mark.parametrize("use_gidx", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sym_rtn_matches_exact_search(g, use_gidx, seed):
    g_idx = _gidx_random(8, g, seed) if use_gidx else None
    w = _plant_special_groups(_tile(seed, 8, 8), g, g_idx)
    c, S = oracle.rtn_quantize_sym(w, g, g_idx)
    ce, Se = quantize_exact_sym(w, g, g_idx)
    assert np.array_equal(c, ce)
    assert all(Fraction(float(S[a, n])) == Se[a][n] for a in range(S.shape[0]) for n in range(S.shape[1]))


def test_sym_rtn_with_awq_scale_matches_exact_search():
    w = _tile(4, 8, 8, scale=0.05)
    s = np.random.default_rng([9, 4]).uniform(0.3, 3.0, 8)
    c, S = oracle.rtn_quantize_sym(w, 4, None, s)
    ce, Se = quantize_exact_sym(w, 4, None, s)
    assert np.array_equal(c, ce)
    assert all(Fraction(float(S[a, n])) == Se[a][n] for a in range(2) for n in range(8))


@pytest.mark.parametrize("name", ["c1", "c3", "c5"])
def test_sym_rtn_invariants_on_configs(name):
    cfg = wl.CONFIGS[name]
    rows = np.linspace(0, cfg.N - 1, 24).astype(np.int64)
    w = wl.weights(cfg, rows)
    g = cfg.group_size
    g_idx = oracle.act_order(wl.calibration(cfg), g)[0] if cfg.act_order else None
    codes, S = oracle.rtn_quantize_sym(w, g, g_idx)
    Z = oracle.sym_zeros(cfg.G, len(rows))
    W = w.astype(np.float64)
    gid = oracle.group_index(cfg.K, g, g_idx)
    Sk = S.astype(np.float64)[gid, :].T
    What = oracle.dequant(codes, S, Z, g, g_idx)
    assert np.all(np.abs(W - What) <= Sk / 2)            # within half a step
    assert codes.min() >= 1 and codes.max() <= 15        # the grid is -7 .. 7
    for gam in range(cfg.G):
        members = np.nonzero(gid == gam)[0]
        a = np.abs(W[:, members]).max(1)
        prev = np.nextafter(S[gam], np.float16(0)).astype(np.float64)
        assert np.all(S[gam].astype(np.float64) * 7 >= a) and np.all(prev * 7 < a)
        # the largest magnitude lands on an end of the grid
        top = codes[np.arange(len(rows)), members[np.argmax(np.abs(W[:, members]), axis=1)]]
        assert np.all((top == 1) | (top == 15))
    # sign symmetry: -w has the same scales and the mirrored codes (round half even is odd)
    c_neg, S_neg = oracle.rtn_quantize_sym(-w, g, g_idx)
    assert np.array_equal(S_neg.view(np.uint16), S.view(np.uint16))
    assert np.array_equal(c_neg.astype(int), 16 - codes.astype(int))


# --- 8-bit weights ---------------------------------------------------------------------

@pytest.mark.parametrize("g", [4, 8])
@pytest.mark.parametrize("seed", [0, 1])
def test_rtn8_matches_exact_search(g, seed):
    w = _plant_special_groups(_tile(seed, 8, 8), g, None)
    c, S, Z = oracle.rtn_quantize(w, g, bits=8)
    ce, Se, Ze = quantize_exact(w, g, top=255)
    assert np.array_equal(c, ce) and np.array_equal(Z, Ze)
    assert all(Fraction(float(S[a, n])) == Se[a][n] for a in range(S.shape[0]) for n in range(8))
    c, S = oracle.rtn_quantize_sym(w, g, bits=8)
    ce, Se = quantize_exact_sym(w, g, half=128)
    assert np.array_equal(c, ce)
    assert all(Fraction(float(S[a, n])) == Se[a][n] for a in range(S.shape[0]) for n in range(8))


def test_sym8_is_the_int8_absmax_grid():
    """At 8 bits the symmetric scheme is the pages' int8 absmax code on each group
    (scale absmax / 127, round half even, clamp to -127..127), with the scale held in
    binary16 rounded up: on groups whose absmax / 127 is a binary16 value the codes are
    exactly round(w / (absmax / 127)) + 128."""
    w = np.zeros((4, 16), np.float16)
    w[0] = np.float16(127.0) * np.linspace(-1, 1, 16).astype(np.float16)   # absmax 127: scale 1
    w[1] = np.float16(0.5) * w[0]                                         # scale 0.5 (power of two)
    w[2] = -w[0]
    w[3, :] = 0
    codes, S = oracle.rtn_quantize_sym(w, 16, bits=8)
    assert S[0, :3].tolist() == [1.0, 0.5, 1.0] and float(S[0, 3]) == 1.0
    a = np.abs(w.astype(np.float64)).max(1)
    for r in range(3):
        expect = np.clip(np.rint(w[r].astype(np.float64) / (a[r] / 127.0)), -127, 127) + 128
        assert np.array_equal(codes[r], expect.astype(np.uint8))
    assert np.all(codes[3] == 128)


@pytest.mark.parametrize("name", ["c1", "c3"])
def test_rtn8_invariants_on_configs(name):
    cfg = wl.CONFIGS[name]
    rows = np.linspace(0, cfg.N - 1, 16).astype(np.int64)
    w = wl.weights(cfg, rows)
    W = w.astype(np.float64)
    g = cfg.group_size
    gid = oracle.group_index(cfg.K, g)
    for sym in (False, True):
        if sym:
            codes, S = oracle.rtn_quantize_sym(w, g, bits=8)
            Z = oracle.sym_zeros(cfg.G, len(rows), bits=8)
        else:
            codes, S, Z = oracle.rtn_quantize(w, g, bits=8)
        Sk = S.astype(np.float64)[gid, :].T
        What = oracle.dequant(codes, S, Z, g)
        assert np.all(np.abs(W - What) <= Sk / 2)
        # 8 bits: at most 1/16 of the 4-bit step on the same group's range
        c4, S4, Z4 = oracle.rtn_quantize(w, g)
        assert np.all(S.astype(np.float64) <= S4.astype(np.float64) * (15.0 / 127.0) * 1.01 if sym
                      else S.astype(np.float64) <= S4.astype(np.float64) * (15.0 / 255.0) * 1.01)


# --- AWQ scale and fold -------------------------------------------------------------

def test_awq_scales_exact_mean_and_sqrt():
    X = (np.random.default_rng(5).standard_normal((37, 11)) * 3).astype(np.float16)
    s = oracle.awq_scales(X)
    assert s.shape == (11,)
    for k in range(11):
        mean = sum(abs(Fraction(float(v))) for v in X[:, k]) / 37
        # float(Fraction) is correctly rounded; s is the correctly rounded square
        # root of that correctly rounded mean
        assert s[k] == np.sqrt(float(mean))


def test_awq_scales_closed_forms():
    X = np.zeros((4, 3), dtype=np.float16)
    X[:, 0] = [4, -4, 4, -4]                   # mean |x| = 4 -> s = 2
    X[:, 1] = [1, 0, 0, 0]                     # mean = 0.25 -> s = 0.5
    s = oracle.awq_scales(X)
    assert s[0] == 2.0 and s[1] == 0.5 and s[2] == 1.0     # all-zero channel -> 1
    assert oracle.awq_scales(X, alpha=1.0)[0] == 4.0


def test_awq_fold_is_exactly_invariant():
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((8, 8)) * 0.1).astype(np.float16)
    x = rng.standard_normal((3, 8)).astype(np.float16)
    # power-of-two scales keep float64 arithmetic exact
    s = 2.0 ** rng.integers(-4, 5, 8).astype(np.float64)
    Wf = oracle.awq_fold_weights(w, s)
    xf = x.astype(np.float64) / s[None, :]
    for m in range(3):
        for n in range(8):
            lhs = sum(Fraction(xf[m, k]) * Fraction(Wf[n, k]) for k in range(8))
            rhs = sum(Fraction(float(x[m, k])) * Fraction(float(w[n, k])) for k in range(8))
            assert lhs == rhs
    # a row (output-channel) scaling would not be invariant
    assert not np.allclose((xf @ (w.astype(np.float64) * s[:, None]).T), x.astype(np.float64) @ w.astype(np.float64).T)


def _fold_pins_hold(fold) -> bool:
    """The activation side of the AWQ fold ("How do GPTQ and AWQ differ...", AWQ:
    protect the salient channels: multiply a weight channel by s, divide the matching
    activation channel by s, the product is unchanged), checked two ways:

    (a) power-of-two s, activations whose quotients stay normal binary16 numbers:
        x/s is exact, so sum_k fold(x)[m,k] * (W diag(s))[n,k] equals x W^T exactly
        (Fractions);
    (b) s from the calibration rule on random data (not powers of two): every element
        is the exact quotient x/s rounded once to the nearest binary16 (exact search).
    """
    rng = np.random.default_rng(31)
    # (a) binary16 activations (1 + f/1024) 2^e with e in [-4, 4]: x/s with s in 2^[-3, 3]
    # stays in [2^-7, 2^8), where binary16 is exact for these significands
    sig = 1.0 + rng.integers(0, 1024, (3, 8)) / 1024.0
    x = (np.where(rng.random((3, 8)) < 0.5, -1.0, 1.0) * sig * 2.0 ** rng.integers(-4, 5, (3, 8))).astype(np.float16)
    w = (rng.standard_normal((5, 8)) * 0.1).astype(np.float16)
    s = 2.0 ** rng.integers(-3, 4, 8).astype(np.float64)
    xf = fold(x, s)
    if xf.dtype != np.float16 or xf.shape != x.shape:
        return False
    Wf = oracle.awq_fold_weights(w, s)
    for m in range(3):
        for n in range(5):
            lhs = sum(Fraction(float(xf[m, k])) * Fraction(float(Wf[n, k])) for k in range(8))
            rhs = sum(Fraction(float(x[m, k])) * Fraction(float(w[n, k])) for k in range(8))
            if lhs != rhs:
                return False
    # (b) quotients that need rounding
    X = (rng.standard_normal((64, 16)) * 3).astype(np.float16)
    s = oracle.awq_scales(X)
    x = (rng.standard_normal((4, 16)) * 2).astype(np.float16)
    xf = fold(x, s)
    rounded = 0
    for m in range(4):
        for k in range(16):
            q = Fraction(float(x[m, k])) / Fraction(float(s[k]))
            r = fp16_round_exact(q)
            rounded += r != q
            if Fraction(float(xf[m, k])) != r:
                return False
    return rounded > 32   # most quotients really were rounded


def test_awq_fold_activations_pinned():
    assert _fold_pins_hold(oracle.awq_fold_activations)


def test_awq_fold_activation_pins_catch_mistakes():
    # planted mistakes (on the CPU, in copies of the step): multiplying instead of
    # dividing, and dropping the fold
    def times_s(x, s):
        return (np.asarray(x, np.float64) * np.asarray(s, np.float64)[None, :]).astype(np.float16)

    def no_fold(x, s):
        return np.asarray(x, np.float16).copy()

    assert not _fold_pins_hold(times_s)
    assert not _fold_pins_hold(no_fold)


@pytest.mark.parametrize("name", ["c2up", "c2down"])
def test_awq_fold_invariant_at_config_scale(name):
    cfg = wl.CONFIGS[name]
    s = oracle.awq_scales(wl.calibration(cfg))
    rows = np.arange(0, cfg.N, cfg.N // 32)
    w = wl.weights(cfg, rows)
    x = wl.activations(cfg, 1)
    y0 = x.astype(np.float64) @ w.astype(np.float64).T
    y1 = (x.astype(np.float64) / s[None, :]) @ oracle.awq_fold_weights(w, s).T
    assert np.max(np.abs(y1 - y0)) <= 1e-13 * np.sqrt(np.mean(y0 ** 2)) * 10
    # the folded activation is binary16(x/s)
    xf = oracle.awq_fold_activations(x, s)
    assert xf.dtype == np.float16
    assert np.array_equal(xf, (x.astype(np.float64) / s).astype(np.float16))


# --- act order ------------------------------------------------------------------------

def test_act_order_h_exact():
    X = (np.random.default_rng(2).standard_normal((23, 9)) * 10).astype(np.float16)
    h = oracle.act_order_h(X)
    for k in range(9):
        exact = sum(Fraction(float(v)) ** 2 for v in X[:, k])
        assert Fraction(h[k], 2 ** 48) == exact


def test_act_order_descending_and_ties():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((16, 12)).astype(np.float16)
    X[:, 7] = X[:, 2]                 # exact tie between channels 2 and 7
    X[:, 9] = -X[:, 2]                # and 9 (same squares)
    g = 4
    g_idx, perm = oracle.act_order(X, g)
    h = [float(v) for v in oracle.act_order_h(X)]
    assert sorted(perm.tolist()) == list(range(12))
    for a, b in zip(perm[:-1], perm[1:]):
        assert h[a] > h[b] or (h[a] == h[b] and a < b)
    pos = {int(k): i for i, k in enumerate(perm)}
    assert pos[2] < pos[7] < pos[9]
    counts = np.bincount(g_idx, minlength=12 // g)
    assert np.all(counts == g)
    for i, k in enumerate(perm):
        assert g_idx[k] == i // g


def test_act_order_config5_is_noncontiguous_and_matches_float64():
    cfg = wl.CONFIGS["c5"]
    X = wl.calibration(cfg)
    g_idx, perm = oracle.act_order(X, cfg.group_size)
    h64 = (X.astype(np.float64) ** 2).sum(0)
    # with well-separated values the float64 sort agrees with the exact one
    order64 = np.argsort(-h64, kind="stable")
    gaps = np.diff(np.sort(h64))
    if gaps.min() > 1e-9 * h64.max():
        assert np.array_equal(order64, perm)
    # the outlier channels come first, and the groups are not contiguous runs
    out = set(wl.outlier_channels(cfg).tolist())
    assert set(perm[:len(out)].tolist()) == out
    assert not np.array_equal(g_idx, np.arange(cfg.K) // cfg.group_size)
    assert np.all(np.bincount(g_idx) == cfg.group_size)
