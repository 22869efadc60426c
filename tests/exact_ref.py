"""Exact brute-force references used to pin the oracle (tests only).

Everything here works in exact rational arithmetic (``fractions.Fraction``) and
by exhaustive search, on tiles small enough for pure-Python loops.  It imports
nothing from the oracle: it restates the definitions independently, by search
instead of by closed-form rounding.

* scale: the smallest binary16 value that is >= range/15, found by scanning the
  sorted list of all positive finite binary16 values.
* zero point: the integer z in [0, 15] nearest to -w_lo/S (ties to even z).
* code: the grid index j in [0, 15] whose grid point (j - Z)*S is nearest to w
  (ties to even j - Z, the rounding of torch.round).
"""

from __future__ import annotations

import bisect
from fractions import Fraction

import numpy as np

_POS_FP16 = None


def positive_fp16() -> list:
    """All positive finite binary16 values as exact Fractions, ascending."""
    global _POS_FP16
    if _POS_FP16 is None:
        bits = np.arange(1, 0x7C00, dtype=np.uint16)
        _POS_FP16 = [Fraction(float(v)) for v in bits.view(np.float16)]
    return _POS_FP16


def fp16_ceil_exact(v: Fraction) -> Fraction:
    vals = positive_fp16()
    i = bisect.bisect_left(vals, v)
    return vals[i]


def _nearest_int_in(lo: int, hi: int, target: Fraction, parity_offset: int = 0) -> int:
    """Integer j in [lo, hi] nearest to target; ties go to even (j - parity_offset)."""
    best = None
    for j in range(lo, hi + 1):
        d = abs(Fraction(j) - target)
        key = (d, (j - parity_offset) % 2)
        if best is None or key < best[0]:
            best = (key, j)
    return best[1]


def quantize_group_exact(ws, top: int = 15):
    """Exact RTN of one group (list of Fractions) on the grid 0..top -> (S, Z, [q...])."""
    lo = min([Fraction(0)] + list(ws))
    hi = max([Fraction(0)] + list(ws))
    if lo == hi:
        return Fraction(1), 0, [0] * len(ws)
    S = fp16_ceil_exact((hi - lo) / top)
    Z = _nearest_int_in(0, top, -lo / S)
    qs = []
    for w in ws:
        # grid point (j - Z)*S nearest to w  <=>  j nearest to w/S + Z
        qs.append(_nearest_int_in(0, top, w / S + Z, parity_offset=Z))
    return S, Z, qs


def quantize_exact(w: np.ndarray, group_size: int, g_idx=None, in_scale=None, top: int = 15):
    """Exact RTN of a small matrix; same return shapes as the oracle (but Fractions
    for the scales).  in_scale multiplies the float64 columns (its float64
    products are what gets quantised, as in the oracle's definition)."""
    N, K = w.shape
    gid = (np.arange(K) // group_size) if g_idx is None else np.asarray(g_idx)
    G = K // group_size
    W = w.astype(np.float64)
    if in_scale is not None:
        W = W * np.asarray(in_scale, dtype=np.float64)[None, :]
    codes = np.zeros((N, K), dtype=np.uint8)
    S = [[None] * N for _ in range(G)]
    Z = np.zeros((G, N), dtype=np.uint8)
    for n in range(N):
        for gam in range(G):
            ks = [k for k in range(K) if gid[k] == gam]
            s, z, qs = quantize_group_exact([Fraction(float(W[n, k])) for k in ks], top)
            S[gam][n] = s
            Z[gam, n] = z
            for k, q in zip(ks, qs):
                codes[n, k] = q
    return codes, S, Z


def linear_exact(x: np.ndarray, codes, S, Z, group_size: int, g_idx=None):
    """y[m][n] = sum_k x[m][k] * (q[n][k] - Z[g(k)][n]) * S[g(k)][n], exact triple loop.
    S may be Fractions or floats (binary16 values)."""
    M, K = x.shape
    N = codes.shape[0]
    gid = (np.arange(K) // group_size) if g_idx is None else np.asarray(g_idx)
    y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                g = int(gid[k])
                s = S[g][n] if isinstance(S, list) else Fraction(float(S[g, n]))
                acc += Fraction(float(x[m, k])) * (int(codes[n, k]) - int(Z[g, n])) * s
            y[m][n] = acc
    return y


def quantize_group_exact_sym(ws, half: int = 8):
    """Exact symmetric RTN of one group (list of Fractions) -> (S, [code...]): S is
    the smallest binary16 with (half - 1) S >= max |w| (found by scan), each code the
    grid index j in [1, 2 half - 1] whose point (j - half) S is nearest to w, ties to
    even j - half (half = 8 at 4 bits, 128 at 8 bits)."""
    a = max([abs(w) for w in ws] + [Fraction(0)])
    if a == 0:
        return Fraction(1), [half] * len(ws)
    S = fp16_ceil_exact(a / (half - 1))
    return S, [_nearest_int_in(1, 2 * half - 1, w / S + half, parity_offset=half) for w in ws]


def quantize_exact_sym(w: np.ndarray, group_size: int, g_idx=None, in_scale=None, half: int = 8):
    """Exact symmetric RTN of a small matrix: (codes uint8 [N][K], scales [G][N] as
    Fractions)."""
    N, K = w.shape
    gid = (np.arange(K) // group_size) if g_idx is None else np.asarray(g_idx)
    G = K // group_size
    W = w.astype(np.float64)
    if in_scale is not None:
        W = W * np.asarray(in_scale, dtype=np.float64)[None, :]
    codes = np.zeros((N, K), dtype=np.uint8)
    S = [[None] * N for _ in range(G)]
    for n in range(N):
        for gam in range(G):
            members = np.nonzero(gid == gam)[0]
            s, qs = quantize_group_exact_sym([Fraction(float(W[n, k])) for k in members], half)
            S[gam][n] = s
            for k, q in zip(members, qs):
                codes[n, k] = q
    return codes, S



def fp16_round_exact(v: Fraction) -> Fraction:
    """v rounded to the nearest binary16 value, ties to the even significand, found by
    search in the list of all finite binary16 values (no overflow handling: |v| must be
    below the largest finite value)."""
    if v == 0:
        return Fraction(0)
    mag = abs(v)
    vals = positive_fp16()
    assert mag < vals[-1]
    i = bisect.bisect_left(vals, mag)
    hi = vals[i]
    lo = vals[i - 1] if i > 0 else Fraction(0)
    if hi == mag:
        r = hi
    elif mag - lo != hi - mag:
        r = lo if mag - lo < hi - mag else hi
    else:
        # a tie: the neighbour whose bit pattern is even (zero counts as even); the
        # positive binary16 values are listed by ascending bit pattern from 1, so the
        # pattern of vals[j] is j + 1
        r = lo if (i % 2 == 0) else hi
    return r if v > 0 else -r
