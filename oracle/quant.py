"""Quantiser steps of the oracle (test infrastructure only; see package header).

Readings of the pages that are fixed here (each listed with its reason in the
design notes of the repository):

* grid: 4 bits give 16 levels, codes q and zero points Z are unsigned integers
  in [0, 15] ("LLM Quantization: INT8, GPTQ, and AWQ Explained", Round-to-
  nearest, and where it falls apart; "AWQ + GPTQ Quantization, in depth", What
  W4A16 buys: a 4-bit zero point).
* range: the block's range is taken to include zero, w_lo = min(0, min w),
  w_hi = max(0, max w); the scale spreads the 16-level grid over it,
  S = (w_hi - w_lo) / 15 ("INT8, GPTQ, and AWQ Explained", What quantization
  actually does: find the range, pick a scale that spreads the grid, round to
  the nearest grid point).
* scale precision: one binary16 scale per group ("in depth", What W4A16 buys:
  a 16-bit scale), rounded UP to the next binary16 value so that the grid still
  covers the range and every weight is within S/2 of a grid point.
* rounding: round half to even, the rounding of ``torch.round`` in the int8
  absmax code of "INT8, GPTQ, and AWQ Explained", What quantization actually
  does; q = round(w/S) + Z and w ~ (q - Z)*S as in "A Deep Dive", The Math of
  Quantization.
* an all-zero group gets S = 1, Z = 0, q = 0 (reconstructs zero exactly).
* groups run along the input dimension: a group is a run of ``group_size``
  input channels of one output row ("in depth", What W4A16 buys; "How do GPTQ
  and AWQ differ...", The shared setting).  Under act order the group of input
  channel k is g_idx[k].
"""

from __future__ import annotations

import numpy as np

FP16_MAX = 65504.0
LEVELS = 15                 # 2**4 - 1 steps between the 16 grid points


def round_half_even(v: np.ndarray) -> np.ndarray:
    """Round to the nearest integer, ties to even (the rounding of torch.round)."""
    return np.rint(v)


def fp16_ceil(v: np.ndarray) -> np.ndarray:
    """Smallest binary16 value that is >= v, for finite v > 0 (float64 input)."""
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)                         # nearest, ties to even
    below = h.astype(np.float64) < v
    h[below] = np.nextafter(h[below], np.float16(np.inf))
    return h


def group_index(K: int, group_size: int, g_idx=None) -> np.ndarray:
    """Group of every input channel: k // group_size, or g_idx[k] under act order."""
    if g_idx is None:
        return np.arange(K, dtype=np.int64) // group_size
    return np.asarray(g_idx, dtype=np.int64)


def rtn_quantize(w, group_size: int, g_idx=None, in_scale=None, bits: int = 4):
    """Asymmetric round-to-nearest group quantiser, 4-bit (16 levels) or 8-bit (256
    levels: "AWQ + GPTQ Quantization, in depth", 4-bit bigger or 8-bit smaller).

    w        binary16 [N][K] weights (out x in).
    g_idx    optional int [K]: group of every input channel (act order).
    in_scale optional float64 [K]: AWQ per-input-channel scale s; the weights
             quantised are then W*diag(s), formed in float64.

    Returns codes uint8 [N][K], scales binary16 [G][N], zeros uint8 [G][N]
    with G = K / group_size.  Per (row n, group gamma), over the members
    {k : group(k) = gamma}, with L = 2**bits - 1 (15 or 255):
        w_lo = min(0, min w), w_hi = max(0, max w)
        S = smallest binary16 >= (w_hi - w_lo)/L        (S = 1 if w_hi = w_lo)
        Z = clamp(round(-w_lo/S), 0, L)
        q = clamp(round(w/S) + Z, 0, L)
    All arithmetic is float64 on the binary16 inputs.
    """
    assert bits in (4, 8)
    levels = (1 << bits) - 1
    w = np.asarray(w)
    assert w.dtype == np.float16 and w.ndim == 2
    N, K = w.shape
    assert K % group_size == 0
    G = K // group_size
    gid = group_index(K, group_size, g_idx)
    W = w.astype(np.float64)
    if in_scale is not None:
        W = W * np.asarray(in_scale, dtype=np.float64)[None, :]

    codes = np.empty((N, K), dtype=np.uint8)
    scales = np.empty((G, N), dtype=np.float16)
    zeros = np.empty((G, N), dtype=np.uint8)
    for gamma in range(G):
        cols = np.nonzero(gid == gamma)[0]
        assert cols.size == group_size, "every group must have group_size members"
        Wg = W[:, cols]
        lo = np.minimum(Wg.min(axis=1), 0.0)
        hi = np.maximum(Wg.max(axis=1), 0.0)
        flat = hi == lo
        S16 = fp16_ceil(np.where(flat, 1.0, (hi - lo) / levels))
        S16[flat] = np.float16(1.0)
        S = S16.astype(np.float64)
        Z = np.clip(round_half_even(-lo / S), 0, levels)
        Z[flat] = 0
        q = np.clip(round_half_even(Wg / S[:, None]) + Z[:, None], 0, levels)
        codes[:, cols] = q.astype(np.uint8)
        scales[gamma] = S16
        zeros[gamma] = Z.astype(np.uint8)
    return codes, scales, zeros


SYM_LEVELS = 7              # 2**(4-1) - 1: the symmetric grid is -7 .. 7
SYM_ZERO = 8                # stored code of 0 (the implicit zero point)


def rtn_quantize_sym(w, group_size: int, g_idx=None, in_scale=None, bits: int = 4):
    """Symmetric 4-bit round-to-nearest group quantiser: the absmax scheme of "LLM
    Quantization: INT8, GPTQ, and AWQ Explained", What quantization actually does
    (one scale from the block's largest magnitude, round, clamp to the symmetric
    range), on the 4-bit grid -7 .. 7; the GPTQ recipe of "AWQ + GPTQ Quantization, in
    depth", Running it, uses the symmetric W4A16 scheme where the AWQ one is asymmetric.

    Returns codes uint8 [N][K] (the signed value plus 2**(bits-1), so the implicit
    zero point is 8 at 4 bits and 128 at 8 bits) and scales binary16 [G][N].  Per
    (row n, group gamma), with L = 2**(bits-1) - 1 (7, or 127 as in the pages' int8
    absmax code):
        a = max |w|
        S = smallest binary16 >= a / L                  (S = 1 if a = 0)
        q = clamp(round(w / S), -L, L),  code = q + L + 1
    and w ~ (code - L - 1) * S.  Same group membership, AWQ factor and float64
    arithmetic as rtn_quantize.
    """
    assert bits in (4, 8)
    levels = (1 << (bits - 1)) - 1
    zero = levels + 1
    w = np.asarray(w)
    assert w.dtype == np.float16 and w.ndim == 2
    N, K = w.shape
    assert K % group_size == 0
    G = K // group_size
    gid = group_index(K, group_size, g_idx)
    W = w.astype(np.float64)
    if in_scale is not None:
        W = W * np.asarray(in_scale, dtype=np.float64)[None, :]

    codes = np.empty((N, K), dtype=np.uint8)
    scales = np.empty((G, N), dtype=np.float16)
    for gamma in range(G):
        cols = np.nonzero(gid == gamma)[0]
        assert cols.size == group_size, "every group must have group_size members"
        Wg = W[:, cols]
        a = np.abs(Wg).max(axis=1)
        flat = a == 0.0
        S16 = fp16_ceil(np.where(flat, 1.0, a / levels))
        S16[flat] = np.float16(1.0)
        S = S16.astype(np.float64)
        q = np.clip(round_half_even(Wg / S[:, None]), -levels, levels)
        codes[:, cols] = (q + zero).astype(np.uint8)
        scales[gamma] = S16
    return codes, scales


def sym_zeros(G: int, N: int, bits: int = 4) -> np.ndarray:
    """The implicit zero points of a symmetric layer, uint8 [G][N]: 8 (4-bit) or
    128 (8-bit)."""
    return np.full((G, N), 1 << (bits - 1), dtype=np.uint8)


# --- AWQ ------------------------------------------------------------------------

def awq_scales(xcal, alpha: float = 0.5) -> np.ndarray:
    """Per-input-channel AWQ scale s_k = (mean_t |X[t,k]|)**alpha, float64 [K].

    "AWQ + GPTQ Quantization, in depth", The two algorithms, compactly: the
    scale is the channel's mean activation magnitude over the calibration tokens
    raised to a power alpha (found by grid search on that page; fixed here).

    The mean is formed exactly: every binary16 value is an integer multiple of
    2**-24, so sum_t |X| * 2**24 is an exact integer (< 2**53 for T <= 8192);
    one float64 division then gives the mean.  alpha = 0.5 is taken with the
    correctly rounded square root.  A channel whose activations are all zero
    gets s = 1.
    """
    X = np.asarray(xcal)
    assert X.dtype == np.float16 and X.ndim == 2
    T = X.shape[0]
    units = (np.abs(X.astype(np.float64)) * 2.0**24).astype(np.int64)
    total = units.sum(axis=0)
    mean = total.astype(np.float64) / (float(T) * 2.0**24)
    if alpha == 0.5:
        s = np.sqrt(mean)
    else:
        s = mean ** alpha
    s[mean == 0.0] = 1.0
    return s


def awq_fold_weights(w, s) -> np.ndarray:
    """W*diag(s): each input channel (column k) of W multiplied by s_k, float64.

    "How do GPTQ and AWQ differ...", AWQ: protect the salient channels: a weight
    channel multiplied by s and the matching activation channel divided by s
    leave the product unchanged.
    """
    return np.asarray(w, dtype=np.float64) * np.asarray(s, dtype=np.float64)[None, :]


def awq_fold_activations(x, s) -> np.ndarray:
    """binary16(x * diag(1/s)): the activation side of the fold, rounded once."""
    x64 = np.asarray(x, dtype=np.float64)
    return (x64 / np.asarray(s, dtype=np.float64)[None, :]).astype(np.float16)


# --- GPTQ act order ------------------------------------------------------------

def act_order_h(xcal) -> list:
    """diag(X X^T) per input channel, exactly, as Python integers in units of 2**-48.

    ("AWQ + GPTQ Quantization, in depth", The two algorithms, compactly: the
    GPTQ Hessian is H = 2 X X^T; act order visits the columns by descending
    diag(H).  The factor 2 does not change the order and is dropped.)
    """
    X = np.asarray(xcal)
    assert X.dtype == np.float16 and X.ndim == 2
    units = (X.astype(np.float64) * 2.0**24).astype(np.int64).astype(object)
    return list((units * units).sum(axis=0))


def act_order(xcal, group_size: int):
    """GPTQ act-order group assignment.

    perm = input channels by descending diag(X X^T), ties by ascending channel
    index; the i-th channel in that order belongs to group i // group_size.
    Returns (g_idx int32 [K], perm int64 [K]).
    """
    h = act_order_h(xcal)
    K = len(h)
    perm = sorted(range(K), key=lambda k: (-h[k], k))
    g_idx = np.empty(K, dtype=np.int32)
    for i, k in enumerate(perm):
        g_idx[k] = i // group_size
    return g_idx, np.asarray(perm, dtype=np.int64)
