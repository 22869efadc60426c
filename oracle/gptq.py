"""GPTQ error-feedback quantiser of the oracle (test infrastructure only; see the
package header).

What it computes ("AWQ + GPTQ Quantization, in depth", The two algorithms,
compactly, the GPTQ half and its pseudocode; "How do GPTQ and AWQ differ...",
GPTQ: quantize then compensate; "LLM Quantization: INT8, GPTQ, and AWQ
Explained", GPTQ): one linear layer W (out x in) and calibration inputs X,

    H    = 2 X X^T                     (X is in x tokens; the pages' shape)
    H   += damp * mean(diag H) * I
    U    = upper Cholesky factor of H^-1   (H^-1 = U^T U)
    for every input column j, in order (or in act order):
        q      = the column rounded to the 4-bit grid of its group
        err    = (W[:, j] - q) / U[j, j]
        W[:, j+1:] -= err (outer) U[j, j+1:]
    (q in the error is the dequantised value (code - Z) * S.)

Readings of the pages fixed here (each listed in the design notes):

* grid and group parameters: the asymmetric 16-level scheme of the
  round-to-nearest quantiser (range including zero, binary16 scale rounded up,
  Z = clamp(round(-lo/S), 0, 15), round half to even), so GPTQ emits the same
  codes / scales / zeros / g_idx format;
* "scale_of_group(j)": the parameters of a group are computed once, when its
  first column is reached, from the weights as they are then: after the error
  feedback of every earlier column, before any of the group's own;
* act order: the columns are visited by descending diag(H) (exact sums of
  squares, ties by ascending channel index, as ``act_order``), H and W permuted
  to that order before H^-1 is formed; group i // group_size holds the i-th
  visited column, which is the g_idx layout of the act-order path;
* damping: ``damp`` times the mean of diag(H), added before the inverse (the
  pages give 0.01 as the typical value).

Plain float64 numpy, column by column, without the pages' blocking (blocking only
reorders the same updates).  Any group size that divides K is accepted here.
"""

from __future__ import annotations

import numpy as np

from .quant import act_order, fp16_ceil, round_half_even

LEVELS = 15


def gptq_hessian(xcal, damp: float = 0.01) -> np.ndarray:
    """H = 2 X X^T + damp * mean(diag) * I, float64 [K][K], from binary16 [T][K]
    calibration rows (X = xcal^T)."""
    X = np.asarray(xcal).astype(np.float64).T
    H = 2.0 * (X @ X.T)
    H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
    return H


def group_params(cols: np.ndarray):
    """Asymmetric 4-bit grid of one group per row, from float64 [N][g] weights:
    returns (S binary16 [N], S as float64, Z float64 [N])."""
    lo = np.minimum(cols.min(axis=1), 0.0)
    hi = np.maximum(cols.max(axis=1), 0.0)
    flat = hi == lo
    S16 = fp16_ceil(np.where(flat, 1.0, (hi - lo) / LEVELS))
    S16[flat] = np.float16(1.0)
    S = S16.astype(np.float64)
    Z = np.clip(round_half_even(-lo / S), 0, LEVELS)
    Z[flat] = 0.0
    return S16, S, Z


def gptq_quantize(w, xcal, group_size: int, use_act_order: bool = False, damp: float = 0.01,
                  return_trace: bool = False):
    """GPTQ of one layer.

    w     binary16 [N][K] weights (out x in);  xcal binary16 [T][K] calibration rows.
    Returns (codes uint8 [N][K] in the original channel order, scales binary16 [G][N],
    zeros uint8 [G][N], g_idx int32 [K] or None).  With return_trace, also
    (pre float64 [N][K], order int64 [K]): pre[:, i] is the value the i-th visited
    column had just before it was rounded.
    """
    w = np.asarray(w)
    assert w.dtype == np.float16 and w.ndim == 2
    N, K = w.shape
    assert K % group_size == 0
    G = K // group_size
    H = gptq_hessian(xcal, damp)
    if use_act_order:
        g_idx, order = act_order(xcal, group_size)
    else:
        g_idx, order = None, np.arange(K, dtype=np.int64)
    W = w.astype(np.float64)[:, order]
    Hp = H[np.ix_(order, order)]
    U = np.linalg.cholesky(np.linalg.inv(Hp)).T          # upper, H^-1 = U^T U

    codes_p = np.empty((N, K), dtype=np.uint8)
    scales = np.empty((G, N), dtype=np.float16)
    zeros = np.empty((G, N), dtype=np.uint8)
    pre = np.empty((N, K)) if return_trace else None
    S = Z = None
    for j in range(K):
        if j % group_size == 0:
            S16, S, Z = group_params(W[:, j:j + group_size])
            scales[j // group_size] = S16
            zeros[j // group_size] = Z.astype(np.uint8)
        col = W[:, j]
        if pre is not None:
            pre[:, j] = col
        q = np.clip(round_half_even(col / S) + Z, 0, LEVELS)
        deq = (q - Z) * S
        err = (col - deq) / U[j, j]
        W[:, j + 1:] -= np.outer(err, U[j, j + 1:])
        W[:, j] = deq
        codes_p[:, j] = q.astype(np.uint8)

    codes = np.empty_like(codes_p)
    codes[:, order] = codes_p
    if return_trace:
        return codes, scales, zeros, g_idx, pre, order
    return codes, scales, zeros, g_idx


def output_error(w, codes, scales, zeros, group_size: int, g_idx, xcal) -> float:
    """|| (W - W^) X ||_F / || W X ||_F on the calibration rows, float64: the layer
    output error that GPTQ lowers relative to round-to-nearest."""
    from .layer import dequant
    W = np.asarray(w).astype(np.float64)
    What = dequant(codes, scales, zeros, group_size, g_idx)
    X = np.asarray(xcal).astype(np.float64)
    return float(np.linalg.norm((W - What) @ X.T) / np.linalg.norm(W @ X.T))
