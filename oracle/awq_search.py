"""AWQ scale search of the oracle (test infrastructure only; see package header).

"AWQ + GPTQ Quantization, in depth", The two algorithms, compactly: for each alpha
on a grid in [0, 1] the per-input-channel scale is s = (mean over the calibration
tokens of |X|) ** alpha; the weights are quantised as W * diag(s), the scale is
divided back out of the layer (folded into the operation feeding it), and the loss
is the norm of the difference between the layer's outputs before and after; the
alpha with the smallest loss wins.

Readings fixed here: the loss is measured on the calibration activations
themselves; the layer after quantisation is the one the kernel runs, i.e. the
activations divided by s and rounded once to binary16 (awq_fold_activations) times
the dequantised codes of W * diag(s); the norm is the Frobenius norm over all
tokens and outputs; ties go to the first alpha of the grid.
"""

from __future__ import annotations

import numpy as np

from .layer import linear
from .quant import awq_fold_activations, awq_scales, rtn_quantize


def awq_search(w, xcal, group_size: int, alphas):
    """Loss of every alpha and the index of the best one.

    w binary16 [N][K] (out x in), xcal binary16 [T][K].  Returns (losses float64
    [len(alphas)], best int).  For each alpha:
        s      = awq_scales(xcal, alpha)
        codes  = rtn_quantize(w, group_size, in_scale=s)
        y      = binary16(xcal / s) @ dequant(codes)^T          (float64)
        loss   = || xcal @ w^T - y ||_F
    """
    w = np.asarray(w)
    X = np.asarray(xcal)
    y_ref = X.astype(np.float64) @ w.astype(np.float64).T
    losses = np.empty(len(alphas), dtype=np.float64)
    for i, a in enumerate(alphas):
        s = awq_scales(X, float(a))
        codes, S, Z = rtn_quantize(w, group_size, None, s)
        y = linear(awq_fold_activations(X, s), codes, S, Z, group_size)
        losses[i] = np.sqrt(np.sum((y_ref - y) ** 2))
    return losses, int(np.argmin(losses))
