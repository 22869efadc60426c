"""The layer itself: dequantisation and the float64 matmul (test infrastructure only).

"AWQ + GPTQ Quantization, in depth", What W4A16 buys: the kernel expands the
packed 4-bit weights to 16 bits with the group's scale and zero point and
multiplies them with 16-bit activations; the arithmetic is the ordinary matmul.
"A Deep Dive", The Math of Quantization: x_approx = (q - Z)*S.

y = x W^T with W (out x in) as in "in depth", The two algorithms, compactly.
"""

from __future__ import annotations

import numpy as np

from .quant import group_index


def dequant(codes, scales, zeros, group_size: int, g_idx=None) -> np.ndarray:
    """W^[n][k] = (q[n][k] - Z[g(k)][n]) * S[g(k)][n] in float64 (exact: a small
    integer times a binary16 value)."""
    q = np.asarray(codes, dtype=np.float64)
    N, K = q.shape
    gid = group_index(K, group_size, g_idx)
    S = np.asarray(scales, dtype=np.float64)[gid, :].T          # [N][K]
    Z = np.asarray(zeros, dtype=np.float64)[gid, :].T           # [N][K]
    return (q - Z) * S


def dequant_fp16(codes, scales, zeros, group_size: int, g_idx=None) -> np.ndarray:
    """binary16(W^), rounded once to nearest even."""
    return dequant(codes, scales, zeros, group_size, g_idx).astype(np.float16)


def linear(x, codes, scales, zeros, group_size: int, g_idx=None) -> np.ndarray:
    """y = x W^T in float64 for binary16 x [M][K]; returns float64 [M][N]."""
    W = dequant(codes, scales, zeros, group_size, g_idx)
    return np.asarray(x, dtype=np.float64) @ W.T


def rel_err(y, y_ref) -> float:
    """max |y - y_ref| / rms(y_ref), the output parity measure."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = np.sqrt(np.mean(y_ref * y_ref))
    if rms == 0.0:
        return float(np.max(np.abs(y - y_ref), initial=0.0))
    return float(np.max(np.abs(y - y_ref), initial=0.0) / rms)
