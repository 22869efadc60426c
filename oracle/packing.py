"""Reference packing of 4-bit values, eight per 32-bit word (test infrastructure only).

"AWQ + GPTQ Quantization, in depth", What W4A16 buys: the kernel loads packed
4-bit weights.  The word layout is this project's convention: nibble j
(bits 4j..4j+3) of word w holds element 8w + j of the packed axis.

* weights: codes [N][K] -> int32 [N][K/8], packed along the input axis k.
* zero points: zeros [G][N] -> int32 [G][N/8], packed along the output axis n.
* act order: a row's codes are stored in group-sorted input order (the order of
  the stable sort of k by g_idx[k]), and that order, perm, follows the words.
"""

from __future__ import annotations

import numpy as np


def _pack_last_axis(vals: np.ndarray) -> np.ndarray:
    v = np.asarray(vals)
    assert v.ndim == 2 and v.shape[1] % 8 == 0
    assert v.min(initial=0) >= 0 and v.max(initial=0) <= 15
    u = v.astype(np.uint64).reshape(v.shape[0], v.shape[1] // 8, 8)
    words = np.zeros(u.shape[:2], dtype=np.uint64)
    for j in range(8):
        words |= u[:, :, j] << np.uint64(4 * j)
    return words.astype(np.uint32).view(np.int32)


def _unpack_last_axis(words: np.ndarray) -> np.ndarray:
    w = np.asarray(words).view(np.uint32).astype(np.uint64)
    out = np.empty((w.shape[0], w.shape[1], 8), dtype=np.uint8)
    for j in range(8):
        out[:, :, j] = ((w >> np.uint64(4 * j)) & np.uint64(0xF)).astype(np.uint8)
    return out.reshape(w.shape[0], w.shape[1] * 8)


def pack_codes(codes) -> np.ndarray:
    """codes uint8 [N][K] (0..15) -> int32 [N][K/8]."""
    return _pack_last_axis(codes)


def unpack_codes(qweight) -> np.ndarray:
    """int32 [N][K/8] -> codes uint8 [N][K]."""
    return _unpack_last_axis(qweight)


def pack_zeros(zeros) -> np.ndarray:
    """zeros uint8 [G][N] (0..15) -> int32 [G][N/8]."""
    return _pack_last_axis(zeros)


def unpack_zeros(qzeros) -> np.ndarray:
    """int32 [G][N/8] -> zeros uint8 [G][N]."""
    return _unpack_last_axis(qzeros)


def sorted_k_order(g_idx) -> np.ndarray:
    """perm[p] = input channel stored at position p: the stable sort of k by g_idx[k]."""
    g = np.asarray(g_idx, dtype=np.int64)
    return np.array(sorted(range(g.size), key=lambda k: (g[k], k)), dtype=np.int64)


def pack_codes_act_order(codes, g_idx) -> np.ndarray:
    """Act-order packing: words of the group-sorted codes, then perm as int32.

    Returns int32 [N*K/8 + K]: row n's words are codes[n, perm] packed as above,
    and the last K entries are perm.
    """
    perm = sorted_k_order(g_idx)
    c = np.asarray(codes)[:, perm]
    return np.concatenate([pack_codes(c).reshape(-1), perm.astype(np.int32)])


# --- 8-bit weights: four 8-bit values per 32-bit word ------------------------------
# byte j (bits 8j..8j+7) of word w holds element 4w + j of the packed axis.

def _pack4_last_axis(vals: np.ndarray) -> np.ndarray:
    v = np.asarray(vals)
    assert v.ndim == 2 and v.shape[1] % 4 == 0
    assert v.min(initial=0) >= 0 and v.max(initial=0) <= 255
    u = v.astype(np.uint64).reshape(v.shape[0], v.shape[1] // 4, 4)
    words = np.zeros(u.shape[:2], dtype=np.uint64)
    for j in range(4):
        words |= u[:, :, j] << np.uint64(8 * j)
    return words.astype(np.uint32).view(np.int32)


def _unpack4_last_axis(words: np.ndarray) -> np.ndarray:
    w = np.asarray(words).view(np.uint32).astype(np.uint64)
    out = np.empty((w.shape[0], w.shape[1], 4), dtype=np.uint8)
    for j in range(4):
        out[:, :, j] = ((w >> np.uint64(8 * j)) & np.uint64(0xFF)).astype(np.uint8)
    return out.reshape(w.shape[0], w.shape[1] * 4)


def pack_codes8(codes) -> np.ndarray:
    """8-bit codes uint8 [N][K] -> int32 [N][K/4]."""
    return _pack4_last_axis(codes)


def unpack_codes8(qweight) -> np.ndarray:
    """int32 [N][K/4] -> 8-bit codes uint8 [N][K]."""
    return _unpack4_last_axis(qweight)


def pack_zeros8(zeros) -> np.ndarray:
    """8-bit zeros uint8 [G][N] -> int32 [G][N/4]."""
    return _pack4_last_axis(zeros)


def unpack_zeros8(qzeros) -> np.ndarray:
    """int32 [G][N/4] -> 8-bit zeros uint8 [G][N]."""
    return _unpack4_last_axis(qzeros)

