"""Storage cost of a packed W4A16 layer (test infrastructure only).

"AWQ + GPTQ Quantization, in depth", What W4A16 buys: a 16-bit scale per 128
weights adds 0.125 bit per weight and a 4-bit zero point about 0.03 more.  The
byte counts are measured from the buffers the reference packing produces, not
written down as a formula.
"""

from __future__ import annotations

import numpy as np

from .packing import pack_codes, pack_zeros, pack_codes_act_order


def layer_bytes(N: int, K: int, group_size: int, act_order: bool = False) -> int:
    """Bytes of the packed weights, binary16 scales and packed zeros of one layer."""
    G = K // group_size
    codes = np.zeros((N, K), dtype=np.uint8)
    if act_order:
        g_idx = np.arange(K) // group_size
        qweight = pack_codes_act_order(codes, g_idx)
    else:
        qweight = pack_codes(codes)
    scales = np.zeros((G, N), dtype=np.float16)
    qzeros = pack_zeros(np.zeros((G, N), dtype=np.uint8))
    return int(qweight.nbytes + scales.nbytes + qzeros.nbytes)


def bits_per_weight(N: int, K: int, group_size: int, act_order: bool = False) -> float:
    return 8.0 * layer_bytes(N, K, group_size, act_order) / (N * K)
