"""CPU oracle for the W4A16 group-quantised linear layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
bench's CPU-baseline leg may import or run anything in this package; the
product path (the C-ABI library and its Python binding) never does, and it
shares no code, table or helper with it.

What it computes, in plain numpy float64 (slow and obviously correct):

* ``rtn_quantize``   asymmetric round-to-nearest group quantiser,
                     q = round(w/S) + Z, w ~ (q - Z)*S, 4-bit codes, binary16
                     scale and 4-bit zero per group of input channels
                     ("LLM Quantization: A Deep Dive...", The Math of
                     Quantization; "LLM Quantization: INT8, GPTQ, and AWQ
                     Explained", What quantization actually does).
* ``rtn_quantize_sym`` / ``sym_zeros``
                     symmetric round-to-nearest group quantiser (absmax on the
                     4-bit grid -7..7, stored code q + 8, implicit zero point 8;
                     "INT8, GPTQ, and AWQ Explained", What quantization actually
                     does; "AWQ + GPTQ Quantization, in depth", Running it).
* ``awq_scales`` / ``awq_fold_weights`` / ``awq_fold_activations``
                     the AWQ per-input-channel scale s = mean|X|^alpha and its
                     fold W*diag(s), x*diag(1/s) ("AWQ + GPTQ Quantization, in
                     depth", The two algorithms, compactly).
* ``awq_search``     the AWQ grid search over alpha: loss of every alpha on the
                     calibration activations, best alpha (same page and section).
* ``gptq_quantize`` / ``gptq_hessian`` / ``output_error``
                     GPTQ: H = 2 X X^T with damping, the upper Cholesky factor of
                     H^-1, column-by-column rounding with error feedback onto the
                     columns not yet rounded, natural or act order; emits the
                     round-to-nearest quantiser's codes / scales / zeros / g_idx
                     (same page and section, the GPTQ half).
* ``act_order``      GPTQ act-order group assignment g_idx from the calibration
                     activations (same page and section).
* ``pack_codes`` / ``unpack_codes`` / ``pack_zeros`` / ``unpack_zeros``
                     eight 4-bit values per 32-bit word; the ``...8`` variants
                     four 8-bit values per word.  ``rtn_quantize`` and
                     ``rtn_quantize_sym`` take bits=8 for 8-bit weights ("AWQ +
                     GPTQ Quantization, in depth", 4-bit bigger or 8-bit smaller).
* ``dequant`` / ``linear``   W^ = (q - Z)*S and y = x W^T in float64.
* ``layer_bytes`` / ``bits_per_weight``   storage cost of a packed layer.

Pins (tests/test_oracle_*.py, run without a GPU): the S/2 round-trip bound,
code/zero ranges, idempotence, exact brute force with ``fractions.Fraction`` on
small tiles, hand-derived worked groups (tests/golden), the pages' storage
figures (bits per weight at group 128, the 1.5B-model byte budget), the exact
invariance of the AWQ fold, unit-vector and all-ones probes of the matmul, and
known-answer packed words.  Every function here is pinned; none is "parity
unpinned".
"""

from .quant import (round_half_even, fp16_ceil, group_index, rtn_quantize,
                    rtn_quantize_sym, sym_zeros,
                    awq_scales, awq_fold_weights, awq_fold_activations,
                    act_order_h, act_order)
from .awq_search import awq_search
from .gptq import gptq_hessian, gptq_quantize, output_error
from .packing import (pack_codes, unpack_codes, pack_zeros, unpack_zeros,
                      sorted_k_order, pack_codes_act_order,
                      pack_codes8, unpack_codes8, pack_zeros8, unpack_zeros8)
from .layer import dequant, dequant_fp16, linear, rel_err
from .storage import layer_bytes, bits_per_weight

__all__ = [
    "round_half_even", "fp16_ceil", "group_index", "rtn_quantize",
    "awq_scales", "awq_fold_weights", "awq_fold_activations", "act_order_h", "act_order",
    "pack_codes", "unpack_codes", "pack_zeros", "unpack_zeros",
    "sorted_k_order", "pack_codes_act_order",
    "dequant", "dequant_fp16", "linear", "rel_err",
    "awq_search", "gptq_hessian", "gptq_quantize", "output_error",
    "layer_bytes", "bits_per_weight",
]
