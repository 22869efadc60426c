"""Helpers shared by the GPU tests: build a layer both ways from the same seeded inputs.

The product side (``product_layer``) runs only the C-ABI library: its quantiser,
AWQ scale, act-order assignment and packing on the host, then uploads.  The oracle
side (``oracle_layer``) recomputes everything from the same seeded inputs with the
oracle alone, for a chosen subset of output rows.  Nothing flows from the product
side into the oracle side.
"""

from __future__ import annotations

import os
import sys

import numpy as np

import oracle
import w4a16_gemm_amd as w4
import workloads as wl


def note(msg: str) -> None:
    """Name the case about to run on the GPU (flushed first, in case it never returns)."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def set_knob(name: str, value) -> None:
    """Set a W4A16_* environment switch and have the library read the switches again
    (it reads them once, not per call)."""
    os.environ[name] = str(value)
    os.environ["W4A16_TUNE"] = "1"   # the library honours the switches only with this opt-in
    w4.w4a16_reload_env()


def clear_knob(*names: str) -> None:
    for name in names:
        os.environ.pop(name, None)
    w4.w4a16_reload_env()


def device():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm device")
    return torch.device("cuda:0")


def product_layer(cfg: wl.LayerConfig, M: int, x=None):
    """Quantise, pack and upload a configuration's layer with the library."""
    import torch
    dev = device()
    g = cfg.group_size
    g_idx = s = None
    if cfg.act_order or cfg.awq:
        X = wl.calibration(cfg)
        if cfg.act_order:
            g_idx = w4.w4a16_act_order(X, g)
        if cfg.awq:
            s = w4.w4a16_awq_scales(X)
    w = wl.weights(cfg)
    eight = cfg.bits == 8
    if cfg.sym:
        codes, S = (w4.w8a16_quantize_sym if eight else w4.w4a16_quantize_sym)(w, g, g_idx, s)
        Z = None
    else:
        codes, S, Z = (w4.w8a16_quantize if eight else w4.w4a16_quantize)(w, g, g_idx, s)
    if x is None:
        x = wl.activations(cfg, M)
        if s is not None:
            x = w4.w4a16_awq_fold_activations(x, s)
    layer = {
        "cfg": cfg, "M": M, "codes": codes, "g_idx_np": g_idx,
        "x": torch.from_numpy(np.ascontiguousarray(x)).to(dev),
        "qweight": torch.from_numpy((w4.w8a16_pack if eight else w4.w4a16_pack)(codes, g_idx, g)).to(dev),
        "scales": torch.from_numpy(S).to(dev),
        "qzeros": None if Z is None else torch.from_numpy(
            (w4.w8a16_pack_zeros if eight else w4.w4a16_pack_zeros)(Z)).to(dev),
        "g_idx": None if g_idx is None else torch.from_numpy(g_idx).to(dev),
    }
    return layer


def oracle_layer(cfg: wl.LayerConfig, M: int, rows, x=None):
    """Oracle codes/scales/zeros for `rows` and the float64 reference y[:, rows]."""
    g = cfg.group_size
    g_idx = s = None
    if cfg.act_order or cfg.awq:
        X = wl.calibration(cfg)
        if cfg.act_order:
            g_idx, _ = oracle.act_order(X, g)
        if cfg.awq:
            s = oracle.awq_scales(X)
    w = wl.weights(cfg, rows)
    if cfg.sym:
        codes, S = oracle.rtn_quantize_sym(w, g, g_idx, s, bits=cfg.bits)
        Z = oracle.sym_zeros(S.shape[0], S.shape[1], bits=cfg.bits)
    else:
        codes, S, Z = oracle.rtn_quantize(w, g, g_idx, s, bits=cfg.bits)
    if x is None:
        x = wl.activations(cfg, M)
        if s is not None:
            x = oracle.awq_fold_activations(x, s)
    y_ref = oracle.linear(x, codes, S, Z, g, g_idx)
    return {"codes": codes, "scales": S, "zeros": Z, "g_idx": g_idx, "x": x, "y_ref": y_ref,
            "W16": oracle.dequant_fp16(codes, S, Z, g, g_idx)}


def run_gemm(layer, x=None, y=None):
    import torch
    gemm = w4.w8a16_gemm if layer["cfg"].bits == 8 else w4.w4a16_gemm
    out = gemm(layer["x"] if x is None else x, layer["qweight"], layer["scales"], layer["qzeros"],
               layer["g_idx"], layer["cfg"].group_size, y=y)
    torch.cuda.synchronize()
    return out


# The library's weight words keep element e of a word in nibble NIBBLE_OF[e] (its
# private word layout); the oracle's unpacking reads nibble j as element j.
NIBBLE_OF = np.array([0, 4, 1, 5, 2, 6, 3, 7])


def codes_of_library_words(words) -> np.ndarray:
    """Codes u8 [rows][K] held by library weight words int32 [rows][K/8] (contiguous
    groups), decoded with the oracle's unpacking and the layout's nibble order."""
    nat = oracle.unpack_codes(words)
    return np.ascontiguousarray(nat.reshape(nat.shape[0], -1, 8)[:, :, NIBBLE_OF].reshape(nat.shape))


def sample_rows(N: int, count: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng([31, N, seed])
    rows = set(rng.choice(N, size=min(count, N), replace=False).tolist())
    rows.update({0, N - 1})
    return np.array(sorted(rows), dtype=np.int64)
