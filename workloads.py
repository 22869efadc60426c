"""Seeded synthetic workloads for the W4A16 group-quantised linear layer.

This module only draws numbers.  It holds the shapes and value distributions of
the layer configurations and the seeded generators for weights, activations and
calibration activations; no quantisation, scaling, ordering, packing or product
step of the method lives here.  Both the CPU oracle (through the tests) and the
GPU path (through the tests and the bench) take their inputs from it, and from
nowhere else.

Distributions (all drawn in float64, then cast once to binary16 with
round-to-nearest-even):

* weights  W[n][k] ~ N(0, w_std^2)
* activations x[m][k] ~ N(0, 1), except a fixed set of "outlier" input channels
  whose values are multiplied by ``outlier_mult``.  The outlier channels are a
  property of the channel, not of the token (the pages describe a few input
  channels whose activations are orders of magnitude larger than the rest), so
  the activations and the calibration activations of one configuration share
  them.
* calibration activations X_cal[t][k]: same distribution as x, T = 512 tokens
  (the pages' recipes use a few hundred 512-token calibration samples; synthetic
  tokens stand in for that text here).

Seeds: every stream is ``numpy.random.default_rng([0, cfg_id, stream, *sub])``
with stream 0 = weights (one sub-stream per block of 64 rows, so any row subset
can be drawn without drawing the whole matrix), 1 = activations,
2 = outlier channel indices, 3 = calibration activations.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

ROW_BLOCK = 64          # rows per weight sub-stream
CALIB_TOKENS = 512


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    K: int                      # input features (reduction dimension)
    N: int                      # output features
    group_size: int
    w_std: float
    outlier_frac: float
    outlier_mult: float
    M_list: tuple = (1,)        # batch sizes run on this layer
    awq: bool = False           # calibration-derived per-input-channel scale folded in
    act_order: bool = False     # calibration-derived input-channel ordering (g_idx)
    note: str = ""
    sym: bool = False           # symmetric quantisation (no zero points)
    bits: int = 4               # weight bits: 4 or 8

    @property
    def n_outliers(self) -> int:
        return max(1, int(round(self.outlier_frac * self.K)))

    @property
    def G(self) -> int:
        return self.K // self.group_size


CONFIGS = {
    "c1": LayerConfig("c1", 1, K=512, N=512, group_size=128, w_std=0.02,
                      outlier_frac=0.005, outlier_mult=20.0, M_list=(1,),
                      note="single small layer, M=1"),
    "c2up": LayerConfig("c2up", 21, K=3072, N=8192, group_size=128, w_std=0.02,
                        outlier_frac=0.01, outlier_mult=20.0, M_list=(1,), awq=True,
                        note="1-4B-class MLP up-projection decode, AWQ-folded"),
    "c2down": LayerConfig("c2down", 22, K=8192, N=3072, group_size=128, w_std=0.02,
                          outlier_frac=0.01, outlier_mult=20.0, M_list=(1,), awq=True,
                          note="1-4B-class MLP down-projection decode, AWQ-folded"),
    "c3": LayerConfig("c3", 3, K=8192, N=28672, group_size=128, w_std=0.015,
                      outlier_frac=0.001, outlier_mult=50.0, M_list=(1, 2, 4, 8, 16),
                      note="70B-class MLP up-projection decode, batch sweep"),
    "c4": LayerConfig("c4", 4, K=4096, N=14336, group_size=128, w_std=0.02,
                      outlier_frac=0.005, outlier_mult=20.0, M_list=(2048,),
                      note="prefill GEMM"),
    "c5": LayerConfig("c5", 5, K=4096, N=11008, group_size=32, w_std=0.02,
                      outlier_frac=0.005, outlier_mult=20.0, M_list=(1, 512), act_order=True,
                      note="act-order layout, group 32"),
}


# Variants of the configurations above (same weights and activations): the 70B-class
# decode layer quantised symmetrically, the scheme of the GPTQ recipe ("AWQ + GPTQ
# Quantization, in depth", Running it), without stored zero points.
VARIANTS = {
    "c3s": replace(CONFIGS["c3"], name="c3s", sym=True,
                   note="70B-class MLP up-projection, symmetric int4 (no zero points), decode"),
    # the same layer with 8-bit weights ("in depth", 4-bit bigger or 8-bit smaller)
    "c3w8": replace(CONFIGS["c3"], name="c3w8", bits=8,
                    note="70B-class MLP up-projection, asymmetric 8-bit weights, decode"),
    "c4w8": replace(CONFIGS["c4"], name="c4w8", bits=8,
                    note="prefill GEMM, asymmetric 8-bit weights"),
}


def config(name: str) -> LayerConfig:
    """A configuration or a variant by name."""
    return CONFIGS[name] if name in CONFIGS else VARIANTS[name]


def custom_config(name: str, cfg_id: int, K: int, N: int, group_size: int, *,
                  w_std: float = 0.02, outlier_frac: float = 0.005,
                  outlier_mult: float = 20.0, M_list=(1,), awq=False, act_order=False,
                  sym=False, bits=4) -> LayerConfig:
    """A layer of arbitrary shape with the same distributions (used for small
    parity cases that span several tiles and a ragged tail)."""
    return LayerConfig(name, cfg_id, K=K, N=N, group_size=group_size, w_std=w_std,
                       outlier_frac=outlier_frac, outlier_mult=outlier_mult,
                       M_list=tuple(M_list), awq=awq, act_order=act_order, sym=sym, bits=bits)


def _rng(cfg: LayerConfig, stream: int, *sub: int) -> np.random.Generator:
    return np.random.default_rng([0, cfg.cfg_id, stream, *sub])


def weights(cfg: LayerConfig, rows=None) -> np.ndarray:
    """binary16 weights [len(rows)][K] ("out x in"); rows defaults to all N rows.

    Row r is drawn from the sub-stream of its 64-row block, so ``weights(cfg,
    rows)`` equals ``weights(cfg)[rows]`` for any row subset.
    """
    if rows is None:
        rows = np.arange(cfg.N)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, cfg.K), dtype=np.float16)
    blocks = np.unique(rows // ROW_BLOCK)
    for b in blocks:
        lo = int(b) * ROW_BLOCK
        nb = min(ROW_BLOCK, cfg.N - lo)
        blk = _rng(cfg, 0, int(b)).standard_normal((ROW_BLOCK, cfg.K))[:nb] * cfg.w_std
        sel = np.nonzero(rows // ROW_BLOCK == b)[0]
        out[sel] = blk[rows[sel] - lo].astype(np.float16)
    return out


def outlier_channels(cfg: LayerConfig) -> np.ndarray:
    """Sorted indices of the outlier input channels (drawn without replacement)."""
    idx = _rng(cfg, 2).choice(cfg.K, size=cfg.n_outliers, replace=False)
    return np.sort(idx)


def _act(cfg: LayerConfig, rng: np.random.Generator, rows: int) -> np.ndarray:
    a = rng.standard_normal((rows, cfg.K))
    a[:, outlier_channels(cfg)] *= cfg.outlier_mult
    return a.astype(np.float16)


def activations(cfg: LayerConfig, M: int | None = None) -> np.ndarray:
    """binary16 activations [M][K]; the first M rows of the configuration's
    largest batch, so smaller batches are prefixes of larger ones."""
    Mmax = max(cfg.M_list)
    M = Mmax if M is None else M
    x = _act(cfg, _rng(cfg, 1), max(Mmax, M))
    return np.ascontiguousarray(x[:M])


def calibration(cfg: LayerConfig, T: int = CALIB_TOKENS) -> np.ndarray:
    """binary16 calibration activations [T][K]."""
    return _act(cfg, _rng(cfg, 3), T)


def unit_vectors(K: int, ks) -> np.ndarray:
    """binary16 rows e_k (one row per k in ks): probes that select one weight column."""
    ks = np.asarray(ks)
    e = np.zeros((ks.size, K), dtype=np.float16)
    e[np.arange(ks.size), ks] = 1.0
    return e


def random_codes(N: int, K: int, seed: int) -> np.ndarray:
    """Uniform 4-bit codes u8 [N][K] for packing tests."""
    return np.random.default_rng([1, seed]).integers(0, 16, size=(N, K), dtype=np.uint8)


def random_words(rows: int, cols: int, seed: int) -> np.ndarray:
    """Uniform 32-bit words int32 [rows][cols]: eight independent uniform 4-bit values
    per word whatever the nibble order, i.e. a packed matrix of uniform codes (or
    zero points) drawn without packing anything.  Used for layers too large to
    quantise on the host."""
    w = np.random.default_rng([2, seed]).integers(0, 1 << 32, size=(rows, cols), dtype=np.uint32)
    return w.view(np.int32)


def random_scales(G: int, N: int, seed: int, lo: float = 0.002, hi: float = 0.01) -> np.ndarray:
    """binary16 scales [G][N], uniform in [lo, hi)."""
    return np.random.default_rng([3, seed]).uniform(lo, hi, size=(G, N)).astype(np.float16)


def random_activations(M: int, K: int, seed: int) -> np.ndarray:
    """binary16 activations [M][K] ~ N(0, 1)."""
    return np.random.default_rng([4, seed]).standard_normal((M, K)).astype(np.float16)


# --- a whole decode step of a small model -----------------------------------------

@dataclass(frozen=True)
class DecodeStep:
    """The quantised linear layers one decode token at batch one runs through, in
    call order, and the unquantised output head."""
    name: str
    layers: int
    linears: tuple              # (name, K, N) per transformer layer, in call order
    head: tuple                 # (K, N) of the output head, kept in 16-bit floats
    group_size: int
    note: str


# "AWQ + GPTQ Quantization, in depth", Worked example: where the bytes go in a 1.5B
# model: 28 layers, hidden size 1536, MLP width 8960, 12 query and 2 key-value heads of
# dimension 128 (so q, k, v project 1536 -> 1536 + 256 + 256 = 2048 and o 1536 ->
# 1536), vocabulary 151,936 with the head tied to the embedding and kept unquantised;
# linear layers at group size 128.  Gate and up read the same input and run as one
# 1536 -> 2 x 8960 layer.
DECODE_1P5B = DecodeStep(
    "1p5b", 28,
    (("qkv", 1536, 2048), ("o", 1536, 1536), ("gate_up", 1536, 17920), ("down", 8960, 1536)),
    (1536, 151936), 128,
    "1.5B-class model, one decode token at batch one: 28 x (qkv, o, gate+up, down) W4A16 layers")


def decode_step_configs(step: DecodeStep = DECODE_1P5B) -> list:
    """One layer configuration per linear shape of the step (seeded like the others),
    for parity checks of those shapes."""
    return [custom_config(f"{step.name}_{name}", 300 + i, K=K, N=N, group_size=step.group_size)
            for i, (name, K, N) in enumerate(step.linears)]
