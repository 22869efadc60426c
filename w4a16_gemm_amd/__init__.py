"""Python binding of the W4A16 C-ABI library (include/w4a16.h).

Argument marshalling only: every function here checks dtypes and shapes, hands raw
pointers and sizes to the function of the same name in libw4a16.so and turns a
non-zero status into ``W4A16Error``.  Host entry points take and return numpy
arrays; device entry points take torch tensors that live on a ROCm device (torch
provides the memory and the stream, nothing else).  There is no fallback: if the
library is not built, the first call raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a16.so")

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int

_SIGNATURES = {
    "w4a16_abi_version": (_c_int, []),
    "w4a16_last_error": (ctypes.c_char_p, []),
    "w4a16_qweight_words": (ctypes.c_size_t, [_c_int, _c_int, _c_int]),
    "w4a16_quantize": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                _c_void_p, _c_void_p, _c_void_p]),
    "w4a16_quantize_sym": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                    _c_void_p, _c_void_p]),
    "w4a16_awq_scales": (_c_int, [_c_void_p, _c_int, _c_int, ctypes.c_double, _c_void_p]),
    "w4a16_awq_fold_activations": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p, _c_void_p]),
    "w4a16_act_order": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p]),
    "w4a16_pack": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p]),
    "w4a16_unpack": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p]),
    "w4a16_pack_zeros": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p]),
    "w4a16_unpack_zeros": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p]),
    "w4a16_gemm": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                            _c_int, _c_int, _c_int, _c_void_p, _c_void_p]),
    "w4a16_dequant": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                               _c_int, _c_void_p, _c_void_p]),
    "w4a16_reload_env": (_c_int, []),
    "w4a16_gemm_noalloc": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                                    _c_int, _c_int, _c_int, _c_void_p, _c_void_p]),
    "w4a16_quantize_device": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_int, _c_void_p,
                                       _c_void_p, _c_void_p, _c_void_p]),
    "w4a16_awq_search": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_void_p,
                                  _c_int, _c_void_p, _c_void_p, _c_void_p]),
    "w4a16_gptq": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_int, _c_int, ctypes.c_double,
                            _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "w8a16_qweight_words": (ctypes.c_size_t, [_c_int, _c_int, _c_int]),
    "w8a16_quantize": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                _c_void_p, _c_void_p, _c_void_p]),
    "w8a16_quantize_sym": (_c_int, [_c_void_p, _c_int, _c_int, _c_int, _c_void_p, _c_void_p,
                                    _c_void_p, _c_void_p]),
    "w8a16_pack": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p]),
    "w8a16_unpack": (_c_int, [_c_void_p, _c_void_p, _c_int, _c_int, _c_int, _c_void_p]),
    "w8a16_pack_zeros": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p]),
    "w8a16_unpack_zeros": (_c_int, [_c_void_p, _c_int, _c_int, _c_void_p]),
    "w8a16_gemm": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int,
                            _c_int, _c_int, _c_int, _c_void_p, _c_void_p]),
    "w8a16_dequant": (_c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_int, _c_int,
                               _c_int, _c_void_p, _c_void_p]),
}
EXPORTS = tuple(_SIGNATURES)

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_BAD_GIDX, ERR_MISALIGNED, ERR_HIP = range(6)

_lib = None


class W4A16Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"w4a16 status {status}: {message}")
        self.status = status


def load_runtime_first() -> None:
    """Load PyTorch (and with it the HIP runtime it ships) before a library of this
    package: the library's dependency on the HIP runtime then resolves to that same,
    already loaded runtime, so the device pointers and streams torch hands over belong
    to the runtime the library launches on.  Loaded the other way round, the process
    holds two HIP runtimes, and the library's launches fail ("no ROCm-capable device")."""
    import torch  # noqa: F401


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m w4a16_gemm_amd.build` (or __graft_entry__.build())")
        load_runtime_first()
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int) -> None:
    if status != OK:
        raise W4A16Error(status, lib().w4a16_last_error().decode())


def _np(a, dtype, ndim=None) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=dtype)
    if ndim is not None and a.ndim != ndim:
        raise ValueError(f"expected {ndim}-d array, got shape {a.shape}")
    return a


def _ptr(a) -> int | None:
    return None if a is None else a.ctypes.data


# --- host entry points (numpy) ----------------------------------------------------

def w4a16_abi_version() -> int:
    return lib().w4a16_abi_version()


def w4a16_qweight_words(N: int, K: int, act_order: bool) -> int:
    return int(lib().w4a16_qweight_words(N, K, int(bool(act_order))))


def w4a16_quantize(w, group_size: int, g_idx=None, in_scale=None):
    """binary16 w [N][K] -> (codes uint8 [N][K], scales binary16 [G][N], zeros uint8 [G][N])."""
    w = _np(w, np.float16, 2)
    N, K = w.shape
    G = K // group_size if group_size else 0
    gi = None if g_idx is None else _np(g_idx, np.int32, 1)
    sc = None if in_scale is None else _np(in_scale, np.float64, 1)
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((max(G, 1), N), np.float16)
    zeros = np.empty((max(G, 1), N), np.uint8)
    _check(lib().w4a16_quantize(_ptr(w), N, K, group_size, _ptr(gi), _ptr(sc), _ptr(codes),
                                _ptr(scales), _ptr(zeros)))
    return codes, scales, zeros


def w4a16_quantize_sym(w, group_size: int, g_idx=None, in_scale=None):
    """Symmetric: binary16 w [N][K] -> (codes uint8 [N][K] in 1..15, scales binary16
    [G][N]); the zero point is 8 everywhere (pass qzeros=None to the device calls)."""
    w = _np(w, np.float16, 2)
    N, K = w.shape
    G = K // group_size if group_size else 0
    gi = None if g_idx is None else _np(g_idx, np.int32, 1)
    sc = None if in_scale is None else _np(in_scale, np.float64, 1)
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((max(G, 1), N), np.float16)
    _check(lib().w4a16_quantize_sym(_ptr(w), N, K, group_size, _ptr(gi), _ptr(sc), _ptr(codes), _ptr(scales)))
    return codes, scales


def w4a16_awq_scales(xcal, alpha: float = 0.5) -> np.ndarray:
    xcal = _np(xcal, np.float16, 2)
    T, K = xcal.shape
    s = np.empty(K, np.float64)
    _check(lib().w4a16_awq_scales(_ptr(xcal), T, K, float(alpha), _ptr(s)))
    return s


def w4a16_awq_fold_activations(x, s) -> np.ndarray:
    x = _np(x, np.float16, 2)
    s = _np(s, np.float64, 1)
    out = np.empty_like(x)
    _check(lib().w4a16_awq_fold_activations(_ptr(x), x.shape[0], x.shape[1], _ptr(s), _ptr(out)))
    return out


def w4a16_act_order(xcal, group_size: int) -> np.ndarray:
    xcal = _np(xcal, np.float16, 2)
    T, K = xcal.shape
    g_idx = np.empty(K, np.int32)
    _check(lib().w4a16_act_order(_ptr(xcal), T, K, group_size, _ptr(g_idx)))
    return g_idx


def w4a16_pack(codes, g_idx, group_size: int) -> np.ndarray:
    codes = _np(codes, np.uint8, 2)
    N, K = codes.shape
    gi = None if g_idx is None else _np(g_idx, np.int32, 1)
    out = np.empty(max(w4a16_qweight_words(N, K, gi is not None), 1), np.int32)
    _check(lib().w4a16_pack(_ptr(codes), _ptr(gi), group_size, N, K, _ptr(out)))
    return out


def w4a16_unpack(qweight, g_idx, group_size: int, N: int, K: int) -> np.ndarray:
    qweight = _np(qweight, np.int32).reshape(-1)
    gi = None if g_idx is None else _np(g_idx, np.int32, 1)
    if qweight.size < w4a16_qweight_words(N, K, gi is not None):
        raise ValueError("qweight is smaller than the packed size of an N x K layer")
    codes = np.empty((N, K), np.uint8)
    _check(lib().w4a16_unpack(_ptr(qweight), _ptr(gi), group_size, N, K, _ptr(codes)))
    return codes


def w4a16_pack_zeros(zeros) -> np.ndarray:
    zeros = _np(zeros, np.uint8, 2)
    G, N = zeros.shape
    out = np.empty((G, max(N // 8, 1)), np.int32)
    _check(lib().w4a16_pack_zeros(_ptr(zeros), G, N, _ptr(out)))
    return out


def w4a16_unpack_zeros(qzeros, G: int, N: int) -> np.ndarray:
    qzeros = _np(qzeros, np.int32, 2)
    if qzeros.shape != (G, N // 8):
        raise ValueError(f"qzeros shape {qzeros.shape} != {(G, N // 8)}")
    out = np.empty((G, N), np.uint8)
    _check(lib().w4a16_unpack_zeros(_ptr(qzeros), G, N, _ptr(out)))
    return out


# --- device entry points (torch tensors on a ROCm device) --------------------------

def w4a16_reload_env() -> None:
    """Re-read the W4A16_* environment switches (the library reads them once)."""
    _check(lib().w4a16_reload_env())


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous {dtype} tensor")
    if not t.is_cuda:
        raise TypeError(f"{name} must live on a ROCm device")
    return t


def _shape(t, shape, name):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _layer_shapes(qweight, scales, qzeros, g_idx, group_size: int, K: int, bits: int):
    """Check every weight-side tensor against the layer (N from scales, K given) before
    anything is launched, so that a mis-shaped tensor is refused instead of read past
    its end.  Returns N."""
    import torch
    for t, dt, name in ((qweight, torch.int32, "qweight"), (scales, torch.float16, "scales"),
                        (qzeros, torch.int32, "qzeros"), (g_idx, torch.int32, "g_idx")):
        if t is not None and (not isinstance(t, torch.Tensor) or t.dtype != dt):
            raise TypeError(f"{name} must be a {dt} tensor")
    if scales.dim() != 2:
        raise ValueError(f"scales must be [G][N], got shape {tuple(scales.shape)}")
    G, N = scales.shape
    if group_size <= 0 or K <= 0 or K % group_size != 0:
        raise ValueError(f"K={K} is not a positive multiple of group_size={group_size}")
    _shape(scales, (K // group_size, N), "scales")
    if qzeros is not None:
        _shape(qzeros, (G, N // (32 // bits)), "qzeros")
    if g_idx is not None:
        _shape(g_idx, (K,), "g_idx")
    words = (w4a16_qweight_words if bits == 4 else w8a16_qweight_words)(N, K, g_idx is not None)
    if words == 0 or qweight.numel() < words:
        raise ValueError(f"qweight has {qweight.numel()} words, the packed {N} x {K} layer needs {words}")
    return N


def _layer_call(fn, x, qweight, scales, qzeros, g_idx, group_size, y, stream, bits):
    import torch
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-d tensor [M][K]")
    M, K = x.shape
    N = _layer_shapes(qweight, scales, qzeros, g_idx, group_size, K, bits)
    if y is not None:
        _shape(y, (M, N), "y")
    _dev(x, torch.float16, "x")
    _dev(qweight, torch.int32, "qweight")
    _dev(scales, torch.float16, "scales")
    if qzeros is not None:                      # None: symmetric weights
        _dev(qzeros, torch.int32, "qzeros")
    if g_idx is not None:
        _dev(g_idx, torch.int32, "g_idx")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float16, device=x.device)
    _dev(y, torch.float16, "y")
    _check(fn(x.data_ptr(), qweight.data_ptr(), scales.data_ptr(),
              None if qzeros is None else qzeros.data_ptr(),
              None if g_idx is None else g_idx.data_ptr(), group_size, M, N, K,
              y.data_ptr(), _stream_handle(stream, x.device)))
    return y


def _dequant_call(fn, qweight, scales, qzeros, g_idx, group_size, K, out, stream, bits):
    import torch
    N = _layer_shapes(qweight, scales, qzeros, g_idx, group_size, K, bits)
    if out is not None:
        _shape(out, (N, K), "out")
    _dev(qweight, torch.int32, "qweight")
    _dev(scales, torch.float16, "scales")
    if qzeros is not None:
        _dev(qzeros, torch.int32, "qzeros")
    if g_idx is not None:
        _dev(g_idx, torch.int32, "g_idx")
    if out is None:
        out = torch.empty((N, K), dtype=torch.float16, device=qweight.device)
    _dev(out, torch.float16, "out")
    _check(fn(qweight.data_ptr(), scales.data_ptr(), None if qzeros is None else qzeros.data_ptr(),
              None if g_idx is None else g_idx.data_ptr(), group_size, N, K,
              out.data_ptr(), _stream_handle(stream, qweight.device)))
    return out


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def w4a16_gemm(x, qweight, scales, qzeros, g_idx, group_size: int, y=None, stream=None):
    """y = x W^T on the device.  x binary16 [M][K]; scales binary16 [G][N];
    qzeros int32 [G][N/8] or None (symmetric); qweight int32 from w4a16_pack; g_idx int32
    [K] or None.  Returns y binary16 [M][N] (allocated unless given)."""
    return _layer_call(lib().w4a16_gemm, x, qweight, scales, qzeros, g_idx, group_size, y, stream, 4)


def w4a16_gemm_noalloc(x, qweight, scales, qzeros, g_idx, group_size: int, y, stream=None):
    """w4a16_gemm with scratch from the library's fixed per-GPU array: allocates no
    device memory (y must be given)."""
    if y is None:
        raise ValueError("w4a16_gemm_noalloc needs the output tensor y")
    return _layer_call(lib().w4a16_gemm_noalloc, x, qweight, scales, qzeros, g_idx, group_size, y, stream, 4)


def w4a16_dequant(qweight, scales, qzeros, g_idx, group_size: int, K: int, out=None, stream=None):
    """binary16 (q - Z) * S as [N][K] in the original input-channel order."""
    return _dequant_call(lib().w4a16_dequant, qweight, scales, qzeros, g_idx, group_size, K, out, stream, 4)


__all__ = ["LIB_PATH", "EXPORTS", "W4A16Error", "lib"] + [n for n in EXPORTS if n != "w4a16_last_error"]


# --- 8-bit weights (same conventions; codes and zero points are bytes) --------------

def w8a16_qweight_words(N: int, K: int, act_order: bool) -> int:
    return int(lib().w8a16_qweight_words(N, K, int(bool(act_order))))


def w8a16_quantize(w, group_size: int, g_idx=None, in_scale=None):
    """binary16 w [N][K] -> (codes uint8 [N][K], scales binary16 [G][N], zeros uint8 [G][N]),
    256 levels."""
    w = _np(w, np.float16, 2)
    N, K = w.shape
    G = K // group_size if group_size else 0
    gi = None if g_idx is None else _np(g_idx, np.int32, 1)
    sc = None if in_scale is None else _np(in_scale, np.float64, 1)
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((max(G, 1), N), np.float16)
    zeros = np.empty((max(G, 1), N), np.uint8)
    _check(lib().w8a16_quantize(_ptr(w), N, K, group_size, _ptr(gi), _ptr(sc), _ptr(codes),
                                _ptr(scales), _ptr(zeros)))
    return codes, scales, zeros


def w8a16_quantize_sym(w, group_size: int, g_idx=None, in_scale=None):
    """Symmetric 8-bit (int8 absmax per group): (codes uint8 [N][K] in 1..255, scales
    binary16 [G][N]); the zero point is 128 everywhere (qzeros=None on the device)."""
    w = _np(w, np.float16, 2)
    N, K = w.shape
    G = K // group_size if group_size else 0
    gi = None if g_idx is None else _np(g_idx, np.int32, 1)
    sc = None if in_scale is None else _np(in_scale, np.float64, 1)
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((max(G, 1), N), np.float16)
    _check(lib().w8a16_quantize_sym(_ptr(w), N, K, group_size, _ptr(gi), _ptr(sc), _ptr(codes), _ptr(scales)))
    return codes, scales


def w8a16_pack(codes, g_idx, group_size: int) -> np.ndarray:
    codes = _np(codes, np.uint8, 2)
    N, K = codes.shape
    gi = None if g_idx is None else _np(g_idx, np.int32, 1)
    out = np.empty(max(w8a16_qweight_words(N, K, gi is not None), 1), np.int32)
    _check(lib().w8a16_pack(_ptr(codes), _ptr(gi), group_size, N, K, _ptr(out)))
    return out


def w8a16_unpack(qweight, g_idx, group_size: int, N: int, K: int) -> np.ndarray:
    qweight = _np(qweight, np.int32).reshape(-1)
    gi = None if g_idx is None else _np(g_idx, np.int32, 1)
    if qweight.size < w8a16_qweight_words(N, K, gi is not None):
        raise ValueError("qweight is smaller than the packed size of an N x K 8-bit layer")
    codes = np.empty((N, K), np.uint8)
    _check(lib().w8a16_unpack(_ptr(qweight), _ptr(gi), group_size, N, K, _ptr(codes)))
    return codes


def w8a16_pack_zeros(zeros) -> np.ndarray:
    zeros = _np(zeros, np.uint8, 2)
    G, N = zeros.shape
    out = np.empty((G, max(N // 4, 1)), np.int32)
    _check(lib().w8a16_pack_zeros(_ptr(zeros), G, N, _ptr(out)))
    return out


def w8a16_unpack_zeros(qzeros, G: int, N: int) -> np.ndarray:
    qzeros = _np(qzeros, np.int32, 2)
    if qzeros.shape != (G, N // 4):
        raise ValueError(f"qzeros shape {qzeros.shape} != {(G, N // 4)}")
    out = np.empty((G, N), np.uint8)
    _check(lib().w8a16_unpack_zeros(_ptr(qzeros), G, N, _ptr(out)))
    return out


def w8a16_gemm(x, qweight, scales, qzeros, g_idx, group_size: int, y=None, stream=None):
    """y = x W^T for 8-bit weights on the device (qzeros int32 [G][N/4] or None)."""
    return _layer_call(lib().w8a16_gemm, x, qweight, scales, qzeros, g_idx, group_size, y, stream, 8)


def w8a16_dequant(qweight, scales, qzeros, g_idx, group_size: int, K: int, out=None, stream=None):
    """binary16 (q - Z) * S of an 8-bit weight buffer as [N][K] in the original order."""
    return _dequant_call(lib().w8a16_dequant, qweight, scales, qzeros, g_idx, group_size, K, out, stream, 8)


def w4a16_awq_search(w, xcal, group_size: int, alphas, stream=None):
    """AWQ alpha search on the device: (losses float64 [len(alphas)], best index).
    w binary16 [N][K] and xcal binary16 [T][K] on the host."""
    import torch
    w = _np(w, np.float16, 2)
    X = _np(xcal, np.float16, 2)
    N, K = w.shape
    T = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("xcal must have K columns")
    a = _np(alphas, np.float64, 1)
    losses = np.empty(a.size, np.float64)
    best = ctypes.c_int(-1)
    _check(lib().w4a16_awq_search(_ptr(w), _ptr(X), N, K, T, group_size, _ptr(a), a.size, _ptr(losses),
                                  ctypes.addressof(best), _stream_handle(stream, torch.device("cuda:0"))))
    return losses, best.value


def w4a16_gptq(w, xcal, group_size: int, act_order: bool = False, damp: float = 0.01, stream=None):
    """GPTQ on the device: (codes uint8 [N][K], scales binary16 [G][N], zeros uint8
    [G][N], g_idx int32 [K] or None), the formats of w4a16_quantize.  w binary16 [N][K]
    and xcal binary16 [T][K] on the host."""
    import torch
    w = _np(w, np.float16, 2)
    X = _np(xcal, np.float16, 2)
    N, K = w.shape
    T = X.shape[0]
    if X.shape[1] != K:
        raise ValueError("xcal must have K columns")
    G = K // group_size if group_size > 0 and K % group_size == 0 else 0
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((G, N), np.float16)
    zeros = np.empty((G, N), np.uint8)
    g_idx = np.empty(K, np.int32) if act_order else None
    _check(lib().w4a16_gptq(_ptr(w), _ptr(X), N, K, T, group_size, int(bool(act_order)), float(damp),
                            _ptr(codes), _ptr(scales), _ptr(zeros), None if g_idx is None else _ptr(g_idx),
                            _stream_handle(stream, torch.device("cuda:0"))))
    return codes, scales, zeros, g_idx


def w4a16_quantize_device(w, group_size: int, in_scale=None, sym: bool = False, stream=None):
    """Quantise and pack binary16 w [N][K] (a device tensor) on the device: (qweight int32
    [N*K/8], scales binary16 [G][N], qzeros int32 [G][N/8] or None when symmetric), the
    same bits as the host quantiser and packing.  in_scale: float64 device tensor [K]."""
    import torch
    _dev(w, torch.float16, "w")
    if in_scale is not None:
        _dev(in_scale, torch.float64, "in_scale")
    N, K = w.shape
    G = K // group_size
    qweight = torch.empty(N * K // 8, dtype=torch.int32, device=w.device)
    scales = torch.empty((G, N), dtype=torch.float16, device=w.device)
    qzeros = None if sym else torch.empty((G, N // 8), dtype=torch.int32, device=w.device)
    _check(lib().w4a16_quantize_device(w.data_ptr(), N, K, group_size,
                                       None if in_scale is None else in_scale.data_ptr(), int(bool(sym)),
                                       qweight.data_ptr(), scales.data_ptr(),
                                       None if qzeros is None else qzeros.data_ptr(), _stream_handle(stream, w.device)))
    return qweight, scales, qzeros

