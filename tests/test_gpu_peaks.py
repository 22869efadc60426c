"""The achievable-peak probes the bench reports beside the nominal peaks (needs an
MI355X): the streaming read touches every 16-byte chunk of its buffer exactly once
(the XOR of the per-thread results equals the XOR of all words of the buffer), and
the MFMA loop launches and gives the same output on every run."""

import ctypes

import numpy as np
import pytest

from gpu_common import device, note

pytestmark = pytest.mark.gpu


def _lib():
    import w4a16_gemm_amd as w4
    from w4a16_gemm_amd import build
    w4.load_runtime_first()
    lib = ctypes.CDLL(build.PEAKS_LIB)
    lib.w4a16_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_void_p]
    lib.w4a16_peak_mfma_f16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.w4a16_peaks_last_error.restype = ctypes.c_char_p
    return lib


@pytest.mark.parametrize("words,blocks", [(4 * 1000003, 7), (1 << 22, 256), (4 * 37, 3)])
def test_stream_read_reads_every_chunk_once(words, blocks):
    import torch
    lib = _lib()
    note(f"stream read words={words} blocks={blocks}")
    host = np.random.default_rng([5, words]).integers(0, 1 << 32, size=words, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(device())
    out = torch.zeros(blocks * 512, dtype=torch.int32, device=device())
    assert lib.w4a16_peak_stream_read(buf.data_ptr(), 4 * words, out.data_ptr(), blocks, None) == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_stream_read_rejects_bad_arguments():
    import torch
    lib = _lib()
    buf = torch.zeros(64, dtype=torch.int32, device=device())
    out = torch.zeros(512, dtype=torch.int32, device=device())
    assert lib.w4a16_peak_stream_read(buf.data_ptr(), 100, out.data_ptr(), 1, None) == 1   # not a multiple of 16
    assert lib.w4a16_peak_stream_read(buf.data_ptr(), 256, out.data_ptr(), 0, None) == 1
    assert lib.w4a16_peak_stream_read(None, 256, out.data_ptr(), 1, None) == 1
    assert lib.w4a16_peaks_last_error()


def test_mfma_loop_is_deterministic():
    import torch
    lib = _lib()
    note("mfma loop")
    outs = []
    for _ in range(2):
        out = torch.zeros(4 * 512, dtype=torch.float32, device=device())
        assert lib.w4a16_peak_mfma_f16(out.data_ptr(), 50, 4, None) == 0
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.isfinite(outs[0]).all() and np.abs(outs[0]).sum() > 0
    assert np.array_equal(outs[0], outs[1])
