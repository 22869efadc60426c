"""The C-ABI library without a GPU: it loads, exports every declared symbol, and its
host-side (offline) entry points agree bit-exactly with the oracle.  Device entry
points are only exercised on their argument checks (no kernel is launched here)."""

import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle
import w4a16_gemm_amd as w4
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w[48]a16_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = w4.lib()
    declared = _declared_functions()
    assert len(declared) == 28
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(w4.EXPORTS) == declared


def test_peaks_library_exports_every_declared_symbol():
    from w4a16_gemm_amd import build
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "w4a16_peaks.h")).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(w4a16_peak\w*)\s*\(", text)))
    assert declared == ["w4a16_peak_mfma_f16", "w4a16_peak_stream_read", "w4a16_peaks_last_error"]
    lib = ctypes.CDLL(build.PEAKS_LIB)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version():
    assert w4.w4a16_abi_version() == 1


def test_qweight_words():
    assert w4.w4a16_qweight_words(16, 256, False) == 16 * 32
    assert w4.w4a16_qweight_words(16, 256, True) == 16 * 32 + 256
    assert w4.lib().w4a16_qweight_words(0, 256, 0) == 0


# --- quantiser ------------------------------------------------------------------

def _assert_same_quant(a, b):
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint16), b[1].view(np.uint16))
    assert np.array_equal(a[2], b[2])


@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_quantize_bit_exact_on_config_rows(name):
    cfg = wl.CONFIGS[name]
    rows = np.linspace(0, cfg.N - 1, 24).astype(np.int64)
    w = wl.weights(cfg, rows)
    g_idx = s = None
    if cfg.act_order:
        g_idx, _ = oracle.act_order(wl.calibration(cfg), cfg.group_size)
    if cfg.awq:
        s = oracle.awq_scales(wl.calibration(cfg))
    _assert_same_quant(w4.w4a16_quantize(w, cfg.group_size, g_idx, s),
                       oracle.rtn_quantize(w, cfg.group_size, g_idx, s))


def test_quantize_bit_exact_on_special_groups():
    import json
    data = json.load(open(os.path.join(ROOT, "tests", "golden", "rtn_worked_groups.json")))
    for grp in data["groups"]:
        w = np.array(grp["w"], dtype=np.float16)
        w = np.tile(w, (8, 32 // w.size + 1))[:, :32]
        _assert_same_quant(w4.w4a16_quantize(w, 32), oracle.rtn_quantize(w, 32))
    rng = np.random.default_rng(0)
    for scale in (1e-6, 1e-3, 1.0, 300.0):       # subnormal scales up to large ones
        w = (rng.standard_normal((16, 128)) * scale).astype(np.float16)
        w[3, :32] = 0
        w[4, 32:64] = np.abs(w[4, 32:64])
        for g in (32, 64, 128):
            _assert_same_quant(w4.w4a16_quantize(w, g), oracle.rtn_quantize(w, g))


@pytest.mark.parametrize("name", ["c1", "c2up", "c3", "c5"])
def test_quantize_sym_bit_exact_on_config_rows(name):
    cfg = wl.CONFIGS[name]
    rows = np.linspace(0, cfg.N - 1, 24).astype(np.int64)
    w = wl.weights(cfg, rows)
    g_idx = s = None
    if cfg.act_order:
        g_idx, _ = oracle.act_order(wl.calibration(cfg), cfg.group_size)
    if cfg.awq:
        s = oracle.awq_scales(wl.calibration(cfg))
    c, S = w4.w4a16_quantize_sym(w, cfg.group_size, g_idx, s)
    co, So = oracle.rtn_quantize_sym(w, cfg.group_size, g_idx, s)
    assert np.array_equal(c, co) and np.array_equal(S.view(np.uint16), So.view(np.uint16))


def test_quantize_sym_bit_exact_on_special_groups():
    import json
    data = json.load(open(os.path.join(ROOT, "tests", "golden", "rtn_sym_worked_groups.json")))
    rng = np.random.default_rng(1)
    for grp in data["groups"]:
        if "w_bits" in grp:
            w = np.array([int(b, 16) for b in grp["w_bits"]], dtype=np.uint16).view(np.float16)
        else:
            w = np.array(grp["w"], dtype=np.float16)
        w = np.tile(w, (8, 32 // w.size + 1))[:, :32]
        c, S = w4.w4a16_quantize_sym(w, 32)
        co, So = oracle.rtn_quantize_sym(w, 32)
        assert np.array_equal(c, co) and np.array_equal(S.view(np.uint16), So.view(np.uint16))
    for scale in (1e-6, 1e-3, 1.0, 300.0):
        w = (rng.standard_normal((16, 128)) * scale).astype(np.float16)
        w[3, :32] = 0
        w[4, 32:64] = -np.abs(w[4, 32:64])
        for g in (32, 64, 128):
            c, S = w4.w4a16_quantize_sym(w, g)
            co, So = oracle.rtn_quantize_sym(w, g)
            assert np.array_equal(c, co) and np.array_equal(S.view(np.uint16), So.view(np.uint16))


def test_awq_scales_and_fold_bit_exact():
    cfg = wl.CONFIGS["c2up"]
    X = wl.calibration(cfg)
    s = w4.w4a16_awq_scales(X)
    assert np.array_equal(s, oracle.awq_scales(X))
    x = wl.activations(cfg, 1)
    assert np.array_equal(w4.w4a16_awq_fold_activations(x, s).view(np.uint16),
                          oracle.awq_fold_activations(x, s).view(np.uint16))
    Xz = X[:, :64].copy()
    Xz[:, 5] = 0
    assert np.array_equal(w4.w4a16_awq_scales(Xz), oracle.awq_scales(Xz))
    # alpha = 0.5 (the configurations' value) goes through the correctly rounded square
    # root and is bit-exact; another alpha goes through pow(), which libm and numpy do
    # not round identically, so it agrees to a few ulp only
    np.testing.assert_allclose(w4.w4a16_awq_scales(Xz, 0.25), oracle.awq_scales(Xz, 0.25), rtol=4e-16)


def test_act_order_bit_exact():
    cfg = wl.CONFIGS["c5"]
    X = wl.calibration(cfg)
    assert np.array_equal(w4.w4a16_act_order(X, cfg.group_size), oracle.act_order(X, cfg.group_size)[0])
    Xt = np.random.default_rng(1).standard_normal((16, 64)).astype(np.float16)
    Xt[:, 10] = Xt[:, 3]
    Xt[:, 40] = -Xt[:, 3]
    assert np.array_equal(w4.w4a16_act_order(Xt, 32), oracle.act_order(Xt, 32)[0])


# --- packing ---------------------------------------------------------------------

def test_private_word_layout_known_answer():
    codes = np.arange(8, dtype=np.uint8)[None, :].repeat(8, 0)
    codes = np.concatenate([codes] * 4, axis=1)            # K = 32
    words = w4.w4a16_pack(codes, None, 32).view(np.uint32)
    # element e of a word sits in nibble (0, 4, 1, 5, 2, 6, 3, 7)[e]
    assert int(words[0]) == 0x75316420
    assert np.all(words == 0x75316420)
    assert np.array_equal(w4.w4a16_pack(np.full((8, 32), 15, np.uint8), None, 32).view(np.uint32),
                          np.full(32, 0xFFFFFFFF, np.uint32))


def test_library_word_decoder_used_by_the_gpu_tests():
    """The GPU tests decode random library words with the documented nibble order;
    that decoder inverts w4a16_pack."""
    from gpu_common import codes_of_library_words
    codes = wl.random_codes(16, 256, 3)
    words = w4.w4a16_pack(codes, None, 128).reshape(16, 32)
    assert np.array_equal(codes_of_library_words(words), codes)


@pytest.mark.parametrize("act", [False, True])
@pytest.mark.parametrize("shape", [(8, 64, 32), (24, 256, 64), (40, 512, 128)])
def test_pack_unpack_round_trip(shape, act):
    N, K, g = shape
    codes = wl.random_codes(N, K, seed=K + N)
    g_idx = None
    if act:
        perm = np.random.default_rng(N).permutation(K)
        g_idx = np.empty(K, np.int32)
        g_idx[perm] = np.arange(K) // g
    packed = w4.w4a16_pack(codes, g_idx, g)
    assert packed.size == w4.w4a16_qweight_words(N, K, act)
    assert np.array_equal(w4.w4a16_unpack(packed, g_idx, g, N, K), codes)
    if act:
        assert np.array_equal(packed[N * K // 8:], oracle.sorted_k_order(g_idx))


@pytest.mark.parametrize("K", [96, 1536])
def test_per_channel_quantize_pack_bit_exact(K):
    """group_size = K: one scale (and zero point) per output row."""
    cfg = wl.custom_config("perch", 500 + K, K=K, N=24, group_size=K)
    w = wl.weights(cfg)
    _assert_same_quant(w4.w4a16_quantize(w, K), oracle.rtn_quantize(w, K))
    c, S = w4.w4a16_quantize_sym(w, K)
    co, So = oracle.rtn_quantize_sym(w, K)
    assert np.array_equal(c, co) and np.array_equal(S.view(np.uint16), So.view(np.uint16))
    assert S.shape == (1, 24)
    codes = w4.w4a16_quantize(w, K)[0]
    g_idx = np.zeros(K, np.int32)                 # act order with one group: identity order
    for gi in (None, g_idx):
        packed = w4.w4a16_pack(codes, gi, K)
        assert np.array_equal(w4.w4a16_unpack(packed, gi, K, 24, K), codes)


# --- 8-bit weights -----------------------------------------------------------------

@pytest.mark.parametrize("name", ["c1", "c2up", "c3", "c5"])
def test_quantize8_bit_exact_on_config_rows(name):
    cfg = wl.CONFIGS[name]
    rows = np.linspace(0, cfg.N - 1, 16).astype(np.int64)
    w = wl.weights(cfg, rows)
    g_idx = s = None
    if cfg.act_order:
        g_idx, _ = oracle.act_order(wl.calibration(cfg), cfg.group_size)
    if cfg.awq:
        s = oracle.awq_scales(wl.calibration(cfg))
    _assert_same_quant(w4.w8a16_quantize(w, cfg.group_size, g_idx, s),
                       oracle.rtn_quantize(w, cfg.group_size, g_idx, s, bits=8))
    c, S = w4.w8a16_quantize_sym(w, cfg.group_size, g_idx, s)
    co, So = oracle.rtn_quantize_sym(w, cfg.group_size, g_idx, s, bits=8)
    assert np.array_equal(c, co) and np.array_equal(S.view(np.uint16), So.view(np.uint16))


def test_quantize8_bit_exact_on_special_groups():
    rng = np.random.default_rng(2)
    for scale in (1e-6, 1e-3, 1.0, 300.0):
        w = (rng.standard_normal((16, 128)) * scale).astype(np.float16)
        w[3, :32] = 0
        w[4, 32:64] = np.abs(w[4, 32:64])
        w[5, 64:96] = -np.abs(w[5, 64:96])
        for g in (32, 64, 128):
            _assert_same_quant(w4.w8a16_quantize(w, g), oracle.rtn_quantize(w, g, bits=8))
            c, S = w4.w8a16_quantize_sym(w, g)
            co, So = oracle.rtn_quantize_sym(w, g, bits=8)
            assert np.array_equal(c, co) and np.array_equal(S.view(np.uint16), So.view(np.uint16))


def test_pack8_private_layout_and_round_trip():
    codes = np.tile(np.array([0x01, 0x23, 0x45, 0x67], np.uint8), (8, 8))   # K = 32
    words = w4.w8a16_pack(codes, None, 32).view(np.uint32)
    # element e of a word sits in byte (0, 2, 1, 3)[e]
    assert np.all(words == 0x67234501)
    for act in (False, True):
        N, K, g = 24, 256, 64
        c = np.random.default_rng(7).integers(0, 256, size=(N, K), dtype=np.uint8)
        g_idx = None
        if act:
            perm = np.random.default_rng(8).permutation(K)
            g_idx = np.empty(K, np.int32)
            g_idx[perm] = np.arange(K) // g
        packed = w4.w8a16_pack(c, g_idx, g)
        assert packed.size == w4.w8a16_qweight_words(N, K, act)
        assert np.array_equal(w4.w8a16_unpack(packed, g_idx, g, N, K), c)
        if act:
            assert np.array_equal(packed[N * K // 4:], oracle.sorted_k_order(g_idx))
    z = np.random.default_rng(9).integers(0, 256, size=(6, 32), dtype=np.uint8)
    q = w4.w8a16_pack_zeros(z)
    assert np.array_equal(q, oracle.pack_zeros8(z))
    assert np.array_equal(w4.w8a16_unpack_zeros(q, 6, 32), z)


def test_identity_gidx_packs_like_contiguous():
    codes = wl.random_codes(16, 128, seed=3)
    ident = (np.arange(128) // 32).astype(np.int32)
    a = w4.w4a16_pack(codes, None, 32)
    b = w4.w4a16_pack(codes, ident, 32)
    assert np.array_equal(b[:a.size], a)
    assert np.array_equal(b[a.size:], np.arange(128))


def test_pack_zeros_matches_oracle_format():
    z = wl.random_codes(12, 64, seed=9)          # [G][N]
    q = w4.w4a16_pack_zeros(z)
    assert np.array_equal(q, oracle.pack_zeros(z))
    assert np.array_equal(w4.w4a16_unpack_zeros(q, 12, 64), z)


# --- error codes -------------------------------------------------------------------

def _status(fn, *args):
    with pytest.raises(w4.W4A16Error) as e:
        fn(*args)
    return e.value.status


def test_error_codes_host():
    codes = wl.random_codes(8, 64, seed=1)
    assert _status(w4.w4a16_pack, codes, None, 48) == w4.ERR_UNSUPPORTED
    assert _status(w4.w4a16_pack, codes[:, :48], None, 48) == w4.ERR_INVALID_ARG   # per-channel, K % 32
    assert _status(w4.w4a16_pack, codes, None, 256) == w4.ERR_UNSUPPORTED          # neither g nor K
    assert _status(w4.w4a16_pack, codes[:, :48], None, 32) == w4.ERR_INVALID_ARG   # K % g
    assert _status(w4.w4a16_pack, codes[:4], None, 32) == w4.ERR_INVALID_ARG       # N % 8
    bad = codes.copy()
    bad[0, 0] = 16
    assert _status(w4.w4a16_pack, bad, None, 32) == w4.ERR_INVALID_ARG
    g_idx = (np.arange(64) // 32).astype(np.int32)
    g2 = g_idx.copy()
    g2[0] = 2
    assert _status(w4.w4a16_pack, codes, g2, 32) == w4.ERR_BAD_GIDX               # out of range
    g3 = g_idx.copy()
    g3[0] = 1
    assert _status(w4.w4a16_pack, codes, g3, 32) == w4.ERR_BAD_GIDX               # group sizes 31/33
    packed = w4.w4a16_pack(codes, g_idx, 32)
    packed[-1] = packed[-2]
    assert _status(w4.w4a16_unpack, packed, g_idx, 32, 8, 64) == w4.ERR_BAD_GIDX   # not a permutation
    w = np.zeros((8, 64), np.float16)
    w[0, 0] = np.inf
    assert _status(w4.w4a16_quantize, w, 32) == w4.ERR_INVALID_ARG
    assert _status(w4.w4a16_quantize, np.zeros((8, 64), np.float16), 32, None, np.zeros(64)) == w4.ERR_INVALID_ARG
    rc = w4.lib().w4a16_pack(bad.ctypes.data, None, 32, 8, 64, np.empty(64, np.int32).ctypes.data)
    assert rc == w4.ERR_INVALID_ARG and "above 15" in w4.lib().w4a16_last_error().decode()


def test_error_codes_device_argument_checks():
    """Argument checks run before any HIP call, so they are testable without a GPU."""
    lib = w4.lib()
    buf = (ctypes.c_uint8 * 4096)()
    base = (ctypes.addressof(buf) + 15) & ~15
    ok = ctypes.c_void_p(base)
    mis = ctypes.c_void_p(base + 2)
    assert lib.w4a16_gemm(None, ok, ok, ok, None, 128, 1, 8, 128, ok, None) == w4.ERR_INVALID_ARG
    assert lib.w4a16_gemm(ok, ok, ok, ok, None, 128, 0, 8, 128, ok, None) == w4.ERR_INVALID_ARG
    assert lib.w4a16_gemm(ok, ok, ok, ok, None, 96, 1, 8, 192, ok, None) == w4.ERR_UNSUPPORTED
    assert lib.w4a16_gemm(ok, ok, ok, ok, None, 128, 1, 12, 128, ok, None) == w4.ERR_INVALID_ARG
    assert lib.w4a16_gemm(ok, ok, ok, ok, None, 128, 1, 8, 192, ok, None) == w4.ERR_INVALID_ARG
    assert lib.w4a16_gemm(mis, ok, ok, ok, None, 128, 1, 8, 128, ok, None) == w4.ERR_MISALIGNED
    assert lib.w4a16_dequant(ok, ok, ok, None, 64, 8, 128, mis, None) == w4.ERR_MISALIGNED
    assert lib.w4a16_dequant(ok, None, ok, None, 64, 8, 128, ok, None) == w4.ERR_INVALID_ARG
    assert lib.w4a16_gemm(mis, ok, ok, ok, None, 128, 1, 8, 128, ok, None) == w4.ERR_MISALIGNED
    assert "aligned" in lib.w4a16_last_error().decode()


def test_gptq_rejects_bad_arguments_before_any_device_work():
    """Argument checks of w4a16_gptq run on the host, before any device call."""
    import ctypes
    L = w4.lib()
    N, K, T, g = 16, 64, 8, 32
    w = np.zeros((N, K), np.float16)
    x = np.ones((T, K), np.float16)
    c = np.empty((N, K), np.uint8)
    s = np.empty((K // g, N), np.float16)
    z = np.empty((K // g, N), np.uint8)
    gi = np.empty(K, np.int32)
    P = lambda a: a.ctypes.data_as(ctypes.c_void_p)

    def call(N=N, K=K, T=T, g=g, act=0, damp=0.01, w=w, x=x, gidx=gi):
        return L.w4a16_gptq(P(w), P(x), N, K, T, g, act, damp, P(c), P(s), P(z),
                            None if gidx is None else P(gidx), None)

    assert call(T=0) == w4.ERR_INVALID_ARG
    assert call(damp=-1.0) == w4.ERR_INVALID_ARG
    assert call(damp=float("nan")) == w4.ERR_INVALID_ARG
    assert call(g=48) == w4.ERR_UNSUPPORTED
    assert call(N=12) == w4.ERR_INVALID_ARG
    assert call(act=1, gidx=None) == w4.ERR_INVALID_ARG
    wn = w.copy()
    wn[3, 7] = np.inf
    assert call(w=wn) == w4.ERR_INVALID_ARG
    xn = x.copy()
    xn[1, 2] = np.nan
    assert call(x=xn) == w4.ERR_INVALID_ARG
    assert b"finite" in L.w4a16_last_error()


# --- binding argument checks (refused before anything reaches the device) ----------

def _layer_tensors(N=64, K=256, g=64, act=False, bits=4):
    import torch
    G = K // g
    words = (w4.w4a16_qweight_words if bits == 4 else w4.w8a16_qweight_words)(N, K, act)
    return dict(
        x=torch.zeros((2, K), dtype=torch.float16),
        qweight=torch.zeros(words, dtype=torch.int32),
        scales=torch.zeros((G, N), dtype=torch.float16),
        qzeros=torch.zeros((G, N // (8 if bits == 4 else 4)), dtype=torch.int32),
        g_idx=torch.zeros(K, dtype=torch.int32) if act else None,
    )


@pytest.mark.parametrize("bits", [4, 8])
def test_binding_refuses_misshaped_layer_tensors(bits):
    import torch
    gemm = w4.w4a16_gemm if bits == 4 else w4.w8a16_gemm
    deq = w4.w4a16_dequant if bits == 4 else w4.w8a16_dequant
    g = 64

    def call(**over):
        t = _layer_tensors(act=True, bits=bits)
        t.update(over)
        return gemm(t["x"], t["qweight"], t["scales"], t["qzeros"], t["g_idx"], g, y=over.get("y"))

    K, N = 256, 64
    bad = {
        "scales": torch.zeros((K // g + 1, N), dtype=torch.float16),          # wrong group count
        "qzeros": torch.zeros((K // g, N // 8 + 1 if bits == 4 else N // 4 + 1), dtype=torch.int32),
        "g_idx": torch.zeros(K - 1, dtype=torch.int32),
        "qweight": torch.zeros(10, dtype=torch.int32),
        "y": torch.zeros((2, N + 1), dtype=torch.float16),
    }
    for name, t in bad.items():
        with pytest.raises(ValueError, match=name):
            call(**{name: t})
    with pytest.raises(ValueError):
        call(x=torch.zeros((2, K + 32), dtype=torch.float16))   # K from x: scales no longer match
    t = _layer_tensors(bits=bits)
    with pytest.raises(ValueError, match="out"):
        deq(t["qweight"], t["scales"], t["qzeros"], None, g, K, out=torch.zeros((N, K - 8), dtype=torch.float16))
    with pytest.raises(ValueError, match="qweight"):
        deq(torch.zeros(8, dtype=torch.int32), t["scales"], t["qzeros"], None, g, K)
    with pytest.raises(ValueError, match="scales"):
        deq(t["qweight"], t["scales"], t["qzeros"], None, g, 2 * K)
    # dtypes
    with pytest.raises(TypeError):
        call(scales=torch.zeros((K // g, N), dtype=torch.float32))
    # well-shaped host tensors pass every shape check and stop at the device check
    with pytest.raises(TypeError, match="ROCm device"):
        call()


def test_reload_env_is_exported_and_succeeds():
    w4.w4a16_reload_env()


def test_library_shares_the_hip_runtime_torch_loads():
    # loaded before anything touches torch, the library must still end up on the HIP
    # runtime torch ships (one runtime in the process), or its launches fail
    code = ("import w4a16_gemm_amd as w4\n"
            "w4.lib()\n"
            "import torch\n"
            "libs = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
            "print(len(libs), sorted(libs))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.startswith("1 "), out.stdout
