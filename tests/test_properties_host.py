"""Property tests (hypothesis) of the library's host entry points against the oracle
over random layer shapes, group sizes and act-order group maps (no GPU): the library's
quantiser writes the oracle's codes, scales and zero points bit for bit, packing and
unpacking are inverse for codes and zero points, and the act-order packing stores
every group as one contiguous run of the oracle's group-sorted order."""

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import w4a16_gemm_amd as w4

SETTINGS = settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])


@st.composite
def layers(draw):
    g = draw(st.sampled_from([32, 64, 128, 0]))        # 0: one group per row (g = K)
    groups = draw(st.integers(1, 4))
    K = (g if g else 32 * draw(st.integers(1, 8))) * (groups if g else 1)
    if g == 0:
        g = K
    N = 8 * draw(st.integers(1, 6))
    seed = draw(st.integers(0, 2**31 - 1))
    act = draw(st.booleans()) and K // g > 1
    scale = draw(st.sampled_from([1e-3, 0.02, 0.5, 3.0]))
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * scale).astype(np.float16)
    if draw(st.booleans()):                              # a few special groups
        w[0, :g] = 0
        w[-1, :g] = np.abs(w[-1, :g])
    g_idx = None
    if act:
        perm = rng.permutation(K)
        g_idx = np.empty(K, np.int32)
        g_idx[perm] = np.arange(K) // g
    return w, g, g_idx


@SETTINGS
@given(layers())
def test_quantiser_matches_oracle(layer):
    w, g, g_idx = layer
    codes, S, Z = w4.w4a16_quantize(w, g, g_idx)
    rc, rs, rz = oracle.rtn_quantize(w, g, g_idx)
    assert np.array_equal(codes, rc)
    assert np.array_equal(S.view(np.uint16), rs.view(np.uint16))
    assert np.array_equal(Z, rz)


@SETTINGS
@given(layers())
def test_symmetric_quantiser_matches_oracle(layer):
    w, g, g_idx = layer
    codes, S = w4.w4a16_quantize_sym(w, g, g_idx)
    rc, rs = oracle.rtn_quantize_sym(w, g, g_idx)
    assert np.array_equal(codes, rc)
    assert np.array_equal(S.view(np.uint16), rs.view(np.uint16))


@SETTINGS
@given(layers())
def test_pack_unpack_round_trip(layer):
    w, g, g_idx = layer
    codes, S, Z = w4.w4a16_quantize(w, g, g_idx)
    N, K = codes.shape
    qw = w4.w4a16_pack(codes, g_idx, g)
    assert qw.size == w4.w4a16_qweight_words(N, K, g_idx is not None)
    assert np.array_equal(w4.w4a16_unpack(qw, g_idx, g, N, K), codes)
    qz = w4.w4a16_pack_zeros(Z)
    assert np.array_equal(w4.w4a16_unpack_zeros(qz, Z.shape[0], N), Z)
    # zero points pack along N exactly as the oracle's canonical packing
    assert np.array_equal(qz.view(np.uint32), oracle.pack_zeros(Z).view(np.uint32))
    if g_idx is not None:
        # the stored order is the oracle's group-sorted order (stable sort of k by
        # g_idx[k]): group i occupies stored positions [i g, (i + 1) g)
        stored = qw[N * K // 8:]
        assert np.array_equal(stored, oracle.sorted_k_order(g_idx).astype(np.int32))
        assert np.array_equal(g_idx[stored], np.arange(K) // g)
