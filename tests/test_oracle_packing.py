"""Pins of the oracle's reference packing (no GPU): known-answer words and round trips."""

import numpy as np
import pytest

import oracle
import workloads as wl


def test_known_answer_words():
    codes = np.array([[0, 1, 2, 3, 4, 5, 6, 7, 15, 15, 15, 15, 15, 15, 15, 15]], dtype=np.uint8)
    words = oracle.pack_codes(codes).view(np.uint32)
    assert words.tolist() == [[0x76543210, 0xFFFFFFFF]]
    one = np.zeros((1, 8), dtype=np.uint8)
    for j in range(8):
        one[:] = 0
        one[0, j] = 0xA
        assert int(oracle.pack_codes(one).view(np.uint32)[0, 0]) == 0xA << (4 * j)


def test_zeros_pack_along_outputs():
    zeros = np.zeros((2, 16), dtype=np.uint8)
    zeros[1, 9] = 7                                  # group 1, output 9 -> word [1][1], nibble 1
    q = oracle.pack_zeros(zeros).view(np.uint32)
    assert q.shape == (2, 2)
    assert q.tolist() == [[0, 0], [0, 0x70]]


@pytest.mark.parametrize("shape", [(1, 8), (8, 64), (33, 256)])
def test_round_trip(shape):
    c = wl.random_codes(*shape, seed=shape[1])
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(c)), c)
    z = wl.random_codes(shape[1] // 8, shape[0] * 8, seed=shape[0])
    assert np.array_equal(oracle.unpack_zeros(oracle.pack_zeros(z)), z)


def test_act_order_packing():
    K, g = 64, 16
    perm = np.random.default_rng(3).permutation(K)
    g_idx = np.empty(K, dtype=np.int32)
    g_idx[perm] = np.arange(K) // g
    c = wl.random_codes(5, K, seed=4)
    packed = oracle.pack_codes_act_order(c, g_idx)
    assert packed.shape == (5 * K // 8 + K,)
    p = packed[-K:].astype(np.int64)
    assert sorted(p.tolist()) == list(range(K))
    # sorted position p belongs to group p // g, and ties keep ascending k
    assert np.array_equal(g_idx[p], np.arange(K) // g)
    for a, b in zip(p[:-1], p[1:]):
        assert (g_idx[a], a) < (g_idx[b], b)
    words = packed[:-K].reshape(5, K // 8)
    assert np.array_equal(oracle.unpack_codes(words)[:, np.argsort(p)], c)
    # identity g_idx: the words are the plain packing
    ident = (np.arange(K) // g).astype(np.int32)
    packed_id = oracle.pack_codes_act_order(c, ident)
    assert np.array_equal(packed_id[:-K].reshape(5, K // 8), oracle.pack_codes(c))
    assert np.array_equal(packed_id[-K:], np.arange(K))


def test_pack8_known_words_and_round_trip():
    codes = np.array([[0x01, 0x23, 0x45, 0x67, 0x89, 0xAB, 0xCD, 0xEF]], dtype=np.uint8)
    words = oracle.pack_codes8(codes).view(np.uint32)
    assert words.tolist() == [[0x67452301, 0xEFCDAB89]]      # byte j of a word = element 4w + j
    rng = np.random.default_rng(5)
    c = rng.integers(0, 256, size=(8, 64), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_codes8(oracle.pack_codes8(c)), c)
    z = rng.integers(0, 256, size=(3, 32), dtype=np.uint8)
    assert np.array_equal(oracle.unpack_zeros8(oracle.pack_zeros8(z)), z)

