"""Pins of the oracle's storage accounting against the figures the pages print (no GPU).

The figures and their citations are in tests/golden/page_figures.json.
"""

import json
import os

import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                     "golden", "page_figures.json")))


def test_bits_per_weight_g128_in_printed_range():
    b = GOLDEN["bits_per_weight_g128"]
    bpw = oracle.bits_per_weight(1024, 4096, 128)
    assert b["printed_low"] <= bpw <= b["printed_high"]
    assert bpw == 4 + 16 / 128 + 4 / 128            # 4.15625
    scale_part = 16 / 128
    assert scale_part == GOLDEN["scale_bits_per_weight_g128"]["printed"]
    zero_part = bpw - 4 - scale_part
    z = GOLDEN["zero_bits_per_weight_g128_about"]
    assert abs(zero_part - z["printed"]) <= z["tolerance"]


@pytest.mark.parametrize("g", [32, 64, 128])
def test_bits_per_weight_formula(g):
    assert oracle.bits_per_weight(256, 1024, g) == 4 + 16 / g + 4 / g
    # the act-order permutation adds one int32 per input channel
    assert oracle.bits_per_weight(256, 1024, g, act_order=True) == pytest.approx(4 + 20 / g + 32 / 256)


def test_groups_per_row():
    f = GOLDEN["groups_per_row_at_hidden_1536"]
    assert f["hidden"] // f["group_size"] == f["printed"]


def test_1p5b_byte_budget():
    f = GOLDEN["model_1p5b"]
    h, L, I, V = f["hidden"], f["layers"], f["mlp"], f["vocab"]
    q_out = f["q_heads"] * f["head_dim"]
    kv_out = f["kv_heads"] * f["head_dim"]
    # (out, in) of every linear layer of one transformer block
    shapes = [(q_out, h), (kv_out, h), (kv_out, h), (h, q_out),   # q, k, v, o
              (I, h), (I, h), (h, I)]                               # gate, up, down
    attn = sum(n * k for n, k in shapes[:4])
    mlp = sum(n * k for n, k in shapes[4:])
    assert attn == h * 3584 and round(attn / 1e6, 1) == 5.5
    assert mlp == 3 * h * I and round(mlp / 1e6, 1) == 41.3
    linear = L * (attn + mlp)
    embed = V * h
    total = linear + embed
    assert round(linear / 1e9, 2) == f["linear_weights_printed_billions"]
    assert round(embed / 1e6) == f["embedding_printed_millions"]
    assert round(total / 1e9, 2) == f["total_params_printed_billions"]
    assert round(2 * total / 1e9, 2) == f["bf16_gb_printed"]
    g = f["group_size"]
    lin_bytes = L * sum(oracle.layer_bytes(n, k, g) for n, k in shapes)
    emb_bytes = 2 * embed
    q_total = lin_bytes + emb_bytes
    assert round(lin_bytes / 1e9, 2) == f["w4a16_linear_gb_printed"]
    assert round(emb_bytes / 1e9, 2) == f["embedding_bf16_gb_printed"]
    assert abs(q_total / 1e9 - f["w4a16_total_gb_printed"]) <= f["w4a16_total_gb_tolerance_rel"] * f["w4a16_total_gb_printed"]
    assert round(2 * total / q_total, 1) == f["shrink_factor_printed"]
    assert round(100 * embed / total) == f["embedding_share_of_params_pct_printed"]
    assert round(100 * emb_bytes / q_total) == f["embedding_share_of_quantized_file_pct_printed"]
