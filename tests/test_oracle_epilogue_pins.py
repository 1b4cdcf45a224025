"""Pins of the oracle's output options (CPU only): the residual addition
(iamjaehka13.blog §14 and the residual row of its §23 shape table) and the
attention weights nn.MultiheadAttention returns (molayo1419.me: head-averaged
(N, L, S) by default, per head (N, h, L, S) with average_attn_weights=False)."""

import math

import numpy as np
import pytest
import torch

from oracle import mha_oracle as mo


def _problem(rng, B, Tq, D, h, Tk=None, cross=False):
    return dict(x_q=rng.standard_normal((B, Tq, D)),
                x_kv=rng.standard_normal((B, Tk, D)) if cross else None,
                w_qkv=rng.standard_normal((D, 3 * D)) / math.sqrt(D),
                b_qkv=rng.standard_normal(3 * D) * 0.1,
                w_o=rng.standard_normal((D, D)) / math.sqrt(D),
                b_o=rng.standard_normal(D) * 0.1)


def test_residual_with_zero_output_projection_is_the_input():
    rng = np.random.default_rng(1)
    p = _problem(rng, 2, 7, 16, 4)
    y = mo.mha_forward(p["x_q"], p["w_qkv"], p["b_qkv"], np.zeros((16, 16)), np.zeros(16), 4,
                       causal=True, residual=True)
    assert np.array_equal(y, p["x_q"])


@pytest.mark.parametrize("cross", [False, True])
def test_residual_adds_the_query_side_input(cross):
    rng = np.random.default_rng(2 + cross)
    p = _problem(rng, 2, 9, 32, 4, Tk=13, cross=cross)
    args = (p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], 4)
    y0 = mo.mha_forward(*args, x_kv=p["x_kv"])
    y1 = mo.mha_forward(*args, x_kv=p["x_kv"], residual=True)
    assert np.max(np.abs((y1 - y0) - p["x_q"])) <= 1e-12 * max(1.0, np.max(np.abs(y0)))
    rows = mo.mha_forward_rows(*args, {0: [0, 4], 1: [8]}, x_kv=p["x_kv"], residual=True)
    assert np.max(np.abs(rows[0] - y1[0, [0, 4]])) <= 1e-13
    assert np.max(np.abs(rows[1] - y1[1, [8]])) <= 1e-13


@pytest.mark.parametrize("average", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_attention_weights_match_torch(average, causal):
    rng = np.random.default_rng(5 + 2 * average + causal)
    D, h, B, T = 32, 4, 3, 11
    p = _problem(rng, B, T, D, h)
    mask = np.zeros((B, T), dtype=np.uint8)
    mask[1, 7:] = 1
    m = torch.nn.MultiheadAttention(D, h, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        m.in_proj_weight.copy_(torch.from_numpy(p["w_qkv"].T.copy()))
        m.in_proj_bias.copy_(torch.from_numpy(p["b_qkv"]))
        m.out_proj.weight.copy_(torch.from_numpy(p["w_o"].T.copy()))
        m.out_proj.bias.copy_(torch.from_numpy(p["b_o"]))
    m.train()
    x = torch.from_numpy(p["x_q"])
    am = torch.ones(T, T, dtype=torch.bool).triu(1) if causal else None
    with torch.no_grad():
        _, w = m(x, x, x, key_padding_mask=torch.from_numpy(mask != 0), attn_mask=am,
                 need_weights=True, average_attn_weights=average)
    a = mo.attention_weights(p["x_q"], p["w_qkv"], p["b_qkv"], h, causal=causal,
                             key_padding_mask=mask, average=average)
    assert a.shape == tuple(w.shape)
    assert np.max(np.abs(a - w.numpy())) <= 1e-13


def test_attention_weights_rows_sum_to_one_and_respect_masks():
    rng = np.random.default_rng(9)
    p = _problem(rng, 2, 6, 16, 2)
    mask = np.zeros((2, 6), dtype=np.uint8)
    mask[0, 4:] = 1
    a = mo.attention_weights(p["x_q"], p["w_qkv"], p["b_qkv"], 2, causal=True,
                             key_padding_mask=mask)
    assert np.allclose(a.sum(-1), 1.0, atol=1e-14)
    assert np.all(a[0, :, :, 4:] == 0.0)
    assert np.all(np.triu(np.ones((6, 6)), 1)[None, None] * a == 0.0)
