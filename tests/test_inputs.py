"""Seeded input generator: determinism, shapes, distributions, mask structure."""

import hashlib
import math

import torch

from mha_inputs import ALL_WORKLOADS, GROUPED_WORKLOADS, WORKLOADS, HEADLINE, make_inputs


def _digest(inp):
    h = hashlib.sha256()
    for k in ("x_q", "x_kv", "w_qkv", "b_qkv", "w_o", "b_o", "key_padding_mask"):
        t = inp[k]
        if t is not None:
            h.update(t.contiguous().view(torch.uint8).numpy().tobytes())
    return h.hexdigest()


def test_deterministic_per_seed_and_distinct_across_seeds():
    w = WORKLOADS["cross_pad_bf16_d512_h8_b32_tq512_tk2048"].shrink(B=3, T_q=40, T_k=300,
                                                                     padding=(10, 300))
    a, b, c = make_inputs(w, 0), make_inputs(w, 0), make_inputs(w, 1)
    assert _digest(a) == _digest(b)
    assert _digest(a) != _digest(c)


def test_shapes_and_dtypes_of_every_workload():
    for name, w in ALL_WORKLOADS.items():
        small = w.shrink(B=min(w.B, 2), T_q=min(w.T_q, 64), T_k=min(w.T_k, 64),
                         padding=None if w.padding is None else (8, 64))
        inp = make_inputs(small, 0)
        dt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
        assert inp["x_q"].shape == (small.B, small.T_q, w.D) and inp["x_q"].dtype == dt
        n_qkv = w.D + 2 * (w.h if w.n_kv is None else w.n_kv) * (w.D // w.h)
        assert inp["w_qkv"].shape == (w.D, n_qkv) and inp["b_qkv"].shape == (n_qkv,)
        assert inp["w_o"].shape == (w.D, w.D)
        assert (inp["x_kv"] is not None) == w.cross
        assert (inp["key_padding_mask"] is not None) == (w.padding is not None)
        if w.bias_std is None:
            assert not inp["b_qkv"].any() and not inp["b_o"].any()


def test_xavier_bounds_and_normal_std():
    w = WORKLOADS[HEADLINE].shrink(B=1, T_q=8, T_k=8)
    inp = make_inputs(w, 0)
    D = w.D
    a_qkv = math.sqrt(6.0 / (4 * D))
    a_o = math.sqrt(6.0 / (2 * D))
    wq = inp["w_qkv"].float()
    assert wq.abs().max() <= a_qkv * (1 + 2 ** -8)
    assert abs(wq.std().item() - a_qkv / math.sqrt(3)) < 0.01 * a_qkv
    assert inp["w_o"].float().abs().max() <= a_o * (1 + 2 ** -8)
    w5 = WORKLOADS["causal_bf16_d4096_h32_b1_t8192"].shrink(T_q=4, T_k=4)
    inp5 = make_inputs(w5, 0)
    assert abs(inp5["w_o"].float().std().item() - 1 / 64) < 1e-4


def test_padding_mask_is_trailing_with_lengths_in_range():
    w = WORKLOADS["cross_pad_bf16_d512_h8_b32_tq512_tk2048"].shrink(T_q=8)
    inp = make_inputs(w, 0)
    m, L = inp["key_padding_mask"], inp["lengths"]
    assert m.dtype == torch.uint8 and m.shape == (w.B, w.T_k)
    assert ((L >= 256) & (L <= 2048)).all()
    for b in range(w.B):
        assert int(m[b].sum()) == w.T_k - int(L[b])
        assert not m[b, : int(L[b])].any()


def test_flop_formula_headline():
    w = WORKLOADS[HEADLINE]
    assert abs(w.flops() / 1e9 - 549.7558) < 1e-3


def test_grouped_workloads_shapes_and_flops():
    gqa = GROUPED_WORKLOADS["gqa4_causal_bf16_d1024_h16_b8_t4096"]
    mqa = GROUPED_WORKLOADS["mqa_causal_bf16_d1024_h16_b8_t4096"]
    assert (gqa.n_g, gqa.n_qkv) == (4, 1024 + 2 * 4 * 64)
    assert (mqa.n_g, mqa.n_qkv) == (1, 1024 + 2 * 64)
    # Q and output projections 4TD^2, K and V 4TD n_g d_k, attention 2T^2D (causal)
    T, D, B = 4096, 1024, 8
    for w in (gqa, mqa):
        expect = B * (4 * T * D * D + 4 * T * D * w.n_g * 64 + 2 * T * T * D)
        assert abs(w.flops() - expect) < 1
    # plain MHA draws are unchanged by the grouped-head field
    small = WORKLOADS[HEADLINE].shrink(B=1, T_q=8, T_k=8)
    assert make_inputs(small, 0)["w_qkv"].shape == (1024, 3072)


def test_decode_inputs_shapes_lengths_and_unused_rows():
    from mha_inputs import DECODE_WORKLOADS, make_decode_inputs
    import pytest
    for name, w in DECODE_WORKLOADS.items():
        small = w.shrink(B=3, T_max=96, lengths=(0, 96 - w.T_new))
        inp = make_decode_inputs(small, 0)
        assert inp["x"].shape == (3, w.T_new, w.D) and inp["x"].dtype == torch.bfloat16
        assert inp["w_qkv"].shape == (w.D, w.n_qkv)
        assert inp["k_cache"].shape == (3, w.n_g, 96, w.d_k)
        L = inp["cache_len"]
        assert L.dtype == torch.int32 and ((L >= 0) & (L <= 96 - w.T_new)).all()
        for b in range(3):
            assert torch.isnan(inp["k_cache"][b, :, int(L[b]):].float()).all()
            assert torch.isfinite(inp["v_cache"][b, :, :int(L[b])].float()).all()
    with pytest.raises(ValueError):
        make_decode_inputs(w.shrink(T_max=64, lengths=(0, 64)), 0)
