"""Pins of the oracle's grouped key/value heads (GQA, MQA) on the CPU.

itwiki "멀티 헤드 어텐션", 추론 비용과 변형: every variant keeps n_h query heads;
MQA shares one key/value set among all of them, GQA shares n_g sets, one per
group of query heads. The pins tie the oracle to brute force, to torch's
scaled_dot_product_attention with enable_gqa (float64), to plain multi-head
attention with each set's weights copied to its heads, to the table's cache
sizes and to a closed form.
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mha_oracle as mo
from oracle.brute import brute_force_mha

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _problem(rng, B, Tq, D, h, n_g, Tk=None, cross=False):
    d = D // h
    n_qkv = D + 2 * n_g * d
    return dict(
        x_q=rng.standard_normal((B, Tq, D)),
        x_kv=rng.standard_normal((B, Tk, D)) if cross else None,
        w_qkv=rng.standard_normal((D, n_qkv)) / math.sqrt(D),
        b_qkv=rng.standard_normal(n_qkv) * 0.1,
        w_o=rng.standard_normal((D, D)) / math.sqrt(D),
        b_o=rng.standard_normal(D) * 0.1,
    )


def _run(p, h, n_g, causal=False, mask=None, **kw):
    return mo.mha_forward(p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], h,
                          x_kv=p["x_kv"], causal=causal, key_padding_mask=mask,
                          n_kv_heads=n_g, **kw)


def _rel_err(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("h,n_g", [(2, 1), (4, 1), (4, 2)])
@pytest.mark.parametrize("T", [1, 3, 4])
@pytest.mark.parametrize("masking", ["none", "causal", "padding"])
@pytest.mark.parametrize("cross", [False, True])
def test_grouped_matches_brute_force(h, n_g, T, masking, cross):
    causal = masking == "causal"
    Tk = T + 1 if (cross and not causal) else T
    rng = np.random.default_rng(100 * h + 10 * n_g + T + (7 if cross else 0))
    p = _problem(rng, 2, T, 8, h, n_g, Tk=Tk, cross=cross)
    mask = None
    if masking == "padding" and Tk > 1:
        mask = np.zeros((2, Tk), dtype=np.uint8)
        mask[0, Tk - 1] = 1
        mask[1, 0] = 1
    y = _run(p, h, n_g, causal, mask)
    yb = brute_force_mha(
        p["x_q"].tolist(), p["w_qkv"].tolist(), p["b_qkv"].tolist(), p["w_o"].tolist(),
        p["b_o"].tolist(), h, x_kv=None if p["x_kv"] is None else p["x_kv"].tolist(),
        causal=causal, key_padding_mask=None if mask is None else mask.tolist(),
        n_kv_heads=n_g)
    assert _rel_err(y, yb) <= 1e-12


def _torch_sdpa_gqa(p, h, n_g, causal, mask):
    """The same layer with torch's projections and grouped SDPA (float64)."""
    t = lambda a: None if a is None else torch.from_numpy(np.asarray(a, dtype=np.float64))
    x_q, w, b, w_o, b_o = t(p["x_q"]), t(p["w_qkv"]), t(p["b_qkv"]), t(p["w_o"]), t(p["b_o"])
    x_kv = x_q if p["x_kv"] is None else t(p["x_kv"])
    B, Tq, D = x_q.shape
    Tk = x_kv.shape[1]
    d = D // h
    dkv = n_g * d
    q = F.linear(x_q, w[:, :D].T, b[:D]).view(B, Tq, h, d).transpose(1, 2)
    k = F.linear(x_kv, w[:, D:D + dkv].T, b[D:D + dkv]).view(B, Tk, n_g, d).transpose(1, 2)
    v = F.linear(x_kv, w[:, D + dkv:].T, b[D + dkv:]).view(B, Tk, n_g, d).transpose(1, 2)
    attn_mask = None
    if mask is not None:   # SDPA's boolean mask: True = may attend
        attn_mask = torch.from_numpy(mask == 0)[:, None, None, :]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=attn_mask, is_causal=causal,
                                       enable_gqa=True)
    o = o.transpose(1, 2).reshape(B, Tq, D)
    return F.linear(o, w_o.T, b_o).numpy()


@pytest.mark.parametrize("h,n_g", [(8, 1), (8, 2), (8, 4), (8, 8), (16, 4)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_grouped_matches_torch_sdpa_enable_gqa(h, n_g, causal, padded):
    rng = np.random.default_rng(7 * h + n_g + (100 if causal else 0) + (1000 if padded else 0))
    D = 16 * h if h == 8 else 8 * h
    T = 23
    p = _problem(rng, 3, T, D, h, n_g)
    mask = None
    if padded:
        mask = np.zeros((3, T), dtype=np.uint8)
        mask[0, 17:] = 1
        mask[1, 5:9] = 1
    y = _run(p, h, n_g, causal, mask)
    yt = _torch_sdpa_gqa(p, h, n_g, causal, mask)
    assert _rel_err(y, yt) <= 1e-12


def test_grouped_cross_attention_matches_torch_sdpa():
    rng = np.random.default_rng(5)
    h, n_g, D = 8, 2, 128
    p = _problem(rng, 2, 11, D, h, n_g, Tk=29, cross=True)
    mask = np.zeros((2, 29), dtype=np.uint8)
    mask[1, 20:] = 1
    assert _rel_err(_run(p, h, n_g, False, mask), _torch_sdpa_gqa(p, h, n_g, False, mask)) <= 1e-12


@pytest.mark.parametrize("h,n_g", [(4, 1), (4, 2), (8, 2)])
def test_grouped_equals_mha_with_shared_weights_copied(h, n_g):
    """A query head reading set g equals plain multi-head attention whose
    head i has set g's key and value weights; heads i of one group are the
    consecutive run [g*h/n_g, (g+1)*h/n_g)."""
    rng = np.random.default_rng(11 * h + n_g)
    D, d = 8 * h, 8
    p = _problem(rng, 2, 9, D, h, n_g)
    w, b = p["w_qkv"], p["b_qkv"]
    dkv = n_g * d
    wk, wv = w[:, D:D + dkv], w[:, D + dkv:]
    bk, bv = b[D:D + dkv], b[D + dkv:]
    per = h // n_g
    cols = [np.arange(d) + (i // per) * d for i in range(h)]
    wk_full = np.concatenate([wk[:, c] for c in cols], axis=1)
    wv_full = np.concatenate([wv[:, c] for c in cols], axis=1)
    bk_full = np.concatenate([bk[c] for c in cols])
    bv_full = np.concatenate([bv[c] for c in cols])
    q = dict(p, w_qkv=np.concatenate([w[:, :D], wk_full, wv_full], axis=1),
             b_qkv=np.concatenate([b[:D], bk_full, bv_full]))
    for causal in (False, True):
        y = _run(p, h, n_g, causal)
        y_mha = mo.mha_forward(q["x_q"], q["w_qkv"], q["b_qkv"], q["w_o"], q["b_o"], h,
                               causal=causal)
        assert _rel_err(y, y_mha) <= 1e-13


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [[int(v) for v in line.split()] for line in f
                if line.strip() and not line.startswith("#")]


def test_kv_elements_per_token_golden():
    rng = np.random.default_rng(3)
    for D, n_h, n_g, d_h, elements in _golden_rows("kv_cache_elements.txt"):
        assert D // n_h == d_h
        assert mo.kv_elements_per_token(D, n_h, n_g) == elements
        if D <= 512:
            p = _problem(rng, 1, 3, D, n_h, n_g)
            _, inter = _run(p, n_h, n_g, return_intermediates=True)
            B, g, T, d = inter["k"].shape
            assert inter["v"].shape == inter["k"].shape
            assert 2 * g * d == elements and T == 3


def test_mqa_single_key_closed_form():
    """One key per sequence: every head's weights are [1], so every head's
    output is the one shared value row v = x W_V + b_V, and
    Y = [v, v, ..., v] W_O + b_O."""
    rng = np.random.default_rng(9)
    h, D = 4, 32
    d = D // h
    p = _problem(rng, 2, 1, D, h, 1)
    y = _run(p, h, 1)
    wv = p["w_qkv"][:, D + d:]
    bv = p["b_qkv"][D + d:]
    v = p["x_q"][:, 0, :] @ wv + bv                      # (B, d)
    o = np.concatenate([v] * h, axis=1)                   # (B, D)
    expect = o @ p["w_o"] + p["b_o"]
    assert _rel_err(y[:, 0, :], expect) <= 1e-13


def test_rows_function_grouped():
    rng = np.random.default_rng(21)
    h, n_g, D = 8, 2, 64
    p = _problem(rng, 2, 13, D, h, n_g)
    y = _run(p, h, n_g, causal=True)
    rows = {0: [0, 5, 12], 1: [3]}
    got = mo.mha_forward_rows(p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], h, rows,
                              causal=True, n_kv_heads=n_g)
    for b, ts in rows.items():
        assert _rel_err(got[b], y[b, ts]) <= 1e-13


def test_bad_group_counts_are_errors():
    rng = np.random.default_rng(1)
    p = _problem(rng, 1, 2, 32, 4, 2)
    with pytest.raises(ValueError):
        _run(p, 4, 3)                       # 3 does not divide 4
    with pytest.raises(ValueError):
        _run(p, 4, 1)                       # W_QKV width is for n_g = 2
    with pytest.raises(ValueError):
        mo.kv_elements_per_token(32, 4, 0)


def test_planted_interleaved_groups_are_caught(monkeypatch):
    """Head i -> set i mod n_g (a plausible mistake) disagrees with torch."""
    rng = np.random.default_rng(2)
    h, n_g = 8, 2
    p = _problem(rng, 2, 10, 128, h, n_g)
    yt = _torch_sdpa_gqa(p, h, n_g, True, None)
    assert _rel_err(_run(p, h, n_g, True), yt) <= 1e-12
    monkeypatch.setattr(mo, "kv_head_of", lambda hh, g: np.arange(hh) % g)
    assert _rel_err(_run(p, h, n_g, True), yt) > 1e-3


def test_planted_v_block_offset_is_caught(monkeypatch):
    """Values taken from the neighbouring set (an off-by-one-head offset into
    the V block) disagree with torch."""
    rng = np.random.default_rng(4)
    h, n_g, D = 8, 4, 64
    p = _problem(rng, 2, 6, D, h, n_g)
    yt = _torch_sdpa_gqa(p, h, n_g, False, None)
    orig = mo._qkv

    def wrong(x_q, x_kv, w_qkv, b_qkv, D_):
        q, k, v = orig(x_q, x_kv, w_qkv, b_qkv, D_)
        return q, k, np.roll(v, 8, axis=-1)
    monkeypatch.setattr(mo, "_qkv", wrong)
    assert _rel_err(_run(p, h, n_g, False), yt) > 1e-3
