"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test ties the oracle to a fact the pages fix, a closed form, brute force,
or an independent library routine (torch.nn.MultiheadAttention in float64).
"""

import concurrent.futures
import math
import os

import numpy as np
import pytest
import torch

from oracle import mha_oracle as mo
from oracle.brute import brute_force_mha

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(v) for v in line.split()])
    return rows


def _rand_problem(rng, B, Tq, D, h, Tk=None, cross=False, scale=1.0, bias=True):
    x_q = rng.standard_normal((B, Tq, D))
    x_kv = rng.standard_normal((B, Tk, D)) if cross else None
    w_qkv = rng.standard_normal((D, 3 * D)) * scale / math.sqrt(D)
    w_o = rng.standard_normal((D, D)) / math.sqrt(D)
    b_qkv = rng.standard_normal(3 * D) * 0.1 if bias else None
    b_o = rng.standard_normal(D) * 0.1 if bias else None
    return dict(x_q=x_q, x_kv=x_kv, w_qkv=w_qkv, b_qkv=b_qkv, w_o=w_o, b_o=b_o)


def _run(p, h, causal=False, mask=None, **kw):
    return mo.mha_forward(p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], h,
                          x_kv=p["x_kv"], causal=causal, key_padding_mask=mask, **kw)


def _rel_err(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ---------------------------------------------------------------- brute force

MASKS = ["none", "causal", "padding", "causal+padding"]


@pytest.mark.parametrize("T", [1, 2, 3, 4])
@pytest.mark.parametrize("h", [1, 2, 4])
@pytest.mark.parametrize("mode", ["self", "cross"])
@pytest.mark.parametrize("masking", MASKS)
def test_oracle_matches_brute_force(T, h, mode, masking):
    cross = mode == "cross"
    causal = "causal" in masking
    Tk = T if (causal or not cross) else T + 1   # causal needs T_q == T_k
    rng = np.random.default_rng(1000 * T + 10 * h + MASKS.index(masking) + (5 if cross else 0))
    D = 8
    p = _rand_problem(rng, 2, T, D, h, Tk=Tk, cross=cross)
    mask = None
    if "padding" in masking:
        mask = np.zeros((2, Tk), dtype=np.uint8)
        mask[0, Tk - 1] = 1 if Tk > 1 else 0      # keep >= 1 valid key per row
        mask[1, 0] = 1 if Tk > 1 else 0
        if causal:
            mask[1, 0] = 0                         # causal row 0 sees key 0 only
    y = _run(p, h, causal, mask)
    yb = brute_force_mha(
        p["x_q"].tolist(), p["w_qkv"].tolist(), p["b_qkv"].tolist(), p["w_o"].tolist(),
        p["b_o"].tolist(), h, x_kv=None if p["x_kv"] is None else p["x_kv"].tolist(),
        causal=causal, key_padding_mask=None if mask is None else mask.tolist())
    assert _rel_err(y, yb) <= 1e-12


def test_brute_force_all_masked_row_is_nan_in_both():
    rng = np.random.default_rng(7)
    p = _rand_problem(rng, 2, 3, 8, 2)
    mask = np.zeros((2, 3), dtype=np.uint8)
    mask[1, :] = 1
    y = _run(p, 2, False, mask)
    yb = np.array(brute_force_mha(p["x_q"].tolist(), p["w_qkv"].tolist(), p["b_qkv"].tolist(),
                                  p["w_o"].tolist(), p["b_o"].tolist(), 2,
                                  key_padding_mask=mask.tolist()))
    assert np.isnan(y[1]).all() and np.isnan(yb[1]).all()
    assert np.isfinite(y[0]).all()
    assert _rel_err(y[0], yb[0]) <= 1e-12


# ------------------------------------------------- independent library routine

def _torch_mha(p, h, causal, mask):
    D = p["w_qkv"].shape[0]
    m = torch.nn.MultiheadAttention(D, h, batch_first=True, dtype=torch.float64)
    with torch.no_grad():
        m.in_proj_weight.copy_(torch.from_numpy(p["w_qkv"].T.copy()))
        m.in_proj_bias.copy_(torch.from_numpy(p["b_qkv"]))
        m.out_proj.weight.copy_(torch.from_numpy(p["w_o"].T.copy()))
        m.out_proj.bias.copy_(torch.from_numpy(p["b_o"]))
    m.train()   # keep the plain math path; dropout is 0
    xq = torch.from_numpy(p["x_q"])
    xkv = xq if p["x_kv"] is None else torch.from_numpy(p["x_kv"])
    Tq, Tk = xq.shape[1], xkv.shape[1]
    attn_mask = torch.ones(Tq, Tk, dtype=torch.bool).triu(1) if causal else None
    kpm = None if mask is None else torch.from_numpy(mask != 0)
    with torch.no_grad():
        y, w = m(xq, xkv, xkv, key_padding_mask=kpm, attn_mask=attn_mask,
                 need_weights=True, average_attn_weights=False)
    return y.numpy(), w.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
@pytest.mark.parametrize("cross", [False, True])
def test_oracle_matches_torch_multihead_attention_fp64(causal, padded, cross):
    if causal and cross:
        Tk = 24
    else:
        Tk = 37 if cross else 24
    rng = np.random.default_rng(11 + 2 * causal + 4 * padded + 8 * cross)
    p = _rand_problem(rng, 3, 24, 32, 4, Tk=Tk, cross=cross, scale=3.0)
    mask = None
    if padded:
        lengths = [Tk, Tk - 5, 3]
        mask = (np.arange(Tk)[None, :] >= np.array(lengths)[:, None]).astype(np.uint8)
    y, inter = _run(p, 4, causal, mask, return_intermediates=True)
    yt, wt = _torch_mha(p, 4, causal, mask)
    assert _rel_err(y, yt) <= 1e-12
    assert _rel_err(inter["a"], wt) <= 1e-12


# -------------------------------------------------------- invariants (pages)

def test_softmax_rows_sum_to_one_and_nonnegative():
    rng = np.random.default_rng(3)
    p = _rand_problem(rng, 2, 40, 32, 4, scale=4.0)
    for causal in (False, True):
        _, inter = _run(p, 4, causal, return_intermediates=True)
        a = inter["a"]
        assert (a >= 0).all()
        assert np.max(np.abs(a.sum(-1) - 1.0)) <= 1e-12


def test_causal_future_weights_exactly_zero_and_prefix_independence():
    rng = np.random.default_rng(4)
    p = _rand_problem(rng, 2, 33, 32, 4)
    y, inter = _run(p, 4, True, return_intermediates=True)
    a = inter["a"]
    T = a.shape[-1]
    future = np.triu(np.ones((T, T), dtype=bool), 1)
    assert (a[..., future] == 0.0).all()
    t = 17
    p2 = dict(p)
    p2["x_q"] = p["x_q"].copy()
    p2["x_q"][:, t + 1:] += rng.standard_normal(p["x_q"][:, t + 1:].shape)
    y2 = _run(p2, 4, True)
    assert np.array_equal(y[:, :t + 1], y2[:, :t + 1])
    assert not np.array_equal(y[:, t + 1:], y2[:, t + 1:])


def test_key_padding_ignores_masked_keys_bitwise():
    rng = np.random.default_rng(5)
    p = _rand_problem(rng, 2, 16, 32, 4, Tk=40, cross=True)
    mask = np.zeros((2, 40), dtype=np.uint8)
    mask[0, 30:] = 1
    mask[1, ::3] = 1
    y = _run(p, 4, False, mask)
    p2 = dict(p)
    p2["x_kv"] = p["x_kv"].copy()
    p2["x_kv"][mask != 0] += 100.0
    assert np.array_equal(y, _run(p2, 4, False, mask))


def test_batch_independence_bitwise():
    rng = np.random.default_rng(6)
    p = _rand_problem(rng, 4, 10, 32, 4)
    y = _run(p, 4, True)
    p2 = dict(p)
    p2["x_q"] = p["x_q"].copy()
    p2["x_q"][1] = rng.standard_normal(p["x_q"][1].shape)
    y2 = _run(p2, 4, True)
    assert np.array_equal(y[0], y2[0]) and np.array_equal(y[2:], y2[2:])
    assert not np.array_equal(y[1], y2[1])


def test_all_masked_row_gives_nan_only_there():
    rng = np.random.default_rng(8)
    p = _rand_problem(rng, 3, 6, 16, 2, Tk=9, cross=True)
    mask = np.zeros((3, 9), dtype=np.uint8)
    mask[2, :] = 1
    y = _run(p, 2, False, mask)
    assert np.isnan(y[2]).all()
    assert np.isfinite(y[:2]).all()


def test_embed_dim_not_divisible_is_an_error():
    rng = np.random.default_rng(9)
    p = _rand_problem(rng, 1, 3, 12, 1)
    with pytest.raises(ValueError):
        _run(p, 5)
    with pytest.raises(ValueError):
        mo.param_count(12, 5)


# ---------------------------------------------------- printed values (golden)

def test_param_count_golden_and_head_independent():
    (E, h1, head_dim, with_bias, without_bias), = _golden_rows("param_count.txt")
    assert E // h1 == head_dim
    for h in (1, 2, 4, 8, 16):
        assert mo.param_count(E, h) == with_bias
        assert mo.param_count(E, h, bias=False) == without_bias
        m = torch.nn.MultiheadAttention(E, h)
        assert sum(t.numel() for t in m.parameters()) == with_bias
    assert with_bias == 4 * E * E + 4 * E


def test_concat_width_golden():
    (h, d_v, width), = _golden_rows("concat_width.txt")
    D = h * d_v
    rng = np.random.default_rng(10)
    p = _rand_problem(rng, 2, 5, D, h)
    y, inter = _run(p, h, False, return_intermediates=True)
    o = inter["o"]
    assert o.shape == (2, 5, width)
    # head i computed on its own lands in columns [i*d_v, (i+1)*d_v)
    for i in range(h):
        cols = slice(i * d_v, (i + 1) * d_v)
        q = p["x_q"] @ p["w_qkv"][:, :D][:, cols] + p["b_qkv"][:D][cols]
        k = p["x_q"] @ p["w_qkv"][:, D:2 * D][:, cols] + p["b_qkv"][D:2 * D][cols]
        v = p["x_q"] @ p["w_qkv"][:, 2 * D:][:, cols] + p["b_qkv"][2 * D:][cols]
        s = np.einsum("btc,bsc->bts", q, k) / math.sqrt(d_v)
        a = np.exp(s) / np.exp(s).sum(-1, keepdims=True)
        assert _rel_err(o[..., cols], a @ v) <= 1e-12


def test_original_setting_golden():
    (d_model, h, d_k, d_v), = _golden_rows("original_setting.txt")
    assert d_model // h == d_k == d_v
    rng = np.random.default_rng(12)
    p = _rand_problem(rng, 1, 3, d_model, h)
    _, inter = _run(p, h, False, return_intermediates=True)
    assert inter["q"].shape == (1, h, 3, d_k)


# ------------------------------------------------------------- closed forms

def test_single_head_is_plain_scaled_dot_product_attention():
    """h = 1: iamjaehka13.blog §16 single-head formula (without the residual)."""
    rng = np.random.default_rng(13)
    D, T = 24, 11
    p = _rand_problem(rng, 2, T, D, 1)
    y = _run(p, 1, True)
    Wq, Wk, Wv = p["w_qkv"][:, :D], p["w_qkv"][:, D:2 * D], p["w_qkv"][:, 2 * D:]
    bq, bk, bv = p["b_qkv"][:D], p["b_qkv"][D:2 * D], p["b_qkv"][2 * D:]
    M = np.where(np.triu(np.ones((T, T), dtype=bool), 1), -np.inf, 0.0)
    for b in range(2):
        X = p["x_q"][b]
        Q, K, V = X @ Wq + bq, X @ Wk + bk, X @ Wv + bv
        S = Q @ K.T / math.sqrt(D) + M
        A = np.exp(S - S.max(1, keepdims=True))
        A /= A.sum(1, keepdims=True)
        assert _rel_err(y[b], (A @ V) @ p["w_o"] + p["b_o"]) <= 1e-12


def test_per_head_matrices_equal_fused_matrix():
    """MultiHead with h separate (W_i^Q, W_i^K, W_i^V) equals one D x 3D matrix."""
    rng = np.random.default_rng(14)
    D, h, T = 32, 4, 9
    d = D // h
    p = _rand_problem(rng, 2, T, D, h)
    y = _run(p, h, False)
    heads = []
    for i in range(h):
        Wq = p["w_qkv"][:, i * d:(i + 1) * d]
        Wk = p["w_qkv"][:, D + i * d:D + (i + 1) * d]
        Wv = p["w_qkv"][:, 2 * D + i * d:2 * D + (i + 1) * d]
        bq = p["b_qkv"][i * d:(i + 1) * d]
        bk = p["b_qkv"][D + i * d:D + (i + 1) * d]
        bv = p["b_qkv"][2 * D + i * d:2 * D + (i + 1) * d]
        Q = (p["x_q"] @ Wq + bq)[:, None]
        K = (p["x_q"] @ Wk + bk)[:, None]
        V = (p["x_q"] @ Wv + bv)[:, None]
        o, _ = mo.attention(Q, K, V)
        heads.append(o[:, 0])
    o_cat = np.concatenate(heads, axis=-1)
    assert _rel_err(y, o_cat @ p["w_o"] + p["b_o"]) <= 1e-12


def test_single_key_output_is_projected_value():
    rng = np.random.default_rng(15)
    D = 16
    p = _rand_problem(rng, 3, 5, D, 4, Tk=1, cross=True)
    y = _run(p, 4, False)
    v = p["x_kv"] @ p["w_qkv"][:, 2 * D:] + p["b_qkv"][2 * D:]       # (B, 1, D)
    expect = np.broadcast_to(v @ p["w_o"] + p["b_o"], y.shape)
    assert _rel_err(y, expect) <= 1e-12


def test_zero_query_weights_give_uniform_prefix_mean():
    rng = np.random.default_rng(16)
    D, T = 16, 12
    p = _rand_problem(rng, 2, T, D, 4)
    p["w_qkv"][:, :D] = 0.0
    p["b_qkv"][:D] = 0.0
    y = _run(p, 4, True)
    V = p["x_q"] @ p["w_qkv"][:, 2 * D:] + p["b_qkv"][2 * D:]
    prefix_mean = np.cumsum(V, axis=1) / np.arange(1, T + 1)[None, :, None]
    assert _rel_err(y, prefix_mean @ p["w_o"] + p["b_o"]) <= 1e-12
    y_nc = _run(p, 4, False)
    full_mean = V.mean(axis=1, keepdims=True)
    assert _rel_err(y_nc, np.broadcast_to(full_mean @ p["w_o"] + p["b_o"], y_nc.shape)) <= 1e-12


def test_identical_keys_give_uniform_weights():
    rng = np.random.default_rng(17)
    D = 16
    p = _rand_problem(rng, 1, 4, D, 2, Tk=6, cross=True)
    p["x_kv"][:] = p["x_kv"][:, :1]
    _, inter = _run(p, 2, False, return_intermediates=True)
    assert np.max(np.abs(inter["a"] - 1.0 / 6.0)) <= 1e-15


def test_permutation_equivariance_non_causal():
    rng = np.random.default_rng(18)
    p = _rand_problem(rng, 2, 13, 32, 4)
    y = _run(p, 4, False)
    perm = rng.permutation(13)
    p2 = dict(p)
    p2["x_q"] = p["x_q"][:, perm]
    assert _rel_err(_run(p2, 4, False), y[:, perm]) <= 1e-12


def test_rows_function_equals_full_forward_rows():
    rng = np.random.default_rng(19)
    for cross, causal in ((False, True), (True, False)):
        p = _rand_problem(rng, 3, 20, 32, 4, Tk=20 if causal else 27, cross=cross)
        mask = None
        if cross:
            mask = (np.arange(27)[None, :] >= np.array([27, 9, 1])[:, None]).astype(np.uint8)
        y = _run(p, 4, causal, mask)
        rows = {0: [0, 5, 19], 2: [3, 4]}
        got = mo.mha_forward_rows(p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], 4,
                                  rows, x_kv=p["x_kv"], causal=causal, key_padding_mask=mask)
        for b, ts in rows.items():
            assert _rel_err(got[b], y[b, ts]) <= 1e-12


@pytest.mark.parametrize("rows_per_block", [1, 3, 7, 64])
def test_blocked_function_equals_full_forward(rows_per_block):
    """The row-blocked evaluation used for full-size comparisons returns the
    whole of mha_forward's Y (NaN rows included), for self/cross, causal,
    padded (leading, interior and all-masked rows), grouped and residual."""
    rng = np.random.default_rng(40 + rows_per_block)
    cases = []
    p = _rand_problem(rng, 3, 20, 32, 4)
    mask = np.zeros((3, 20), dtype=np.uint8)
    mask[0, :5] = 1            # leading keys: causal rows 0..4 see none -> NaN
    mask[1, 7:12] = 1
    cases.append((p, True, mask, {}))
    p = _rand_problem(rng, 2, 11, 32, 4, Tk=17, cross=True)
    mask = np.zeros((2, 17), dtype=np.uint8)
    mask[1, :] = 1             # every key of batch element 1 ignored
    cases.append((p, False, mask, dict(residual=True)))
    p = _rand_problem(rng, 2, 13, 32, 4)
    d_k = 8
    p["w_qkv"] = rng.standard_normal((32, 32 + 2 * 2 * d_k)) / math.sqrt(32)
    p["b_qkv"] = rng.standard_normal(32 + 2 * 2 * d_k) * 0.1
    cases.append((p, True, None, dict(n_kv_heads=2)))
    for p, causal, mask, kw in cases:
        y = _run(p, 4, causal, mask, **kw)
        calls = []
        got = mo.mha_forward_blocked(p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], 4,
                                     x_kv=p["x_kv"], causal=causal, key_padding_mask=mask,
                                     rows_per_block=rows_per_block,
                                     progress=lambda b, t0, t1: calls.append((b, t0, t1)), **kw)
        assert np.array_equal(np.isnan(got), np.isnan(y))
        ok = ~np.isnan(y)
        assert _rel_err(got[ok], y[ok]) <= 1e-12
        B, T = y.shape[:2]
        assert calls[-1] == (B - 1, (T - 1) // rows_per_block * rows_per_block, T)
        # blocks evaluated concurrently: the same values, bit for bit
        with concurrent.futures.ThreadPoolExecutor(4) as ex:
            par = mo.mha_forward_blocked(p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], 4,
                                         x_kv=p["x_kv"], causal=causal, key_padding_mask=mask,
                                         rows_per_block=rows_per_block, map_blocks=ex.map, **kw)
        assert np.array_equal(par, got, equal_nan=True)
    # the leading-padding case really produced NaN rows
    assert np.isnan(_run(cases[0][0], 4, True, cases[0][2])[0, :5]).all()


def test_blocked_function_matches_brute_force():
    """Pinned directly too: brute force at T <= 4 (causal + padding, cross)."""
    rng = np.random.default_rng(48)
    for cross, causal in ((False, True), (True, False)):
        Tk = 4 if causal else 3
        p = _rand_problem(rng, 2, 4, 8, 2, Tk=Tk, cross=cross)
        mask = np.zeros((2, Tk), dtype=np.uint8)
        mask[1, 1] = 1
        got = mo.mha_forward_blocked(p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], 2,
                                     x_kv=p["x_kv"], causal=causal, key_padding_mask=mask,
                                     rows_per_block=3)
        yb = brute_force_mha(
            p["x_q"].tolist(), p["w_qkv"].tolist(), p["b_qkv"].tolist(), p["w_o"].tolist(),
            p["b_o"].tolist(), 2, x_kv=None if p["x_kv"] is None else p["x_kv"].tolist(),
            causal=causal, key_padding_mask=mask.tolist())
        assert _rel_err(got, yb) <= 1e-12


# ------------------------------------------------ planted mistakes are caught

def test_planted_wrong_scale_is_caught(monkeypatch):
    """The d_k (not sqrt(d_k)) denominator printed on one page must fail."""
    rng = np.random.default_rng(20)
    p = _rand_problem(rng, 2, 8, 16, 2, scale=3.0)
    yt, _ = _torch_mha(p, 2, False, None)
    orig = mo.masked_scores

    def wrong(q, k, causal, kpm, q_pos=None):
        return orig(q, k, causal, kpm, q_pos) / math.sqrt(q.shape[-1])

    monkeypatch.setattr(mo, "masked_scores", wrong)
    assert _rel_err(_run(p, 2), yt) > 1e-3


def test_planted_zero_mask_is_caught(monkeypatch):
    """Masking with 0 instead of -inf leaves weight on future keys."""
    rng = np.random.default_rng(21)
    p = _rand_problem(rng, 1, 6, 16, 2)
    yb = brute_force_mha(p["x_q"].tolist(), p["w_qkv"].tolist(), p["b_qkv"].tolist(),
                         p["w_o"].tolist(), p["b_o"].tolist(), 2, causal=True)

    def zero_masked(q, k, causal, kpm, q_pos=None):
        s = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(q.shape[-1])
        if causal:
            T = s.shape[-1]
            s = np.where(np.triu(np.ones((T, T), dtype=bool), 1), 0.0, s)
        return s

    monkeypatch.setattr(mo, "masked_scores", zero_masked)
    assert _rel_err(_run(p, 2, True), yb) > 1e-3


def test_planted_swapped_kv_blocks_are_caught(monkeypatch):
    rng = np.random.default_rng(22)
    p = _rand_problem(rng, 1, 4, 8, 2)
    yb = brute_force_mha(p["x_q"].tolist(), p["w_qkv"].tolist(), p["b_qkv"].tolist(),
                         p["w_o"].tolist(), p["b_o"].tolist(), 2)
    orig = mo._qkv

    def swapped(x_q, x_kv, w, b, D):
        q, k, v = orig(x_q, x_kv, w, b, D)
        return q, v, k

    monkeypatch.setattr(mo, "_qkv", swapped)
    assert _rel_err(_run(p, 2), yb) > 1e-3


def test_planted_head_transpose_is_caught(monkeypatch):
    """Splitting columns as (d_k, h) instead of (h, d_k) must fail."""
    rng = np.random.default_rng(23)
    p = _rand_problem(rng, 1, 4, 8, 2)
    yb = brute_force_mha(p["x_q"].tolist(), p["w_qkv"].tolist(), p["b_qkv"].tolist(),
                         p["w_o"].tolist(), p["b_o"].tolist(), 2)

    def wrong_split(y, h):
        B, T, D = y.shape
        return y.reshape(B, T, D // h, h).transpose(0, 3, 1, 2)

    monkeypatch.setattr(mo, "split_heads", wrong_split)
    assert _rel_err(_run(p, 2), yb) > 1e-3
