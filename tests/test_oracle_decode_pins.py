"""Pins of the oracle's generation step against a KV cache (CPU only).

iamjaehka13.blog §21 and itwiki "멀티 헤드 어텐션", 추론 비용과 변형: earlier
tokens' keys and values are kept in a cache, so a step projects only the new
tokens and attends over cached plus new keys. The defining property pinned
here: with the cache holding exactly the earlier tokens' keys and values, the
step's outputs equal the corresponding rows of the full causal forward pass.
Also pinned: brute force, torch's grouped SDPA with an explicit mask, and
that cache rows past the valid length are never read.
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mha_oracle as mo
from oracle.brute import brute_force_decode


def _weights(rng, D, h, n_g):
    d = D // h
    n_qkv = D + 2 * n_g * d
    return dict(w_qkv=rng.standard_normal((D, n_qkv)) / math.sqrt(D),
                b_qkv=rng.standard_normal(n_qkv) * 0.1,
                w_o=rng.standard_normal((D, D)) / math.sqrt(D),
                b_o=rng.standard_normal(D) * 0.1)


def _rel_err(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def _decode(p, h, n_g, x_new, kc, vc, lens):
    return mo.mha_decode(x_new, p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], h, kc, vc, lens,
                         n_kv_heads=n_g)


@pytest.mark.parametrize("h,n_g", [(2, 2), (2, 1), (4, 2)])
@pytest.mark.parametrize("T_new", [1, 2, 3])
def test_decode_matches_brute_force(h, n_g, T_new):
    rng = np.random.default_rng(10 * h + n_g + 100 * T_new)
    D, T_max = 8, 6
    p = _weights(rng, D, h, n_g)
    lens = [0, 3]
    x_new = rng.standard_normal((2, T_new, D))
    kc = rng.standard_normal((2, n_g, T_max, D // h))
    vc = rng.standard_normal((2, n_g, T_max, D // h))
    y, _, _ = _decode(p, h, n_g, x_new, kc, vc, lens)
    yb = brute_force_decode(x_new.tolist(), p["w_qkv"].tolist(), p["b_qkv"].tolist(),
                            p["w_o"].tolist(), p["b_o"].tolist(), h, kc.tolist(), vc.tolist(),
                            lens, n_kv_heads=n_g)
    assert _rel_err(y, yb) <= 1e-12


@pytest.mark.parametrize("h,n_g", [(4, 4), (4, 1), (8, 2)])
@pytest.mark.parametrize("T_new", [1, 4])
def test_decode_with_exact_cache_equals_full_causal_forward(h, n_g, T_new):
    """Cache = the prefix's own keys and values: the step reproduces rows
    L .. L + T_new - 1 of the causal forward pass over prefix + new tokens."""
    rng = np.random.default_rng(7 * h + n_g + T_new)
    D = 8 * h
    p = _weights(rng, D, h, n_g)
    lens = [0, 5, 13]
    T_max = 16
    B = len(lens)
    x_new = rng.standard_normal((B, T_new, D))
    kc = np.full((B, n_g, T_max, D // h), np.nan)
    vc = np.full((B, n_g, T_max, D // h), np.nan)
    prefixes = []
    for b, L in enumerate(lens):
        x_pre = rng.standard_normal((1, L, D))
        prefixes.append(x_pre)
        if L:
            _, inter = mo.mha_forward(x_pre, p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], h,
                                      causal=True, return_intermediates=True, n_kv_heads=n_g)
            kc[b, :, :L] = inter["k"][0]
            vc[b, :, :L] = inter["v"][0]
    y, k_new, v_new = _decode(p, h, n_g, x_new, kc, vc, lens)
    for b, L in enumerate(lens):
        x_full = np.concatenate([prefixes[b], x_new[b:b + 1]], axis=1)
        y_full, inter = mo.mha_forward(x_full, p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], h,
                                       causal=True, return_intermediates=True, n_kv_heads=n_g)
        assert _rel_err(y[b], y_full[0, L:]) <= 1e-12
        assert _rel_err(k_new[b], inter["k"][0, :, L:]) <= 1e-13
        assert _rel_err(v_new[b], inter["v"][0, :, L:]) <= 1e-13


def _torch_decode(p, h, n_g, x_new, kc, vc, lens):
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    w, b, w_o, b_o = t(p["w_qkv"]), t(p["b_qkv"]), t(p["w_o"]), t(p["b_o"])
    B, T_new, D = x_new.shape
    d = D // h
    dkv = n_g * d
    x = t(x_new)
    q = F.linear(x, w[:, :D].T, b[:D]).view(B, T_new, h, d).transpose(1, 2)
    k = F.linear(x, w[:, D:D + dkv].T, b[D:D + dkv]).view(B, T_new, n_g, d).transpose(1, 2)
    v = F.linear(x, w[:, D + dkv:].T, b[D + dkv:]).view(B, T_new, n_g, d).transpose(1, 2)
    out = []
    for bb in range(B):
        L = lens[bb]
        kk = torch.cat([t(kc[bb, :, :L]), k[bb]], dim=1)[None]
        vv = torch.cat([t(vc[bb, :, :L]), v[bb]], dim=1)[None]
        pos_q = L + torch.arange(T_new)[:, None]
        pos_k = torch.arange(L + T_new)[None, :]
        o = F.scaled_dot_product_attention(q[bb:bb + 1], kk, vv, attn_mask=pos_k <= pos_q,
                                           enable_gqa=True)
        out.append(o.transpose(1, 2).reshape(1, T_new, D))
    return F.linear(torch.cat(out), w_o.T, b_o).numpy()


@pytest.mark.parametrize("h,n_g", [(8, 8), (8, 2), (16, 1)])
@pytest.mark.parametrize("T_new", [1, 3])
def test_decode_matches_torch_sdpa(h, n_g, T_new):
    rng = np.random.default_rng(3 * h + n_g + T_new)
    D = 8 * h
    p = _weights(rng, D, h, n_g)
    lens = [0, 1, 17, 40]
    T_max = 48
    x_new = rng.standard_normal((4, T_new, D))
    kc = rng.standard_normal((4, n_g, T_max, D // h))
    vc = rng.standard_normal((4, n_g, T_max, D // h))
    y, _, _ = _decode(p, h, n_g, x_new, kc, vc, lens)
    assert _rel_err(y, _torch_decode(p, h, n_g, x_new, kc, vc, lens)) <= 1e-12


def test_empty_cache_equals_causal_forward_of_new_tokens():
    rng = np.random.default_rng(5)
    h, n_g, D = 4, 2, 32
    p = _weights(rng, D, h, n_g)
    x_new = rng.standard_normal((2, 5, D))
    kc = np.zeros((2, n_g, 8, 8))
    y, _, _ = _decode(p, h, n_g, x_new, kc, kc, [0, 0])
    y_full = mo.mha_forward(x_new, p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], h, causal=True,
                            n_kv_heads=n_g)
    assert _rel_err(y, y_full) <= 1e-13


def test_rows_past_cache_length_are_never_read():
    rng = np.random.default_rng(6)
    h, n_g, D = 4, 1, 32
    p = _weights(rng, D, h, n_g)
    x_new = rng.standard_normal((2, 2, D))
    kc = rng.standard_normal((2, n_g, 10, 8))
    vc = rng.standard_normal((2, n_g, 10, 8))
    lens = [4, 7]
    y1, _, _ = _decode(p, h, n_g, x_new, kc, vc, lens)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[0, :, 4:] = np.nan
    vc2[0, :, 4:] = 1e300
    kc2[1, :, 7:] = np.inf
    y2, _, _ = _decode(p, h, n_g, x_new, kc2, vc2, lens)
    assert np.array_equal(y1, y2)


def test_cache_length_out_of_range_is_an_error():
    rng = np.random.default_rng(8)
    p = _weights(rng, 32, 4, 4)
    kc = np.zeros((1, 4, 6, 8))
    with pytest.raises(ValueError):
        _decode(p, 4, 4, rng.standard_normal((1, 1, 32)), kc, kc, [7])


def test_planted_position_shift_is_caught(monkeypatch):
    """Placing the new tokens one position late (a new token seeing the next
    new token) breaks the full-forward equality."""
    rng = np.random.default_rng(9)
    h, n_g, D = 4, 2, 32
    p = _weights(rng, D, h, n_g)
    x_new = rng.standard_normal((1, 3, D))
    kc = np.zeros((1, n_g, 4, 8))
    y_ref = mo.mha_forward(x_new, p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], h, causal=True,
                           n_kv_heads=n_g)
    orig = mo._attend_grouped

    def shifted(qh, kh, vh, g, causal, mask, q_pos=None):
        return orig(qh, kh, vh, g, causal, mask, None if q_pos is None else q_pos + 1)
    monkeypatch.setattr(mo, "_attend_grouped", shifted)
    y, _, _ = _decode(p, h, n_g, x_new, kc, kc, [0])
    assert _rel_err(y, y_ref) > 1e-3
