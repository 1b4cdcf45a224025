"""Pins of the oracle's gated attention (CPU only).

itwiki "멀티 헤드 어텐션", 추론 비용과 변형, last paragraph: the scaled
dot-product attention output of each head is multiplied by a sigmoid gate of
its own. Reading taken (the page does not say what the gate is computed
from): one gate per batch element, query position and head, sigma(x_q . W_G
+ b_G) with W_G (D, h), multiplying head i's output before the concat.

* brute force (scalar formulas in Python floats) at T <= 4;
* gate -> 1 (large positive b_G) is bitwise the ungated layer;
* gate = 1/2 (W_G = 0, b_G = 0) halves every head's output, so
  Y - b_O is half of the ungated Y - b_O;
* gate -> 0 leaves only b_O (NaN rows stay NaN);
* grouped key/value heads: the gate belongs to the query head;
* the row-wise and row-blocked evaluations agree with the full one;
* planted mistakes (gate indexed by key/value set instead of query head,
  query positions reversed, applied without the sigmoid) fail the
  brute-force pin.
"""

import math

import numpy as np
import pytest

from oracle import mha_oracle as mo
from oracle.brute import brute_force_mha


def _problem(rng, B, Tq, D, h, Tk=None, cross=False, n_g=None):
    d_k = D // h
    n_g = h if n_g is None else n_g
    n_qkv = D + 2 * n_g * d_k
    return dict(x_q=rng.standard_normal((B, Tq, D)),
                x_kv=rng.standard_normal((B, Tk, D)) if cross else None,
                w_qkv=rng.standard_normal((D, n_qkv)) / math.sqrt(D),
                b_qkv=rng.standard_normal(n_qkv) * 0.1,
                w_o=rng.standard_normal((D, D)) / math.sqrt(D),
                b_o=rng.standard_normal(D) * 0.1,
                gate_w=rng.standard_normal((D, h)) / math.sqrt(D) * 2.0,
                gate_b=rng.standard_normal(h) * 0.5)


def _run(p, h, causal=False, mask=None, gate=True, **kw):
    return mo.mha_forward(p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], h,
                          x_kv=p["x_kv"], causal=causal, key_padding_mask=mask,
                          gate_w=p["gate_w"] if gate else None,
                          gate_b=p["gate_b"] if gate else None, **kw)


def _brute(p, h, causal=False, mask=None, n_g=None):
    tl = lambda a: None if a is None else a.tolist()
    return np.array(brute_force_mha(tl(p["x_q"]), tl(p["w_qkv"]), tl(p["b_qkv"]), tl(p["w_o"]),
                                    tl(p["b_o"]), h, x_kv=tl(p["x_kv"]), causal=causal,
                                    key_padding_mask=tl(mask), n_kv_heads=n_g,
                                    gate_w=tl(p["gate_w"]), gate_b=tl(p["gate_b"])))


def _rel(a, b):
    ok = ~np.isnan(b)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    return float(np.max(np.abs(a[ok] - b[ok])) / max(np.max(np.abs(b[ok])), 1e-300))


@pytest.mark.parametrize("T", [1, 2, 4])
@pytest.mark.parametrize("h,n_g", [(1, 1), (2, 2), (4, 4), (4, 2), (4, 1)])
@pytest.mark.parametrize("mode", ["self causal", "cross padded"])
def test_gate_matches_brute_force(T, h, n_g, mode):
    rng = np.random.default_rng(100 * T + 10 * h + n_g + (5 if "cross" in mode else 0))
    D = 8
    cross = "cross" in mode
    Tk = T + 1 if cross else T
    p = _problem(rng, 2, T, D, h, Tk=Tk, cross=cross, n_g=n_g)
    mask = None
    if cross:
        mask = np.zeros((2, Tk), dtype=np.uint8)
        mask[1, 0] = 1
    y = _run(p, h, causal=not cross, mask=mask, n_kv_heads=n_g)
    assert _rel(y, _brute(p, h, causal=not cross, mask=mask, n_g=n_g)) <= 1e-12


def test_gate_of_one_is_the_ungated_layer():
    rng = np.random.default_rng(1)
    p = _problem(rng, 2, 9, 32, 4)
    p["gate_b"] = np.full(4, 60.0)          # sigma(>= 37) == 1.0 in float64
    p["gate_w"] = p["gate_w"] * 1e-3
    assert np.array_equal(_run(p, 4, causal=True), _run(p, 4, causal=True, gate=False))


def test_gate_of_one_half_halves_the_heads():
    rng = np.random.default_rng(2)
    p = _problem(rng, 2, 9, 32, 4, Tk=11, cross=True)
    p["gate_w"] = np.zeros((32, 4))
    p["gate_b"] = np.zeros(4)
    yg = _run(p, 4)
    y = _run(p, 4, gate=False)
    assert np.max(np.abs((yg - p["b_o"]) - 0.5 * (y - p["b_o"]))) <= 1e-14 * np.max(np.abs(y))


def test_gate_of_zero_leaves_the_bias_and_nan_rows():
    rng = np.random.default_rng(3)
    p = _problem(rng, 2, 6, 16, 2, Tk=6, cross=True)
    p["gate_w"] = np.zeros((16, 2))
    p["gate_b"] = np.full(2, -800.0)        # exp(800) overflows: sigma = 0 exactly
    mask = np.zeros((2, 6), dtype=np.uint8)
    mask[1, :] = 1                          # batch element 1: every key ignored
    y = _run(p, 2, mask=mask)
    assert np.array_equal(y[0], np.broadcast_to(p["b_o"], y[0].shape))
    assert np.isnan(y[1]).all()


def test_gate_changes_only_its_head():
    """Changing the gate column of head 1 changes Y by (delta sigma) times that
    head's ungated output through its rows of W_O (head 1 alone: W_O rows of
    the other heads zeroed)."""
    rng = np.random.default_rng(4)
    D, h = 32, 4
    p = _problem(rng, 2, 7, D, h)
    p2 = dict(p)
    p2["gate_w"] = p["gate_w"].copy()
    p2["gate_w"][:, 1] += rng.standard_normal(D)
    d = _run(p2, h, causal=True) - _run(p, h, causal=True)
    only1 = dict(p)
    w1 = np.zeros_like(p["w_o"])
    w1[8:16] = p["w_o"][8:16]
    only1["w_o"], only1["b_o"] = w1, np.zeros(D)
    s1 = mo.head_gates(p["x_q"], p["gate_w"], p["gate_b"])[..., 1]
    s2 = mo.head_gates(p["x_q"], p2["gate_w"], p2["gate_b"])[..., 1]
    y1 = _run(only1, h, causal=True, gate=False)      # head 1's ungated contribution
    assert np.max(np.abs(d - (s2 - s1)[..., None] * y1)) <= 1e-13 * np.max(np.abs(y1))


def test_grouped_gate_belongs_to_the_query_head():
    """n_g sets: equal to plain MHA whose heads carry copies of their set's K
    and V weights, with the same per-query-head gates."""
    rng = np.random.default_rng(5)
    D, h, n_g = 32, 4, 2
    d_k = D // h
    p = _problem(rng, 2, 8, D, h, n_g=n_g)
    sel = np.arange(h) // (h // n_g)
    cols_k = np.concatenate([D + g * d_k + np.arange(d_k) for g in sel])
    cols_v = np.concatenate([D + n_g * d_k + g * d_k + np.arange(d_k) for g in sel])
    cols = np.concatenate([np.arange(D), cols_k, cols_v])
    plain = dict(p, w_qkv=p["w_qkv"][:, cols], b_qkv=p["b_qkv"][cols])
    assert _rel(_run(p, h, causal=True, n_kv_heads=n_g), _run(plain, h, causal=True)) <= 1e-13


def test_rows_and_blocked_agree_with_full():
    rng = np.random.default_rng(6)
    p = _problem(rng, 3, 13, 32, 4, Tk=17, cross=True)
    mask = np.zeros((3, 17), dtype=np.uint8)
    mask[2, 5:] = 1
    y = _run(p, 4, mask=mask, residual=True)
    kw = dict(x_kv=p["x_kv"], key_padding_mask=mask, residual=True, gate_w=p["gate_w"],
              gate_b=p["gate_b"])
    args = (p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], 4)
    rows = mo.mha_forward_rows(*args, {0: [0, 12], 2: [3]}, **kw)
    assert _rel(rows[0], y[0, [0, 12]]) <= 1e-13 and _rel(rows[2], y[2, [3]]) <= 1e-13
    assert _rel(mo.mha_forward_blocked(*args, rows_per_block=5, **kw), y) <= 1e-13


@pytest.mark.parametrize("mistake", ["by set", "reversed positions", "no sigmoid"])
def test_planted_gate_mistakes_are_caught(monkeypatch, mistake):
    rng = np.random.default_rng(7)
    D, h, n_g = 16, 4, 2
    p = _problem(rng, 2, 4, D, h, n_g=n_g)
    p["x_kv"] = rng.standard_normal((2, 4, D))
    yb = _brute(p, h, causal=True, n_g=n_g)
    orig = mo.apply_gates

    if mistake == "by set":
        def wrong(o, gates):
            return orig(o, gates[..., np.arange(o.shape[1]) // (o.shape[1] // n_g)])
        monkeypatch.setattr(mo, "apply_gates", wrong)
    elif mistake == "reversed positions":
        def wrong(o, gates):
            return orig(o, gates[:, ::-1])
        monkeypatch.setattr(mo, "apply_gates", wrong)
    else:
        monkeypatch.setattr(mo, "sigmoid", lambda x: np.asarray(x, dtype=np.float64))
    y = mo.mha_forward(p["x_q"], p["w_qkv"], p["b_qkv"], p["w_o"], p["b_o"], h, causal=True,
                       n_kv_heads=n_g, gate_w=p["gate_w"], gate_b=p["gate_b"])
    assert _rel(y, yb) > 1e-3
