"""Pins of the storage-plan rounding emulator (oracle/precision_plan.py).

* The rounding function against the library casts that implement the same
  IEEE formats (numpy's float16 and float32, torch's bfloat16), and against
  hand-worked ties and overflow values.
* With no rounding the emulator is the oracle's forward pass; prescaling Q
  into log2 units changes nothing in exact arithmetic.
* One storage point at a time: Y rounded is the oracle's Y rounded; V
  rounded is the oracle's weights times rounded V; P rounded stays inside
  the bound that a relative perturbation of at most u = 2^-11 of every
  numerator allows (each normalised weight moves by at most 2u/(1-u) of
  itself, so |dO| <= 2u/(1-u) max |v|).
* The early-row correction: rows t < R0 of causal self-attention at fp32
  level, the other rows untouched; hi + lo keeps 22 significant bits (down
  to an absolute 2^-25 where the remainder is below the fp16 normal range).
* The budget the plan was chosen by: on the d512/h8/t1024 causal workload
  (two batch elements), 16-bit bf16 storage exceeds the 2e-2 tolerance,
  fp16 storage stays inside it, the early-row correction shrinks it further.
"""

import math

import numpy as np
import pytest
import torch

from mha_inputs import WORKLOADS, as_float64_numpy, make_inputs
from oracle import mha_oracle as mo
from oracle.precision_plan import (KERNEL_PLAN, PLANS, Plan, emulate, max_abs_over_rms,
                                   round_to, split_hi_lo)

U16 = 2.0 ** -11


def _spread(rng, n, lo, hi):
    mant = rng.uniform(0.5, 1.0, n) * np.where(rng.uniform(size=n) < 0.5, -1.0, 1.0)
    return np.ldexp(mant, rng.integers(lo, hi, n))


def test_round_to_fp16_matches_numpy_half():
    rng = np.random.default_rng(0)
    x = _spread(rng, 200_000, -30, 18)
    # exact ties: odd multiples of half a quantum at several binades
    e = rng.integers(-24, 16, 20_000)
    ties = np.ldexp(2.0 * rng.integers(1024, 2048, 20_000) + 1.0, e - 11)
    x = np.concatenate([x, ties, -ties, [0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99,
                                         65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25]])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).astype(np.float64)
    got = round_to(x, "fp16")
    assert np.array_equal(got, ref)
    assert np.array_equal(np.signbit(got), np.signbit(ref))


def test_round_to_fp32_matches_numpy_single():
    rng = np.random.default_rng(1)
    x = _spread(rng, 200_000, -155, 129)
    ties = np.ldexp(2.0 * rng.integers(2 ** 23, 2 ** 24, 20_000) + 1.0,
                    rng.integers(-140, 100, 20_000) - 24)
    x = np.concatenate([x, ties])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float32).astype(np.float64)
    assert np.array_equal(round_to(x, "fp32"), ref)


def test_round_to_bf16_matches_torch_bfloat16():
    rng = np.random.default_rng(2)
    x = _spread(rng, 200_000, -120, 120).astype(np.float32)      # fp32-representable
    ties = (np.ldexp(2.0 * rng.integers(128, 256, 20_000) + 1.0,
                     rng.integers(-100, 100, 20_000) - 8)).astype(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).double().numpy()
    assert np.array_equal(round_to(x.astype(np.float64), "bf16"), ref)


def test_round_to_hand_values():
    # fp16: 1 + half an ulp ties to 1 (even); 1 + 3 half-ulps ties up to 1 + 2 ulps
    assert round_to(1.0 + 2.0 ** -11, "fp16") == 1.0
    assert round_to(1.0 + 3 * 2.0 ** -11, "fp16") == 1.0 + 2.0 ** -9
    # the largest finite fp16 is 65504; 65520 is the tie with 2^16 and overflows
    assert round_to(65519.0, "fp16") == 65504.0
    assert math.isinf(round_to(65520.0, "fp16"))
    # subnormal quantum 2^-24
    assert round_to(1.4 * 2.0 ** -24, "fp16") == 2.0 ** -24
    # bf16 keeps 8 significant bits: 1 + 2^-8 ties to 1, 1 + 2^-7 is exact
    assert round_to(1.0 + 2.0 ** -8, "bf16") == 1.0
    assert round_to(1.0 + 2.0 ** -7, "bf16") == 1.0 + 2.0 ** -7
    assert round_to(np.nan, "fp16") != round_to(np.nan, "fp16")


def test_split_hi_lo_keeps_22_bits():
    rng = np.random.default_rng(3)
    x = _spread(rng, 100_000, -8, 8)
    hi, lo = split_hi_lo(x, "fp16")
    assert np.array_equal(hi, round_to(x, "fp16"))
    # lo is rounded with relative error 2^-11 of |x - hi| <= 2^-11 |x|, unless
    # it falls below the smallest normal fp16 (absolute error 2^-25 there)
    assert np.all(np.abs(hi + lo - x) <= np.maximum(2.0 ** -22 * np.abs(x), 2.0 ** -25))
    big = np.abs(x) >= 2.0 ** -2
    assert np.all(np.abs(hi + lo - x)[big] <= 2.0 ** -22 * np.abs(x)[big])


def _case(name, seed=0, **shrink):
    w = WORKLOADS[name].shrink(**shrink) if shrink else WORKLOADS[name]
    inp = make_inputs(w, seed=seed)
    f = as_float64_numpy
    mask = inp["key_padding_mask"]
    args = (f(inp["x_q"]), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]), f(inp["b_o"]), w.h)
    kw = dict(x_kv=f(inp["x_kv"]), causal=w.causal,
              key_padding_mask=None if mask is None else mask.numpy(), n_kv_heads=w.n_g,
              gate_w=f(inp["gate_w"]), gate_b=f(inp["gate_b"]))
    return w, args, kw


CASES = [
    ("causal", "causal_bf16_d512_h8_b16_t1024", dict(B=2, T_q=150, T_k=150)),
    ("padded cross", "cross_pad_bf16_d512_h8_b32_tq512_tk2048",
     dict(B=3, T_q=70, T_k=200, padding=(40, 200))),
    ("grouped causal", "causal_bf16_d512_h8_b16_t1024", dict(B=2, T_q=90, T_k=90, n_kv=2)),
    ("gated causal", "causal_bf16_d512_h8_b16_t1024", dict(B=2, T_q=90, T_k=90, gate=True)),
]


@pytest.mark.parametrize("label,name,shrink", CASES, ids=[c[0] for c in CASES])
def test_exact_plan_is_the_oracle(label, name, shrink):
    _, args, kw = _case(name, **shrink)
    ref = mo.mha_forward(*args, **kw)
    y = emulate(PLANS["exact"], *args, **kw)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.nanmax(np.abs(ref)), equal_nan=True)
    rows = np.array([0, 1, 7, shrink["T_q"] - 1])
    ys = emulate(PLANS["exact"], *args, rows=rows, rows_per_block=3, **kw)
    assert np.allclose(ys, ref[:, rows], rtol=1e-12, atol=1e-12 * np.nanmax(np.abs(ref)),
                       equal_nan=True)
    yp = emulate(Plan(q_prescaled=True, l_from_stored_p=True), *args, **kw)
    assert np.allclose(yp, ref, rtol=1e-12, atol=1e-12 * np.nanmax(np.abs(ref)), equal_nan=True)


def test_y_storage_point():
    _, args, kw = _case("causal_bf16_d512_h8_b16_t1024", B=2, T_q=100, T_k=100)
    ref = mo.mha_forward(*args, **kw)
    y = emulate(Plan(y="bf16"), *args, **kw)
    assert np.array_equal(y, round_to(ref, "bf16"))


def test_v_storage_point():
    w, args, kw = _case("causal_bf16_d512_h8_b16_t1024", B=2, T_q=100, T_k=100)
    x_q, w_qkv, b_qkv, _, _, h = args
    D = w.D
    eye = np.eye(D)
    ref, inter = mo.mha_forward(x_q, w_qkv, b_qkv, eye, None, h, causal=True,
                                return_intermediates=True)
    o = inter["a"] @ round_to(inter["v"], "fp16")
    y = emulate(Plan(v="fp16"), x_q, w_qkv, b_qkv, eye, None, h, causal=True)
    assert np.allclose(y, mo.concat_heads(o), rtol=1e-12, atol=1e-14)
    vmax = np.max(np.abs(inter["v"]))
    assert np.max(np.abs(y - ref)) <= U16 * vmax


@pytest.mark.parametrize("from_stored", [False, True])
def test_p_storage_point_bound(from_stored):
    w, args, kw = _case("causal_bf16_d512_h8_b16_t1024", B=2, T_q=100, T_k=100)
    x_q, w_qkv, b_qkv, _, _, h = args
    eye = np.eye(w.D)
    ref, inter = mo.mha_forward(x_q, w_qkv, b_qkv, eye, None, h, causal=True,
                                return_intermediates=True)
    # the numerators stay normal fp16 values (relative rounding <= u)
    s = mo.masked_scores(inter["q"], inter["k"], True, None)
    spread = np.max(s, axis=-1, keepdims=True) - np.where(np.isinf(s), np.nan, s)
    assert np.nanmax(spread) < 9.0            # exp(-9) > 2^-14
    y = emulate(Plan(p="fp16", l_from_stored_p=from_stored), x_q, w_qkv, b_qkv, eye, None, h,
                causal=True)
    vmax = np.max(np.abs(inter["v"]), axis=2)                  # (B, h, d)
    bound = 2 * U16 / (1 - U16) * mo.concat_heads(vmax[:, :, None, :].repeat(100, axis=2))
    err = np.abs(y - ref)
    assert np.all(err <= bound)
    assert np.max(err / bound) > 0.01        # it did round


def test_early_rows_correction():
    w, args, kw = _case("causal_bf16_d512_h8_b16_t1024", B=2, T_q=200, T_k=200)
    ref = mo.mha_forward(*args, **kw)
    rms = math.sqrt(float(np.mean(ref ** 2)))
    y16 = emulate(PLANS["fp16"], *args, **kw)
    ye = emulate(PLANS["fp16 + early rows 64"], *args, **kw)
    assert np.array_equal(ye[:, 64:], y16[:, 64:])
    assert np.max(np.abs(ye[:, :64] - ref[:, :64])) <= 1e-5 * rms
    assert np.max(np.abs(y16[:, :64] - ref[:, :64])) > 1e-3 * rms
    # no effect without a causal self-attention
    _, a2, k2 = _case("cross_pad_bf16_d512_h8_b32_tq512_tk2048", B=2, T_q=80, T_k=100,
                      padding=(50, 100))
    assert np.array_equal(emulate(PLANS["fp16 + early rows 64"], *a2, **k2),
                          emulate(PLANS["fp16"], *a2, **k2))


def test_budget_on_the_d512_causal_workload():
    """The storage-plan budget on two full batch elements of the d512/h8/
    t1024 causal workload: bf16 everywhere fails the 2e-2 tolerance, so does
    bf16 Y; fp16 passes, the early-row correction shrinks it, and the path's
    own plan keeps at least a 2.5x margin."""
    _, args, kw = _case("causal_bf16_d512_h8_b16_t1024", B=2)
    ref = mo.mha_forward_blocked(*args, **kw)
    err = {p: max_abs_over_rms(emulate(PLANS[p], *args, **kw), ref)
           for p in ("bf16", "fp16, bf16 Y", "fp16", "fp16 + early rows 64", KERNEL_PLAN)}
    assert err["bf16"] > 2e-2
    assert err["fp16, bf16 Y"] > 2e-2
    assert err["fp16"] < 2e-2
    assert err["fp16 + early rows 64"] < err["fp16"] / 2
    assert err[KERNEL_PLAN] < 2e-2 / 2.5
