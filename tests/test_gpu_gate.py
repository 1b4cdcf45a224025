"""GPU parity of gated attention (itwiki "멀티 헤드 어텐션", 추론 비용과 변형,
last paragraph: each head's scaled dot-product attention output times a
sigmoid gate of its own; here sigma(x_q . W_G + b_G) per query row and head)
through the C ABI, against the fp64 oracle, every element compared.

Covers both dtypes, causal (the fp32 early rows and the fp16 rows past them
are gated in different kernels), cross-attention with padding, grouped
key/value heads, d_k 64 and 128, gates near 0 and 1 and all-masked (NaN)
rows, together with the residual and bf16-y options, a NULL gate bias, and
that a gate of 1 gives the ungated result. The full-size gated workload is
in test_gpu_parity.py (test_full_size_workload)."""

import math
import sys

import numpy as np
import pytest
import torch

from mha_inputs import WORKLOADS, make_inputs, as_float64_numpy
from oracle import mha_oracle as mo

pytestmark = pytest.mark.gpu

W = WORKLOADS
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import transformer_head_attention_amd as m
    return m


def _dev(t):
    return None if t is None else t.to("cuda:0")


def _gpu(lib, w, inp, residual=False, y_dtype="fp32", gate_b=True):
    m = lib.MultiHeadAttention(w.D, w.h, w.dtype, num_kv_heads=w.n_g)
    y = m.forward(_dev(inp["x_q"]), _dev(inp["w_qkv"]), _dev(inp["w_o"]),
                  b_qkv=_dev(inp["b_qkv"]), b_o=_dev(inp["b_o"]), x_kv=_dev(inp["x_kv"]),
                  causal=inp["causal"], key_padding_mask=_dev(inp["key_padding_mask"]),
                  residual=residual, y_dtype=y_dtype, gate_w=_dev(inp["gate_w"]),
                  gate_b=_dev(inp["gate_b"]) if gate_b else None)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy()


def _oracle(inp, residual=False, gate_b=True):
    f = as_float64_numpy
    m = inp["key_padding_mask"]
    return mo.mha_forward(f(inp["x_q"]), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]),
                          f(inp["b_o"]), inp["h"], x_kv=f(inp["x_kv"]), causal=inp["causal"],
                          key_padding_mask=None if m is None else m.numpy(),
                          n_kv_heads=inp["n_kv"], residual=residual,
                          gate_w=f(inp["gate_w"]), gate_b=f(inp["gate_b"]) if gate_b else None)


def _err(y, ref):
    assert np.array_equal(np.isnan(y), np.isnan(ref)), "NaN positions differ"
    ok = ~np.isnan(ref)
    return float(np.max(np.abs(y[ok] - ref[ok]))) / math.sqrt(float(np.mean(ref[ok] ** 2)))


CASES = [
    ("bf16 causal d1024 ragged", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=2, T_q=300, T_k=300)),
    ("bf16 causal d_k=128", W["causal_bf16_d4096_h32_b1_t8192"], dict(D=1024, h=8, B=2, T_q=200,
                                                                      T_k=200, bias_std=0.02)),
    ("bf16 non-causal self", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=2, T_q=257, T_k=257,
                                                                        causal=False)),
    ("bf16 cross padded", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=3, T_q=200, T_k=333, padding=(40, 333), bias_std=0.02)),
    ("bf16 GQA g4 causal", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=1, T_q=400, T_k=400,
                                                                      n_kv=4)),
    ("bf16 MQA cross padded", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=2, T_q=77, T_k=201, padding=(40, 201), n_kv=1, bias_std=0.02)),
    ("bf16 causal D=128 h=2", W["causal_bf16_d512_h8_b16_t1024"], dict(D=128, h=2, B=2, T_q=150,
                                                                       T_k=150, bias_std=0.02)),
    ("fp32 self", W["self_fp32_d512_h8_b2_t128"], dict()),
    ("fp32 causal GQA g2", W["self_fp32_d512_h8_b2_t128"], dict(T_q=201, T_k=201, causal=True,
                                                               n_kv=2)),
    ("fp32 cross padded d_k=128", W["self_fp32_d512_h8_b2_t128"],
     dict(D=1024, h=8, B=3, T_q=77, T_k=150, cross=True, padding=(1, 150))),
]


@pytest.mark.parametrize("name,base,kw", CASES, ids=[c[0] for c in CASES])
def test_gated_parity(lib, name, base, kw):
    w = base.shrink(name=name, gate=True, **kw)
    _say(f"[gate] {name}: {w}")
    inp = make_inputs(w, seed=31)
    y = _gpu(lib, w, inp)
    ref = _oracle(inp)
    ung = mo.mha_forward(*[as_float64_numpy(inp[k]) for k in ("x_q", "w_qkv", "b_qkv", "w_o",
                                                              "b_o")], inp["h"],
                         x_kv=as_float64_numpy(inp["x_kv"]), causal=inp["causal"],
                         key_padding_mask=None if inp["key_padding_mask"] is None
                         else inp["key_padding_mask"].numpy(), n_kv_heads=inp["n_kv"])
    # the gate really changes the result (gates spread over (0, 1))
    assert np.max(np.abs(ung - ref)) > 0.1 * math.sqrt(float(np.mean(ref ** 2)))
    err = _err(y, ref)
    _say(f"[gate] {name}: err/rms = {err:.3e} (tol {TOL[w.dtype]})")
    assert err <= TOL[w.dtype]


def test_gate_extremes_nan_rows_and_options(lib):
    """Gate biases of +-30 (gates ~1 and ~0) on alternate heads, leading keys
    masked so some causal rows are NaN, residual and bf16 y; then a NULL gate
    bias; then gates of exactly 1 (bias +60) give the ungated result."""
    w = W["causal_bf16_d1024_h16_b8_t4096"].shrink(B=2, T_q=200, T_k=200, gate=True)
    inp = make_inputs(w, seed=32)
    b = inp["gate_b"].float().clone()
    b[0::2] += 30.0
    b[1::2] -= 30.0
    inp["gate_b"] = b.to(torch.bfloat16)
    mask = torch.zeros(2, 200, dtype=torch.uint8)
    mask[0, :20] = 1
    inp["key_padding_mask"] = mask
    ref = _oracle(inp, residual=True)
    y = _gpu(lib, w, inp, residual=True, y_dtype="bf16")
    bar = TOL["bf16"] + 2.0 ** -8 * float(np.nanmax(np.abs(ref))) / math.sqrt(
        float(np.nanmean(ref ** 2)))
    err = _err(y, ref)
    _say(f"[gate] extremes + NaN rows + residual + bf16 y: err/rms = {err:.3e}")
    assert np.isnan(ref[0, :20]).all() and err <= bar
    err = _err(_gpu(lib, w, inp, gate_b=False), _oracle(inp, gate_b=False))
    _say(f"[gate] NULL gate bias: err/rms = {err:.3e}")
    assert err <= TOL["bf16"]
    inp["gate_b"] = torch.full((w.h,), 60.0).to(torch.bfloat16)
    inp["gate_w"] = (inp["gate_w"].float() * 0.0).to(torch.bfloat16)
    m = lib.MultiHeadAttention(w.D, w.h, "bf16")
    y_plain = m.forward(_dev(inp["x_q"]), _dev(inp["w_qkv"]), _dev(inp["w_o"]),
                        b_qkv=_dev(inp["b_qkv"]), b_o=_dev(inp["b_o"]), causal=True,
                        key_padding_mask=_dev(mask))
    torch.cuda.synchronize()
    y_one = _gpu(lib, w, inp)
    assert np.array_equal(y_one, y_plain.cpu().double().numpy(), equal_nan=True)
