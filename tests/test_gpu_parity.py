"""GPU parity: the HIP path through the C ABI vs the fp64 oracle.

Error metric (the workloads' tolerance contract): max |Y_gpu - Y_ref| divided
by the RMS of Y_ref, <= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs.
NaN positions (rows whose keys are all masked) must match exactly.

* Mid-size cases compare every output element; their sizes span several
  tiles and end in ragged tails.
* Grouped key/value heads (GQA, MQA): the same mid-size shapes with n_g < h
  sets, plus two full-size grouped workloads.
* The full-size workloads run exactly as the benchmark launches them and
  every output element is compared; the oracle evaluates them one batch
  element and one block of query rows at a time (the same steps, bounded
  memory).
"""

import concurrent.futures
import math
import os
import sys
import time

import numpy as np
import pytest
import torch
from threadpoolctl import threadpool_limits

from mha_inputs import ALL_WORKLOADS, WORKLOADS, make_inputs, as_float64_numpy
from oracle import mha_oracle as mo

pytestmark = pytest.mark.gpu

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


def run_gpu(lib, w, inp, stream=None, none_bias=False, mod=None):
    m = mod or lib.MultiHeadAttention(w.D, w.h, w.dtype, num_kv_heads=w.n_g)
    y = m.forward(_dev(inp["x_q"]), _dev(inp["w_qkv"]), _dev(inp["w_o"]),
                  b_qkv=None if none_bias else _dev(inp["b_qkv"]),
                  b_o=None if none_bias else _dev(inp["b_o"]),
                  x_kv=_dev(inp["x_kv"]), causal=inp["causal"],
                  key_padding_mask=_dev(inp["key_padding_mask"]), stream=stream,
                  gate_w=_dev(inp.get("gate_w")),
                  gate_b=None if none_bias else _dev(inp.get("gate_b")))
    torch.cuda.synchronize()
    return y.cpu().double().numpy()


def _np_mask(inp):
    m = inp["key_padding_mask"]
    return None if m is None else m.numpy()


def oracle_full(inp):
    f = as_float64_numpy
    return mo.mha_forward(f(inp["x_q"]), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]),
                          f(inp["b_o"]), inp["h"], x_kv=f(inp["x_kv"]), causal=inp["causal"],
                          key_padding_mask=_np_mask(inp), n_kv_heads=inp["n_kv"],
                          gate_w=f(inp.get("gate_w")), gate_b=f(inp.get("gate_b")))


def oracle_rows(inp, rows):
    f = as_float64_numpy
    return mo.mha_forward_rows(f(inp["x_q"]), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]),
                               f(inp["b_o"]), inp["h"], rows, x_kv=f(inp["x_kv"]),
                               causal=inp["causal"], key_padding_mask=_np_mask(inp),
                               n_kv_heads=inp["n_kv"])


def rel_err(y, ref, rms=None):
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(y), nan_ref), "NaN positions differ"
    ok = ~nan_ref
    if rms is None:
        rms = math.sqrt(float(np.mean(ref[ok] ** 2)))
    return float(np.max(np.abs(y[ok] - ref[ok]))) / rms


# ---------------------------------------------------------------- mid-size

W = WORKLOADS
MID = [
    ("fp32 self, the full d512/h8/b2/t128 workload", W["self_fp32_d512_h8_b2_t128"], {}),
    ("fp32 causal ragged", W["self_fp32_d512_h8_b2_t128"], dict(T_q=201, T_k=201, causal=True)),
    ("fp32 cross padded", W["self_fp32_d512_h8_b2_t128"],
     dict(B=3, T_q=77, T_k=150, cross=True, padding=(1, 150))),
    ("fp32 d_k=128", W["self_fp32_d512_h8_b2_t128"], dict(D=1024, h=8, T_q=99, T_k=99,
                                                          causal=True)),
    ("bf16 causal d512 ragged", W["causal_bf16_d512_h8_b16_t1024"], dict(B=2, T_q=300, T_k=300)),
    ("bf16 causal d1024 ragged", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=1, T_q=777,
                                                                            T_k=777)),
    ("bf16 non-causal self", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=2, T_q=257, T_k=257,
                                                                        causal=False)),
    # the single [Q|K|V] launch with a ragged last row band and sequence
    # boundaries inside tiles: 8400 rows give 396 tiles of 256 x 256 (a last
    # round more than half full: those tiles); 7000 rows give 336 (a last
    # round at most half full: 256 x 128 tiles, two workgroups per CU)
    ("bf16 causal d1024 single QKV launch, big tiles, ragged", W["causal_bf16_d1024_h16_b8_t4096"],
     dict(B=8, T_q=1050, T_k=1050)),
    ("bf16 causal d1024 single QKV launch, mid tiles, ragged", W["causal_bf16_d1024_h16_b8_t4096"],
     dict(B=7, T_q=1000, T_k=1000)),
    # the cross-attention [K|V] launch (17000 rows of X_kv: 268 big tiles)
    ("bf16 cross padded single [K|V] launch ragged", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=17, T_q=90, T_k=1000, padding=(100, 1000))),
    ("bf16 cross padded ragged", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=3, T_q=200, T_k=333, padding=(40, 333))),
    ("bf16 causal d_k=128", W["causal_bf16_d4096_h32_b1_t8192"], dict(T_q=300, T_k=300)),
    ("bf16 causal + padding", W["causal_bf16_d512_h8_b16_t1024"],
     dict(B=3, T_q=190, T_k=190, padding=(150, 190))),
    # more batch elements than the extent ranking takes: natural order
    ("bf16 cross padded B=1100", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=1100, T_q=5, T_k=12, padding=(1, 12))),
    ("bf16 T=1 causal", W["causal_bf16_d512_h8_b16_t1024"], dict(B=3, T_q=1, T_k=1)),
    ("bf16 T=1 self", W["causal_bf16_d512_h8_b16_t1024"], dict(B=3, T_q=1, T_k=1, causal=False)),
    ("bf16 T_q=1 cross", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=2, T_q=1, T_k=5, padding=(1, 5))),
    ("bf16 T=65 causal", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=2, T_q=65, T_k=65)),
    ("bf16 T=129 causal d_k=128", W["causal_bf16_d4096_h32_b1_t8192"], dict(D=1024, h=8,
                                                                              T_q=129, T_k=129)),
    # small d_model: the early-row projection's 64-deep K chunks are dealt
    # unevenly to its four waves (D=128: two chunks, D=384: 2/2/1/1)
    ("bf16 causal D=128 h=2", W["causal_bf16_d512_h8_b16_t1024"], dict(D=128, h=2, B=2, T_q=150,
                                                                       T_k=150)),
    ("bf16 causal D=128 h=1 d_k=128", W["causal_bf16_d4096_h32_b1_t8192"],
     dict(D=128, h=1, B=2, T_q=70, T_k=70)),
    ("bf16 causal D=384 h=6 ragged", W["causal_bf16_d512_h8_b16_t1024"],
     dict(D=384, h=6, B=2, T_q=211, T_k=211)),
    # grouped key/value heads
    ("bf16 GQA g4 causal d1024 ragged", W["causal_bf16_d1024_h16_b8_t4096"],
     dict(B=1, T_q=777, T_k=777, n_kv=4)),
    ("bf16 GQA g8 non-causal d1024", W["causal_bf16_d1024_h16_b8_t4096"],
     dict(B=2, T_q=257, T_k=257, causal=False, n_kv=8)),
    ("bf16 MQA causal d512 (64-wide K, V blocks)", W["causal_bf16_d512_h8_b16_t1024"],
     dict(B=2, T_q=300, T_k=300, n_kv=1)),
    ("bf16 MQA causal + padding d512", W["causal_bf16_d512_h8_b16_t1024"],
     dict(B=3, T_q=190, T_k=190, padding=(150, 190), n_kv=1)),
    ("bf16 GQA g2 cross padded ragged", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=3, T_q=200, T_k=333, padding=(40, 333), n_kv=2)),
    ("bf16 MQA cross padded ragged", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=2, T_q=77, T_k=201, padding=(40, 201), n_kv=1)),
    ("bf16 GQA g2 causal d_k=128", W["causal_bf16_d4096_h32_b1_t8192"],
     dict(D=1024, h=8, T_q=300, T_k=300, n_kv=2)),
    ("bf16 MQA causal d_k=128 T=129", W["causal_bf16_d4096_h32_b1_t8192"],
     dict(D=1024, h=8, T_q=129, T_k=129, n_kv=1)),
    ("bf16 GQA T=1 causal", W["causal_bf16_d512_h8_b16_t1024"], dict(B=3, T_q=1, T_k=1, n_kv=2)),
    # causal cross-attention (T_q == T_k): early rows take Q from x_q, K and V from x_kv
    ("bf16 causal cross padded", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=3, T_q=150, T_k=150, causal=True, padding=(100, 150))),
    ("bf16 causal cross GQA d_k=128", W["causal_bf16_d4096_h32_b1_t8192"],
     dict(D=1024, h=8, B=2, T_q=140, T_k=140, cross=True, n_kv=2)),
    ("fp32 causal cross", W["self_fp32_d512_h8_b2_t128"],
     dict(T_q=90, T_k=90, cross=True, causal=True)),
    ("fp32 GQA g2 causal ragged", W["self_fp32_d512_h8_b2_t128"],
     dict(T_q=201, T_k=201, causal=True, n_kv=2)),
    ("fp32 MQA cross padded", W["self_fp32_d512_h8_b2_t128"],
     dict(B=3, T_q=77, T_k=150, cross=True, padding=(1, 150), n_kv=1)),
    ("fp32 GQA g4 d_k=128", W["self_fp32_d512_h8_b2_t128"],
     dict(D=1024, h=8, T_q=99, T_k=99, causal=True, n_kv=4)),
]


@pytest.mark.parametrize("name,base,kw", MID, ids=[m[0] for m in MID])
def test_mid_size_parity(lib, name, base, kw):
    w = base.shrink(name=name, **kw)
    _say(f"[parity] {name}: {w}")
    inp = make_inputs(w, seed=3)
    y = run_gpu(lib, w, inp)
    ref = oracle_full(inp)
    err = rel_err(y, ref)
    _say(f"[parity] {name}: err/rms = {err:.3e} (tol {TOL[w.dtype]})")
    assert err <= TOL[w.dtype]


def test_all_masked_rows_are_nan(lib):
    w = W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"].shrink(B=3, T_q=70, T_k=90, padding=None)
    _say(f"[parity] all-masked batch element: {w}")
    inp = make_inputs(w, seed=4)
    mask = torch.zeros(3, 90, dtype=torch.uint8)
    mask[1, :] = 1          # every key of batch element 1 ignored
    mask[2, 50:] = 1
    inp["key_padding_mask"] = mask
    y = run_gpu(lib, w, inp)
    assert np.isnan(y[1]).all()
    assert np.isfinite(y[0]).all() and np.isfinite(y[2]).all()
    assert rel_err(y, oracle_full(inp)) <= TOL["bf16"]


def test_interior_mask_holes(lib):
    """A general (non-trailing) padding mask, masking whole 64-key tiles too."""
    w = W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"].shrink(B=2, T_q=100, T_k=300, padding=None)
    _say(f"[parity] interior mask holes: {w}")
    inp = make_inputs(w, seed=5)
    mask = torch.zeros(2, 300, dtype=torch.uint8)
    mask[0, 0:64] = 1
    mask[0, 100:190] = 1
    mask[1, ::3] = 1
    inp["key_padding_mask"] = mask
    assert rel_err(run_gpu(lib, w, inp), oracle_full(inp)) <= TOL["bf16"]


# Causal attention with a padding mask that hides the leading keys: query
# rows before the first unmasked key see no key at all and must be NaN, both
# among the early rows (evaluated in fp32 on the bf16 path) and past them
# (several all-masked 64-key tiles before the first live key); plus causal
# masks with interior holes.
LEADING = [
    ("bf16 d_k=64 leading 40", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=3, T_q=300, T_k=300),
     "lead", 40),
    ("bf16 d_k=64 leading 150", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=3, T_q=300, T_k=300),
     "lead", 150),
    ("bf16 d_k=128 leading 40", W["causal_bf16_d4096_h32_b1_t8192"],
     dict(D=1024, h=8, B=3, T_q=300, T_k=300), "lead", 40),
    ("bf16 d_k=128 leading 150", W["causal_bf16_d4096_h32_b1_t8192"],
     dict(D=1024, h=8, B=3, T_q=300, T_k=300), "lead", 150),
    ("bf16 GQA g4 leading 150", W["causal_bf16_d1024_h16_b8_t4096"],
     dict(B=3, T_q=300, T_k=300, n_kv=4), "lead", 150),
    ("fp32 leading 40", W["self_fp32_d512_h8_b2_t128"], dict(B=3, T_q=201, T_k=201,
                                                             causal=True), "lead", 40),
    ("fp32 leading 150", W["self_fp32_d512_h8_b2_t128"], dict(B=3, T_q=201, T_k=201,
                                                              causal=True), "lead", 150),
    ("bf16 d_k=64 causal holes", W["causal_bf16_d1024_h16_b8_t4096"],
     dict(B=3, T_q=300, T_k=300), "holes", 0),
    ("bf16 d_k=128 causal holes", W["causal_bf16_d4096_h32_b1_t8192"],
     dict(D=1024, h=8, B=3, T_q=300, T_k=300), "holes", 0),
    ("fp32 causal holes", W["self_fp32_d512_h8_b2_t128"], dict(B=3, T_q=201, T_k=201,
                                                               causal=True), "holes", 0),
]


@pytest.mark.parametrize("name,base,kw,kind,k", LEADING, ids=[c[0] for c in LEADING])
def test_causal_masked_keys(lib, name, base, kw, kind, k):
    w = base.shrink(name=name, padding=None, **kw)
    _say(f"[parity] {name}: {w}")
    inp = make_inputs(w, seed=12)
    mask = torch.zeros(w.B, w.T_k, dtype=torch.uint8)
    if kind == "lead":
        mask[0, :k] = 1                 # rows 0..k-1 of batch element 0 see no key
        mask[1, :k // 2] = 1
        mask[1, k + 10:k + 90] = 1
        mask[2, :] = 1                  # every key of batch element 2 ignored
    else:
        mask[0, 0:64] = 1
        mask[0, 100:190] = 1
        mask[1, 1::3] = 1
        mask[2, 64:128] = 1
        mask[2, 250:] = 1
    inp["key_padding_mask"] = mask
    y = run_gpu(lib, w, inp)
    ref = oracle_full(inp)
    if kind == "lead":
        assert np.isnan(ref[0, :k]).all() and np.isfinite(ref[0, k:]).all()
        assert np.isnan(ref[2]).all()
    err = rel_err(y, ref)
    _say(f"[parity] {name}: err/rms = {err:.3e}, NaN rows {int(np.isnan(ref[..., 0]).sum())}")
    assert err <= TOL[w.dtype]


# Causal launches whose query blocks are interleaved over groups of G units
# (batch element, head) longest first: G = 8 (D=1024, h=16, B=4: 64 units, 8
# per XCD) and G = 16 with a partial last group (D=512, h=8, B=17: 136 units,
# 17 per XCD, 8.5 groups). Every element compared.
GROUPS = [
    ("bf16 causal G=8 d1024 h16 B=4", W["causal_bf16_d1024_h16_b8_t4096"],
     dict(B=4, T_q=300, T_k=300)),
    ("bf16 causal G=16 partial d512 h8 B=17", W["causal_bf16_d512_h8_b16_t1024"],
     dict(B=17, T_q=300, T_k=300)),
    ("bf16 causal G=16 d512 h8 B=16 T=1024 ragged", W["causal_bf16_d512_h8_b16_t1024"],
     dict(B=16, T_q=1000, T_k=1000)),
    ("bf16 causal G=4 d_k=128 h8 B=5", W["causal_bf16_d4096_h32_b1_t8192"],
     dict(D=1024, h=8, B=5, T_q=260, T_k=260)),
]


@pytest.mark.parametrize("name,base,kw", GROUPS, ids=[g[0] for g in GROUPS])
def test_causal_interleave_groups(lib, name, base, kw):
    w = base.shrink(name=name, **kw)
    _say(f"[parity] {name}: {w}")
    inp = make_inputs(w, seed=13)
    y = run_gpu(lib, w, inp)
    err = rel_err(y, oracle_full(inp))
    _say(f"[parity] {name}: err/rms = {err:.3e} (tol {TOL[w.dtype]})")
    assert err <= TOL[w.dtype]


# Inputs reshaped so the online softmax leaves its common case: the kernel
# keeps a row's reference at 0 while its first tile's maximum lies in [0, 8]
# (log2 units) and otherwise moves it to that maximum, and afterwards moves it
# whenever a score exceeds it by more than 8. The synthetic workloads' scores
# stay within about 4, so these cases scale them: "scale" multiplies the
# inputs by 3 (first maxima above 8), "grow" multiplies position t by
# 1 + t/96 (rows start at reference 0 and move later), "negative" adds +a to
# the Q bias and -a to the K bias, which lowers every score of a query by the
# same amount (first maxima below 0; the attention output is unchanged).
def _reshape_inputs(w, inp, how):
    inp = dict(inp)
    if how == "scale":
        for k in ("x_q", "x_kv"):
            if inp[k] is not None:
                inp[k] = (inp[k].float() * 3.0).to(inp[k].dtype)
    elif how == "grow":
        for k in ("x_q", "x_kv"):
            if inp[k] is not None:
                t = inp[k].shape[1]
                fac = (1.0 + torch.arange(t, dtype=torch.float32) / 96.0).view(1, t, 1)
                inp[k] = (inp[k].float() * fac).to(inp[k].dtype)
    else:
        b = inp["b_qkv"].float().clone()
        b[:w.D] += 1.5
        b[w.D:2 * w.D] -= 1.5
        inp["b_qkv"] = b.to(inp["b_qkv"].dtype)
    return inp


def _score_regime(w, inp):
    """Per (b, head, row): the maximum score over the first 64 keys and over
    all keys, in log2 units, float64, for the rows the fp16 kernel evaluates
    (rows >= 64 under the causal mask). Masked keys excluded."""
    f = as_float64_numpy
    x_q = f(inp["x_q"])
    x_kv = f(inp["x_kv"]) if inp["x_kv"] is not None else x_q
    W_, b_ = f(inp["w_qkv"]), f(inp["b_qkv"])
    D, h = w.D, w.h
    dk = D // h
    q = (x_q @ W_[:, :D] + b_[:D]).reshape(w.B, w.T_q, h, dk).transpose(0, 2, 1, 3)
    k = (x_kv @ W_[:, D:2 * D] + b_[D:2 * D]).reshape(w.B, w.T_k, h, dk).transpose(0, 2, 1, 3)
    s = q @ k.transpose(0, 1, 3, 2) * (math.log2(math.e) / math.sqrt(dk))
    if inp["causal"]:
        s = np.where(np.triu(np.ones((w.T_q, w.T_k), bool), 1), -np.inf, s)
    if inp["key_padding_mask"] is not None:
        s = np.where(_np_mask(inp)[:, None, None, :], -np.inf, s)
    r0 = 64 if inp["causal"] else 0
    return s[:, :, r0:, :64].max(-1), s[:, :, r0:, :].max(-1)


REF_PATHS = [
    ("scale, causal d_k=64", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=2, T_q=300, T_k=300),
     "scale"),
    ("scale, causal d_k=128", W["causal_bf16_d4096_h32_b1_t8192"],
     dict(D=1024, h=8, B=2, T_q=300, T_k=300), "scale"),
    ("grow, causal d_k=64", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=2, T_q=300, T_k=300),
     "grow"),
    ("grow, cross padded", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=3, T_q=200, T_k=333, padding=(100, 333)), "grow"),
    ("negative, causal d_k=64", W["causal_bf16_d1024_h16_b8_t4096"],
     dict(B=2, T_q=300, T_k=300), "negative"),
]


@pytest.mark.parametrize("name,base,kw,how", REF_PATHS, ids=[r[0] for r in REF_PATHS])
def test_softmax_reference_paths(lib, name, base, kw, how):
    w = base.shrink(name=name, **kw)
    _say(f"[parity] {name}: {w}")
    inp = _reshape_inputs(w, make_inputs(w, seed=9), how)
    first, full = _score_regime(w, inp)
    ok = np.isfinite(first)
    if how == "scale":
        assert np.mean(first[ok] > 8) > 0.25
    elif how == "grow":
        assert np.mean((first[ok] >= 0) & (first[ok] <= 8)) > 0.2
        assert np.mean(full[ok] - np.maximum(first[ok], 0) > 8) > 0.05
    else:
        assert np.all(first[ok] < 0)
    y = run_gpu(lib, w, inp)
    err = rel_err(y, oracle_full(inp))
    _say(f"[parity] {name}: err/rms = {err:.3e} (tol {TOL['bf16']})")
    assert err <= TOL["bf16"]


def test_deterministic_and_null_bias_equals_zero_bias(lib):
    w = W["causal_bf16_d512_h8_b16_t1024"].shrink(B=2, T_q=333, T_k=333)
    _say(f"[parity] determinism / null bias: {w}")
    inp = make_inputs(w, seed=6)       # zero biases
    y1 = run_gpu(lib, w, inp)
    y2 = run_gpu(lib, w, inp)
    y3 = run_gpu(lib, w, inp, none_bias=True)
    assert np.array_equal(y1, y2)
    assert np.array_equal(y1, y3)


def test_side_stream_and_workspace_reuse(lib):
    w = W["causal_bf16_d1024_h16_b8_t4096"].shrink(B=1, T_q=400, T_k=400)
    _say(f"[parity] side stream + reused workspace: {w}")
    m = lib.MultiHeadAttention(w.D, w.h, "bf16")
    inp = make_inputs(w, seed=7)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y_big = run_gpu(lib, w, inp, stream=s.cuda_stream, mod=m)
    w2 = w.shrink(T_q=130, T_k=130)
    inp2 = make_inputs(w2, seed=8)
    y_small = run_gpu(lib, w2, inp2, mod=m)     # smaller call into the larger workspace
    assert rel_err(y_big, oracle_full(inp)) <= TOL["bf16"]
    assert rel_err(y_small, oracle_full(inp2)) <= TOL["bf16"]


# -------------------------------------------------------------- full sizes

def oracle_blocked(inp, w, label):
    """The whole oracle output, one batch element and one block of query rows
    at a time (score blocks of about 64 MiB). Blocks are evaluated by a pool
    of threads, each with a single-threaded BLAS (numpy's elementwise passes
    over the score blocks release the GIL); the per-batch projections run
    between the pooled phases with the BLAS's own threads."""
    f = as_float64_numpy
    rows = max(16, (64 << 20) // (w.h * w.T_k * 8))
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    t_start = time.time()
    last = [t_start]

    def progress(b, t0, t1):
        now = time.time()
        if now - last[0] >= 10.0 or (b == w.B - 1 and t1 == w.T_q):
            _say(f"[parity] {label}: oracle at batch element {b + 1}/{w.B}, row {t1}/{w.T_q} "
                 f"({now - t_start:.0f} s)")
            last[0] = now

    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        def map_blocks(fn, it):
            with threadpool_limits(1):
                return list(ex.map(fn, it))

        return mo.mha_forward_blocked(f(inp["x_q"]), f(inp["w_qkv"]), f(inp["b_qkv"]),
                                      f(inp["w_o"]), f(inp["b_o"]), inp["h"],
                                      x_kv=f(inp["x_kv"]), causal=inp["causal"],
                                      key_padding_mask=_np_mask(inp), n_kv_heads=inp["n_kv"],
                                      gate_w=f(inp.get("gate_w")), gate_b=f(inp.get("gate_b")),
                                      rows_per_block=rows, progress=progress,
                                      map_blocks=map_blocks)


@pytest.mark.parametrize("name", list(ALL_WORKLOADS))
def test_full_size_workload(lib, name):
    """Every element of every batch element, RMS over the whole output."""
    w = ALL_WORKLOADS[name]
    _say(f"[parity] full size {name}")
    inp = make_inputs(w, seed=0)
    y = run_gpu(lib, w, inp)
    _say(f"[parity] full size {name}: GPU done, oracle on every row")
    ref = oracle_blocked(inp, w, name)
    err = rel_err(y, ref)
    _say(f"[parity] full size {name}: err/rms = {err:.3e} over {y.size} elements "
         f"(tol {TOL[w.dtype]})")
    assert np.isfinite(y).all()
    assert err <= TOL[w.dtype]


def test_grouped_with_one_set_per_head_equals_plain(lib):
    """num_kv_heads = num_heads runs the same kernels as mha_create: bitwise
    equal results."""
    w = W["causal_bf16_d512_h8_b16_t1024"].shrink(B=2, T_q=200, T_k=200, bias_std=0.02)
    _say(f"[parity] grouped handle with n_g = h vs plain handle: {w}")
    inp = make_inputs(w, seed=9)
    plain = lib.MultiHeadAttention(w.D, w.h, "bf16")
    grouped = lib.MultiHeadAttention(w.D, w.h, "bf16", num_kv_heads=w.h)
    assert np.array_equal(run_gpu(lib, w, inp, mod=plain), run_gpu(lib, w, inp, mod=grouped))
