"""mha_forward_noalloc (no workspace argument; the library's per-GPU scratch)
against mha_forward_ex with a caller workspace: the same kernels on the same
inputs, so the outputs must be bitwise equal, and both within the oracle
tolerance. Calls follow each other on one GPU with a smaller problem after a
larger one (the scratch keeps the previous call's contents), on bf16 and
fp32 handles, with and without options."""

import math
import sys

import numpy as np
import pytest
import torch

from mha_inputs import WORKLOADS, make_inputs, as_float64_numpy
from oracle import mha_oracle as mo

pytestmark = pytest.mark.gpu

W = WORKLOADS


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import transformer_head_attention_amd as m
    return m


def _ptr(t):
    return None if t is None else t.data_ptr()


def _call(lib, m, w, inp, noalloc, opts=None, y_dtype=torch.float32):
    dev = torch.device("cuda:0")
    t = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    y = torch.full((w.B, w.T_q, w.D), float("nan"), dtype=y_dtype, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (m.handle, _ptr(t["x_q"]), _ptr(t["x_kv"]), _ptr(t["w_qkv"]), _ptr(t["b_qkv"]),
            _ptr(t["w_o"]), _ptr(t["b_o"]), w.B, w.T_q, w.T_k, 1 if w.causal else 0,
            _ptr(t["key_padding_mask"]), y.data_ptr())
    if noalloc:
        st = lib.mha_forward_noalloc(*args, opts, stream)
    else:
        n = lib.mha_workspace_size(m.handle, w.B, w.T_q, w.T_k)
        ws = torch.empty(n, dtype=torch.uint8, device=dev)
        st = lib.mha_forward_ex(*args, ws.data_ptr(), n, opts, stream)
    assert st == lib.MHA_OK, lib.mha_status_string(st)
    torch.cuda.synchronize()
    return y.float().cpu().double().numpy()


def _oracle(inp, residual=False):
    f = as_float64_numpy
    m = inp["key_padding_mask"]
    return mo.mha_forward(f(inp["x_q"]), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]),
                          f(inp["b_o"]), inp["h"], x_kv=f(inp["x_kv"]), causal=inp["causal"],
                          key_padding_mask=None if m is None else m.numpy(),
                          n_kv_heads=inp["n_kv"], residual=residual)


def _err(y, ref):
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    ok = ~np.isnan(ref)
    return float(np.max(np.abs(y[ok] - ref[ok]))) / math.sqrt(float(np.mean(ref[ok] ** 2)))


CALLS = [
    # (label, workload, options (residual, y_bf16), tolerance)
    ("bf16 causal d1024 B=2 T=300", W["causal_bf16_d1024_h16_b8_t4096"].shrink(B=2, T_q=300,
                                                                                 T_k=300),
     (0, 0), 2e-2),
    ("bf16 GQA g2 cross padded B=2 77x150, residual", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"]
     .shrink(B=2, T_q=77, T_k=150, padding=(40, 150), n_kv=2), (1, 0), 2e-2),
    ("bf16 causal d_k=128 B=1 T=129, bf16 y", W["causal_bf16_d4096_h32_b1_t8192"]
     .shrink(D=1024, h=8, T_q=129, T_k=129), (0, 1), 2e-2),
    ("fp32 causal B=2 T=90", W["self_fp32_d512_h8_b2_t128"].shrink(T_q=90, T_k=90, causal=True),
     (0, 0), 1e-4),
]


def test_noalloc_matches_workspace_entry_point(lib):
    handles = {}
    results = []
    for label, w, (resid, ybf), tol in CALLS:
        _say(f"[noalloc] {label}: {w}")
        key = (w.D, w.h, w.dtype, w.n_g)
        if key not in handles:
            handles[key] = lib.MultiHeadAttention(w.D, w.h, w.dtype, num_kv_heads=w.n_g)
        m = handles[key]
        assert lib.mha_workspace_size(m.handle, w.B, w.T_q, w.T_k) <= lib.MHA_NOALLOC_SCRATCH_BYTES
        inp = make_inputs(w, seed=21)
        opts = lib.mha_forward_options(resid, ybf, None, 0)
        ydt = torch.bfloat16 if ybf else torch.float32
        y_na = _call(lib, m, w, inp, True, opts, ydt)
        y_ws = _call(lib, m, w, inp, False, opts, ydt)
        assert np.array_equal(y_na, y_ws, equal_nan=True), label
        ref = _oracle(inp, residual=bool(resid))
        err = _err(y_na, ref)
        bar = tol + (2.0 ** -8 * float(np.max(np.abs(ref))) / math.sqrt(float(np.mean(ref ** 2)))
                     if ybf else 0.0)
        _say(f"[noalloc] {label}: bitwise equal to mha_forward_ex, err/rms {err:.3e}")
        assert err <= bar
        results.append((label, w, inp, opts, ydt, y_na))
    # again, each call now following a different (larger or smaller) one
    for label, w, inp, opts, ydt, y_first in reversed(results):
        key = (w.D, w.h, w.dtype, w.n_g)
        y = _call(lib, handles[key], w, inp, True, opts, ydt)
        assert np.array_equal(y, y_first, equal_nan=True), label
    _say("[noalloc] repeated calls in reverse order: bitwise equal")


def test_noalloc_rejects_sizes_beyond_scratch(lib):
    w = W["causal_bf16_d1024_h16_b8_t4096"]
    m = lib.MultiHeadAttention(w.D, w.h, "bf16")
    assert lib.mha_workspace_size(m.handle, w.B, w.T_q, w.T_k) > lib.MHA_NOALLOC_SCRATCH_BYTES
    dev = torch.device("cuda:0")
    x = torch.zeros(w.B, w.T_q, w.D, dtype=torch.bfloat16, device=dev)
    wq = torch.zeros(w.D, 3 * w.D, dtype=torch.bfloat16, device=dev)
    wo = torch.zeros(w.D, w.D, dtype=torch.bfloat16, device=dev)
    y = torch.zeros(w.B, w.T_q, w.D, dtype=torch.float32, device=dev)
    st = lib.mha_forward_noalloc(m.handle, x.data_ptr(), None, wq.data_ptr(), None,
                                 wo.data_ptr(), None, w.B, w.T_q, w.T_k, 1, None, y.data_ptr(),
                                 None, torch.cuda.current_stream(dev).cuda_stream)
    assert st == lib.MHA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0     # nothing was enqueued
