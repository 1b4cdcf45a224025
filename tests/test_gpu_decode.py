"""GPU parity of the generation step against a KV cache (C ABI mha_decode)
vs the fp64 oracle.

Tolerance: max |y_gpu - y_ref| / RMS(y_ref) <= 2e-2 (bf16 contract). The
rows a step appends to the caches must be the oracle's new keys and values
rounded to bf16: within one bf16 unit in the last place plus twice the fp32
accumulation bound (K + 2) 2^-24 (|x| . |W| + |b|) of the value (the GPU
projects in fp32, so a value near a rounding boundary may round the other
way, and a value that cancels to near zero carries the sum's absolute
rounding error); every
other cache row must be left bitwise unchanged (rows past a sequence's
length hold NaN on entry and must never be read).
"""

import math
import sys

import numpy as np
import pytest
import torch

from mha_inputs import DECODE_WORKLOADS, as_float64_numpy, make_decode_inputs
from oracle import mha_oracle as mo

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import transformer_head_attention_amd as m
    return m


def _gpu_step(lib, w, inp, mod=None):
    dev = "cuda:0"
    m = mod or lib.MultiHeadAttention(w.D, w.h, "bf16", num_kv_heads=w.n_g)
    kc, vc = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    y = m.decode(inp["x"].to(dev), inp["w_qkv"].to(dev), inp["w_o"].to(dev), kc, vc,
                 inp["cache_len"].to(dev), b_qkv=inp["b_qkv"].to(dev), b_o=inp["b_o"].to(dev))
    torch.cuda.synchronize()
    return y.cpu().double().numpy(), kc.cpu(), vc.cpu()


def _oracle_step(inp, batch=None):
    f = as_float64_numpy
    sl = slice(None) if batch is None else batch
    return mo.mha_decode(f(inp["x"][sl]), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]),
                         f(inp["b_o"]), inp["h"], f(inp["k_cache"][sl]), f(inp["v_cache"][sl]),
                         inp["cache_len"][sl].numpy(), n_kv_heads=inp["n_kv"])


def _err(y, ref):
    assert np.isfinite(y).all()
    rms = math.sqrt(float(np.mean(ref ** 2)))
    return float(np.max(np.abs(y - ref))) / rms


def _check_cache(before, after, new_ref, lens, T_new, acc_err=None):
    """Appended rows: within one bf16 ulp of the oracle plus, where given,
    (1 + 2^-8) times the fp32 accumulation bound a of each value; all others
    unchanged.

    The kernel stores bf16(v), v its fp32 value with |v - v_ref| <= a. Round
    to nearest even moves v by at most half an ulp, 2^-8 |v| <= 2^-8
    (|v_ref| + a), so |bf16(v) - v_ref| <= 2^-8 |v_ref| + (1 + 2^-8) a; the
    test allows a full ulp (2^-7 |v_ref|) for the rounding term."""
    b4 = before.view(torch.int16).numpy()
    af = after.view(torch.int16).numpy()
    aft = after.double().numpy()
    B = before.shape[0]
    for b in range(B):
        L = int(lens[b])
        keep = np.ones(before.shape[2], dtype=bool)
        keep[L:L + T_new] = False
        assert np.array_equal(b4[b][:, keep], af[b][:, keep]), f"batch {b}: untouched rows changed"
        got = aft[b][:, L:L + T_new]
        ref = new_ref[b]
        ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7
        if acc_err is not None:
            ulp = ulp + (1.0 + 2.0 ** -8) * acc_err[b]
        bad = np.abs(got - ref) > ulp
        if bad.any():
            i = np.unravel_index(np.argmax(np.abs(got - ref) - ulp), ref.shape)
            raise AssertionError(
                f"batch {b}: {int(bad.sum())} appended values off by more than the bound; "
                f"worst at {i}: got {got[i]!r} ref {ref[i]!r} bound {ulp[i]!r}")


def _acc_bound(inp, w, batch=None):
    """fp32 accumulation error bound of the projected K and V values:
    (K + 2) * 2^-24 * (|x| . |W| + |b|), per (batch, set, new token, channel)."""
    sl = slice(None) if batch is None else batch
    x = np.abs(as_float64_numpy(inp["x"][sl]))
    wq = np.abs(as_float64_numpy(inp["w_qkv"]))
    bq = np.abs(as_float64_numpy(inp["b_qkv"]))
    mag = x @ wq + bq                                          # (B, T_new, N_qkv)
    gam = (w.D + 2) * 2.0 ** -24
    d, dkv = w.d_k, w.n_g * w.d_k
    kk = mag[..., w.D:w.D + dkv].reshape(x.shape[0], x.shape[1], w.n_g, d).transpose(0, 2, 1, 3)
    vv = mag[..., w.D + dkv:].reshape(x.shape[0], x.shape[1], w.n_g, d).transpose(0, 2, 1, 3)
    return gam * kk, gam * vv


def _run_case(lib, w, lens=None, seed=11):
    # Full-length draws (no NaN rows yet); rows past the given lengths become NaN.
    full = w.T_max - w.T_new
    inp = make_decode_inputs(w.shrink(lengths=(full, full) if lens else (0, full)), seed)
    if lens is not None:
        inp["cache_len"] = torch.tensor(lens, dtype=torch.int32)
        pos = torch.arange(w.T_max)
        unused = (pos[None, :] >= inp["cache_len"][:, None].long())[:, None, :, None]
        for k in ("k_cache", "v_cache"):
            inp[k] = torch.where(unused, torch.full_like(inp[k], float("nan")), inp[k])
    y, kc, vc = _gpu_step(lib, w, inp)
    ref, k_new, v_new = _oracle_step(inp)
    err = _err(y, ref)
    _say(f"[decode] {w.name}: lens {inp['cache_len'].tolist()[:8]} err/rms = {err:.3e}")
    assert err <= TOL
    ek, ev = _acc_bound(inp, w)
    _check_cache(inp["k_cache"], kc, k_new, inp["cache_len"], w.T_new, ek)
    _check_cache(inp["v_cache"], vc, v_new, inp["cache_len"], w.T_new, ev)


BASE = DECODE_WORKLOADS["decode_bf16_d1024_h16_b32_t4096"]
MID = [
    ("mha d1024 T_new=1 ragged lengths", BASE.shrink(B=7, T_max=300),
     [0, 1, 63, 64, 65, 257, 299]),
    ("gqa4 d1024 T_new=3", BASE.shrink(B=4, T_new=3, T_max=400, n_kv=4), [0, 5, 128, 397]),
    ("mqa d512 h8 T_new=4 (32 query rows)", BASE.shrink(D=512, h=8, B=3, T_new=4, T_max=500,
                                                        n_kv=1), [2, 191, 496]),
    ("mqa d512 h8 T_new=5 (two query blocks)", BASE.shrink(D=512, h=8, B=3, T_new=5, T_max=333,
                                                           n_kv=1), [0, 100, 328]),
    ("mha d_k=128 T_new=2", BASE.shrink(D=1024, h=8, B=3, T_new=2, T_max=700), [1, 333, 698]),
    ("gqa2 d_k=128 T_new=1", BASE.shrink(D=1024, h=8, B=2, T_new=1, T_max=1000, n_kv=2),
     [999, 640]),
    ("empty caches, T_new = T_max", BASE.shrink(D=512, h=8, B=2, T_new=6, T_max=6, n_kv=2),
     [0, 0]),
    ("B=1 long cache", BASE.shrink(B=1, T_max=3000, n_kv=4), [2999]),
    ("no biases", BASE.shrink(B=2, T_max=200, bias_std=None), [10, 150]),
]


@pytest.mark.parametrize("name,w,lens", MID, ids=[m[0] for m in MID])
def test_decode_mid_size(lib, name, w, lens):
    _say(f"[decode] {name}: {w}")
    _run_case(lib, w.shrink(name=name), lens)


def test_decode_deterministic_and_reuses_handle(lib):
    w = BASE.shrink(B=3, T_new=2, T_max=256, n_kv=4, lengths=(0, 254))
    _say(f"[decode] determinism: {w}")
    inp = make_decode_inputs(w, 5)
    m = lib.MultiHeadAttention(w.D, w.h, "bf16", num_kv_heads=w.n_g)
    y1, k1, v1 = _gpu_step(lib, w, inp, mod=m)
    y2, k2, v2 = _gpu_step(lib, w, inp, mod=m)
    assert np.array_equal(y1, y2)
    assert torch.equal(k1.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v1.view(torch.int16), v2.view(torch.int16))


def test_decode_three_steps_against_oracle_cache(lib):
    """Three steps in a row, each side keeping its own cache: the GPU's
    caches are written by the library; the oracle's by appending its own new
    keys and values rounded to bf16."""
    w = BASE.shrink(B=3, T_new=2, T_max=200, n_kv=4, lengths=(0, 190))
    _say(f"[decode] three steps: {w}")
    inp = make_decode_inputs(w, 6)
    dev = "cuda:0"
    m = lib.MultiHeadAttention(w.D, w.h, "bf16", num_kv_heads=w.n_g)
    kc_g, vc_g = inp["k_cache"].to(dev), inp["v_cache"].to(dev)
    kc_o, vc_o = inp["k_cache"].clone(), inp["v_cache"].clone()
    lens = inp["cache_len"].clone()
    g = torch.Generator().manual_seed(99)
    for step in range(3):
        x = torch.randn(w.B, w.T_new, w.D, generator=g).to(torch.bfloat16)
        y = m.decode(x.to(dev), inp["w_qkv"].to(dev), inp["w_o"].to(dev), kc_g, vc_g,
                     lens.to(dev), b_qkv=inp["b_qkv"].to(dev), b_o=inp["b_o"].to(dev))
        torch.cuda.synchronize()
        f = as_float64_numpy
        ref, k_new, v_new = mo.mha_decode(f(x), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]),
                                          f(inp["b_o"]), w.h, f(kc_o), f(vc_o), lens.numpy(),
                                          n_kv_heads=w.n_g)
        err = _err(y.cpu().double().numpy(), ref)
        _say(f"[decode] step {step}: err/rms = {err:.3e}")
        assert err <= TOL
        for b in range(w.B):
            L = int(lens[b])
            kc_o[b, :, L:L + w.T_new] = torch.from_numpy(k_new[b]).to(torch.bfloat16)
            vc_o[b, :, L:L + w.T_new] = torch.from_numpy(v_new[b]).to(torch.bfloat16)
        lens += w.T_new


@pytest.mark.parametrize("name", list(DECODE_WORKLOADS))
def test_decode_full_size_workload(lib, name):
    """The benchmark's configurations; the oracle evaluates four batch
    elements (every row, head and the appended cache rows of each)."""
    w = DECODE_WORKLOADS[name]
    _say(f"[decode] full size {name}")
    inp = make_decode_inputs(w, 0)
    y, kc, vc = _gpu_step(lib, w, inp)
    picks = sorted({0, 1, w.B // 2, w.B - 1})
    refs = [_oracle_step(inp, slice(b, b + 1)) for b in picks]
    ref = np.concatenate([r[0] for r in refs])
    err = _err(y[picks], ref)
    _say(f"[decode] full size {name}: err/rms = {err:.3e}")
    assert np.isfinite(y).all()
    assert err <= TOL
    for i, b in enumerate(picks):
        ek, ev = _acc_bound(inp, w, slice(b, b + 1))
        _check_cache(inp["k_cache"][b:b + 1], kc[b:b + 1], refs[i][1], inp["cache_len"][b:b + 1],
                     w.T_new, ek)
        _check_cache(inp["v_cache"][b:b + 1], vc[b:b + 1], refs[i][2], inp["cache_len"][b:b + 1],
                     w.T_new, ev)
