"""The fp16_overflow option of the forward pass (C ABI mha_forward_ex).

The bf16 path stores W_O and the projected Q (times log2(e)/sqrt(d_k)), K and
V in fp16; the flag must become 1 when one of those stored values is not
finite (magnitude 65520 or more before rounding, or NaN) and stay as it was
otherwise. Every case first checks on the CPU, from the fp64 projection,
which stored values overflow, so that each case isolates one store: W_O's
conversion, the Q and K epilogue, the V epilogue's staged tiles, the V
epilogue's element-wise tail, the key/value projection of cross-attention.
"""

import math
import sys

import numpy as np
import pytest
import torch

from mha_inputs import WORKLOADS, as_float64_numpy, make_inputs

pytestmark = pytest.mark.gpu

F16_INF_FROM = 65520.0


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import transformer_head_attention_amd as m
    return m


def _dev(t):
    return None if t is None else t.to("cuda:0")


def _run(lib, w, inp, flag=None):
    m = lib.MultiHeadAttention(w.D, w.h, w.dtype, num_kv_heads=w.n_g)
    y = m.forward(_dev(inp["x_q"]), _dev(inp["w_qkv"]), _dev(inp["w_o"]),
                  b_qkv=_dev(inp["b_qkv"]), b_o=_dev(inp["b_o"]), x_kv=_dev(inp["x_kv"]),
                  causal=inp["causal"], key_padding_mask=_dev(inp["key_padding_mask"]),
                  gate_w=_dev(inp.get("gate_w")), gate_b=_dev(inp.get("gate_b")),
                  fp16_overflow=flag)
    torch.cuda.synchronize()
    return y.cpu()


def _flag(v=0):
    return torch.full((1,), v, dtype=torch.int32, device="cuda:0")


def _stored_maxima(w, inp):
    """Largest |value| the bf16 path stores in fp16: Q (prescaled), K, V per
    row range, and W_O (fp64 projection of the bf16 inputs)."""
    f = as_float64_numpy
    D, dk = w.D, w.D // w.h
    x_q = f(inp["x_q"])
    x_kv = x_q if inp["x_kv"] is None else f(inp["x_kv"])
    wq, bq = f(inp["w_qkv"]), f(inp["b_qkv"])
    q = (x_q @ wq[:, :D] + bq[:D]) * (math.log2(math.e) / math.sqrt(dk))
    kv = x_kv @ wq[:, D:] + bq[D:]
    dkv = kv.shape[-1] // 2
    return {"q": np.abs(q), "k": np.abs(kv[..., :dkv]), "v": np.abs(kv[..., dkv:]),
            "w_o": float(np.max(np.abs(f(inp["w_o"]))))}


def _base(name, **shrink):
    w = WORKLOADS[name].shrink(**shrink)
    return w, make_inputs(w, seed=0)


def _w_o_big(w, inp):
    inp["w_o"][3, 5] = 131072.0                                 # 2^17, exact in bf16


def _q_bias_big(w, inp):
    inp["b_qkv"][0] = 524288.0                                  # 2^19 x 0.18 > 65520


def _k_bias_big(w, inp):
    inp["b_qkv"][w.D + 1] = 131072.0


def _v_big_rows(lo, hi):
    """V's first column scaled by 128 and x rows [lo, hi) by 512 (powers of
    two, exact in bf16): only V values of those rows leave the fp16 range."""
    def edit(w, inp):
        D, dkv = w.D, w.n_g * (w.D // w.h)
        inp["w_qkv"][:, D + dkv] *= 128.0
        src = inp["x_q"] if inp["x_kv"] is None else inp["x_kv"]
        src[:, lo:hi] *= 512.0
    return edit


def _nan_input(w, inp):
    inp["x_q"][1, 7, 9] = float("nan")


CASES = [
    # label, workload, shrink, edit, which stored values overflow
    ("W_O conversion", "causal_bf16_d512_h8_b16_t1024", dict(B=2, T_q=256, T_k=256),
     _w_o_big, "w_o"),
    ("Q epilogue", "causal_bf16_d512_h8_b16_t1024", dict(B=2, T_q=256, T_k=256),
     _q_bias_big, "q"),
    ("K epilogue", "causal_bf16_d512_h8_b16_t1024", dict(B=2, T_q=256, T_k=256),
     _k_bias_big, "k"),
    ("V epilogue, staged tiles", "causal_bf16_d512_h8_b16_t1024", dict(B=2, T_q=300, T_k=300),
     _v_big_rows(0, 64), "v"),
    ("V epilogue, ragged tail", "causal_bf16_d512_h8_b16_t1024", dict(B=2, T_q=300, T_k=300),
     _v_big_rows(256, 300), "v"),
    ("cross-attention V", "cross_pad_bf16_d512_h8_b32_tq512_tk2048",
     dict(B=2, T_q=96, T_k=200, padding=(100, 200)), _v_big_rows(0, 200), "v"),
]


@pytest.mark.parametrize("label,name,shrink,edit,which", CASES, ids=[c[0] for c in CASES])
def test_flag_set_by_each_fp16_store(lib, label, name, shrink, edit, which):
    w, inp = _base(name, **shrink)
    edit(w, inp)
    mx = _stored_maxima(w, inp)
    over = {k: (mx[k] >= F16_INF_FROM) if k == "w_o" else bool(np.any(mx[k] >= F16_INF_FROM))
            for k in ("q", "k", "v", "w_o")}
    assert over[which] and sum(over.values()) == 1, over      # exactly the one store
    if label == "V epilogue, ragged tail":                    # only rows of the tail tile
        assert not np.any(mx["v"][:, :256] >= F16_INF_FROM)
    if label == "V epilogue, staged tiles":
        assert not np.any(mx["v"][:, 64:] >= F16_INF_FROM)
    _say(f"[overflow] {label}")
    flag = _flag(0)
    _run(lib, w, inp, flag)
    assert int(flag.item()) == 1


def test_nan_input_sets_the_flag(lib):
    w, inp = _base("causal_bf16_d512_h8_b16_t1024", B=2, T_q=128, T_k=128)
    _nan_input(w, inp)
    flag = _flag(0)
    _run(lib, w, inp, flag)
    assert int(flag.item()) == 1


WORKLOAD_CASES = [
    ("causal", "causal_bf16_d512_h8_b16_t1024", dict(B=2, T_q=300, T_k=300)),
    ("padded cross", "cross_pad_bf16_d512_h8_b32_tq512_tk2048",
     dict(B=3, T_q=96, T_k=200, padding=(100, 200))),
    ("gated d1024", "gated_causal_bf16_d1024_h16_b8_t4096", dict(B=1, T_q=200, T_k=200)),
]


@pytest.mark.parametrize("label,name,shrink", WORKLOAD_CASES, ids=[c[0] for c in WORKLOAD_CASES])
def test_flag_untouched_in_range_and_output_unchanged(lib, label, name, shrink):
    from mha_inputs import ALL_WORKLOADS
    w = ALL_WORKLOADS[name].shrink(**shrink)
    inp = make_inputs(w, seed=0)
    _say(f"[overflow] in range: {label}")
    flag = _flag(0)
    y = _run(lib, w, inp, flag)
    assert int(flag.item()) == 0
    assert torch.equal(y, _run(lib, w, inp))                 # the flag changes nothing else


def test_flag_is_never_cleared(lib):
    w, inp = _base("causal_bf16_d512_h8_b16_t1024", B=2, T_q=128, T_k=128)
    flag = _flag(1)
    _run(lib, w, inp, flag)
    assert int(flag.item()) == 1
    flag = _flag(5)
    _run(lib, w, inp, flag)
    assert int(flag.item()) == 5


def test_fp32_path_never_writes_the_flag(lib):
    w, inp = _base("self_fp32_d512_h8_b2_t128", T_q=100, T_k=100, causal=True)
    inp["b_qkv"][0] = 1e6                                      # fine in fp32
    flag = _flag(7)
    y = _run(lib, w, inp, flag)
    assert int(flag.item()) == 7
    assert torch.isfinite(y).all()
