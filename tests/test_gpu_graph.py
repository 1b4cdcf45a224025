"""HIP graph capture of the library's calls.

A forward pass (causal, padded cross-attention, grouped heads, fp32) and a
decode step are captured with torch.cuda.CUDAGraph on the capture stream and
replayed several times, with eager work (the output overwritten) and a
synchronisation between replays. Every replay must equal the eager result
bit for bit: the kernels are deterministic and a call allocates nothing,
synchronises nothing and records no memset node, so the captured launches
are the whole call.
"""

import sys

import pytest
import torch

from mha_inputs import DECODE_WORKLOADS, WORKLOADS, make_decode_inputs, make_inputs

pytestmark = pytest.mark.gpu

W = WORKLOADS
FORWARD = [
    ("bf16 causal d1024", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=2, T_q=300, T_k=300)),
    ("bf16 cross padded", W["cross_pad_bf16_d512_h8_b32_tq512_tk2048"],
     dict(B=3, T_q=200, T_k=333, padding=(40, 333))),
    ("bf16 GQA g4 causal", W["causal_bf16_d1024_h16_b8_t4096"], dict(B=1, T_q=257, T_k=257,
                                                                     n_kv=4)),
    ("fp32 causal", W["self_fp32_d512_h8_b2_t128"], dict(T_q=130, T_k=130, causal=True)),
]


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    import transformer_head_attention_amd as m
    return m


def _dev(t):
    return None if t is None else t.to("cuda:0")


def _same_bits(a, b):
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                       b.view(torch.int32) if b.dtype == torch.float32 else b)


@pytest.mark.parametrize("name,base,kw", FORWARD, ids=[f[0] for f in FORWARD])
def test_forward_graph_replays_equal_eager(lib, name, base, kw):
    w = base.shrink(name=name, **kw)
    _say(f"[graph] {name}: {w}")
    inp = make_inputs(w, seed=5)
    d = {k: _dev(v) if isinstance(v, torch.Tensor) else v for k, v in inp.items()}
    m = lib.MultiHeadAttention(w.D, w.h, w.dtype, num_kv_heads=w.n_g)
    ws = m.workspace(w.B, w.T_q, w.T_k, torch.device("cuda:0"))
    y_eager = torch.empty(w.B, w.T_q, w.D, dtype=torch.float32, device="cuda:0")
    y_graph = torch.empty_like(y_eager)

    def call(out):
        m.forward(d["x_q"], d["w_qkv"], d["w_o"], b_qkv=d["b_qkv"], b_o=d["b_o"],
                  x_kv=d["x_kv"], causal=d["causal"], key_padding_mask=d["key_padding_mask"],
                  out=out, workspace=ws)

    call(y_eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(y_graph)
    for rep in range(3):
        y_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"[graph] {name}: replay {rep}")
        assert _same_bits(y_graph, y_eager), f"replay {rep} differs from the eager call"


def test_decode_graph_replays_equal_eager(lib):
    w = DECODE_WORKLOADS["decode_bf16_d1024_h16_b32_t4096"].shrink(B=4, T_new=2, T_max=600,
                                                                   n_kv=4, lengths=(100, 598))
    _say(f"[graph] decode: {w}")
    inp = make_decode_inputs(w, seed=5)
    d = {k: _dev(v) if isinstance(v, torch.Tensor) else v for k, v in inp.items()}
    m = lib.MultiHeadAttention(w.D, w.h, "bf16", num_kv_heads=w.n_g)
    y_eager = torch.empty(w.B, w.T_new, w.D, dtype=torch.float32, device="cuda:0")
    y_graph = torch.empty_like(y_eager)

    def call(out):
        # the step rewrites the same cache rows each time (cache_len is not advanced)
        m.decode(d["x"], d["w_qkv"], d["w_o"], d["k_cache"], d["v_cache"], d["cache_len"],
                 b_qkv=d["b_qkv"], b_o=d["b_o"], out=out)

    call(y_eager)
    torch.cuda.synchronize()
    k_after = d["k_cache"].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(y_graph)
    for rep in range(3):
        y_graph.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _say(f"[graph] decode: replay {rep}")
        assert _same_bits(y_graph, y_eager), f"replay {rep} differs from the eager call"
        # bit patterns: rows past a sequence's length hold NaN by construction
        assert torch.equal(d["k_cache"].view(torch.int16), k_after.view(torch.int16))
