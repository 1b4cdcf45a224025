"""Operands above 2 GiB: the projections' copies switch from buffer loads
(32-bit byte offsets) to 64-bit global addresses once an operand (X, or the
fp16 attention output O) exceeds 2 GiB. A causal D=1024 forward with B=528,
T=2048 has X and O at 2.06 GiB each; batch elements 0 and B-1 are compared
element by element with the fp64 oracle (the workloads' 2e-2 bound on
max |err| / RMS).

X is drawn on the GPU (seeded) and the two compared batch elements are copied
back for the oracle; the weights and biases come from the shared seeded input
generator.
"""

import math
import sys

import numpy as np
import pytest
import torch

from mha_inputs import WORKLOADS, as_float64_numpy, make_inputs
from oracle import mha_oracle as mo

pytestmark = pytest.mark.gpu

B, T = 528, 2048


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_operands_above_2gib():
    import transformer_head_attention_amd as lib
    w = WORKLOADS["causal_bf16_d1024_h16_b8_t4096"].shrink(B=1, T_q=64, T_k=64)
    inp = make_inputs(w, seed=5)                     # weights and biases
    D = w.D
    assert B * T * D * 2 > (1 << 31)                 # X and O above 2 GiB
    _say(f"[large] causal D={D} h={w.h} B={B} T={T}: X {B * T * D * 2 / 2**30:.2f} GiB")
    g = torch.Generator(device="cuda:0")
    g.manual_seed(11)
    x = torch.randn((B, T, D), generator=g, device="cuda:0", dtype=torch.float32)
    x = x.to(torch.bfloat16)
    d = lambda t: t.to("cuda:0")
    m = lib.MultiHeadAttention(D, w.h, "bf16")
    y = m.forward(x, d(inp["w_qkv"]), d(inp["w_o"]), b_qkv=d(inp["b_qkv"]), b_o=d(inp["b_o"]),
                  causal=True)
    torch.cuda.synchronize()
    f = as_float64_numpy
    for b in (0, B - 1):
        xb = x[b:b + 1].cpu()
        ref = mo.mha_forward(f(xb), f(inp["w_qkv"]), f(inp["b_qkv"]), f(inp["w_o"]),
                             f(inp["b_o"]), w.h, causal=True)
        yb = y[b:b + 1].cpu().double().numpy()
        rms = math.sqrt(float(np.mean(ref ** 2)))
        err = float(np.max(np.abs(yb - ref))) / rms
        _say(f"[large] batch element {b}: err/rms = {err:.3e}")
        assert np.isfinite(yb).all()
        assert err <= 2e-2
    del x, y
    torch.cuda.empty_cache()
