"""Seeded synthetic inputs for the multi-head attention forward pass.

This module is shared by the fp64 oracle's tests, the GPU parity tests, the
benchmark and the smoke check. It holds workload descriptions and random
draws only: none of the attention arithmetic lives here.

Workloads follow the pages' own settings where they give them:

* d_model = 512, h = 8, d_k = d_v = 64 is the original paper's setting quoted
  by itwiki "멀티 헤드 어텐션", section 수식, and by molayo1419.me
  "MHA란 무엇인가?", closing references.
* Batch-first (B, T, D) inputs, as in the tensor-shape table of itwiki
  "멀티 헤드 어텐션", section 텐서 모양으로 본 계산.
* Cross-attention takes queries from one sequence and keys/values from
  another (itwiki, section 수식, last paragraph; iamjaehka13.blog
  "[Deep Learning 5] Attention의 내부 계산", §19).
* A key-padding mask marks keys to IGNORE with a nonzero value, the
  nn.MultiheadAttention convention described in molayo1419.me, trap 2.
* Grouped key/value heads (itwiki, 추론 비용과 변형, variants table): n_g
  key/value sets for n_h query heads; W_QKV is then (D, D + 2 n_g d_k).

Readings taken where the workload text is silent (each is listed in the
design notes):

* "Xavier-uniform" is U(-a, a), a = sqrt(6 / (fan_in + fan_out)), gain 1.
  For the fused (D, 3D) projection fan_in = D, fan_out = 3D (D + 2 n_g d_k
  with grouped key/value heads).
* "N(0, s)" names the standard deviation s.
* Key padding is trailing: keys j >= len_b of batch element b are masked,
  with len_b an integer drawn uniformly from [256, 2048] inclusive.
* Values are drawn in fp32 and rounded once, round-to-nearest-even, to the
  workload's dtype; everything downstream sees those rounded values.

Draw order from one CPU ``torch.Generator`` seeded with ``seed``:
X (or X_q then X_kv), W_QKV, W_O, b_QKV, b_O, then the valid lengths, then
(gated attention only) W_G and b_G.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    """One attention problem: sizes, dtype, masks and the input distributions."""

    name: str
    dtype: str            # "fp32" or "bf16": the input/weight storage type
    D: int                # d_model
    h: int                # number of heads
    B: int                # batch
    T_q: int              # query length
    T_k: int              # key/value length (== T_q for self-attention)
    cross: bool = False   # keys/values from a second sequence X_kv
    causal: bool = False
    padding: Optional[tuple] = None   # (lo, hi) inclusive range of valid key lengths
    weight_init: str = "xavier"       # "xavier" or ("normal", std)
    weight_std: float = 0.0
    bias_std: Optional[float] = None  # None -> zero biases
    n_kv: Optional[int] = None        # key/value sets n_g (None -> h, plain MHA)
    gate: bool = False                # gated attention: W_G (D, h), b_G (h)

    @property
    def d_k(self) -> int:
        return self.D // self.h

    @property
    def n_g(self) -> int:
        return self.h if self.n_kv is None else self.n_kv

    @property
    def n_qkv(self) -> int:
        """Width of the fused projection: D + 2 n_g d_k."""
        return self.D + 2 * self.n_g * self.d_k

    def flops(self) -> float:
        """Formula FLOPs: projections 4*T_q*D^2 + 4*T_k*D^2 (8*T*D^2 when
        T_q == T_k) plus 4*T_q*T_k*D for scores and weighted sum, halved
        under a causal mask, per batch element (itwiki, 매개변수와 계산량).
        With n_g key/value sets the K and V projections are n_g d_k wide:
        4*T_k*D*n_g*d_k instead of 4*T_k*D^2. Gated attention adds the gate
        projection, 2*T_q*D*h."""
        proj = 4.0 * self.T_q * self.D ** 2 + 4.0 * self.T_k * self.D * self.n_g * self.d_k
        attn = 4.0 * self.T_q * self.T_k * self.D
        if self.causal:
            attn *= 0.5
        gate = 2.0 * self.T_q * self.D * self.h if self.gate else 0.0
        return self.B * (proj + attn + gate)

    def shrink(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads this path is checked and measured on, named by content.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("self_fp32_d512_h8_b2_t128", "fp32", 512, 8, 2, 128, 128,
                 bias_std=0.02),
        Workload("causal_bf16_d512_h8_b16_t1024", "bf16", 512, 8, 16, 1024, 1024,
                 causal=True),
        Workload("causal_bf16_d1024_h16_b8_t4096", "bf16", 1024, 16, 8, 4096, 4096,
                 causal=True, bias_std=0.02),
        Workload("cross_pad_bf16_d512_h8_b32_tq512_tk2048", "bf16", 512, 8, 32, 512,
                 2048, cross=True, padding=(256, 2048)),
        Workload("causal_bf16_d4096_h32_b1_t8192", "bf16", 4096, 32, 1, 8192, 8192,
                 causal=True, weight_init="normal", weight_std=1.0 / 64.0),
    ]
}

# Grouped key/value heads at the d_model = 1024 causal shape: GQA with 4 sets
# of 4 query heads, and MQA (one set shared by all 16 heads).
GROUPED_WORKLOADS = {
    w.name: w
    for w in [
        Workload("gqa4_causal_bf16_d1024_h16_b8_t4096", "bf16", 1024, 16, 8, 4096, 4096,
                 causal=True, bias_std=0.02, n_kv=4),
        Workload("mqa_causal_bf16_d1024_h16_b8_t4096", "bf16", 1024, 16, 8, 4096, 4096,
                 causal=True, bias_std=0.02, n_kv=1),
    ]
}
# Gated attention (itwiki, 추론 비용과 변형, last paragraph) at the d_model =
# 1024 causal shape: W_G Xavier-uniform (fan_in D, fan_out h), b_G N(0, 0.02).
GATED_WORKLOADS = {
    w.name: w
    for w in [
        Workload("gated_causal_bf16_d1024_h16_b8_t4096", "bf16", 1024, 16, 8, 4096, 4096,
                 causal=True, bias_std=0.02, gate=True),
    ]
}
ALL_WORKLOADS = {**WORKLOADS, **GROUPED_WORKLOADS, **GATED_WORKLOADS}

HEADLINE = "causal_bf16_d1024_h16_b8_t4096"

_TORCH_DTYPE = {"fp32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(w: Workload) -> torch.dtype:
    return _TORCH_DTYPE[w.dtype]


def _uniform(g, shape, a):
    return torch.rand(shape, generator=g, dtype=torch.float32) * (2.0 * a) - a


def _normal(g, shape, std):
    return torch.randn(shape, generator=g, dtype=torch.float32) * std


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Draw the inputs of workload ``w`` on the CPU.

    Returns a dict of CPU tensors in the workload dtype (the mask is uint8,
    nonzero = ignore this key) plus the scalar settings. Zero biases are
    returned as zero tensors.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    D = w.D
    x_q = _normal(g, (w.B, w.T_q, D), 1.0)
    x_kv = _normal(g, (w.B, w.T_k, D), 1.0) if w.cross else None
    n_qkv = w.n_qkv
    if w.weight_init == "xavier":
        w_qkv = _uniform(g, (D, n_qkv), math.sqrt(6.0 / (D + n_qkv)))
        w_o = _uniform(g, (D, D), math.sqrt(6.0 / (D + D)))
    else:
        w_qkv = _normal(g, (D, n_qkv), w.weight_std)
        w_o = _normal(g, (D, D), w.weight_std)
    if w.bias_std is None:
        b_qkv = torch.zeros(n_qkv)
        b_o = torch.zeros(D)
    else:
        b_qkv = _normal(g, (n_qkv,), w.bias_std)
        b_o = _normal(g, (D,), w.bias_std)
    mask = None
    lengths = None
    if w.padding is not None:
        lo, hi = w.padding
        lengths = torch.randint(lo, hi + 1, (w.B,), generator=g)
        j = torch.arange(w.T_k)
        mask = (j[None, :] >= lengths[:, None]).to(torch.uint8)
    gate_w = gate_b = None
    if w.gate:
        # drawn last, so the other inputs equal those of the ungated workload
        gate_w = _uniform(g, (D, w.h), math.sqrt(6.0 / (D + w.h)))
        gate_b = torch.zeros(w.h) if w.bias_std is None else _normal(g, (w.h,), w.bias_std)
    dt = torch_dtype(w)
    out = {
        "x_q": x_q.to(dt),
        "x_kv": None if x_kv is None else x_kv.to(dt),
        "w_qkv": w_qkv.to(dt),
        "b_qkv": b_qkv.to(dt),
        "w_o": w_o.to(dt),
        "b_o": b_o.to(dt),
        "key_padding_mask": mask,
        "lengths": lengths,
        "gate_w": None if gate_w is None else gate_w.to(dt),
        "gate_b": None if gate_b is None else gate_b.to(dt),
        "h": w.h,
        "n_kv": w.n_g,
        "causal": w.causal,
    }
    return out


@dataclass(frozen=True)
class DecodeWorkload:
    """One generation step against a KV cache (bf16): B sequences with
    cached lengths drawn uniformly from ``lengths`` (inclusive), T_new new
    tokens each, caches of capacity T_max."""

    name: str
    D: int
    h: int
    B: int
    T_new: int
    T_max: int
    lengths: tuple
    n_kv: Optional[int] = None
    bias_std: Optional[float] = 0.02
    dtype: str = "bf16"

    @property
    def d_k(self) -> int:
        return self.D // self.h

    @property
    def n_g(self) -> int:
        return self.h if self.n_kv is None else self.n_kv

    @property
    def n_qkv(self) -> int:
        return self.D + 2 * self.n_g * self.d_k

    def flops(self, lengths) -> float:
        """Projections of the new tokens (2 D N_qkv + 2 D^2 per token) plus
        scores and weighted sum over (cached + causal new) keys, 4 d_k per
        (query head, key) pair."""
        tok = self.B * self.T_new
        proj = tok * (2.0 * self.D * self.n_qkv + 2.0 * self.D * self.D)
        pairs = sum(int(L) * self.T_new + self.T_new * (self.T_new + 1) // 2 for L in lengths)
        return proj + 4.0 * self.d_k * self.h * pairs

    def cache_bytes(self, lengths) -> float:
        """bf16 key and value bytes a step must read (cached rows only)."""
        return 2.0 * 2.0 * self.n_g * self.d_k * float(sum(int(L) for L in lengths))

    def shrink(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


DECODE_WORKLOADS = {
    w.name: w
    for w in [
        DecodeWorkload("decode_bf16_d1024_h16_b32_t4096", 1024, 16, 32, 1, 4096, (2048, 4095)),
        DecodeWorkload("decode_gqa4_bf16_d1024_h16_b32_t4096", 1024, 16, 32, 1, 4096,
                       (2048, 4095), n_kv=4),
        DecodeWorkload("decode_mqa_bf16_d1024_h16_b32_t4096", 1024, 16, 32, 1, 4096,
                       (2048, 4095), n_kv=1),
        DecodeWorkload("decode_bf16_d4096_h32_b8_t8192", 4096, 32, 8, 1, 8192, (4096, 8191),
                       bias_std=None),
    ]
}


def make_decode_inputs(w: DecodeWorkload, seed: int = 0) -> dict:
    """Draw a generation step's inputs on the CPU (bf16 tensors, int32 lengths).

    Draw order: x_new, W_QKV, W_O, b_QKV, b_O, lengths, K cache, V cache.
    Weights are Xavier-uniform as for the forward workloads; cached keys and
    values are N(0, s) with s the standard deviation of a projected value
    under those distributions, sqrt(D a^2 / 3) for the W_QKV bound a. Cache
    rows at or past a sequence's length are filled with NaN: they must never
    be read.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    D, n_qkv = w.D, w.n_qkv
    x = _normal(g, (w.B, w.T_new, D), 1.0)
    a = math.sqrt(6.0 / (D + n_qkv))
    w_qkv = _uniform(g, (D, n_qkv), a)
    w_o = _uniform(g, (D, D), math.sqrt(6.0 / (D + D)))
    if w.bias_std is None:
        b_qkv, b_o = torch.zeros(n_qkv), torch.zeros(D)
    else:
        b_qkv = _normal(g, (n_qkv,), w.bias_std)
        b_o = _normal(g, (D,), w.bias_std)
    lo, hi = w.lengths
    if not 0 <= lo <= hi <= w.T_max - w.T_new:
        raise ValueError("cached lengths must lie in [0, T_max - T_new]")
    lengths = torch.randint(lo, hi + 1, (w.B,), generator=g).to(torch.int32)
    s = math.sqrt(D * a * a / 3.0)
    shape = (w.B, w.n_g, w.T_max, w.d_k)
    k_cache = _normal(g, shape, s)
    v_cache = _normal(g, shape, s)
    pos = torch.arange(w.T_max)
    unused = (pos[None, :] >= lengths[:, None].long())[:, None, :, None]
    k_cache = torch.where(unused, torch.full_like(k_cache, float("nan")), k_cache)
    v_cache = torch.where(unused, torch.full_like(v_cache, float("nan")), v_cache)
    dt = torch.bfloat16
    return {"x": x.to(dt), "w_qkv": w_qkv.to(dt), "w_o": w_o.to(dt), "b_qkv": b_qkv.to(dt),
            "b_o": b_o.to(dt), "k_cache": k_cache.to(dt), "v_cache": v_cache.to(dt),
            "cache_len": lengths, "h": w.h, "n_kv": w.n_g}


def as_float64_numpy(t):
    """Exact upcast of a (bf16 or fp32) CPU tensor to a float64 numpy array."""
    if t is None:
        return None
    return t.to(torch.float64).numpy()
