"""Rounding emulator for a GPU storage plan of the multi-head attention forward.

TEST INFRASTRUCTURE ONLY (like the rest of this package): the product path
never imports it.

The forward pass of ``mha_oracle`` (itwiki "멀티 헤드 어텐션", 수식 and 텐서
모양으로 본 계산; iamjaehka13.blog "[Deep Learning 5]", §7-§18) evaluated in
fp64, except that values are rounded to a narrower floating-point format at
the points where a GPU implementation stores them between its kernels or
feeds them to a 16-bit matrix unit:

* the projected Q, K (``plan.qk``) and V (``plan.v``);
* the softmax numerators P = exp(s - max) (``plan.p``);
* each head's output O (``plan.o``), and W_O (``plan.w_o``);
* the final Y (``plan.y``).

Everything between two storage points is exact (fp64), which models an fp32
accumulation as error-free: the result isolates what the storage formats
cost. The pages fix no precision for any of this; the emulator exists to
choose one before writing kernels (the tolerance is max |dY| / RMS(Y)).

Options that describe how a GPU path can organise the same steps:

* ``q_prescaled``: Q is multiplied by log2(e)/sqrt(d_k) before it is rounded,
  so the score products come out in log2 units and P = 2^(s2 - max2); in
  exact arithmetic the weights are unchanged, only the rounding of Q differs.
* ``l_from_stored_p``: the row sum l adds the rounded numerators (what a sum
  computed from the stored P gives) rather than the exact ones.
* ``early_rows`` = R0 > 0 (causal self-attention only): query rows t < R0 are
  evaluated from fp32-rounded Q, K, V with exact weights, their O rounded to
  fp32 and then split into an fp16 high part and an fp16 remainder, which
  together enter the output projection (about 22 significant bits). Rows
  t >= R0 follow the plan's formats unchanged. This is the precaution for
  the first causal rows, whose outputs average few keys and so are many
  times the tensor RMS.

Rounding is round-to-nearest-even with gradual underflow, and overflow to
infinity past the largest finite value, for the binary formats fp32
(24 significand bits, smallest normal 2^-126), fp16 (11, 2^-14, largest
65504) and bf16 (8, 2^-126).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

from .mha_oracle import (_as64, _kv_width, concat_heads, head_gates, kv_head_of, linear,
                         split_heads)

# significand bits (with the leading one), exponent of the smallest normal,
# exponent of the largest finite
FORMATS = {
    "fp32": (24, -126, 127),
    "fp16": (11, -14, 15),
    "bf16": (8, -126, 127),
}


def round_to(x, fmt: str) -> np.ndarray:
    """x (float64) rounded to the nearest value of format fmt, ties to even.

    A value of magnitude in [2^E, 2^(E+1)) has the quantum 2^(E - p + 1);
    below the smallest normal the quantum stays that of the smallest normal
    binade (gradual underflow). Results beyond the largest finite value
    become +-inf. fmt "fp64" returns x unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    if fmt == "fp64":
        return x
    p, emin, emax = FORMATS[fmt]
    _, e = np.frexp(x)                    # |x| in [2^(e-1), 2^e)
    E = np.maximum(e - 1, emin)
    q = np.ldexp(1.0, E - (p - 1))
    with np.errstate(invalid="ignore"):
        r = np.rint(x / q) * q            # exact: q is a power of two
    largest = math.ldexp(2.0 - math.ldexp(1.0, 1 - p), emax)
    r = np.where(np.abs(r) > largest, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def split_hi_lo(x, fmt: str = "fp16"):
    """x as hi + lo with hi = round(x) and lo = round(x - hi) in fmt."""
    hi = round_to(x, fmt)
    return hi, round_to(x - hi, fmt)


@dataclasses.dataclass(frozen=True)
class Plan:
    """Storage formats at each rounding point ("fp64" = not rounded)."""
    qk: str = "fp64"
    v: str = "fp64"
    p: str = "fp64"
    o: str = "fp64"
    y: str = "fp64"
    w_o: str = "fp64"
    early_rows: int = 0
    q_prescaled: bool = False
    l_from_stored_p: bool = False


_BF16 = dict(qk="bf16", v="bf16", p="bf16", o="bf16", y="fp32", w_o="bf16")
_FP16 = dict(qk="fp16", v="fp16", p="fp16", o="fp16", y="fp32", w_o="fp16")

PLANS = {
    "exact": Plan(),
    # fp32 storage everywhere (the plan of an all-fp32 path)
    "fp32": Plan(qk="fp32", v="fp32", p="fp32", o="fp32", y="fp32", w_o="fp32"),
    # 16-bit storage of every intermediate, fp32 Y
    "bf16": Plan(**_BF16),
    "bf16 Q/K, fp16 V/P/O": Plan(**{**_FP16, "qk": "bf16"}),
    "fp16": Plan(**_FP16),
    "fp16, bf16 Y": Plan(**{**_FP16, "y": "bf16"}),
    "fp16 + early rows 64": Plan(**_FP16, early_rows=64),
    "bf16 + early rows 64": Plan(**_BF16, early_rows=64),
    # the fp16 plan as the HIP path organises it: Q prescaled into log2
    # units before rounding, row sums of the stored numerators
    "fp16 + early rows 64, prescaled Q, l from stored P":
        Plan(**_FP16, early_rows=64, q_prescaled=True, l_from_stored_p=True),
}
KERNEL_PLAN = "fp16 + early rows 64, prescaled Q, l from stored P"


def _attend_rounded(plan, qh, kh, vh, t_pos, causal, mask_b, fmt_qk, fmt_v, fmt_p,
                    prescale):
    """Per-head attention of query rows at positions t_pos with the given
    roundings. qh (h, n, d), kh/vh (h, T_k, d) (already one set per query
    head). Returns O (h, n, d), unrounded."""
    d_k = qh.shape[-1]
    if prescale:
        c = math.log2(math.e) / math.sqrt(d_k)
        q_r = round_to(qh * c, fmt_qk)
        s = (q_r @ np.swapaxes(round_to(kh, fmt_qk), -1, -2)) * math.log(2.0)
    else:
        q_r = round_to(qh, fmt_qk)
        s = (q_r @ np.swapaxes(round_to(kh, fmt_qk), -1, -2)) / math.sqrt(d_k)
    T_k = s.shape[-1]
    if causal:
        future = np.arange(T_k)[None, :] > np.asarray(t_pos)[:, None]
        s = np.where(future[None], -np.inf, s)
    if mask_b is not None:
        s = np.where((np.asarray(mask_b) != 0)[None, None, :], -np.inf, s)
    m = np.max(s, axis=-1, keepdims=True)
    m = np.where(np.isneginf(m), 0.0, m)
    e = np.exp(s - m)
    e_r = round_to(e, fmt_p)
    l = np.sum(e_r if plan.l_from_stored_p else e, axis=-1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        return (e_r @ round_to(vh, fmt_v)) / l


def emulate(plan: Plan, x_q, w_qkv, b_qkv, w_o, b_o, h, x_kv=None, causal=False,
            key_padding_mask=None, n_kv_heads=None, gate_w=None, gate_b=None, rows=None,
            rows_per_block=256):
    """Y with ``plan``'s roundings, for the inputs of ``mha_forward``.

    ``rows``: query positions to evaluate in every batch element (default
    all); the keys and values are always projected in full. Returns
    (B, len(rows), D) float64. Rows are evaluated in blocks of
    ``rows_per_block`` (each row is independent of the others).
    """
    x_q, x_kv, w_qkv, b_qkv, w_o, b_o = map(_as64, (x_q, x_kv, w_qkv, b_qkv, w_o, b_o))
    gate_w, gate_b = _as64(gate_w), _as64(gate_b)
    B, T_q, D = x_q.shape
    n_g = _kv_width(w_qkv, D, h, n_kv_heads)
    d_k = D // h
    d_kv = n_g * d_k
    sel = kv_head_of(h, n_g)
    rows = np.arange(T_q) if rows is None else np.asarray(rows, dtype=np.int64)
    R0 = plan.early_rows if (causal and x_kv is None) else 0
    w_o_r = round_to(w_o, plan.w_o)
    bq = None if b_qkv is None else b_qkv[:D]
    bkv = None if b_qkv is None else b_qkv[D:]
    out = np.empty((B, len(rows), D))
    for b in range(B):
        src = (x_q if x_kv is None else x_kv)[b]
        kv = linear(src, w_qkv[:, D:], bkv)                       # (T_k, 2 D_kv)
        kh = split_heads(kv[None, :, :d_kv], n_g)[0][sel]         # (h, T_k, d)
        vh = split_heads(kv[None, :, d_kv:], n_g)[0][sel]
        mask_b = None if key_padding_mask is None else np.asarray(key_padding_mask)[b]
        for r0 in range(0, len(rows), rows_per_block):
            t = rows[r0:r0 + rows_per_block]
            xq = x_q[b][t]
            qh = split_heads(linear(xq, w_qkv[:, :D], bq)[None], h)[0]   # (h, n, d)
            o = _attend_rounded(plan, qh, kh, vh, t, causal, mask_b, plan.qk, plan.v,
                                plan.p, plan.q_prescaled)
            gates = None
            if gate_w is not None:
                gates = np.transpose(head_gates(xq, gate_w, gate_b))[..., None]   # (h, n, 1)
                o = o * gates
            o = round_to(o, plan.o)
            early = np.nonzero(t < R0)[0]
            if early.size:
                # fp32 Q/K/V and weights, O in fp32 and then hi + lo in fp16
                oe = _attend_rounded(plan, round_to(qh[:, early], "fp32"),
                                     round_to(kh, "fp32"), round_to(vh, "fp32"), t[early],
                                     causal, mask_b, "fp64", "fp64", "fp64", False)
                oe = round_to(oe, "fp32")
                if gates is not None:
                    oe = round_to(oe * gates[:, early], "fp32")
                hi, lo = split_hi_lo(oe, "fp16")
                o[:, early] = hi + lo
            y = linear(concat_heads(o[None])[0], w_o_r, b_o)
            out[b, r0:r0 + len(t)] = round_to(y, plan.y)
    return out


def max_abs_over_rms(y, ref, rms=None) -> float:
    """max |y - ref| / RMS(ref) over the entries where ref is not NaN (the
    tolerance metric); ``rms`` overrides the RMS (e.g. one taken over more
    rows than were compared)."""
    ok = ~np.isnan(ref)
    if rms is None:
        rms = math.sqrt(float(np.mean(ref[ok] ** 2)))
    return float(np.max(np.abs(y[ok] - ref[ok]))) / rms
