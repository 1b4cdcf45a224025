"""Scalar brute-force multi-head attention for tiny inputs (T <= 4).

TEST INFRASTRUCTURE ONLY. Pure Python floats and ``math.exp``: no matrix
library and no max-shift, so it shares no arithmetic shape with
``mha_oracle``. Each quantity is the page formula evaluated element by element:

* q_i = x_i W_Q + b_Q (per head, columns of the fused matrix), likewise k_j, v_j
  (itwiki "멀티 헤드 어텐션", 수식 and 구현).
* s_ij = q_i . k_j / sqrt(d_k), and s_ij = -inf for masked keys
  (iamjaehka13.blog "[Deep Learning 5]", §7-§9).
* A_ij = exp(s_ij) / sum_m exp(s_im) (same page, §10); all keys masked gives
  0/0, returned as NaN (molayo1419.me "MHA란 무엇인가?", trap 3).
* o_i = sum_j A_ij v_j (§13); concat over heads and y = o W_O + b_O (§18).
* With n_g key/value sets (itwiki, 추론 비용과 변형, variants table), query
  head i takes its keys and values from set i // (h / n_g): columns
  D + g*d_k ... of the K block and D + n_g*d_k + g*d_k ... of the V block.
* Gated attention (same itwiki section, last paragraph): head i's o_i is
  multiplied by 1 / (1 + exp(-z)), z = x_q . W_G[:, i] + b_G[i].
"""

from __future__ import annotations

import math


def _matvec(x, w, col0, ncol, b):
    """Row vector x (list) times columns [col0, col0+ncol) of w, plus bias."""
    out = []
    for c in range(col0, col0 + ncol):
        acc = 0.0
        for r in range(len(x)):
            acc += x[r] * w[r][c]
        if b is not None:
            acc += b[c]
        out.append(acc)
    return out


def _gate(z):
    """Logistic function of a Python float, without overflow for large |z|."""
    if z >= 0.0:
        return 1.0 / (1.0 + math.exp(-z))
    e = math.exp(z)
    return e / (1.0 + e)


def brute_force_mha(x_q, w_qkv, b_qkv, w_o, b_o, h, x_kv=None, causal=False,
                    key_padding_mask=None, n_kv_heads=None, gate_w=None, gate_b=None):
    """Nested lists in, nested list Y[b][t][c] out. Inputs are plain floats."""
    D = len(w_qkv)
    d = D // h
    n_g = h if n_kv_heads is None else n_kv_heads
    per_group = h // n_g
    B = len(x_q)
    src = x_q if x_kv is None else x_kv
    y_all = []
    for b in range(B):
        Tq, Tk = len(x_q[b]), len(src[b])
        y_b = []
        for i in range(Tq):
            o_cat = []
            for head in range(h):
                g = head // per_group
                q = _matvec(x_q[b][i], w_qkv, head * d, d, b_qkv)
                weights = []
                for j in range(Tk):
                    masked = (causal and j > i) or (
                        key_padding_mask is not None and key_padding_mask[b][j] != 0)
                    if masked:
                        weights.append(0.0)          # exp(-inf)
                        continue
                    k = _matvec(src[b][j], w_qkv, D + g * d, d, b_qkv)
                    s = sum(q[c] * k[c] for c in range(d)) / math.sqrt(d)
                    weights.append(math.exp(s))
                total = sum(weights)
                o = [0.0] * d
                for j in range(Tk):
                    if weights[j] == 0.0:
                        continue
                    v = _matvec(src[b][j], w_qkv, D + n_g * d + g * d, d, b_qkv)
                    for c in range(d):
                        o[c] += weights[j] * v[c]
                if total == 0.0:
                    o = [float("nan")] * d
                else:
                    o = [oc / total for oc in o]
                if gate_w is not None:
                    z = sum(x_q[b][i][r] * gate_w[r][head] for r in range(D))
                    if gate_b is not None:
                        z += gate_b[head]
                    o = [oc * _gate(z) for oc in o]
                o_cat.extend(o)
            y_b.append(_matvec(o_cat, w_o, 0, D, b_o))
        y_all.append(y_b)
    return y_all


def brute_force_decode(x_new, w_qkv, b_qkv, w_o, b_o, h, k_cache, v_cache, cache_len,
                       n_kv_heads=None):
    """One generation step from nested lists: y[b][j][c] for new token j of
    batch b at position cache_len[b] + j. Its keys are the cached rows
    k_cache[b][g][0 .. cache_len[b]-1] followed by the new tokens 0..j, each
    new key and value projected from x_new (iamjaehka13.blog §21: the cache
    holds earlier tokens' keys and values)."""
    D = len(w_qkv)
    d = D // h
    n_g = h if n_kv_heads is None else n_kv_heads
    per_group = h // n_g
    y_all = []
    for b in range(len(x_new)):
        L = cache_len[b]
        y_b = []
        for j in range(len(x_new[b])):
            o_cat = []
            for head in range(h):
                g = head // per_group
                q = _matvec(x_new[b][j], w_qkv, head * d, d, b_qkv)
                keys = [k_cache[b][g][p] for p in range(L)]
                vals = [v_cache[b][g][p] for p in range(L)]
                for jj in range(j + 1):
                    keys.append(_matvec(x_new[b][jj], w_qkv, D + g * d, d, b_qkv))
                    vals.append(_matvec(x_new[b][jj], w_qkv, D + n_g * d + g * d, d, b_qkv))
                weights = [math.exp(sum(q[c] * kk[c] for c in range(d)) / math.sqrt(d))
                           for kk in keys]
                total = sum(weights)
                o = [sum(wt * vv[c] for wt, vv in zip(weights, vals)) / total for c in range(d)]
                o_cat.extend(o)
            y_b.append(_matvec(o_cat, w_o, 0, D, b_o))
        y_all.append(y_b)
    return y_all
