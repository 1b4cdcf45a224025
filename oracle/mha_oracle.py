"""Multi-head attention forward, fp64, from the definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Sources (pages as titled; sections / equations named, no line numbers):

* itwiki "멀티 헤드 어텐션", 수식: Attention(Q,K,V) = softmax(QK^T/sqrt(d_k)) V and
  MultiHead = Concat(head_1..head_h) W^O, with W_i^Q, W_i^K in R^{d_model x d_k},
  W_i^V in R^{d_model x d_v}, W^O in R^{h d_v x d_model}.
* itwiki, 텐서 모양으로 본 계산: the three D x D projections are usually one
  D x 3D matrix; a "head" is a slice of that output, split by view+transpose
  to (B, h, T, d_k); scores (B, h, T, T); softmax over the last axis; weighted
  sum (B, h, T, d_k); concat by transpose+reshape to (B, T, D); output
  projection W^O.
* iamjaehka13.blog "[Deep Learning 5] Attention의 내부 계산", §9: causal mask
  M_ij = 0 for j <= i and -inf for j > i, added to the scaled scores, so a
  future key's weight is exactly exp(-inf) = 0; §10: row-wise softmax, rows
  non-negative and summing to 1; §13: O = A V; §18: concat then one
  d_model x d_model W_O; §19: cross-attention takes Q from the target
  sequence and K, V from the source sequence.
* molayo1419.me "MHA란 무엇인가?", trap 2: key_padding_mask True = ignore
  this key; trap 3: a row whose keys are all ignored becomes 0/0 = NaN.
* itwiki "멀티 헤드 어텐션", 추론 비용과 변형 (variants table): MQA keeps n_h
  query heads and one key/value set shared by every head; GQA keeps n_g
  key/value sets, each shared by a group of query heads; the key/value
  elements per token and layer are 2 n_h d_h (MHA), 2 d_h (MQA), 2 n_g d_h
  (GQA).
* iamjaehka13.blog §14 and §23 (shape table, residual row): the layer's
  output can be added to its input, X' = X + O W_O (with the bias b_O, and X
  the query-side input under cross-attention).
* molayo1419.me, nn.MultiheadAttention's return values: the attention
  weights, averaged over heads (N, L, S) by default or per head (N, h, L, S).
* Same itwiki section, first paragraph, and iamjaehka13.blog §21: during
  autoregressive generation the keys and values of earlier tokens are kept in
  a KV cache, so a step computes only the new tokens' projections and reads
  every cached key and value.
* Same itwiki section, last paragraph (gated attention): the scaled
  dot-product attention output of each head is multiplied by a sigmoid gate
  of its own.

Conventions (readings where the pages leave a step open):

* Weights are stored as y = x . W: W_QKV is (D, 3D) with column blocks
  [Q | K | V]; inside each block head i owns columns [i*d_k, (i+1)*d_k).
* Cross-attention with one fused W_QKV: Q = X_q W_QKV[:, :D] + b[:D] and
  [K | V] = X_kv W_QKV[:, D:] + b[D:].
* Grouped key/value heads (n_g = n_kv_heads sets, n_g divides h): the fused
  matrix is (D, D + 2 n_g d_k) with column blocks [Q | K | V], set g owning
  columns [g*d_k, (g+1)*d_k) of the K and of the V block, and query head i
  uses set i // (h / n_g) (consecutive query heads form a group). n_g = h is
  plain multi-head attention, n_g = 1 multi-query attention.
* The scale is 1/sqrt(d_k) (one page prints QK^T/d_k; every other statement,
  including the variance argument of §8 on iamjaehka13.blog, has the root).
* Gated attention (the page does not say what the gate is computed from):
  one gate value per batch element, query position and head, from the
  query-side input like the projections, sigma(x_q . W_G + b_G) with W_G of
  shape (D, h) and b_G of shape (h,); head i's output O_i (the weighted sum
  of its values) is multiplied by column i of it before the concat. Without
  W_G there is no gate.
* softmax subtracts the row maximum before exponentiating. In exact
  arithmetic this changes nothing (the factor exp(-max) cancels); it only
  keeps exp() in range. A row with every key masked is 0/0 = NaN.
"""

from __future__ import annotations

import math

import numpy as np


def linear(x: np.ndarray, w: np.ndarray, b) -> np.ndarray:
    """y = x . W + b for x (..., D_in), W (D_in, D_out), b (D_out,) or None."""
    y = x @ w
    if b is not None:
        y = y + b
    return y


def split_heads(y: np.ndarray, h: int) -> np.ndarray:
    """(B, T, D) -> (B, h, T, d_k): head i is columns [i*d_k, (i+1)*d_k)."""
    B, T, D = y.shape
    if D % h != 0:
        raise ValueError("embed_dim must be divisible by num_heads")
    return y.reshape(B, T, h, D // h).transpose(0, 2, 1, 3)


def concat_heads(o: np.ndarray) -> np.ndarray:
    """(B, h, T, d_v) -> (B, T, h*d_v): head i lands in columns [i*d_v, (i+1)*d_v)."""
    B, h, T, d = o.shape
    return o.transpose(0, 2, 1, 3).reshape(B, T, h * d)


def masked_scores(q: np.ndarray, k: np.ndarray, causal: bool, key_padding_mask,
                  q_pos=None) -> np.ndarray:
    """QK^T / sqrt(d_k) + M for q (B, h, Tq, d_k), k (B, h, Tk, d_k).

    ``causal`` puts -inf at key j > query position i. ``key_padding_mask``
    (B, Tk), nonzero = ignore, puts -inf at those keys. ``q_pos`` gives the
    sequence positions of the query rows (default 0..Tq-1), so that a subset
    of rows can be evaluated on its own.
    """
    d_k = q.shape[-1]
    s = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(d_k)
    Tq, Tk = s.shape[-2], s.shape[-1]
    if causal:
        i = np.arange(Tq) if q_pos is None else np.asarray(q_pos)
        future = np.arange(Tk)[None, :] > i[:, None]          # (Tq, Tk)
        s = np.where(future[None, None], -np.inf, s)
    if key_padding_mask is not None:
        ignore = np.asarray(key_padding_mask) != 0              # (B, Tk)
        s = np.where(ignore[:, None, None, :], -np.inf, s)
    return s


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Softmax over the last axis; an all -inf row gives 0/0 = NaN."""
    m = np.max(s, axis=-1, keepdims=True)
    m = np.where(np.isneginf(m), 0.0, m)   # all-masked row: exp(-inf - 0) = 0
    e = np.exp(s - m)
    with np.errstate(invalid="ignore", divide="ignore"):
        return e / np.sum(e, axis=-1, keepdims=True)


def attention(q, k, v, causal=False, key_padding_mask=None, q_pos=None):
    """softmax(QK^T/sqrt(d_k) + M) V per (batch, head). Returns (O, A)."""
    a = softmax_rows(masked_scores(q, k, causal, key_padding_mask, q_pos))
    return a @ v, a


def sigmoid(x):
    """1 / (1 + exp(-x)); for very negative x, exp overflows to inf and the
    result is 1/inf = 0."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def head_gates(x_q, gate_w, gate_b) -> np.ndarray:
    """Gate of every head at every query position: sigma(x_q . W_G + b_G),
    (B, T_q, h) for x_q (B, T_q, D), W_G (D, h), b_G (h,) or None."""
    return sigmoid(linear(x_q, gate_w, gate_b))


def apply_gates(o: np.ndarray, gates: np.ndarray) -> np.ndarray:
    """O (B, h, T, d_v) with head i's rows multiplied by gates (B, T, h)[..., i]."""
    return o * np.transpose(gates, (0, 2, 1))[..., None]


def _as64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def kv_head_of(h: int, n_kv_heads: int) -> np.ndarray:
    """Key/value set used by each query head: head i -> i // (h / n_g)."""
    if n_kv_heads < 1 or h % n_kv_heads != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    return np.arange(h) // (h // n_kv_heads)


def _qkv(x_q, x_kv, w_qkv, b_qkv, D):
    """Fused projection: one D x (D + 2 D_kv) matrix for self-attention; for
    cross-attention Q comes from x_q and K, V from x_kv. D_kv = n_g d_k
    (= D for plain multi-head attention)."""
    d_kv = (w_qkv.shape[1] - D) // 2
    if x_kv is None:
        y = linear(x_q, w_qkv, b_qkv)
        return y[..., :D], y[..., D:D + d_kv], y[..., D + d_kv:]
    bq = None if b_qkv is None else b_qkv[:D]
    bkv = None if b_qkv is None else b_qkv[D:]
    q = linear(x_q, w_qkv[:, :D], bq)
    kv = linear(x_kv, w_qkv[:, D:], bkv)
    return q, kv[..., :d_kv], kv[..., d_kv:]


def _kv_width(w_qkv, D, h, n_kv_heads):
    n_g = h if n_kv_heads is None else n_kv_heads
    kv_head_of(h, n_g)
    if w_qkv.shape[1] != D + 2 * n_g * (D // h):
        raise ValueError("W_QKV must be (D, D + 2 n_kv_heads d_k)")
    return n_g


def _attend_grouped(qh, kh, vh, n_g, causal, mask, q_pos=None):
    """Attention with key/value set kv_head_of(h, n_g)[i] for query head i."""
    h = qh.shape[1]
    sel = kv_head_of(h, n_g)
    return attention(qh, kh[:, sel], vh[:, sel], causal, mask, q_pos)


def mha_forward(x_q, w_qkv, b_qkv, w_o, b_o, h, x_kv=None, causal=False,
                key_padding_mask=None, return_intermediates=False, n_kv_heads=None,
                residual=False, gate_w=None, gate_b=None):
    """Y = Concat(head_1..head_h) W^O + b_O for batch-first inputs.

    x_q (B, T_q, D); x_kv (B, T_k, D) or None for self-attention;
    w_qkv (D, D + 2 n_g d_k) (3D wide for n_kv_heads None = h);
    b_qkv (D + 2 n_g d_k,) or None; w_o (D, D); b_o (D,) or None;
    key_padding_mask (B, T_k), nonzero = ignore, or None. ``residual`` adds
    x_q to the result. ``gate_w`` (D, h) and ``gate_b`` (h,) or None: gated
    attention, head i's output times sigma(x_q . W_G + b_G)[..., i].
    Everything is evaluated in float64.
    """
    x_q, x_kv, w_qkv, b_qkv, w_o, b_o = map(_as64, (x_q, x_kv, w_qkv, b_qkv, w_o, b_o))
    gate_w, gate_b = _as64(gate_w), _as64(gate_b)
    B, T_q, D = x_q.shape
    if D % h != 0:
        raise ValueError("embed_dim must be divisible by num_heads")
    if causal and x_kv is not None and x_kv.shape[1] != T_q:
        raise ValueError("causal mask needs T_q == T_k")
    n_g = _kv_width(w_qkv, D, h, n_kv_heads)
    q, k, v = _qkv(x_q, x_kv, w_qkv, b_qkv, D)
    qh = split_heads(q, h)
    kh, vh = split_heads(k, n_g), split_heads(v, n_g)
    o, a = _attend_grouped(qh, kh, vh, n_g, causal, key_padding_mask)
    if gate_w is not None:
        o = apply_gates(o, head_gates(x_q, gate_w, gate_b))
    o_cat = concat_heads(o)
    y = linear(o_cat, w_o, b_o)
    if residual:
        y = x_q + y
    if return_intermediates:
        return y, {"q": qh, "k": kh, "v": vh, "a": a, "o": o_cat}
    return y


def attention_weights(x_q, w_qkv, b_qkv, h, x_kv=None, causal=False, key_padding_mask=None,
                      n_kv_heads=None, average=False):
    """The softmax weights A of every head, (B, h, T_q, T_k), or their mean
    over heads, (B, T_q, T_k), for the same inputs as ``mha_forward``."""
    x_q, x_kv, w_qkv, b_qkv = map(_as64, (x_q, x_kv, w_qkv, b_qkv))
    D = x_q.shape[2]
    n_g = _kv_width(w_qkv, D, h, n_kv_heads)
    q, k, v = _qkv(x_q, x_kv, w_qkv, b_qkv, D)
    _, a = _attend_grouped(split_heads(q, h), split_heads(k, n_g), split_heads(v, n_g), n_g,
                           causal, key_padding_mask)
    return a.mean(axis=1) if average else a


def mha_forward_rows(x_q, w_qkv, b_qkv, w_o, b_o, h, rows, x_kv=None,
                     causal=False, key_padding_mask=None, n_kv_heads=None, residual=False,
                     gate_w=None, gate_b=None):
    """Y[b, t, :] for selected query rows only.

    ``rows`` maps a batch index b to a 1-D array of query positions t. The
    keys and values of batch b are projected in full; only the selected query
    rows are projected, attended and output-projected. Each row's result is
    the same as that row of ``mha_forward`` (rows are independent).
    Returns {b: (len(rows[b]), D) float64 array}.
    """
    w_qkv, b_qkv, w_o, b_o = map(_as64, (w_qkv, b_qkv, w_o, b_o))
    gate_w, gate_b = _as64(gate_w), _as64(gate_b)
    D = w_qkv.shape[0]
    n_g = _kv_width(w_qkv, D, h, n_kv_heads)
    d_kv = n_g * (D // h)
    out = {}
    for b, ts in rows.items():
        ts = np.asarray(ts, dtype=np.int64)
        xq_b = _as64(x_q[b])[ts][None]                       # (1, n, D)
        xkv_b = _as64((x_q if x_kv is None else x_kv)[b])[None]
        bq = None if b_qkv is None else b_qkv[:D]
        bkv = None if b_qkv is None else b_qkv[D:]
        q = linear(xq_b, w_qkv[:, :D], bq)
        kv = linear(xkv_b, w_qkv[:, D:], bkv)
        k, v = kv[..., :d_kv], kv[..., d_kv:]
        mask_b = None if key_padding_mask is None else np.asarray(key_padding_mask)[b:b + 1]
        qh = split_heads(q, h)
        kh, vh = split_heads(k, n_g), split_heads(v, n_g)
        o, _ = _attend_grouped(qh, kh, vh, n_g, causal, mask_b, q_pos=ts)
        if gate_w is not None:
            o = apply_gates(o, head_gates(xq_b, gate_w, gate_b))
        out[b] = linear(concat_heads(o), w_o, b_o)[0]
        if residual:
            out[b] = xq_b[0] + out[b]
    return out


def mha_forward_blocked(x_q, w_qkv, b_qkv, w_o, b_o, h, x_kv=None, causal=False,
                        key_padding_mask=None, n_kv_heads=None, residual=False,
                        gate_w=None, gate_b=None, rows_per_block=256, progress=None,
                        map_blocks=map):
    """The whole of ``mha_forward``'s Y, evaluated one batch element and one
    block of query rows at a time so that the score tensor held at once is
    (h, rows_per_block, T_k) instead of (B, h, T_q, T_k).

    The same steps as ``mha_forward``: per batch element the fused projection
    of all its rows (Q from x_q, K and V from x_kv or x_q), the head split,
    then per block of query rows the masked scores at those rows' positions,
    the row softmax, the weighted sum, the concat and W_O. Rows are
    independent, so every row equals that row of ``mha_forward``, whatever
    order the blocks are evaluated in: ``map_blocks`` (default the builtin
    map) may evaluate them concurrently, e.g. a thread pool's map.
    ``progress(b, t0, t1)`` is called after each block, if given.
    """
    w_qkv, b_qkv, w_o, b_o = map(_as64, (w_qkv, b_qkv, w_o, b_o))
    gate_w, gate_b = _as64(gate_w), _as64(gate_b)
    B, T_q, D = x_q.shape
    if D % h != 0:
        raise ValueError("embed_dim must be divisible by num_heads")
    if causal and x_kv is not None and x_kv.shape[1] != T_q:
        raise ValueError("causal mask needs T_q == T_k")
    n_g = _kv_width(w_qkv, D, h, n_kv_heads)
    y = np.empty((B, T_q, D), dtype=np.float64)
    for b in range(B):
        xq_b = _as64(x_q[b])[None]
        xkv_b = None if x_kv is None else _as64(x_kv[b])[None]
        q, k, v = _qkv(xq_b, xkv_b, w_qkv, b_qkv, D)
        qh = split_heads(q, h)
        kh, vh = split_heads(k, n_g), split_heads(v, n_g)
        mask_b = None if key_padding_mask is None else np.asarray(key_padding_mask)[b:b + 1]

        def rows_block(t0, qh=qh, kh=kh, vh=vh, mask_b=mask_b, xq_b=xq_b):
            t1 = min(T_q, t0 + rows_per_block)
            o, _ = _attend_grouped(qh[:, :, t0:t1], kh, vh, n_g, causal, mask_b,
                                   q_pos=np.arange(t0, t1))
            if gate_w is not None:
                o = apply_gates(o, head_gates(xq_b[:, t0:t1], gate_w, gate_b))
            yb = linear(concat_heads(o), w_o, b_o)[0]
            if residual:
                yb = xq_b[0, t0:t1] + yb
            return t0, t1, yb

        for t0, t1, yb in map_blocks(rows_block, range(0, T_q, rows_per_block)):
            y[b, t0:t1] = yb
            if progress is not None:
                progress(b, t0, t1)
    return y


def mha_decode(x_new, w_qkv, b_qkv, w_o, b_o, h, k_cache, v_cache, cache_len,
               n_kv_heads=None):
    """One generation step against a KV cache, batch-first.

    x_new (B, T_new, D): the new tokens; batch element b holds positions
    cache_len[b] .. cache_len[b] + T_new - 1. k_cache, v_cache (B, n_g, T_max,
    d_k): rows [0, cache_len[b]) of batch b are the keys and values of its
    earlier tokens (later rows are ignored). The new tokens' keys and values
    are projected from x_new and appended after the cached ones; new token j
    attends to every cached key and to new tokens 0..j (the causal mask at its
    position). Returns (y (B, T_new, D), k_new, v_new (B, n_g, T_new, d_k)),
    k_new and v_new being what the step appends to the cache.
    """
    x_new, w_qkv, b_qkv, w_o, b_o = map(_as64, (x_new, w_qkv, b_qkv, w_o, b_o))
    k_cache, v_cache = _as64(k_cache), _as64(v_cache)
    B, T_new, D = x_new.shape
    if D % h != 0:
        raise ValueError("embed_dim must be divisible by num_heads")
    n_g = _kv_width(w_qkv, D, h, n_kv_heads)
    q, k, v = _qkv(x_new, None, w_qkv, b_qkv, D)
    qh = split_heads(q, h)
    k_new, v_new = split_heads(k, n_g), split_heads(v, n_g)
    lens = np.asarray(cache_len, dtype=np.int64)
    o = np.empty_like(qh)
    for b in range(B):
        L = int(lens[b])
        if L < 0 or L > k_cache.shape[2]:
            raise ValueError("cache_len out of range")
        kb = np.concatenate([k_cache[b, :, :L], k_new[b]], axis=1)[None]
        vb = np.concatenate([v_cache[b, :, :L], v_new[b]], axis=1)[None]
        o[b:b + 1], _ = _attend_grouped(qh[b:b + 1], kb, vb, n_g, True, None,
                                        q_pos=L + np.arange(T_new))
    y = linear(concat_heads(o), w_o, b_o)
    return y, k_new, v_new


def param_count(D: int, h: int, bias: bool = True, n_kv_heads=None) -> int:
    """Number of parameters of one MHA layer as this module stores them:
    W_QKV (D x (D + 2 n_g d_k)), W_O (D x D) and, with ``bias``, b_QKV and
    b_O. With n_g = h the head count only slices the same matrices
    (molayo1419.me, parameter table: 4E^2 + 4E for every num_heads)."""
    if D % h != 0:
        raise ValueError("embed_dim must be divisible by num_heads")
    n_g = h if n_kv_heads is None else n_kv_heads
    kv_head_of(h, n_g)
    n_qkv = D + 2 * n_g * (D // h)
    shapes = [(D, n_qkv), (D, D)] + ([(n_qkv,), (D,)] if bias else [])
    return int(sum(np.prod(s) for s in shapes))


def kv_elements_per_token(D: int, h: int, n_kv_heads=None) -> int:
    """Key and value elements one token leaves per layer: the widths of the
    K and V blocks of the projection output."""
    n_g = h if n_kv_heads is None else n_kv_heads
    kv_head_of(h, n_g)
    return 2 * n_g * (D // h)
