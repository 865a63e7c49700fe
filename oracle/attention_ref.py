"""Plain fp64 CPU oracle for multi-head scaled dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests, the smoke check and the bench's CPU-baseline leg
use it. It shares no code with the HIP library or its Python binding.

What it computes is the pages' definition written out, one step at a time,
in float64, materialising the full score matrix:

* Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V, the softmax taken over
  each row (one query against all keys) -- "The Transformer"
  (hoshank.vercel.app), "The Mathematics", the Attention equation and its
  symbol table; the same formula in "How Transformers Work"
  (worksonmygpu.com), "Scaled dot-product attention", steps 1-4.
* MultiHead(Q, K, V) = Concat(head_1..head_h) W^O with
  head_i = Attention(Q W_i^Q, K W_i^K, V W_i^V) -- same page, the MultiHead
  equation and its symbol table, written out head by head: W_i is the i-th
  block of d_k columns of the stored projection matrix, and Concat lays the
  heads side by side in order.
* The causal mask is an additive matrix, 0 on and below the diagonal and -inf
  above it, added to the scores before the softmax, so a blocked key gets a
  weight of exactly 0 -- "The Transformer" (rayaq.ca), "Masks: who may look at
  whom", with its printed 4x4 example.

* A key-padding mask works the same way, one row per batch item: every key
  at or past the item's length gets -inf for every query -- same page, same
  section, on the *_key_padding_mask arguments. The length is given as a
  number of valid keys, so no boolean polarity is involved.

Readings where the pages are silent (each is listed in the design notes):
the softmax subtracts the row maximum before exponentiating (softmax is
unchanged by a per-row shift; it only avoids overflow); no biases in the
projections; weights are stored (in, out) so Q = X W; the causal mask is only
defined for N_q == N_k; a row whose keys are all masked (length 0) has no
softmax, and its output is taken as 0 with a log-sum-exp of -inf.

Every function here is pinned by tests/test_oracle.py against properties the
pages fix (rows sum to 1, permutation equivariance, the printed mask, closed
forms, brute force on tiny inputs, an independent library routine).
"""
from __future__ import annotations

import math

import numpy as np


def causal_mask(n: int) -> np.ndarray:
    """Additive causal mask: 0 where key j <= query i, -inf where j > i.

    "The Transformer" (rayaq.ca), "Masks: who may look at whom": the decoder's
    mask is the strictly upper triangle filled with -inf, diagonal kept.
    """
    m = np.zeros((n, n), dtype=np.float64)
    for i in range(n):
        for j in range(i + 1, n):
            m[i, j] = -np.inf
    return m


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row-wise softmax over the last axis: each row becomes weights summing to 1.

    "The Transformer" (hoshank.vercel.app), "The Mathematics", symbol table
    entry for softmax. Subtracting the row maximum first leaves the result
    unchanged and keeps exp() finite.
    """
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention_weights_ref(q: np.ndarray, k: np.ndarray, *, causal: bool = False,
                          scale: float | None = None, rows=None) -> np.ndarray:
    """P = softmax(scale * Q K^T (+ causal mask)) for one (batch, head).

    q: (N_q, d_k), k: (N_k, d_k). rows: optional query positions; only those
    rows of P are formed, each one complete over all keys.
    Default scale is 1/sqrt(d_k) ("The Transformer" (hoshank.vercel.app),
    "The Mathematics"; "32 Transformer", "Why we divide by sqrt(dk)").
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d_k = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    pos = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = np.matmul(q[pos], k.T) * scale            # every query dotted with every key
    if causal:
        if q.shape[0] != k.shape[0]:
            raise ValueError("the causal mask is defined for N_q == N_k only")
        s = s + causal_mask(k.shape[0])[pos]
    return softmax_rows(s)


def key_padding_mask_row(n_k: int, length: int) -> np.ndarray:
    """Additive key-padding row of one batch item: 0 for keys j < length,
    -inf for j >= length ("The Transformer" (rayaq.ca), "Masks: who may look
    at whom": padding masks, one row per batch item)."""
    m = np.zeros((n_k,), dtype=np.float64)
    m[int(length):] = -np.inf
    return m


def attention_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool = False,
                  scale: float | None = None, rows=None, kv_len=None):
    """O = softmax(scale * Q K^T (+ mask)) V over every (batch, head).

    q: (B, H, N_q, d_k), k: (B, H, N_k, d_k), v: (B, H, N_k, d_v); any float
    dtype, widened exactly to float64. rows: optional sorted query positions
    (the same for every (b, h)); the outputs then hold only those rows.
    kv_len: optional per-batch number of valid keys (clamped to [0, N_k]);
    keys at or past it are masked for every query and head of that item.
    A row with no unmasked key gets O = 0, rowsum = 0 and lse = -inf.

    Returns (O, rowsum, lse):
      O      (B, H, R, d_v)  attention output
      rowsum (B, H, R)       sum of each weight row (1 up to rounding)
      lse    (B, H, R)       natural log of sum_j exp(scale * q_i . k_j) over
                             the unmasked keys
    The weighted sum of values: "How Transformers Work", "Scaled dot-product
    attention", step 4.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, n_q, d_k = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    R = n_q if rows is None else len(rows)
    o = np.empty((B, H, R, v.shape[-1]), dtype=np.float64)
    rowsum = np.empty((B, H, R), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    pos = np.arange(n_q) if rows is None else np.asarray(rows)
    for b in range(B):
        for h in range(H):
            s = np.matmul(q[b, h][pos], k[b, h].T) * scale
            if causal:
                if n_q != k.shape[2]:
                    raise ValueError("the causal mask is defined for N_q == N_k only")
                s = s + causal_mask_rows(k.shape[2], pos)
            if kv_len is not None:
                length = min(max(int(kv_len[b]), 0), k.shape[2])
                s = s + key_padding_mask_row(k.shape[2], length)[None, :]
            dead = np.all(s == -np.inf, axis=-1)       # rows with no unmasked key
            s = np.where(dead[:, None], 0.0, s)         # placeholder, overwritten below
            m = np.max(s, axis=-1, keepdims=True)
            e = np.exp(s - m)
            l = np.sum(e, axis=-1, keepdims=True)
            p = e / l
            p[dead] = 0.0
            o[b, h] = np.matmul(p, v[b, h])
            rowsum[b, h] = np.sum(p, axis=-1)
            lse[b, h] = np.where(dead, -np.inf, (m + np.log(l))[:, 0])
    return o, rowsum, lse


def attention_backward_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray, *, causal: bool = False,
                           scale: float | None = None, kv_len=None, error_scale: bool = False):
    """Gradients of the attention output with respect to Q, K and V.

    The pages motivate the 1/sqrt(d_k) scale by the gradient that flows back
    through the softmax: a saturated (nearly one-hot) row passes almost none
    ("32 Transformer" (ml-canon-en.vercel.app), "Why we divide by sqrt(dk)";
    "How Transformers Work" (worksonmygpu.com), "Scaled dot-product
    attention", step 2; "The Transformer" (hoshank.vercel.app), "The
    Breakthrough"). This is that backward pass, the chain rule written out for
    a loss whose gradient with respect to O is `do`:

      O = P V                    ->  dV = P^T dO,    dP = dO V^T
      P_i = softmax(S_i), each row ->  dS_i = J_i dP_i with the softmax Jacobian
                                     J_i = diag(P_i) - P_i P_i^T, that is
                                     dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
      S = scale Q K^T (+ masks)  ->  dQ = scale dS K,  dK = scale dS^T Q

    Masked scores are constants (-inf), so no gradient reaches them: their
    weights are 0 and so is dS there. A row with no visible key has P = 0 and
    passes nothing. q, k, do: as in attention_ref; returns (dQ, dK, dV) of the
    shapes of q, k and v, in float64.

    error_scale: also return (E_dQ, E_dK, E_dV), the sums of the absolute
    values of the terms each gradient element adds up -- the scale that
    rounding errors in those terms are proportional to (for tests):
      E_dV = P^T |dO|,  g_ij = |dS_ij| + P_ij sum_d |dO_id O_id|,
      E_dQ = |scale| g |K|,  E_dK = |scale| g^T |Q|.
    The second part of g covers delta, whose terms are dO_id O_id.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, n_q, d_k = q.shape
    n_k = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    if causal and n_q != n_k:
        raise ValueError("the causal mask is defined for N_q == N_k only")
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    eq, ek, ev = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            s = np.matmul(q[b, h], k[b, h].T) * scale
            if causal:
                s = s + causal_mask(n_q)
            if kv_len is not None:
                s = s + key_padding_mask_row(n_k, min(max(int(kv_len[b]), 0), n_k))[None, :]
            dead = np.all(s == -np.inf, axis=-1)
            s = np.where(dead[:, None], 0.0, s)
            e = np.exp(s - np.max(s, axis=-1, keepdims=True))
            p = e / np.sum(e, axis=-1, keepdims=True)
            p[dead] = 0.0
            dp = np.matmul(do[b, h], v[b, h].T)
            ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
            dv[b, h] = np.matmul(p.T, do[b, h])
            dq[b, h] = scale * np.matmul(ds, k[b, h])
            dk[b, h] = scale * np.matmul(ds.T, q[b, h])
            if error_scale:
                o = np.matmul(p, v[b, h])
                g = np.abs(ds) + p * np.sum(np.abs(do[b, h] * o), axis=-1, keepdims=True)
                ev[b, h] = np.matmul(p.T, np.abs(do[b, h]))
                eq[b, h] = abs(scale) * np.matmul(g, np.abs(k[b, h]))
                ek[b, h] = abs(scale) * np.matmul(g.T, np.abs(q[b, h]))
    if error_scale:
        return dq, dk, dv, (eq, ek, ev)
    return dq, dk, dv


def attention_backward_sampled_ref(q, k, v, do, rows, keys, *, causal: bool = False, scale: float | None = None,
                                   kv_len=None, chunk: int = 512, error_scale: bool = False):
    """attention_backward_ref restricted to query rows `rows` (dQ) and key rows
    `keys` (dK, dV), for sizes where the full score matrix is too large.

    The softmax statistics come from the forward oracle, chunk by chunk of
    query rows: lse_i, and delta_i = dO_i . O_i (equal to sum_j P_ij dP_ij,
    since O_i = sum_j P_ij V_j). Then dQ_i = scale sum_j dS_ij K_j over a
    sampled row, and dV_j = sum_i P_ij dO_i, dK_j = scale sum_i dS_ij Q_i over
    a sampled key column, with P_ij = exp(scale q_i.k_j - lse_i) and
    dS_ij = P_ij (dO_i . V_j - delta_i). Returns (dQ (B,H,R,d), dK (B,H,C,d),
    dV (B,H,C,d)) for the R rows and C keys, and with error_scale the term
    magnitudes of attention_backward_ref for them."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows, keys = np.asarray(rows), np.asarray(keys)
    lse = np.empty((B, H, n_q))
    delta = np.empty((B, H, n_q))
    dabs = np.empty((B, H, n_q))
    for c0 in range(0, n_q, chunk):
        r = np.arange(c0, min(c0 + chunk, n_q))
        o, _, l = attention_ref(q, k, v, causal=causal, scale=scale, rows=r, kv_len=kv_len)
        lse[:, :, r] = l
        delta[:, :, r] = np.sum(do[:, :, r] * o, axis=-1)
        dabs[:, :, r] = np.sum(np.abs(do[:, :, r] * o), axis=-1)
    dq = np.zeros((B, H, len(rows), d))
    dk = np.zeros((B, H, len(keys), d))
    dv = np.zeros((B, H, len(keys), v.shape[-1]))
    eq, ek, ev = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for b in range(B):
        length = n_k if kv_len is None else min(max(int(kv_len[b]), 0), n_k)
        for h in range(H):
            # sampled rows: every key
            s = np.matmul(q[b, h][rows], k[b, h].T) * scale
            vis = np.arange(n_k)[None, :] < length
            if causal:
                vis = vis & (np.arange(n_k)[None, :] <= rows[:, None])
            p = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse[b, h][rows][:, None]), 0.0)
            ds = p * (np.matmul(do[b, h][rows], v[b, h].T) - delta[b, h][rows][:, None])
            dq[b, h] = scale * np.matmul(ds, k[b, h])
            if error_scale:
                g = np.abs(ds) + p * dabs[b, h][rows][:, None]
                eq[b, h] = abs(scale) * np.matmul(g, np.abs(k[b, h]))
            # sampled keys: every query
            s = np.matmul(q[b, h], k[b, h][keys].T) * scale
            vis = np.broadcast_to(keys[None, :] < length, s.shape)
            if causal:
                vis = vis & (keys[None, :] <= np.arange(n_q)[:, None])
            p = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse[b, h][:, None]), 0.0)
            ds = p * (np.matmul(do[b, h], v[b, h][keys].T) - delta[b, h][:, None])
            dv[b, h] = np.matmul(p.T, do[b, h])
            dk[b, h] = scale * np.matmul(ds.T, q[b, h])
            if error_scale:
                g = np.abs(ds) + p * dabs[b, h][:, None]
                ev[b, h] = np.matmul(p.T, np.abs(do[b, h]))
                ek[b, h] = abs(scale) * np.matmul(g.T, np.abs(q[b, h]))
    if error_scale:
        return dq, dk, dv, (eq, ek, ev)
    return dq, dk, dv


def causal_mask_rows(n: int, rows) -> np.ndarray:
    """The rows `rows` of causal_mask(n), formed without the full n x n matrix."""
    rows = np.asarray(rows)
    j = np.arange(n)[None, :]
    out = np.zeros((len(rows), n), dtype=np.float64)
    out[j > rows[:, None]] = -np.inf
    return out


def mha_ref(xq: np.ndarray, xk: np.ndarray, xv: np.ndarray, wq: np.ndarray, wk: np.ndarray,
            wv: np.ndarray, wo: np.ndarray, heads: int, *, causal: bool = False,
            rows=None, kv_len=None, bq=None, bk=None, bv=None, bo=None) -> np.ndarray:
    """MultiHead(Xq, Xk, Xv) = Concat(head_1, ..., head_h) W^O with
    head_i = Attention(Xq W_i^Q, Xk W_i^K, Xv W_i^V).

    "The Transformer" (hoshank.vercel.app), "The Mathematics": the MultiHead
    equation and its symbol table (W_i^Q, W_i^K, W_i^V are d_model x d_k,
    W^O is h d_v x d_model, d_k = d_v = d_model / h). Written out head by
    head: W_i^Q is column block i of the stored (d_model, d_model) matrix
    (head i owns columns [i d_k, (i + 1) d_k)), each head runs Attention on
    its own projections, Concat lays head_1 .. head_h side by side in that
    order, and the result is multiplied by W^O.

    xq: (B, N_q, d_model); xk, xv: (B, N_k, d_model); w*: (d_model, d_model)
    stored (in, out). Scale is 1/sqrt(d_model / heads). Self-attention passes
    the same x three times; cross-attention passes the decoder state as xq and
    the encoder memory as xk and xv ("The Transformer" (rayaq.ca), "The decoder
    stack").
    rows: optional query positions; only those output rows are returned.
    kv_len: optional per-batch number of valid key/value positions of the
    xk/xv sequence (a key-padding mask, as in attention_ref).
    bq, bk, bv, bo: optional biases (d_model,) added after each projection, as
    in the encoder layer's attention module ("The Transformer" (rayaq.ca), "In
    PyTorch": nn.MultiheadAttention, whose parameters the printed count
    includes). The MultiHead equation itself has none.
    """
    xq = np.asarray(xq, dtype=np.float64)
    xk = np.asarray(xk, dtype=np.float64)
    xv = np.asarray(xv, dtype=np.float64)
    d_model = xq.shape[-1]
    if d_model % heads:
        raise ValueError("d_model must be divisible by the number of heads")
    d = d_model // heads

    def proj(x, w, b, cols=slice(None)):
        y = np.matmul(x, np.asarray(w, dtype=np.float64)[:, cols])
        return y if b is None else y + np.asarray(b, dtype=np.float64)[cols]

    head_outputs = []
    for i in range(heads):
        cols = slice(i * d, (i + 1) * d)
        qi, ki, vi = proj(xq, wq, bq, cols), proj(xk, wk, bk, cols), proj(xv, wv, bv, cols)
        # one head: attention_ref takes (B, H, N, d), here with H = 1
        oi, _, _ = attention_ref(qi[:, None], ki[:, None], vi[:, None], causal=causal,
                                 scale=1.0 / math.sqrt(d), rows=rows, kv_len=kv_len)
        head_outputs.append(oi[:, 0])
    concat = np.concatenate(head_outputs, axis=-1)  # head_1 in columns [0, d), then head_2, ...
    return proj(concat, wo, bo)


def layer_norm_ref(x: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    """LayerNorm over the last axis: each position's d_model numbers are
    shifted to mean 0 and scaled to variance 1 (the population variance, the
    mean of squared deviations), then scaled by gamma and shifted by beta
    ("The Transformer" (rayaq.ca), "Residuals and LayerNorm"). eps is added to
    the variance under the square root; the pages print no value (reading in
    the design notes: 1e-5, the default of the nn.LayerNorm their code uses)."""
    x = np.asarray(x, dtype=np.float64)
    mean = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mean) ** 2, axis=-1, keepdims=True)
    return (x - mean) / np.sqrt(var + eps) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def ffn_ref(x: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray, b2: np.ndarray) -> np.ndarray:
    """Position-wise feed-forward network FFN(x) = max(0, x W1 + b1) W2 + b2,
    widening d_model -> d_ff and back ("The Transformer" (hoshank.vercel.app),
    "The Mathematics", the FFN equation and its symbol table). Weights (in, out)."""
    x = np.asarray(x, dtype=np.float64)
    h = np.maximum(0.0, np.matmul(x, np.asarray(w1, np.float64)) + np.asarray(b1, np.float64))
    return np.matmul(h, np.asarray(w2, np.float64)) + np.asarray(b2, np.float64)


def encoder_layer_ref(x: np.ndarray, p: dict, heads: int, *, eps: float = 1e-5, causal: bool = False,
                      kv_len=None) -> np.ndarray:
    """One encoder layer, post-norm: h = LayerNorm(x + MHA(x)), then
    out = LayerNorm(h + FFN(h)) ("The Transformer" (hoshank.vercel.app), "The
    Mathematics": output = LayerNorm(x + Sublayer(x)) around both sub-layers;
    "The Transformer" (rayaq.ca), "In PyTorch", the EncoderLayer forward, in
    eval mode, so without dropout).

    p holds wq, wk, wv, wo, bq, bk, bv, bo (attention), ln1_g, ln1_b, w1, b1,
    w2, b2, ln2_g, ln2_b, all (in, out). kv_len: optional key-padding lengths
    for the self-attention, as in attention_ref.
    """
    x = np.asarray(x, dtype=np.float64)
    a = mha_ref(x, x, x, p["wq"], p["wk"], p["wv"], p["wo"], heads, causal=causal, kv_len=kv_len,
                bq=p["bq"], bk=p["bk"], bv=p["bv"], bo=p["bo"])
    h = layer_norm_ref(x + a, p["ln1_g"], p["ln1_b"], eps)
    f = ffn_ref(h, p["w1"], p["b1"], p["w2"], p["b2"])
    return layer_norm_ref(h + f, p["ln2_g"], p["ln2_b"], eps)


def gather_pages(pool: np.ndarray, block_table, page_size: int, length: int) -> np.ndarray:
    """Keys (or values) 0..length-1 of one sequence stored in fixed-size pages:
    logical position j sits in page block_table[j // page_size] at row
    j % page_size. pool: (num_pages, page_size, H, d) -> (H, length, d)."""
    pool = np.asarray(pool, dtype=np.float64)
    rows = [pool[int(block_table[j // page_size]), j % page_size] for j in range(length)]
    if not rows:
        return np.zeros((pool.shape[2], 0, pool.shape[3]))
    return np.stack(rows, axis=1)


def decode_ref(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, kv_len, *, scale: float | None = None):
    """One decoding step: each (batch, head) query attends to the first
    kv_len[b] cached keys and values -- the newest row of causal attention,
    where position i sees keys j <= i: decoder-only models generate left to
    right ("How Transformers Work" (worksonmygpu.com), "What changed since
    2017"), the decoder's masked self-attention covers the tokens generated so
    far ("The Transformer" (hoshank.vercel.app), "The Breakthrough"), and the
    causal mask is "The Transformer" (rayaq.ca), "Masks: who may look at
    whom". q: (B, H, d); k_cache, v_cache: (B, H, N_max, d). Returns (O (B, H, d), lse (B, H)); a length of 0 gives O = 0, lse = -inf."""
    q = np.asarray(q, dtype=np.float64)
    o, _, lse = attention_ref(q[:, :, None, :], k_cache, v_cache, scale=scale, kv_len=kv_len)
    return o[:, :, 0, :], lse[:, :, 0]


def linear_ref(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """One projection Y = X W (no bias), the per-head projection of the
    MultiHead equation ("The Transformer" (hoshank.vercel.app), "The
    Mathematics"), in float64."""
    return np.matmul(np.asarray(x, dtype=np.float64), np.asarray(w, dtype=np.float64))
