"""Pins for the fp64 oracle: properties and values the pages and mathematics fix.

Each check takes the attention function under test (signature of
oracle.attention_ref) and, where needed, the multi-head function (signature of
oracle.mha_ref), and raises AssertionError when the property fails. The
pin tests run them on the oracle; the mutant tests run them on deliberately
broken copies of the oracle to show that each plausible mistake is caught.

Pages cited: "32 Transformer" (ml-canon-en.vercel.app); "How Transformers Work"
(worksonmygpu.com); "The Transformer" (hoshank.vercel.app); "Transformer: The
Starting Point of Everything" (chenyuan1125.github.io); "The Transformer"
(rayaq.ca).
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _qkv(seed, B=2, H=3, nq=7, nk=7, d=5, dv=None):
    r = _rng(seed)
    dv = d if dv is None else dv
    return (r.standard_normal((B, H, nq, d)), r.standard_normal((B, H, nk, d)),
            r.standard_normal((B, H, nk, dv)))


def read_golden_matrix(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([float(t) for t in line.split()])
    return np.array(rows)


def read_golden_table(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split()
            out[key] = int(val)
    return out


# ------------------------------------------------------------------ P1 rows sum to 1
def check_rows_sum_to_one(attn):
    """Softmax rows are probability distributions ("The Transformer"
    (hoshank.vercel.app), "The Mathematics", softmax row of the symbol table).
    Checked with V = identity so that O *is* the weight matrix, independently
    of the rowsum the function reports."""
    for causal in (False, True):
        q, k, _ = _qkv(11)
        n = k.shape[2]
        eye = np.broadcast_to(np.eye(n), (q.shape[0], q.shape[1], n, n)).copy()
        p, rowsum, _ = attn(q, k, eye, causal=causal)
        assert np.all(p >= 0), "negative attention weight"
        assert np.allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12), "weight rows do not sum to 1"
        assert np.allclose(rowsum, 1.0, rtol=0, atol=1e-12), "reported row sums differ from 1"


# ------------------------------------------------------------------ P2 permutation equivariance
def check_permutation_equivariance(attn):
    """Swapping tokens swaps the outputs and changes nothing else ("The
    Transformer" (rayaq.ca), "Embeddings and positions"); permuting keys and
    values together leaves every output unchanged ("32 Transformer",
    "Positional encodings": attention alone knows no order)."""
    q, k, v = _qkv(12, nq=9, nk=9)
    perm = _rng(13).permutation(9)
    o, _, _ = attn(q, k, v)
    o_p, _, _ = attn(q[:, :, perm], k[:, :, perm], v[:, :, perm])
    assert np.allclose(o_p, o[:, :, perm], rtol=0, atol=1e-12), "not permutation-equivariant"
    o_kv, _, _ = attn(q, k[:, :, perm], v[:, :, perm])
    assert np.allclose(o_kv, o, rtol=0, atol=1e-12), "key/value order changed the output"


# ------------------------------------------------------------------ P3 convex combination
def check_constant_v_and_convex_hull(attn):
    """Weights are >= 0 and sum to 1, so O is a convex combination of V's rows:
    constant V gives constant O, and every O lies between min and max of V."""
    q, k, v = _qkv(14, nq=8, nk=8)
    c = _rng(15).standard_normal(v.shape[-1])
    vc = np.broadcast_to(c, v.shape).copy()
    for causal in (False, True):
        o, _, _ = attn(q, k, vc, causal=causal)
        assert np.allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-12), "constant V not kept"
    o, _, _ = attn(q, k, v)
    lo = v.min(axis=2, keepdims=True)
    hi = v.max(axis=2, keepdims=True)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12), "output outside the hull of V"


# ------------------------------------------------------------------ P4 causal locality
def check_causal_locality(attn):
    """With the causal mask, output row i depends only on rows <= i ("How
    Transformers Work", "What changed since 2017"; "The Transformer"
    (hoshank.vercel.app), "The Breakthrough": the mask removes future
    positions). Perturbing rows > i of Q, K and V must leave rows <= i
    bitwise unchanged."""
    q, k, v = _qkv(16, nq=10, nk=10)
    o, _, _ = attn(q, k, v, causal=True)
    for i in (0, 3, 8):
        r = _rng(17 + i)
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[:, :, i + 1:] += r.standard_normal(q2[:, :, i + 1:].shape)
        k2[:, :, i + 1:] += r.standard_normal(k2[:, :, i + 1:].shape)
        v2[:, :, i + 1:] += r.standard_normal(v2[:, :, i + 1:].shape)
        o2, _, _ = attn(q2, k2, v2, causal=True)
        assert np.array_equal(o2[:, :, :i + 1], o[:, :, :i + 1]), f"row <= {i} saw the future"
    # and the mask does matter: without it, row 0 changes when later keys change
    o_full, _, _ = attn(q, k, v, causal=False)
    assert not np.allclose(o_full[:, :, 0], o[:, :, 0]), "causal flag had no effect"


# ------------------------------------------------------------------ P5 the printed mask
def check_printed_mask(mask_fn):
    """The mask for n = 4 equals the tensor printed on "The Transformer"
    (rayaq.ca), "Masks: who may look at whom"."""
    want = read_golden_matrix("causal_mask_n4.txt")
    got = mask_fn(4)
    assert got.shape == want.shape
    assert np.array_equal(np.isinf(got), np.isinf(want)), "mask pattern differs from the page"
    assert np.all(got[np.isfinite(want)] == 0)
    assert np.all(got[np.isinf(want)] < 0)


def check_masked_weight_is_zero(attn):
    """A blocked key gets a weight of exactly 0 ("The Transformer" (rayaq.ca),
    "Masks"): with V = identity the strict upper triangle of O is 0."""
    q, k, _ = _qkv(18, nq=6, nk=6)
    eye = np.broadcast_to(np.eye(6), (2, 3, 6, 6)).copy()
    p, _, _ = attn(q, k, eye, causal=True)
    iu = np.triu_indices(6, 1)
    assert np.all(p[:, :, iu[0], iu[1]] == 0.0), "masked weight not exactly zero"
    assert np.all(p[:, :, np.arange(6), np.arange(6)] > 0), "diagonal must stay visible"


# ------------------------------------------------------------------ P6 closed forms
def check_closed_forms(attn):
    q, k, v = _qkv(19, nq=5, nk=5)
    # one key: the only weight is 1, O = V
    o, _, _ = attn(q, k[:, :, :1], v[:, :, :1])
    assert np.allclose(o, np.broadcast_to(v[:, :, :1], o.shape), rtol=0, atol=1e-14), "N_k = 1"
    # zero queries: uniform weights, O = mean of V (unmasked), prefix mean (causal)
    z = np.zeros_like(q)
    o, _, _ = attn(z, k, v)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-14)
    o, _, _ = attn(z, k, v, causal=True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, 6)[None, None, :, None]
    assert np.allclose(o, prefix, rtol=0, atol=1e-14), "causal prefix mean"
    # scale 0 gives uniform weights too
    o, _, _ = attn(q, k, v, scale=0.0)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-14)
    # causal row 0 sees only key 0
    o, _, _ = attn(q, k, v, causal=True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0]), "causal row 0 must equal V_0"
    # all keys equal: uniform weights
    ke = np.broadcast_to(k[:, :, :1], k.shape).copy()
    o, _, _ = attn(q, ke, v)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape), atol=1e-14)
    # two keys: weight of key 1 is the logistic function of the scaled score gap
    q1, k2, v2 = q[:, :, :3], k[:, :, :2], np.zeros((2, 3, 2, 1))
    v2[:, :, 0, 0] = 1.0
    o, _, _ = attn(q1, k2, v2)
    s = np.einsum("bhid,bhjd->bhij", q1, k2) / math.sqrt(q.shape[-1])
    want = 1.0 / (1.0 + np.exp(-(s[..., 0] - s[..., 1])))
    assert np.allclose(o[..., 0], want, rtol=0, atol=1e-14), "two-key logistic form"


# ------------------------------------------------------------------ P7 temperature
def check_low_temperature_argmax(attn):
    """A large scale (low temperature) collapses each row onto its single best
    key ("The Transformer" (rayaq.ca), "Worked example")."""
    q, k, v = _qkv(20, nq=6, nk=12)
    s = np.einsum("bhid,bhjd->bhij", q, k)
    srt = np.sort(s, axis=-1)
    gap = srt[..., -1] - srt[..., -2]
    assert gap.min() > 1e-3  # inputs chosen without near ties
    o, _, _ = attn(q, k, v, scale=1e5)
    best = np.argmax(s, axis=-1)
    want = np.take_along_axis(v, best[..., None], axis=2)
    assert np.allclose(o, want, rtol=0, atol=1e-12), "low temperature must pick the best key"


# ------------------------------------------------------------------ P8 the scale divides by sqrt(d_k)
def check_default_scale(attn):
    """The default scale divides the scores by sqrt(d_k) ("32 Transformer",
    "Why we divide by sqrt(dk)"; "The Transformer" (hoshank.vercel.app), "The
    Mathematics"). With two keys, log(w1/w2) recovers the scaled score gap; for
    unit-normal q, k in d_k = 64 that gap has variance 2 (two unit-variance
    scaled scores), not 2 * 64."""
    d = 64
    r = _rng(21)
    q = r.standard_normal((1, 1, 4096, d))
    k = r.standard_normal((1, 1, 2, d))
    v = np.zeros((1, 1, 2, 1))
    v[..., 0, 0] = 1.0
    o, _, _ = attn(q, k, v)
    w1 = o[0, 0, :, 0]
    gap = np.log(w1) - np.log1p(-w1)
    want = (q[0, 0] @ (k[0, 0, 0] - k[0, 0, 1])) / math.sqrt(d)
    assert np.allclose(gap, want, rtol=1e-9, atol=1e-9), "score gap is not q.(k1-k2)/sqrt(d)"
    # the page's variance argument: with unit-normal queries the scaled gap has
    # variance |k1 - k2|^2 / d_k (about 2 here), i.e. unit variance per scaled score
    ratio = gap.var() / (np.sum((k[0, 0, 0] - k[0, 0, 1]) ** 2) / d)
    assert 0.9 < ratio < 1.1, "scaled scores do not have unit variance"


# ------------------------------------------------------------------ P10 brute force and a hand example
def _brute_attention(q, k, v, causal, scale):
    """Pure-Python loops with math.exp, one query at a time."""
    nq, nk, d, dv = len(q), len(k), len(q[0]), len(v[0])
    out = []
    for i in range(nq):
        scores = []
        for j in range(nk):
            if causal and j > i:
                scores.append(None)
                continue
            scores.append(scale * sum(q[i][t] * k[j][t] for t in range(d)))
        finite = [s for s in scores if s is not None]
        m = max(finite)
        w = [0.0 if s is None else math.exp(s - m) for s in scores]
        tot = sum(w)
        out.append([sum(w[j] / tot * v[j][c] for j in range(nk)) for c in range(dv)])
    return out


def check_brute_force(attn):
    r = _rng(22)
    for trial in range(12):
        n = int(r.integers(1, 5))
        nk = n if trial % 2 else int(r.integers(1, 5))
        d = int(r.integers(1, 4))
        causal = bool(trial % 2)
        q = r.integers(-3, 4, size=(n, d)).astype(float)
        k = r.integers(-3, 4, size=(nk, d)).astype(float)
        v = r.integers(-3, 4, size=(nk, 2)).astype(float)
        want = _brute_attention(q.tolist(), k.tolist(), v.tolist(), causal, 1 / math.sqrt(d))
        got, _, _ = attn(q[None, None], k[None, None], v[None, None], causal=causal)
        assert np.allclose(got[0, 0], np.array(want), rtol=0, atol=1e-12), f"brute force trial {trial}"


def check_hand_example(attn):
    """q = (1, 0); k1 = (1, 0); k2 = (0, 1); d = 2. Scores 1/sqrt(2) and 0, so the
    weights are sigma(1/sqrt(2)) and 1 - sigma(1/sqrt(2)), worked by hand."""
    q = np.array([[[[1.0, 0.0]]]])
    k = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    v = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    o, _, lse = attn(q, k, v)
    w1 = 1.0 / (1.0 + math.exp(-1.0 / math.sqrt(2.0)))
    assert abs(o[0, 0, 0, 0] - w1) < 1e-15 and abs(o[0, 0, 0, 1] - (1 - w1)) < 1e-15
    assert abs(lse[0, 0, 0] - math.log(math.exp(1 / math.sqrt(2)) + 1.0)) < 1e-15


# ------------------------------------------------------------------ P11 linearity and shift invariance
def check_linearity_and_shift(attn):
    q, k, v = _qkv(23)
    v2 = _qkv(24)[2]
    a, b = 1.7, -0.4
    o1, _, _ = attn(q, k, v)
    o2, _, _ = attn(q, k, v2)
    o12, _, _ = attn(q, k, a * v + b * v2)
    assert np.allclose(o12, a * o1 + b * o2, rtol=0, atol=1e-12), "not linear in V"
    c = _rng(25).standard_normal(k.shape[-1])
    for causal in (False, True):
        o, _, _ = attn(q, k, v, causal=causal)
        os_, _, _ = attn(q, k + c, v, causal=causal)
        assert np.allclose(os_, o, rtol=0, atol=1e-12), "shifting every key changed O"


# ------------------------------------------------------------------ P12 multi-head structure
def check_mha_structure(mha, attn):
    r = _rng(26)
    B, N, dm = 2, 5, 6
    x = r.standard_normal((B, N, dm))
    # h = 1 with identity weights is plain attention on x
    eye = np.eye(dm)
    o = mha(x, x, x, eye, eye, eye, eye, 1)
    want, _, _ = attn(x[:, None], x[:, None], x[:, None])
    assert np.allclose(o, want[:, 0], rtol=0, atol=1e-12), "h=1, W=I is not attention(x,x,x)"
    # block decomposition: out = sum_i head_i @ W^O[i*d:(i+1)*d]
    h, d = 3, 2
    wq, wk, wv, wo = (r.standard_normal((dm, dm)) for _ in range(4))
    # cross-attention with N_k != N_q, and with three distinct inputs of equal length
    for xk, xv in ((r.standard_normal((B, 4, dm)),) * 2,
                   (r.standard_normal((B, N, dm)), r.standard_normal((B, N, dm)))):
        out = mha(x, xk, xv, wq, wk, wv, wo, h)
        acc = np.zeros_like(out)
        for i in range(h):
            cols = slice(i * d, (i + 1) * d)
            head, _, _ = attn((x @ wq[:, cols])[:, None], (xk @ wk[:, cols])[:, None],
                              (xv @ wv[:, cols])[:, None])
            acc += head[:, 0] @ wo[cols, :]
        assert np.allclose(out, acc, rtol=0, atol=1e-12), "head split/concat order, W orientation or inputs"


# ------------------------------------------------------------------ P9 an independent library routine
def check_torch_sdpa(attn, mha):
    """torch's CPU float64 scaled_dot_product_attention and nn.MultiheadAttention
    compute the same definition ("The Transformer" (rayaq.ca), "Attention, by
    hand" and "In PyTorch"). Used as a cross-check only."""
    import torch
    import torch.nn.functional as F
    q, k, v = _qkv(27, nq=6, nk=9, d=4, dv=3)
    o, _, _ = attn(q, k, v)
    t = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v))
    assert np.allclose(o, t.numpy(), rtol=0, atol=1e-12), "differs from torch sdpa"
    q, k, v = _qkv(28, nq=7, nk=7, d=4)
    o, _, _ = attn(q, k, v, causal=True)
    t = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                       is_causal=True)
    assert np.allclose(o, t.numpy(), rtol=0, atol=1e-12), "differs from torch causal sdpa"
    r = _rng(29)
    B, N, M, dm, h = 2, 5, 7, 8, 2
    xq, xkv = r.standard_normal((B, N, dm)), r.standard_normal((B, M, dm))
    wq, wk, wv, wo = (r.standard_normal((dm, dm)) for _ in range(4))
    m = torch.nn.MultiheadAttention(dm, h, bias=False, batch_first=True).double()
    with torch.no_grad():
        m.in_proj_weight.copy_(torch.from_numpy(np.concatenate([wq.T, wk.T, wv.T])))
        m.out_proj.weight.copy_(torch.from_numpy(wo.T))
    m.eval()
    with torch.no_grad():
        t, _ = m(torch.from_numpy(xq), torch.from_numpy(xkv), torch.from_numpy(xkv), need_weights=False)
    got = mha(xq, xkv, xkv, wq, wk, wv, wo, h)
    assert np.allclose(got, t.numpy(), rtol=0, atol=1e-12), "differs from nn.MultiheadAttention"


# ------------------------------------------------------------------ P13 projection shapes
def check_parameter_counts(mha):
    """A bias-free MHA at the base width holds 4 * d_model^2 weights; adding the
    biases, the FFN and the two LayerNorms of one encoder layer gives the
    count printed on "The Transformer" (rayaq.ca), "In PyTorch"."""
    sizes = read_golden_table("model_sizes.txt")
    dm, h, ff = sizes["base_d_model"], sizes["base_heads"], sizes["ffn_inner"]
    assert dm // h == sizes["base_d_k"] == sizes["base_d_v"]
    assert sizes["big_d_model"] // sizes["big_heads"] == sizes["base_d_k"]
    # the oracle's multi-head function takes four (d_model, d_model) matrices
    r = _rng(30)
    x = r.standard_normal((1, 3, dm))
    ws = [r.standard_normal((dm, dm)) / math.sqrt(dm) for _ in range(4)]
    assert mha(x, x, x, *ws, h).shape == (1, 3, dm)
    mha_weights = sum(w.size for w in ws)
    assert mha_weights == 4 * dm * dm == 1_048_576
    with_bias = mha_weights + 4 * dm
    ffn = dm * ff + ff + ff * dm + dm
    norms = 2 * 2 * dm
    assert with_bias + ffn + norms == sizes["encoder_layer_params"]


# ------------------------------------------------------------------ sampled rows agree with full rows
def check_rows_subset(attn, mha):
    q, k, v = _qkv(31, nq=12, nk=12)
    rows = np.array([0, 5, 11])
    for causal in (False, True):
        full, rs, lse = attn(q, k, v, causal=causal)
        part, rs2, lse2 = attn(q, k, v, causal=causal, rows=rows)
        assert np.allclose(part, full[:, :, rows], rtol=0, atol=1e-14)
        assert np.allclose(lse2, lse[:, :, rows], rtol=0, atol=1e-14)
    r = _rng(32)
    x = r.standard_normal((2, 12, 6))
    ws = [r.standard_normal((6, 6)) for _ in range(4)]
    for causal in (False, True):
        full = mha(x, x, x, *ws, 3, causal=causal)
        part = mha(x, x, x, *ws, 3, causal=causal, rows=rows)
        assert np.allclose(part, full[:, rows], rtol=0, atol=1e-12)


def check_lse(attn):
    """lse_i = log sum_j exp(scale * q_i . k_j) over the unmasked keys."""
    q, k, v = _qkv(33, nq=5, nk=5, d=3)
    for causal in (False, True):
        _, _, lse = attn(q, k, v, causal=causal)
        s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(3)
        if causal:
            s = np.where(np.triu(np.ones((5, 5), bool), 1), -np.inf, s)
        want = np.log(np.sum(np.exp(s), axis=-1))
        assert np.allclose(lse, want, rtol=0, atol=1e-13), "lse"


# ------------------------------------------------------------------ key-padding masks (per-batch key lengths)
def check_key_padding(attn):
    """A key-padding mask blocks, for every query of a batch item, the keys at
    or past that item's length ("The Transformer" (rayaq.ca), "Masks: who may
    look at whom": padding masks work like the causal one, one row per batch
    item). Pinned by an independent route: the same item computed on keys
    truncated to its length, unmasked."""
    q, k, v = _qkv(41, B=4, H=2, nq=6, nk=9, d=4, dv=3)
    lens = [9, 4, 1, 12]  # full, partial, one key, longer than N_k (clamped)
    o, rs, lse = attn(q, k, v, kv_len=lens)
    for b, L in enumerate(lens):
        L = min(L, 9)
        want, wrs, wlse = attn(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L])
        assert np.allclose(o[b], want[0], rtol=0, atol=1e-14), f"padding of item {b} (length {L})"
        assert np.allclose(lse[b], wlse[0], rtol=0, atol=1e-14), "lse under padding"
        assert np.allclose(rs[b], 1.0, rtol=0, atol=1e-12)
    # the padded keys and values are never read: changing them changes nothing, bitwise
    k2, v2 = k.copy(), v.copy()
    k2[1, :, 4:] = 1e3
    v2[1, :, 4:] = -7.0
    o2, _, _ = attn(q, k2, v2, kv_len=lens)
    assert np.array_equal(o2, o), "a padded key or value leaked into the output"
    # causal and padding together: row i sees keys j <= min(i, L - 1)
    q, k, v = _qkv(42, B=2, H=1, nq=7, nk=7, d=3)
    o, _, _ = attn(q, k, v, causal=True, kv_len=[7, 3])
    full, _, _ = attn(q[1:], k[1:], v[1:], causal=True)
    assert np.allclose(o[1, :, :3], full[0, :, :3], rtol=0, atol=1e-14), "causal rows inside the length"
    trunc, _, _ = attn(q[1:, :, 3:], k[1:, :, :3], v[1:, :, :3])
    assert np.allclose(o[1, :, 3:], trunc[0], rtol=0, atol=1e-14), "causal rows past the length see every valid key"
    assert np.allclose(o[0], attn(q[:1], k[:1], v[:1], causal=True)[0][0], rtol=0, atol=1e-14)


def check_fully_masked_rows(attn):
    """A batch item with length 0 has no visible key. The pages define no
    softmax for such a row; the reading adopted here: output 0, row sum 0,
    log-sum-exp -inf (and the other items are unaffected)."""
    q, k, v = _qkv(43, B=3, H=2, nq=4, nk=5, d=3)
    for causal_ok in (False,):
        o, rs, lse = attn(q, k, v, kv_len=[5, 0, 2])
        assert np.array_equal(o[1], np.zeros_like(o[1])), "fully masked rows must give 0"
        assert np.all(rs[1] == 0.0) and np.all(np.isneginf(lse[1])), "row sum 0, lse -inf"
        assert np.all(np.isfinite(o)), "no NaN anywhere"
        ref, _, _ = attn(q[:1], k[:1], v[:1])
        assert np.allclose(o[0], ref[0], rtol=0, atol=1e-14)


def check_torch_padding(attn, mha):
    """torch's float64 scaled_dot_product_attention with a boolean attn_mask
    (True = may attend) and nn.MultiheadAttention with key_padding_mask
    (True = blocked): the two polarities the pages warn about ("Masks: who may
    look at whom"; "Pitfalls"). Cross-check only."""
    import torch
    import torch.nn.functional as F
    q, k, v = _qkv(44, B=3, H=2, nq=5, nk=8, d=4)
    lens = [8, 3, 1]
    o, _, _ = attn(q, k, v, kv_len=lens)
    allow = torch.arange(8)[None, :] < torch.tensor(lens)[:, None]       # True = may attend
    t = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                       attn_mask=allow[:, None, None, :])
    assert np.allclose(o, t.numpy(), rtol=0, atol=1e-12), "differs from torch sdpa with a key mask"
    r = _rng(45)
    B, N, M, dm, h = 3, 4, 6, 8, 2
    xq, xkv = r.standard_normal((B, N, dm)), r.standard_normal((B, M, dm))
    wq, wk, wv, wo = (r.standard_normal((dm, dm)) for _ in range(4))
    m = torch.nn.MultiheadAttention(dm, h, bias=False, batch_first=True).double()
    with torch.no_grad():
        m.in_proj_weight.copy_(torch.from_numpy(np.concatenate([wq.T, wk.T, wv.T])))
        m.out_proj.weight.copy_(torch.from_numpy(wo.T))
    m.eval()
    lens = [6, 2, 5]
    blocked = torch.arange(M)[None, :] >= torch.tensor(lens)[:, None]     # True = blocked
    with torch.no_grad():
        t, _ = m(torch.from_numpy(xq), torch.from_numpy(xkv), torch.from_numpy(xkv),
                 key_padding_mask=blocked, need_weights=False)
    got = mha(xq, xkv, xkv, wq, wk, wv, wo, h, kv_len=lens)
    assert np.allclose(got, t.numpy(), rtol=0, atol=1e-12), "differs from nn.MultiheadAttention with padding"


# ------------------------------------------------------------------ encoder sub-layer (LayerNorm, FFN, residuals)
def encoder_params(seed, d, ff, scale=1.0):
    """Random encoder-layer parameters in the oracle's (in, out) layout."""
    r = _rng(seed)
    p = {n: r.standard_normal((d, d)) / math.sqrt(d) * scale for n in ("wq", "wk", "wv", "wo")}
    p.update({n: r.standard_normal(d) * 0.1 for n in ("bq", "bk", "bv", "bo")})
    p["w1"] = r.standard_normal((d, ff)) / math.sqrt(d)
    p["b1"] = r.standard_normal(ff) * 0.1
    p["w2"] = r.standard_normal((ff, d)) / math.sqrt(ff)
    p["b2"] = r.standard_normal(d) * 0.1
    for n in ("ln1", "ln2"):
        p[n + "_g"] = 1.0 + 0.1 * r.standard_normal(d)
        p[n + "_b"] = 0.1 * r.standard_normal(d)
    return p


def check_layer_norm(ln):
    """Each position's numbers are shifted to mean 0 and scaled to variance 1
    (population variance), then scaled and shifted ("The Transformer"
    (rayaq.ca), "Residuals and LayerNorm")."""
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    eps = 1e-5
    want = (x - 2.5) / math.sqrt(1.25 + eps)         # mean 2.5, mean squared deviation 1.25
    assert np.allclose(ln(x, np.ones(4), np.zeros(4), eps), want, rtol=0, atol=1e-15), "hand example"
    r = _rng(50)
    x = r.standard_normal((3, 5, 64)) * 3.0 + 2.0
    y = ln(x, np.ones(64), np.zeros(64), 0.0)
    assert np.allclose(y.mean(-1), 0.0, atol=1e-13) and np.allclose((y ** 2).mean(-1), 1.0, atol=1e-12)
    g, b = r.standard_normal(64), r.standard_normal(64)
    assert np.allclose(ln(x, g, b, eps), ln(x, np.ones(64), np.zeros(64), eps) * g + b, rtol=0, atol=1e-12)
    # per-row shift and positive scale do not change it (eps = 0)
    assert np.allclose(ln(5.0 * x - 7.0, np.ones(64), np.zeros(64), 0.0), y, rtol=0, atol=1e-12)


def check_ffn(ffn):
    """FFN(x) = max(0, x W1 + b1) W2 + b2 ("The Transformer" (hoshank.vercel.app),
    "The Mathematics"), by hand on integers, one token at a time."""
    x = np.array([[1.0, -2.0], [0.0, 3.0]])
    w1 = np.array([[1.0, 0.0, -1.0], [2.0, 1.0, 0.0]])
    b1 = np.array([0.0, 1.0, 0.5])
    w2 = np.array([[1.0], [-1.0], [2.0]])
    b2 = np.array([0.25])
    want = []
    for t in x:  # position-wise: each token alone
        hid = [max(0.0, sum(t[i] * w1[i, j] for i in range(2)) + b1[j]) for j in range(3)]
        want.append([sum(hid[j] * w2[j, 0] for j in range(3)) + b2[0]])
    assert np.allclose(ffn(x, w1, b1, w2, b2), np.array(want), rtol=0, atol=1e-15), "FFN by hand"


def check_encoder_layer_torch(layer):
    """torch's float64 nn.TransformerEncoderLayer (post-norm, ReLU, eval mode,
    batch_first) with the same parameters computes the same layer ("The
    Transformer" (rayaq.ca), "In PyTorch" and "Residuals and LayerNorm").
    Cross-check only; also with a key-padding mask (True = blocked) and with
    the causal mask."""
    import torch
    d, h, ff = 16, 2, 32
    p = encoder_params(51, d, ff)
    m = torch.nn.TransformerEncoderLayer(d, h, dim_feedforward=ff, dropout=0.0, batch_first=True).double().eval()
    with torch.no_grad():
        m.self_attn.in_proj_weight.copy_(torch.from_numpy(np.concatenate([p["wq"].T, p["wk"].T, p["wv"].T])))
        m.self_attn.in_proj_bias.copy_(torch.from_numpy(np.concatenate([p["bq"], p["bk"], p["bv"]])))
        m.self_attn.out_proj.weight.copy_(torch.from_numpy(p["wo"].T))
        m.self_attn.out_proj.bias.copy_(torch.from_numpy(p["bo"]))
        m.linear1.weight.copy_(torch.from_numpy(p["w1"].T))
        m.linear1.bias.copy_(torch.from_numpy(p["b1"]))
        m.linear2.weight.copy_(torch.from_numpy(p["w2"].T))
        m.linear2.bias.copy_(torch.from_numpy(p["b2"]))
        m.norm1.weight.copy_(torch.from_numpy(p["ln1_g"]))
        m.norm1.bias.copy_(torch.from_numpy(p["ln1_b"]))
        m.norm2.weight.copy_(torch.from_numpy(p["ln2_g"]))
        m.norm2.bias.copy_(torch.from_numpy(p["ln2_b"]))
    assert m.norm1.eps == 1e-5
    x = _rng(52).standard_normal((3, 7, d))
    with torch.no_grad():
        t = m(torch.from_numpy(x)).numpy()
    assert np.allclose(layer(x, p, h), t, rtol=0, atol=1e-12), "differs from nn.TransformerEncoderLayer"
    lens = [7, 3, 5]
    blocked = torch.arange(7)[None, :] >= torch.tensor(lens)[:, None]
    with torch.no_grad():
        t = m(torch.from_numpy(x), src_key_padding_mask=blocked).numpy()
    assert np.allclose(layer(x, p, h, kv_len=lens), t, rtol=0, atol=1e-12), "padding mask"
    causal = torch.triu(torch.full((7, 7), float("-inf"), dtype=torch.float64), diagonal=1)
    with torch.no_grad():
        t = m(torch.from_numpy(x), src_mask=causal).numpy()
    assert np.allclose(layer(x, p, h, causal=True), t, rtol=0, atol=1e-12), "causal mask"


def check_encoder_layer_structure(layer, ln, ffn, mha):
    """The layer is the two wrapped sub-layers in order, post-norm: with the
    attention output projection zeroed (W^O = 0, b^O = 0) the first sub-layer is
    LayerNorm(x); with W2 = 0 and b2 = 0 the second is LayerNorm(h)."""
    d, h, ff = 8, 2, 16
    p = encoder_params(53, d, ff)
    x = _rng(54).standard_normal((2, 5, d))
    q = dict(p, wo=np.zeros((d, d)), bo=np.zeros(d), w2=np.zeros((ff, d)), b2=np.zeros(d))
    want = ln(ln(x, p["ln1_g"], p["ln1_b"], 1e-5), p["ln2_g"], p["ln2_b"], 1e-5)
    assert np.allclose(layer(x, q, h), want, rtol=0, atol=1e-12), "residual + post-norm order"
    a = mha(x, x, x, p["wq"], p["wk"], p["wv"], p["wo"], h, bq=p["bq"], bk=p["bk"], bv=p["bv"], bo=p["bo"])
    hh = ln(x + a, p["ln1_g"], p["ln1_b"], 1e-5)
    want = ln(hh + ffn(hh, p["w1"], p["b1"], p["w2"], p["b2"]), p["ln2_g"], p["ln2_b"], 1e-5)
    assert np.allclose(layer(x, p, h), want, rtol=0, atol=1e-13)


def check_encoder_layer_params():
    """The layer's parameters, in the shapes this build takes them, number
    3,152,384 at the base size: the count printed on "The Transformer"
    (rayaq.ca), "In PyTorch" (tests/golden/model_sizes.txt)."""
    sizes = read_golden_table("model_sizes.txt")
    p = encoder_params(55, sizes["base_d_model"], sizes["ffn_inner"])
    assert sum(v.size for v in p.values()) == sizes["encoder_layer_params"]


# ------------------------------------------------------------------ decoding against a K/V cache
def check_decode_is_last_causal_row(decode, attn):
    """Generating left to right, the newest token's query sees every cached key
    up to and including its own position: one decoding step equals the last row
    of causal attention over the sequence so far ("How Transformers Work"
    (worksonmygpu.com), "What changed since 2017"; "The Transformer"
    (hoshank.vercel.app), "The Breakthrough"; "The Transformer" (rayaq.ca),
    "Masks: who may look at whom")."""
    q, k, v = _qkv(60, B=3, H=2, nq=9, nk=9, d=4)
    full, _, full_lse = attn(q, k, v, causal=True)
    for L in (1, 5, 9):
        o, lse = decode(q[:, :, L - 1], k, v, [L] * 3)
        assert np.allclose(o, full[:, :, L - 1], rtol=0, atol=1e-14), f"decode at length {L}"
        assert np.allclose(lse, full_lse[:, :, L - 1], rtol=0, atol=1e-14)
    o, lse = decode(q[:, :, 0], k, v, [0, 3, 9])
    assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0])), "an empty cache gives 0 and lse -inf"


def check_paged_gather(gather):
    """A sequence stored in pages, in any page order, reads back as the
    contiguous sequence (the cache layout only moves rows, it computes nothing)."""
    r = _rng(61)
    H, d, P = 2, 3, 4
    seq = r.standard_normal((H, 10, d))
    order = [5, 0, 3]                                # logical page i lives in physical page order[i]
    pool = np.zeros((6, P, H, d))
    for i, pg in enumerate(order):
        chunk = seq[:, i * P:(i + 1) * P]
        pool[pg, :chunk.shape[1]] = chunk.transpose(1, 0, 2)
    assert np.array_equal(gather(pool, order, P, 10), seq)
    assert gather(pool, order, P, 0).shape == (H, 0, d)


# ------------------------------------------------------------------ backward pass
def _loss_grad_fd(attn, q, k, v, do, causal, kv_len, h=1e-6):
    """Central differences of L = sum(dO * O) with respect to every element of
    q, k and v, through the (separately pinned) forward oracle."""
    def loss(qq, kk, vv):
        return float(np.sum(do * attn(qq, kk, vv, causal=causal, kv_len=kv_len)[0]))
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(*g.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


def check_backward_finite_differences(bwd, attn):
    """The backward matches central differences of sum(dO * O) through the
    forward, unmasked (N_q != N_k), causal, and with key padding (incl. 0)."""
    r = _rng(70)
    cases = [(dict(causal=False, kv_len=None), (1, 2, 3, 4, 3)),
             (dict(causal=True, kv_len=None), (1, 1, 5, 5, 3)),
             (dict(causal=False, kv_len=[2, 0, 4]), (3, 1, 3, 4, 2)),
             (dict(causal=True, kv_len=[3, 5]), (2, 1, 5, 5, 2))]
    for kw, (B, H, nq, nk, d) in cases:
        q, k, v = r.standard_normal((B, H, nq, d)), r.standard_normal((B, H, nk, d)), r.standard_normal((B, H, nk, d))
        do = r.standard_normal((B, H, nq, d))
        want = _loss_grad_fd(attn, q, k, v, do, kw["causal"], kw["kv_len"])
        got = bwd(q, k, v, do, **kw)
        for name, g, w in zip(("dQ", "dK", "dV"), got, want):
            assert np.allclose(g, w, rtol=0, atol=1e-7), f"{name} vs finite differences ({kw})"


def check_backward_torch(bwd):
    """Cross-check: torch float64 autograd through scaled_dot_product_attention
    (CPU), unmasked, causal, and with a boolean key mask (True = may attend)."""
    import torch
    import torch.nn.functional as F
    r = _rng(71)
    B, H, n, d = 2, 3, 9, 4
    q, k, v = r.standard_normal((B, H, n, d)), r.standard_normal((B, H, n, d)), r.standard_normal((B, H, n, d))
    do = r.standard_normal((B, H, n, d))
    lens = [9, 4]
    for causal, kv_len in ((False, None), (True, None), (False, lens), (True, lens)):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        mask = None
        if kv_len is not None:
            mask = torch.zeros(B, 1, n, n, dtype=torch.bool)
            for b, L in enumerate(kv_len):
                mask[b, :, :, :L] = True
            if causal:
                mask &= torch.ones(n, n, dtype=torch.bool).tril()
        o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, is_causal=causal and mask is None)
        o.backward(torch.tensor(do))
        got = bwd(q, k, v, do, causal=causal, kv_len=kv_len)
        for name, g, t in zip(("dQ", "dK", "dV"), got, (tq, tk, tv)):
            assert np.allclose(g, t.grad.numpy(), rtol=0, atol=1e-12), f"{name} vs torch ({causal}, {kv_len})"


def check_backward_invariants(bwd):
    """Facts that hold for any inputs: every softmax Jacobian row sums to 0, so
    the key gradients sum to 0 over the keys; the weights sum to 1, so the value
    gradients sum to the sum of dO; with one key nothing reaches Q or K; the
    backward is linear in dO; under the causal mask the gradients of keys j and
    later do not depend on earlier queries; padded keys get exactly 0 and the
    rest equal the gradient of the truncated problem."""
    q, k, v = _qkv(72, B=2, H=2, nq=6, nk=6, d=4)
    do = _rng(73).standard_normal(q.shape)
    dq, dk, dv = bwd(q, k, v, do)
    assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-12), "key gradients must sum to 0"
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12), "value gradients must sum to sum(dO)"
    dq1, dk1, dv1 = bwd(q, k[:, :, :1], v[:, :, :1], do)
    assert np.all(np.abs(dq1) < 1e-14) and np.all(np.abs(dk1) < 1e-14), "one key: no gradient to Q or K"
    assert np.allclose(dv1[:, :, 0], do.sum(axis=2), atol=1e-12)
    do2 = _rng(74).standard_normal(q.shape)
    lin = bwd(q, k, v, do + 2.0 * do2)
    for a, b_, c in zip(lin, (dq, dk, dv), bwd(q, k, v, do2)):
        assert np.allclose(a, b_ + 2.0 * c, atol=1e-12), "linear in dO"
    # causal locality: change queries and dO before position j0
    j0 = 3
    base = bwd(q, k, v, do, causal=True)
    q2, do3 = q.copy(), do.copy()
    q2[:, :, :j0] += 5.0
    do3[:, :, :j0] -= 2.0
    moved = bwd(q2, k, v, do3, causal=True)
    assert np.allclose(moved[1][:, :, j0:], base[1][:, :, j0:], atol=1e-13), "causal dK locality"
    assert np.allclose(moved[2][:, :, j0:], base[2][:, :, j0:], atol=1e-13), "causal dV locality"
    # padding
    L = 4
    pq, pk, pv = bwd(q, k, v, do, kv_len=[L, L])
    tq, tk, tv = bwd(q, k[:, :, :L], v[:, :, :L], do)
    assert np.all(pk[:, :, L:] == 0.0) and np.all(pv[:, :, L:] == 0.0), "padded keys get no gradient"
    assert np.allclose(pq, tq, atol=1e-13) and np.allclose(pk[:, :, :L], tk, atol=1e-13)
    assert np.allclose(pv[:, :, :L], tv, atol=1e-13)
    zq, zk, zv = bwd(q, k, v, do, kv_len=[0, 6])
    assert np.all(zq[0] == 0.0) and np.all(zk[0] == 0.0) and np.all(zv[0] == 0.0), "no visible key: no gradient"


def check_backward_saturation(bwd):
    """The pages' reason for the scale: large logits saturate the softmax
    (nearly one-hot rows) and then almost no gradient passes through it. With
    K = I and each query t times a distinct basis vector, row i's scores are
    scale * t at one key and 0 elsewhere: at t = 1 the gradients to Q and K are
    live; at t = 200 the rows are one-hot to within exp(-70), dQ and dK vanish,
    and dV only routes each dO row to its query's key."""
    d = 8
    perm = np.array([3, 0, 7, 1, 6, 2, 5, 4])
    k = np.eye(d)[None, None]
    v = _rng(75).standard_normal((1, 1, d, d))
    do = _rng(76).standard_normal((1, 1, d, d))
    grads = {}
    for t in (1.0, 200.0):
        q = (t * np.eye(d)[perm])[None, None]
        grads[t] = bwd(q, k, v, do)
    live, frozen = grads[1.0], grads[200.0]
    assert np.linalg.norm(live[0]) > 0.05 * np.linalg.norm(do), "gradients to Q live at t = 1"
    assert np.linalg.norm(frozen[0]) < 1e-12 * np.linalg.norm(live[0]), "dQ must vanish at saturation"
    assert np.linalg.norm(frozen[1]) < 1e-12 * np.linalg.norm(live[1]), "dK must vanish at saturation"
    routed = np.zeros((d, d))
    routed[perm] = do[0, 0]                 # key perm[i] receives query i's dO row
    assert np.allclose(frozen[2][0, 0], routed, atol=1e-12), "dV routes dO rows through the one-hot weights"


def check_backward_sampled(sampled, bwd):
    """The sampled backward (statistics from the forward, delta as dO . O)
    equals the full backward on the sampled rows and keys, for every mask;
    rows with no visible key and padded keys give 0."""
    r = _rng(77)
    B, H, n, d = 2, 2, 37, 5
    q, k, v, do = (r.standard_normal((B, H, n, d)) for _ in range(4))
    rows = np.array([0, 1, 17, 35, 36])
    keys = np.array([0, 2, 20, 30, 36])
    for causal, kv_len in ((False, None), (True, None), (False, [37, 21]), (True, [0, 25])):
        full = bwd(q, k, v, do, causal=causal, kv_len=kv_len)
        part = sampled(q, k, v, do, rows, keys, causal=causal, kv_len=kv_len, chunk=8)
        assert np.allclose(part[0], full[0][:, :, rows], rtol=0, atol=1e-12), f"sampled dQ ({causal}, {kv_len})"
        assert np.allclose(part[1], full[1][:, :, keys], rtol=0, atol=1e-12), f"sampled dK ({causal}, {kv_len})"
        assert np.allclose(part[2], full[2][:, :, keys], rtol=0, atol=1e-12), f"sampled dV ({causal}, {kv_len})"



def check_backward_error_scale(bwd, sampled):
    """The term magnitudes bound the gradients (|sum| <= sum |terms|), equal
    them where every term is non-negative (dV with dO >= 0), are 0 exactly
    where no term exists (padded keys, empty rows), and agree between the full
    and the sampled oracle."""
    r = _rng(78)
    B, H, n, d = 2, 2, 21, 4
    q, k, v = (r.standard_normal((B, H, n, d)) for _ in range(3))
    do = r.standard_normal((B, H, n, d))
    for causal, kv_len in ((False, None), (True, [21, 0])):
        *g, e = bwd(q, k, v, do, causal=causal, kv_len=kv_len, error_scale=True)
        for gi, ei in zip(g, e):
            assert np.all(np.abs(gi) <= ei + 1e-12), "term magnitudes bound the gradient"
        rows = keys = np.array([0, 5, 20])
        *gs, es = sampled(q, k, v, do, rows, keys, causal=causal, kv_len=kv_len, chunk=8, error_scale=True)
        for ei, esi, idx in zip(e, es, (rows, keys, keys)):
            assert np.allclose(esi, ei[:, :, idx], rtol=0, atol=1e-12), "sampled term magnitudes"
    *g, e = bwd(q, k, v, np.abs(do), error_scale=True)
    assert np.allclose(e[2], g[2], atol=1e-12), "dV with dO >= 0: magnitude equals the gradient"
    *g, e = bwd(q, k, v, do, kv_len=[7, 0], error_scale=True)
    assert np.all(e[1][0, :, 7:] == 0) and np.all(e[2][0, :, 7:] == 0), "padded keys: no terms"
    assert all(np.all(x[1] == 0) for x in e), "no visible key: no terms"


ATTENTION_PINS = [check_rows_sum_to_one, check_permutation_equivariance,
                  check_constant_v_and_convex_hull, check_causal_locality,
                  check_masked_weight_is_zero, check_closed_forms, check_low_temperature_argmax,
                  check_default_scale, check_brute_force, check_hand_example,
                  check_linearity_and_shift, check_lse, check_key_padding, check_fully_masked_rows]
