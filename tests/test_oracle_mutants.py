"""Plant plausible mistakes in a copy of the oracle and show the pins catch each.

The mutants live here, on the CPU, and never touch the GPU path. Each one is
the plain definition with exactly one mistake; the test passes when at least
one pin rejects the mutant (an AssertionError, or arithmetic that breaks, e.g.
a row left with no visible key).
"""
import math

import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def _mutant_attention(mutation):
    def attn(q, k, v, *, causal=False, scale=None, rows=None, kv_len=None):
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        B, H, nq, d = q.shape
        nk = k.shape[2]
        if scale is None:
            scale = {"scale_times_sqrt_d": math.sqrt(d), "no_scale": 1.0,
                     "scale_one_over_d": 1.0 / d}.get(mutation, 1.0 / math.sqrt(d))
        pos = np.arange(nq) if rows is None else np.asarray(rows)
        o = np.empty((B, H, len(pos), v.shape[-1]))
        rs = np.empty((B, H, len(pos)))
        lse = np.empty((B, H, len(pos)))
        for b in range(B):
            for h in range(H):
                kk = k[b, h]
                s = q[b, h][pos] @ kk.T * scale
                if mutation == "sign_flip":
                    s = -s
                if causal:
                    i = pos[:, None]
                    j = np.arange(nk)[None, :]
                    blocked = {"mask_flipped": j < i, "mask_no_diagonal": j >= i,
                               "mask_off_by_one": j > i + 1}.get(mutation, j > i)
                    if mutation == "mask_after_softmax":
                        pass
                    else:
                        s = np.where(blocked, -np.inf, s)
                if kv_len is not None:
                    L = min(max(int(kv_len[b]), 0), nk)
                    j = np.arange(nk)[None, :]
                    pad = {"pad_keeps_one_more": j > L, "pad_polarity": j < L,
                           "pad_on_queries": np.zeros((1, nk), bool)}.get(mutation, j >= L)
                    s = np.where(pad, -np.inf, s)
                dead = np.all(s == -np.inf, axis=-1)
                if mutation != "pad_dead_rows_nan":
                    s = np.where(dead[:, None], 0.0, s)
                axis = -2 if mutation == "softmax_wrong_axis" else -1
                m = np.max(s, axis=axis, keepdims=True)
                e = np.exp(s - m)
                l = np.sum(e, axis=axis, keepdims=True)
                p = e if mutation == "no_normalise" else e / l
                if causal and mutation == "mask_after_softmax":
                    p = np.where(np.arange(nk)[None, :] > pos[:, None], 0.0, p)
                if mutation != "pad_dead_rows_nan":
                    p[dead] = 0.0
                vv = kk[:, :v.shape[-1]] if mutation == "uses_k_for_v" else v[b, h]
                if mutation == "transposed_p" and p.shape[0] == p.shape[1]:
                    p = p.T
                o[b, h] = p @ vv
                if mutation == "pad_on_queries" and kv_len is not None:
                    o[b, h][pos >= min(max(int(kv_len[b]), 0), nk)] = 0.0
                rs[b, h] = p.sum(-1)
                lse[b, h] = (m + np.log(l))[:, 0] if axis == -1 else np.log(np.exp(s).sum(-1))
                if mutation != "pad_dead_rows_nan":
                    lse[b, h] = np.where(dead, -np.inf, lse[b, h])
        return o, rs, lse
    return attn


ATTENTION_MUTANTS = ["scale_times_sqrt_d", "no_scale", "scale_one_over_d", "sign_flip",
                     "mask_flipped", "mask_no_diagonal", "mask_off_by_one", "mask_after_softmax",
                     "softmax_wrong_axis", "no_normalise", "uses_k_for_v", "transposed_p",
                     "pad_keeps_one_more", "pad_polarity", "pad_on_queries", "pad_dead_rows_nan"]


def _caught(fn):
    import warnings
    try:
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            with np.errstate(all="ignore"):
                fn()
    except (AssertionError, ValueError, FloatingPointError, IndexError):
        return True
    return False


@pytest.mark.parametrize("mutation", ATTENTION_MUTANTS)
def test_attention_mutant_is_caught(mutation):
    attn = _mutant_attention(mutation)
    caught = [c.__name__ for c in pins.ATTENTION_PINS if _caught(lambda c=c: c(attn))]
    assert caught, f"no pin catches the mutant {mutation!r}"


def _mutant_mha(mutation):
    def mha(xq, xk, xv, wq, wk, wv, wo, heads, *, causal=False, rows=None, kv_len=None):
        xq, xk, xv = (np.asarray(t, np.float64) for t in (xq, xk, xv))
        wq, wk, wv, wo = (np.asarray(t, np.float64) for t in (wq, wk, wv, wo))
        if mutation == "weights_transposed":
            wq, wk, wv, wo = wq.T, wk.T, wv.T, wo.T
        B, N, dm = xq.shape
        d = dm // heads

        def split(t):
            b, n, _ = t.shape
            if mutation == "heads_interleaved":
                return t.reshape(b, n, d, heads).transpose(0, 3, 1, 2)
            return t.reshape(b, n, heads, d).transpose(0, 2, 1, 3)

        q, k, v = split(xq @ wq), split(xk @ wk), split(xv @ wv)
        if mutation == "value_from_query_input":
            v = split(xq @ wv)
        o, _, _ = oracle.attention_ref(q, k, v, causal=causal, scale=1 / math.sqrt(d), rows=rows,
                                       kv_len=None if mutation == "padding_dropped" else kv_len)
        if mutation == "concat_reversed":
            o = o[:, ::-1]
        cat = o.transpose(0, 2, 1, 3).reshape(B, o.shape[2], dm)
        if mutation == "no_output_projection":
            return cat
        return cat @ wo
    return mha


MHA_MUTANTS = ["weights_transposed", "heads_interleaved", "concat_reversed",
               "no_output_projection", "value_from_query_input", "padding_dropped"]


@pytest.mark.parametrize("mutation", MHA_MUTANTS)
def test_mha_mutant_is_caught(mutation):
    mha = _mutant_mha(mutation)
    checks = [lambda: pins.check_mha_structure(mha, oracle.attention_ref),
              lambda: pins.check_torch_sdpa(oracle.attention_ref, mha),
              lambda: pins.check_torch_padding(oracle.attention_ref, mha),
              lambda: pins.check_parameter_counts(mha)]
    assert any(_caught(c) for c in checks), f"no pin catches the mutant {mutation!r}"


def test_unmutated_copies_pass():
    """The mutant scaffolding itself, with no mistake planted, passes every pin."""
    attn = _mutant_attention("none")
    for c in pins.ATTENTION_PINS:
        c(attn)
    mha = _mutant_mha("none")
    pins.check_mha_structure(mha, oracle.attention_ref)
    pins.check_torch_sdpa(oracle.attention_ref, mha)
    pins.check_torch_padding(oracle.attention_ref, mha)


def _mutant_layer(mutation):
    """The encoder layer with one planted mistake, built from the oracle's own
    attention (already pinned above)."""
    def ln(x, g, b, eps):
        x = np.asarray(x, np.float64)
        mu = x.mean(-1, keepdims=True)
        dev = x - mu
        n = x.shape[-1] - (1 if mutation == "unbiased_variance" else 0)
        var = (dev ** 2).sum(-1, keepdims=True) / n
        e = 0.0 if mutation == "no_eps" else eps
        if mutation == "gamma_beta_swapped":
            g, b = b, g
        return dev / np.sqrt(var + e) * g + b

    def ffn(x, w1, b1, w2, b2):
        pre = x @ w1 + (0.0 if mutation == "ffn_bias_dropped" else b1)
        hid = pre if mutation == "no_relu" else np.maximum(0.0, pre)
        return hid @ w2 + b2

    def layer(x, p, heads, *, eps=1e-5, causal=False, kv_len=None):
        x = np.asarray(x, np.float64)
        biases = {} if mutation == "attention_biases_dropped" else dict(bq=p["bq"], bk=p["bk"], bv=p["bv"],
                                                                          bo=p["bo"])
        def attn(t):
            return oracle.mha_ref(t, t, t, p["wq"], p["wk"], p["wv"], p["wo"], heads, causal=causal,
                                  kv_len=kv_len, **biases)
        if mutation == "pre_norm":
            h = x + attn(ln(x, p["ln1_g"], p["ln1_b"], eps))
            return h + ffn(ln(h, p["ln2_g"], p["ln2_b"], eps), p["w1"], p["b1"], p["w2"], p["b2"])
        a = attn(x)
        h = ln(a if mutation == "no_residual" else x + a, p["ln1_g"], p["ln1_b"], eps)
        f = ffn(h, p["w1"], p["b1"], p["w2"], p["b2"])
        return ln(h + f, p["ln2_g"], p["ln2_b"], eps)
    return layer, ln, ffn


LAYER_MUTANTS = ["pre_norm", "no_residual", "unbiased_variance", "no_eps", "gamma_beta_swapped",
                 "ffn_bias_dropped", "no_relu", "attention_biases_dropped"]


@pytest.mark.parametrize("mutation", LAYER_MUTANTS)
def test_layer_mutant_is_caught(mutation):
    layer, ln, ffn = _mutant_layer(mutation)
    checks = [lambda: pins.check_layer_norm(ln), lambda: pins.check_ffn(ffn),
              lambda: pins.check_encoder_layer_torch(layer),
              lambda: pins.check_encoder_layer_structure(layer, ln, ffn, oracle.mha_ref)]
    assert any(_caught(c) for c in checks), f"no pin catches the mutant {mutation!r}"


def test_unmutated_layer_passes():
    layer, ln, ffn = _mutant_layer("none")
    pins.check_layer_norm(ln)
    pins.check_ffn(ffn)
    pins.check_encoder_layer_torch(layer)
    pins.check_encoder_layer_structure(layer, ln, ffn, oracle.mha_ref)


def _mutant_decode(mutation):
    """One decoding step or the page gather with one planted mistake."""
    def decode(q, k, v, kv_len, *, scale=None):
        L = np.asarray(kv_len)
        if mutation == "decode_length_minus_one":
            L = np.maximum(L - 1, 0)
        elif mutation == "decode_length_plus_one":
            L = np.minimum(L + 1, np.asarray(k).shape[2])
        qq = np.asarray(q, np.float64)
        if mutation == "decode_scale_missing":
            qq = qq * math.sqrt(qq.shape[-1])
        return oracle.decode_ref(qq, k, v, L, scale=scale)

    def gather(pool, table, P, length):
        pool = np.asarray(pool, np.float64)
        if mutation == "pages_in_logical_order":
            table = list(range(len(table)))
        rows = []
        for j in range(length):
            pg, r = int(table[j // P]), j % P
            if mutation == "page_row_reversed":
                r = P - 1 - r
            rows.append(pool[pg, r])
        if not rows:
            return np.zeros((pool.shape[2], 0, pool.shape[3]))
        out = np.stack(rows, axis=1)
        return out[::-1] if mutation == "heads_swapped" else out
    return decode, gather


DECODE_MUTANTS = ["decode_length_minus_one", "decode_length_plus_one", "decode_scale_missing",
                  "pages_in_logical_order", "page_row_reversed", "heads_swapped"]


@pytest.mark.parametrize("mutation", DECODE_MUTANTS)
def test_decode_mutant_is_caught(mutation):
    decode, gather = _mutant_decode(mutation)
    checks = [lambda: pins.check_decode_is_last_causal_row(decode, oracle.attention_ref),
              lambda: pins.check_paged_gather(gather)]
    assert any(_caught(c) for c in checks), f"no pin catches the mutant {mutation!r}"


def test_unmutated_decode_passes():
    decode, gather = _mutant_decode("none")
    pins.check_decode_is_last_causal_row(decode, oracle.attention_ref)
    pins.check_paged_gather(gather)


def _mutant_backward(mutation):
    """The attention backward with one planted mistake."""
    def bwd(q, k, v, do, *, causal=False, scale=None, kv_len=None):
        q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
        B, H, nq, d = q.shape
        nk = k.shape[2]
        if scale is None:
            scale = 1.0 / math.sqrt(d)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                s = q[b, h] @ k[b, h].T * scale
                if causal and mutation != "causal_dropped":
                    s = np.where(np.arange(nk)[None, :] > np.arange(nq)[:, None], -np.inf, s)
                if kv_len is not None and mutation != "padding_dropped":
                    L = min(max(int(kv_len[b]), 0), nk)
                    s = np.where(np.arange(nk)[None, :] >= L, -np.inf, s)
                dead = np.all(s == -np.inf, axis=-1)
                s = np.where(dead[:, None], 0.0, s)
                e = np.exp(s - s.max(-1, keepdims=True))
                p = e / e.sum(-1, keepdims=True)
                p[dead] = 0.0
                vv = k[b, h] if mutation == "dp_uses_k" else v[b, h]
                dp = do[b, h] @ vv.T
                if mutation == "no_row_term":
                    ds = p * dp
                elif mutation == "row_term_wrong_axis":
                    ds = p * (dp - np.sum(p * dp, axis=0, keepdims=True))
                else:
                    ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
                if mutation == "ds_sign_flip":
                    ds = -ds
                dv[b, h] = (p @ do[b, h]) if mutation == "dv_not_transposed" else p.T @ do[b, h]
                dq[b, h] = (1.0 if mutation == "dq_scale_dropped" else scale) * (ds @ k[b, h])
                sk = scale * scale if mutation == "dk_scale_twice" else scale
                dk[b, h] = sk * ((ds @ q[b, h]) if mutation == "dk_not_transposed" else ds.T @ q[b, h])
        return dq, dk, dv
    return bwd


BACKWARD_MUTANTS = ["dq_scale_dropped", "dk_scale_twice", "no_row_term", "row_term_wrong_axis", "ds_sign_flip",
                    "dv_not_transposed", "dk_not_transposed", "dp_uses_k", "causal_dropped", "padding_dropped"]


@pytest.mark.parametrize("mutation", BACKWARD_MUTANTS)
def test_backward_mutant_is_caught(mutation):
    bwd = _mutant_backward(mutation)
    checks = [lambda: pins.check_backward_finite_differences(bwd, oracle.attention_ref),
              lambda: pins.check_backward_torch(bwd),
              lambda: pins.check_backward_invariants(bwd),
              lambda: pins.check_backward_saturation(bwd)]
    assert any(_caught(c) for c in checks), f"no pin catches the mutant {mutation!r}"


def test_unmutated_backward_passes():
    bwd = _mutant_backward("none")
    pins.check_backward_finite_differences(bwd, oracle.attention_ref)
    pins.check_backward_torch(bwd)
    pins.check_backward_invariants(bwd)
    pins.check_backward_saturation(bwd)
