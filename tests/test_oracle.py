"""The fp64 oracle against what the pages and mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


@pytest.mark.parametrize("check", pins.ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_pin(check):
    check(oracle.attention_ref)


def test_printed_mask():
    pins.check_printed_mask(oracle.causal_mask)


def test_mask_rows_match_full_mask():
    full = oracle.causal_mask(9)
    rows = np.array([0, 4, 8])
    assert np.array_equal(oracle.causal_mask_rows(9, rows), full[rows])


def test_weights_function_matches_attention():
    r = np.random.default_rng(3)
    q, k = r.standard_normal((6, 4)), r.standard_normal((6, 4))
    for causal in (False, True):
        p = oracle.attention_weights_ref(q, k, causal=causal)
        o, _, _ = oracle.attention_ref(q[None, None], k[None, None], np.eye(6)[None, None], causal=causal)
        assert np.allclose(p, o[0, 0], rtol=0, atol=1e-14)
    # with all-zero scores the causal weights are uniform over the visible keys,
    # and their zero pattern is the printed mask's -inf pattern
    p = oracle.attention_weights_ref(np.zeros((4, 1)), np.zeros((4, 1)), causal=True)
    want = pins.read_golden_matrix("causal_mask_n4.txt")
    assert np.array_equal(p == 0, np.isinf(want))
    assert np.allclose(p.sum(1), 1.0) and np.allclose(p[3], 0.25)


def test_mha_structure():
    pins.check_mha_structure(oracle.mha_ref, oracle.attention_ref)


def test_rows_subset():
    pins.check_rows_subset(oracle.attention_ref, oracle.mha_ref)


def test_parameter_counts():
    pins.check_parameter_counts(oracle.mha_ref)


def test_torch_cross_check():
    pins.check_torch_sdpa(oracle.attention_ref, oracle.mha_ref)


def test_torch_padding_cross_check():
    pins.check_torch_padding(oracle.attention_ref, oracle.mha_ref)


def test_padding_row_is_the_printed_form():
    # one row per batch item, 0 where the key may be read and -inf past the length
    row = oracle.key_padding_mask_row(5, 3)
    assert np.array_equal(row[:3], np.zeros(3)) and np.all(np.isneginf(row[3:]))
    assert np.array_equal(oracle.key_padding_mask_row(4, 0), np.full(4, -np.inf))


def test_causal_rejects_cross_shapes():
    r = np.random.default_rng(4)
    q, k = r.standard_normal((1, 1, 3, 2)), r.standard_normal((1, 1, 5, 2))
    with pytest.raises(ValueError):
        oracle.attention_ref(q, k, k, causal=True)


def test_linear_is_the_projection_used_by_mha():
    # h = 1 with W^O = I: mha output = attention over the three projections
    r = np.random.default_rng(5)
    x = r.standard_normal((2, 4, 6))
    wq, wk, wv = (r.standard_normal((6, 6)) for _ in range(3))
    out = oracle.mha_ref(x, x, x, wq, wk, wv, np.eye(6), 1)
    q, k, v = (oracle.linear_ref(x, w)[:, None] for w in (wq, wk, wv))
    o, _, _ = oracle.attention_ref(q, k, v)
    assert np.allclose(out, o[:, 0], rtol=0, atol=1e-12)
    # and it is the row-by-column product: entry (i, j) = sum_t x[i, t] w[t, j]
    a, b = r.standard_normal((3, 5)), r.standard_normal((5, 2))
    y = oracle.linear_ref(a, b)
    assert abs(y[2, 1] - sum(a[2, t] * b[t, 1] for t in range(5))) < 1e-13


def test_layer_norm():
    pins.check_layer_norm(oracle.layer_norm_ref)


def test_ffn():
    pins.check_ffn(oracle.ffn_ref)


def test_encoder_layer_against_torch():
    pins.check_encoder_layer_torch(oracle.encoder_layer_ref)


def test_encoder_layer_structure():
    pins.check_encoder_layer_structure(oracle.encoder_layer_ref, oracle.layer_norm_ref, oracle.ffn_ref,
                                       oracle.mha_ref)


def test_encoder_layer_params():
    pins.check_encoder_layer_params()


def test_decode_is_last_causal_row():
    pins.check_decode_is_last_causal_row(oracle.decode_ref, oracle.attention_ref)


def test_paged_gather():
    pins.check_paged_gather(oracle.gather_pages)


def test_backward_finite_differences():
    pins.check_backward_finite_differences(oracle.attention_backward_ref, oracle.attention_ref)


def test_backward_torch():
    pins.check_backward_torch(oracle.attention_backward_ref)


def test_backward_invariants():
    pins.check_backward_invariants(oracle.attention_backward_ref)


def test_backward_saturation():
    pins.check_backward_saturation(oracle.attention_backward_ref)


def test_backward_sampled():
    pins.check_backward_sampled(oracle.attention_backward_sampled_ref, oracle.attention_backward_ref)


def test_backward_error_scale():
    pins.check_backward_error_scale(oracle.attention_backward_ref, oracle.attention_backward_sampled_ref)
