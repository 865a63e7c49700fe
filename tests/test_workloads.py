"""Seeded input generators: storage rounding and workload bookkeeping (CPU only)."""
import numpy as np
import torch

import workloads


def test_bf16_rounding_matches_torch():
    r = np.random.default_rng(0)
    x = np.concatenate([r.standard_normal(100000) * 10.0 ** r.integers(-6, 6, 100000),
                        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.005859375, 3.0e38, -1e-40])])
    x32 = x.astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.bf16_bits(x), want)
    back = workloads.bf16_bits_to_f32(want)
    assert np.array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_flop_counts():
    w = workloads.WORKLOADS
    assert w["long_causal_bf16_b2_h16_n8192"].attention_flops() == 4 * 2 * 16 * 64 * (8192 * 8193 // 2)
    assert abs(w["long_causal_bf16_b2_h16_n8192"].attention_flops() - 2.749e11) < 1e8
    enc = w["base_encoder_mha_bf16_b32_n512"]
    assert abs(enc.attention_flops() - 1.718e10) < 1e7
    assert abs(enc.total_flops() - 5.154e10) < 1e7
    assert abs(w["decoder_causal_bf16_b16_h8_n1024"].attention_flops() - 1.720e10) < 1e7
    assert abs(w["cross_attn_bf16_b32_h8_nq384_nk512"].attention_flops() - 1.288e10) < 1e7


def test_inputs_are_seeded_and_shaped():
    w = workloads.get("cross")
    a, b = workloads.make_inputs(w), workloads.make_inputs(w)
    assert a["q"].shape == (32, 8, 384, 64) and a["k"].shape == (32, 8, 512, 64)
    assert np.array_equal(a["v"].raw, b["v"].raw)
    ones = workloads.make_inputs(w, v_ones=True)
    assert np.array_equal(ones["q"].raw, a["q"].raw) and np.all(ones["v"].value == 1.0)
    assert abs(a["q"].value.std() - 1.0) < 0.01
    t = workloads.make_inputs(workloads.get("tiny"))
    assert t["x"].dtype == "f32" and t["wq"].shape == (512, 512)
    assert abs(t["wq"].value.std() * np.sqrt(512) - 1.0) < 0.01


def test_sample_rows():
    w = workloads.get("long")
    rows = workloads.sample_rows(w)
    assert len(rows) == 64 == len(set(rows.tolist()))
    assert set(workloads.EDGE_ROWS) <= set(rows.tolist())
    assert np.all(np.diff(rows) > 0) and rows.max() < w.n_q


def test_padded_workload_lengths_and_pairs():
    w = workloads.get("padded")
    lens = w.kv_lengths()
    assert lens.dtype == np.int32 and lens.shape == (32,)
    assert np.array_equal(lens, w.kv_lengths())
    assert lens.min() >= 64 and lens.max() <= 512
    assert w.total_pairs() == int(np.sum(lens)) * w.n_q
    assert w.attention_flops() == 4 * 8 * 64 * w.total_pairs()
    # the causal count under padding equals a brute-force count of visible (i, j)
    import dataclasses
    c = dataclasses.replace(w, causal=True, n_q=40, n_k=40, kv_len_range=(0, 40))
    want = 0
    for L in c.kv_lengths():
        i = np.arange(40)[:, None]
        j = np.arange(40)[None, :]
        want += int(np.sum((j <= i) & (j < L)))
    assert c.total_pairs() == want
    assert workloads.get("encoder").kv_lengths() is None
