"""HIP path vs the fp64 oracle on the same seeded inputs (GPU).

Bars: max-abs error <= 1e-4 (fp32) or <= 2e-2 (bf16) on unit-variance inputs;
softmax row sums within 1e-3 of 1. Everything is called through the C ABI
(via the thin binding). Sizes: every workload at its full size (the long
causal one checked on sampled query positions, all keys each), plus small
ragged shapes that span several tiles and a partial tail.
"""
import math

import numpy as np
import pytest

import oracle
import transformer_scaled_dot_mha_amd as mha
import workloads
from tests.gpu_util import (ENC_TOL, LSE_TOL, ROWSUM_TOL, TOL, assert_close, device, max_abs, say, to_device,
                             to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _attn_inputs(w, dev, v_ones=False):
    x = workloads.make_inputs(w, v_ones=v_ones)
    return x, to_device(x["q"], dev), to_device(x["k"], dev), to_device(x["v"], dev)


def _oracle_rows(w):
    return workloads.sample_rows(w) if w.oracle_rows else None


# ---------------------------------------------------------------- the five workloads
@pytest.mark.parametrize("name", ["decoder", "cross", "long"])
def test_attention_workload_parity(dev, name):
    import torch
    w = workloads.get(name)
    x, q, k, v = _attn_inputs(w, dev)
    say(f"attention_forward {w.name}")
    o, lse = mha.attention_forward(q, k, v, causal=w.causal, return_lse=True)
    torch.cuda.synchronize()
    rows = _oracle_rows(w)
    want, _, want_lse = oracle.attention_ref(x["q"].value, x["k"].value, x["v"].value, causal=w.causal,
                                             rows=rows)
    got = to_f64(o) if rows is None else to_f64(o[:, :, torch.as_tensor(rows, device=dev)])
    got_lse = to_f64(lse) if rows is None else to_f64(lse[:, :, torch.as_tensor(rows, device=dev)])
    err = assert_close(got, want, w.dtype, w.name)
    assert max_abs(got_lse, want_lse) <= LSE_TOL[w.dtype], "log-sum-exp"
    say(f"{w.name}: max-abs {err:.3e}")


@pytest.mark.parametrize("name", ["tiny", "encoder"])
def test_mha_workload_parity(dev, name):
    import torch
    w = workloads.get(name)
    x = workloads.make_inputs(w)
    t = {k_: to_device(s, dev) for k_, s in x.items()}
    say(f"mha_forward {w.name}")
    out = mha.mha_forward(t["x"], t["x"], t["x"], t["wq"], t["wk"], t["wv"], t["wo"], w.heads)
    torch.cuda.synchronize()
    xv = x["x"].value
    want = oracle.mha_ref(xv, xv, xv, x["wq"].value, x["wk"].value, x["wv"].value, x["wo"].value, w.heads)
    err = assert_close(to_f64(out), want, w.dtype, w.name)
    say(f"{w.name}: max-abs {err:.3e}")


# ---------------------------------------------------------------- row sums
@pytest.mark.parametrize("name", ["decoder", "cross", "long"])
def test_row_sums_with_v_ones(dev, name):
    """With V = 1 every output element is the row sum of the weights."""
    import torch
    w = workloads.get(name)
    _, q, k, v = _attn_inputs(w, dev, v_ones=True)
    say(f"row sums {w.name}")
    o = mha.attention_forward(q, k, v, causal=w.causal)
    torch.cuda.synchronize()
    dev_err = float((o.float() - 1.0).abs().max())
    assert dev_err <= ROWSUM_TOL, f"row sum off by {dev_err}"


def test_lse_normalises_the_scores(dev):
    """sum_j exp(scale q_i.k_j - lse_i), evaluated on the host in fp64, is 1 to
    within the normaliser's bf16 rounding bound (exp(LSE_TOL) - 1)."""
    import torch
    w = workloads.get("long")
    x, q, k, v = _attn_inputs(w, dev)
    _, lse = mha.attention_forward(q, k, v, causal=True, return_lse=True)
    torch.cuda.synchronize()
    rows = workloads.sample_rows(w)[::4]
    lse_h = to_f64(lse)
    qv, kv = x["q"].value, x["k"].value
    for b in range(w.batch):
        for h in (0, w.heads - 1):
            s = qv[b, h, rows] @ kv[b, h].T * 0.125
            s = np.where(np.arange(w.n_k)[None, :] > rows[:, None], -np.inf, s)
            tot = np.exp(s - lse_h[b, h, rows][:, None]).sum(-1)
            assert np.max(np.abs(tot - 1.0)) <= math.expm1(LSE_TOL["bf16"])


# ---------------------------------------------------------------- edge shapes
EDGE = [
    # (B, H, n_q, n_k, causal, dtype)
    (1, 1, 1, 1, False, "bf16"),
    (1, 1, 1, 1, True, "bf16"),
    (1, 2, 63, 63, True, "bf16"),
    (2, 1, 65, 65, True, "bf16"),
    (1, 3, 129, 129, False, "bf16"),
    (1, 1, 1000, 1000, True, "bf16"),
    (2, 2, 200, 77, False, "bf16"),
    (1, 2, 5, 300, False, "bf16"),
    (1, 1, 257, 1, False, "bf16"),
    (2, 1, 1500, 1650, False, "bf16"),
    # 64 query rows per wavefront (two 32-row blocks, long query runs: causal from 4096 queries,
    # unmasked from 2048) on both sides of the rule, with ragged tails
    (2, 2, 2048, 2048, True, "bf16"),
    (1, 1, 2049, 2049, True, "bf16"),
    (1, 3, 2600, 2600, True, "bf16"),
    (1, 2, 3000, 3000, True, "bf16"),
    (1, 1, 4095, 4095, True, "bf16"),
    (1, 1, 4096, 4096, True, "bf16"),
    (1, 1, 4100, 4100, True, "bf16"),
    (1, 1, 2500, 2600, False, "bf16"),
    # unmasked query runs that fill whole 256-row workgroups also take 64 rows per wavefront;
    # ragged key counts on either side of a key tile, and 640 rows (which stays at 32)
    (2, 2, 512, 300, False, "bf16"),
    (1, 3, 768, 769, False, "bf16"),
    (1, 1, 1024, 64, False, "bf16"),
    (1, 2, 640, 640, False, "bf16"),
    (1, 1, 1, 1, True, "f32"),
    (2, 3, 65, 65, True, "f32"),
    (1, 2, 100, 37, False, "f32"),
]


@pytest.mark.parametrize("B,H,nq,nk,causal,dtype", EDGE)
def test_edge_shapes(dev, B, H, nq, nk, causal, dtype):
    import torch
    d = 64
    q = workloads.random_tensor((B, H, nq, d), dtype, seed=100 + nq)
    k = workloads.random_tensor((B, H, nk, d), dtype, seed=200 + nk)
    v = workloads.random_tensor((B, H, nk, d), dtype, seed=300 + nk)
    say(f"edge {B}x{H} nq={nq} nk={nk} causal={causal} {dtype}")
    o = mha.attention_forward(to_device(q, dev), to_device(k, dev), to_device(v, dev), causal=causal)
    torch.cuda.synchronize()
    want, _, _ = oracle.attention_ref(q.value, k.value, v.value, causal=causal)
    assert_close(to_f64(o), want, dtype, "edge")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
def test_f32_head_widths(dev, d):
    import torch
    q = workloads.random_tensor((2, 2, 70, d), "f32", seed=400 + d)
    k = workloads.random_tensor((2, 2, 70, d), "f32", seed=500 + d)
    v = workloads.random_tensor((2, 2, 70, d), "f32", seed=600 + d)
    for causal in (False, True):
        say(f"f32 d={d} causal={causal}")
        o = mha.attention_forward(to_device(q, dev), to_device(k, dev), to_device(v, dev), causal=causal)
        torch.cuda.synchronize()
        want, _, _ = oracle.attention_ref(q.value, k.value, v.value, causal=causal)
        assert_close(to_f64(o), want, "f32", f"f32 d={d}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_head_views(dev, dtype):
    """(B, N, H, d) buffers used through transposed views: the head split as strides."""
    import torch
    B, N, H, d = 2, 150, 4, 64
    qs = workloads.random_tensor((B, N, H, d), dtype, seed=7)
    ks = workloads.random_tensor((B, N, H, d), dtype, seed=8)
    vs = workloads.random_tensor((B, N, H, d), dtype, seed=9)
    q, k, v = (to_device(s, dev).transpose(1, 2) for s in (qs, ks, vs))
    out = torch.zeros((B, N, H, d), dtype=q.dtype, device=dev)
    say(f"strided views {dtype}")
    mha.attention_forward(q, k, v, causal=True, out=out.transpose(1, 2))
    torch.cuda.synchronize()
    t = lambda s: s.value.transpose(0, 2, 1, 3)
    want, _, _ = oracle.attention_ref(t(qs), t(ks), t(vs), causal=True)
    assert_close(to_f64(out).transpose(0, 2, 1, 3), want, dtype, "strided")


@pytest.mark.parametrize("scale", [0.0, -0.125, 0.3, 2.0])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_scale_values(dev, scale, dtype):
    """Scale acts as an inverse temperature; 0 gives uniform weights, negative flips the order."""
    import torch
    q = workloads.random_tensor((1, 2, 130, 64), dtype, seed=11)
    k = workloads.random_tensor((1, 2, 130, 64), dtype, seed=12)
    v = workloads.random_tensor((1, 2, 130, 64), dtype, seed=13)
    for causal in (False, True):
        say(f"scale={scale} {dtype} causal={causal}")
        o = mha.attention_forward(to_device(q, dev), to_device(k, dev), to_device(v, dev), causal=causal,
                                  scale=scale)
        torch.cuda.synchronize()
        want, _, _ = oracle.attention_ref(q.value, k.value, v.value, causal=causal, scale=scale)
        assert_close(to_f64(o), want, dtype, f"scale {scale}")


@pytest.mark.parametrize("scale", [1.0, 2.0, -1.5])
@pytest.mark.parametrize("causal", [False, True])
def test_reference_moves_in_long_query_runs(dev, scale, causal):
    """Large scales spread the scores over many binary orders, so a row's running
    reference maximum moves inside a key tile, also on its second 32-key slab.
    N = 2048 (a multiple of 256 rows) takes the kernel form with 64 query rows per
    wavefront, which checks both slabs of a tile before their P V products: the
    weights already computed against the old reference must reach O before O is
    rescaled. (Found wrong in that form, max-abs error 58 at scale 2.)"""
    import torch
    n = 2048
    q = workloads.random_tensor((1, 2, n, 64), "bf16", seed=61)
    k = workloads.random_tensor((1, 2, n, 64), "bf16", seed=62)
    v = workloads.random_tensor((1, 2, n, 64), "bf16", seed=63)
    say(f"reference moves n={n} scale={scale} causal={causal}")
    o, lse = mha.attention_forward(to_device(q, dev), to_device(k, dev), to_device(v, dev), causal=causal,
                                   scale=scale, return_lse=True)
    torch.cuda.synchronize()
    want, _, want_lse = oracle.attention_ref(q.value, k.value, v.value, causal=causal, scale=scale)
    assert_close(to_f64(o), want, "bf16", f"scale {scale} causal {causal}")
    assert max_abs(to_f64(lse), want_lse) <= LSE_TOL["bf16"], "log-sum-exp"


@pytest.mark.parametrize("n,causal", [(300, False), (512, False), (2048, True), (4096, True)])
def test_weights_beyond_the_float_range(dev, n, causal):
    """At scale 12 the scores of one row span several hundred binary orders: a
    row's maximum exceeds the maximum of its first 32 keys by up to ~500 of them
    (274 of the 512 rows, 2947 of the 4096 rows by 128 or more, so weights against
    that first reference would overflow fp32). The running reference must move
    on unmasked tiles without any weight against an outdated reference reaching
    O or the row sum as inf. 512 and 4096 rows take the 64-row kernel form, 300
    and 2048 the 32-row forms (unmasked, and causal with the three-stage ring)."""
    import torch
    q = workloads.random_tensor((1, 1, n, 64), "bf16", seed=71)
    k = workloads.random_tensor((1, 1, n, 64), "bf16", seed=72)
    v = workloads.random_tensor((1, 1, n, 64), "bf16", seed=73)
    say(f"overflowing weights n={n} causal={causal}")
    o, lse = mha.attention_forward(to_device(q, dev), to_device(k, dev), to_device(v, dev), causal=causal,
                                   scale=12.0, return_lse=True)
    torch.cuda.synchronize()
    want, _, want_lse = oracle.attention_ref(q.value, k.value, v.value, causal=causal, scale=12.0)
    assert_close(to_f64(o), want, "bf16", f"scale 12 causal {causal}")
    assert max_abs(to_f64(lse), want_lse) <= LSE_TOL["bf16"], "log-sum-exp"


# ---------------------------------------------------------------- properties on GPU outputs
def test_deterministic(dev):
    import torch
    w = workloads.get("decoder")
    _, q, k, v = _attn_inputs(w, dev)
    say("determinism")
    a = mha.attention_forward(q, k, v, causal=True)
    b = mha.attention_forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_causal_locality_on_gpu(dev):
    """Changing rows > i of Q, K, V leaves GPU output rows <= i bitwise unchanged."""
    import torch
    q = workloads.random_tensor((1, 2, 300, 64), "bf16", seed=21)
    k = workloads.random_tensor((1, 2, 300, 64), "bf16", seed=22)
    v = workloads.random_tensor((1, 2, 300, 64), "bf16", seed=23)
    tq, tk, tv = (to_device(s, dev) for s in (q, k, v))
    o = mha.attention_forward(tq, tk, tv, causal=True)
    for i in (0, 63, 64, 200):
        q2, k2, v2 = tq.clone(), tk.clone(), tv.clone()
        for t in (q2, k2, v2):
            t[:, :, i + 1:] = -t[:, :, i + 1:] * 2
        say(f"causal locality i={i}")
        o2 = mha.attention_forward(q2, k2, v2, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o2[:, :, :i + 1], o[:, :, :i + 1])


def test_key_permutation_invariance_on_gpu(dev):
    import torch
    w = workloads.get("cross")
    _, q, k, v = _attn_inputs(w, dev)
    perm = torch.as_tensor(np.random.default_rng(5).permutation(w.n_k), device=dev)
    say("key permutation")
    a = mha.attention_forward(q, k, v)
    b = mha.attention_forward(q, k[:, :, perm].contiguous(), v[:, :, perm].contiguous())
    torch.cuda.synchronize()
    assert float((a.float() - b.float()).abs().max()) <= TOL["bf16"]


# ---------------------------------------------------------------- projections and full MHA variants
def _linear_tile_rows(m, n, groups=1):
    """Tile height the bf16 projection launcher picks (its rule restated here
    so that each case below is known to reach the form it is meant for): 64
    rows when the 128-row grid has fewer workgroups than CUs, else the height
    whose workgroup count fills whole rounds of resident workgroups best (768
    per round for the 256-row tile, three per CU; 1280 for the 128-row tile,
    five per CU), 128 on ties."""
    tiles_n = (n + 127) // 128
    big = tiles_n * ((m + 255) // 256) * groups
    small = tiles_n * ((m + 127) // 128) * groups
    if small < 256:
        return 64
    fill = lambda w, r: w / (((w + r - 1) // r) * r)
    return 256 if big >= 768 and fill(big, 768) > fill(small, 1280) else 128


LINEAR_CASES = [
    # 64-row tiles (grids smaller than the CU count), ragged m, n and k
    (1, 8, 8, "bf16"), (300, 136, 72, "bf16"), (2048, 512, 512, "bf16"), (257, 520, 136, "bf16"),
    (1000, 1536, 512, "bf16"), (64, 128, 1040, "bf16"),
    # 128-row tiles; grids of at most 512 of them (two per CU) take the 4-stage ring with two k chunks per
    # barrier: 16 chunks, 7 (an odd count, ragged last), 1 and 2 (both ragged)
    (16384, 512, 512, "bf16"), (4100, 1096, 200, "bf16"), (8200, 512, 24, "bf16"), (8200, 512, 40, "bf16"),
    (8000, 2048, 520, "bf16"), (32640, 512, 512, "bf16"),
    # 256-row tiles: 768 workgroups fill one round, with ragged m (the epilogue's
    # second pass partly or wholly past the end) and a partial last k chunk
    (12200, 2048, 520, "bf16"), (49000, 512, 512, "bf16"), (12161, 2048, 512, "bf16"),
    # fp32: split-k form (small grids; k quarters of 16, 48 and 64 with a ragged last one), and the 64 x 64 form
    (37, 20, 12, "f32"), (129, 512, 512, "f32"), (70, 136, 200, "f32"), (3, 4, 260, "f32"), (1100, 1040, 72, "f32"),
]


def _linear_f32_form(m, n, groups=1):
    return "split-k" if ((n + 63) // 64) * ((m + 63) // 64) * groups < 256 else "64x64"


@pytest.mark.parametrize("m,n,k,dtype", LINEAR_CASES)
def test_linear_parity(dev, m, n, k, dtype):
    import torch
    x = workloads.random_tensor((m, k), dtype, seed=31)
    wt = workloads.random_tensor((k, n), dtype, seed=32, scale=1 / math.sqrt(k))
    say(f"linear {m}x{k}x{n} {dtype} ({_linear_tile_rows(m, n)}-row tiles)")
    y = mha.linear_forward(to_device(x, dev), to_device(wt, dev))
    torch.cuda.synchronize()
    assert_close(to_f64(y), oracle.linear_ref(x.value, wt.value), dtype, "linear")


def test_linear_cases_reach_both_tile_heights():
    """The case list above selects both bf16 tile forms and both fp32 forms (a host-side check of the list)."""
    heights = {_linear_tile_rows(m, n) for m, n, k, dt in LINEAR_CASES if dt == "bf16"}
    assert heights == {64, 128, 256}
    assert {_linear_f32_form(m, n) for m, n, k, dt in LINEAR_CASES if dt == "f32"} == {"split-k", "64x64"}


def test_mha_with_256_row_projection_tiles(dev):
    """B * N = 16200 rows: the grouped Q/K/V launch takes 256-row tiles (768
    workgroups, one round against 60 % of two for 1524 of 128 rows), W^O takes
    128-row tiles; the last row tile holds 72 rows, so its second output pass is
    empty."""
    import torch
    B, N, dm, h = 30, 540, 512, 8
    assert B * N == 16200 and _linear_tile_rows(B * N, dm, groups=3) == 256
    x = workloads.random_tensor((B, N, dm), "bf16", seed=1301)
    ws = [workloads.random_tensor((dm, dm), "bf16", seed=1302 + i, scale=1 / math.sqrt(dm)) for i in range(4)]
    t = to_device(x, dev)
    say(f"mha_forward {B}x{N} d_model={dm} (256-row Q/K/V tiles)")
    out = mha.mha_forward(t, t, t, *[to_device(s, dev) for s in ws], h)
    torch.cuda.synchronize()
    want = oracle.mha_ref(x.value, x.value, x.value, *[s.value for s in ws], h)
    err = assert_close(to_f64(out), want, "bf16", "mha 16200 rows")
    say(f"mha 16200 rows: max-abs {err:.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_linear_strided(dev, dtype):
    """Leading dimensions wider than the row: X, W and Y are column slices of wider buffers."""
    import torch
    m, n, k = 333, 200, 264
    xb = workloads.random_tensor((m, k + 24), dtype, seed=33)
    wb = workloads.random_tensor((k, n + 40), dtype, seed=34, scale=1 / math.sqrt(k))
    x, w = to_device(xb, dev)[:, :k], to_device(wb, dev)[:, :n]
    yb = torch.full((m, n + 16), 7.0, dtype=x.dtype, device=dev)
    say(f"linear strided {dtype}")
    mha.linear_forward(x, w, out=yb[:, :n])
    torch.cuda.synchronize()
    assert_close(to_f64(yb[:, :n]), oracle.linear_ref(xb.value[:, :k], wb.value[:, :n]), dtype, "linear strided")
    assert bool((yb[:, n:] == 7.0).all()), "write outside the output view"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mha_cross_and_causal(dev, dtype):
    import torch
    B, nq, nk, dm, h = 2, 70, 130, 256 if dtype == "f32" else 512, 8 if dtype == "bf16" else 4
    xq = workloads.random_tensor((B, nq, dm), dtype, seed=41)
    mem = workloads.random_tensor((B, nk, dm), dtype, seed=42)
    ws = [workloads.random_tensor((dm, dm), dtype, seed=43 + i, scale=1 / math.sqrt(dm)) for i in range(4)]
    tw = [to_device(s, dev) for s in ws]
    say(f"mha cross {dtype}")
    out = mha.mha_forward(to_device(xq, dev), to_device(mem, dev), to_device(mem, dev), *tw, h)
    torch.cuda.synchronize()
    want = oracle.mha_ref(xq.value, mem.value, mem.value, *[s.value for s in ws], h)
    assert_close(to_f64(out), want, dtype, "mha cross")
    say(f"mha causal {dtype}")
    xs = workloads.random_tensor((B, nk, dm), dtype, seed=47)
    t = to_device(xs, dev)
    out = mha.mha_forward(t, t, t, *tw, h, causal=True)
    torch.cuda.synchronize()
    want = oracle.mha_ref(xs.value, xs.value, xs.value, *[s.value for s in ws], h, causal=True)
    assert_close(to_f64(out), want, dtype, "mha causal")


def test_binding_reports_workspace_error(dev):
    import torch
    w = workloads.get("tiny")
    x = {k_: to_device(s, dev) for k_, s in workloads.make_inputs(w).items()}
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(mha.MHAError, match="MHA_ERR_WORKSPACE"):
        mha.mha_forward(x["x"], x["x"], x["x"], x["wq"], x["wk"], x["wv"], x["wo"], 8, workspace=small)


# ---------------------------------------------------------------- key-padding masks (per-batch key lengths)
PADDED = [
    # (B, H, n_q, n_k, causal, dtype, lengths)
    (4, 2, 100, 130, False, "bf16", [130, 65, 0, 1]),
    (3, 2, 129, 129, True, "bf16", [129, 64, 200]),
    (2, 3, 2600, 2600, True, "bf16", [2600, 1000]),
    (2, 1, 2100, 2300, False, "bf16", [0, 2299]),
    # 64 query rows per wavefront (whole 256-row workgroups) under per-item lengths:
    # 0, below one slab, not a multiple of 64, full
    (4, 2, 512, 512, False, "bf16", [512, 300, 37, 0]),
    # the hand-scheduled loop over exactly one tile (150 and 129 keys: tile 1 is both its first and last
    # tile, a ragged tile follows for 150), and not at all (64 keys: only the first tile)
    (3, 2, 512, 512, False, "bf16", [150, 64, 129]),
    (1, 2, 4096, 4096, True, "bf16", [1000]),
    (2, 1, 4096, 4096, True, "bf16", [4096, 2100]),
    # the causal 32-row form under the same kind of lengths, 0 and below one slab included
    (2, 2, 2048, 2048, True, "bf16", [2048, 1000]),
    (3, 2, 300, 300, True, "bf16", [0, 5, 300]),
    # 800 causal 32-row workgroups overflow one round of 768 resident ones: the lightest level goes first
    (50, 8, 256, 256, True, "bf16", [256, 0, 37, 1, 200, 129, 64, 255] * 6 + [256, 100]),
    (3, 1, 768, 1000, False, "bf16", [1000, 63, 513]),
    (3, 2, 70, 90, False, "f32", [90, 33, 0]),
    (2, 2, 65, 65, True, "f32", [65, 7]),
]


@pytest.mark.parametrize("B,H,nq,nk,causal,dtype,lens", PADDED)
def test_padded_attention_parity(dev, B, H, nq, nk, causal, dtype, lens):
    import torch
    q = workloads.random_tensor((B, H, nq, 64), dtype, seed=500 + nq)
    k = workloads.random_tensor((B, H, nk, 64), dtype, seed=600 + nk)
    v = workloads.random_tensor((B, H, nk, 64), dtype, seed=700 + nk)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    say(f"padded {B}x{H} nq={nq} nk={nk} causal={causal} {dtype} lens={lens}")
    o, lse = mha.attention_forward(to_device(q, dev), to_device(k, dev), to_device(v, dev), causal=causal,
                                   kv_len=kv_len, return_lse=True)
    torch.cuda.synchronize()
    want, _, want_lse = oracle.attention_ref(q.value, k.value, v.value, causal=causal, kv_len=lens)
    assert_close(to_f64(o), want, dtype, "padded attention")
    got_lse = to_f64(lse)
    dead = np.isneginf(want_lse)
    assert np.array_equal(np.isneginf(got_lse), dead), "rows with no visible key must report lse = -inf"
    assert max_abs(got_lse[~dead], want_lse[~dead]) <= LSE_TOL[dtype], "log-sum-exp under padding"


@pytest.mark.parametrize("causal", [False, True])
def test_padded_keys_are_never_read(dev, causal):
    """Changing K and V past a batch item's length leaves the output bitwise unchanged."""
    import torch
    B, H, n = 2, 2, 300
    q, k, v = (to_device(workloads.random_tensor((B, H, n, 64), "bf16", seed=800 + i), dev) for i in range(3))
    kv_len = torch.tensor([300, 111], dtype=torch.int32, device=dev)
    say(f"padded keys never read, causal={causal}")
    a = mha.attention_forward(q, k, v, causal=causal, kv_len=kv_len)
    k2, v2 = k.clone(), v.clone()
    k2[1, :, 111:] = 30.0
    v2[1, :, 111:] = float("nan")
    b = mha.attention_forward(q, k2, v2, causal=causal, kv_len=kv_len)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_padded_mha_parity(dev, dtype):
    import torch
    B, nq, nk, dm, h = 3, 40, 75, 512 if dtype == "bf16" else 256, 8 if dtype == "bf16" else 4
    xq = workloads.random_tensor((B, nq, dm), dtype, seed=901)
    mem = workloads.random_tensor((B, nk, dm), dtype, seed=902)
    ws = [workloads.random_tensor((dm, dm), dtype, seed=903 + i, scale=1 / math.sqrt(dm)) for i in range(4)]
    tw = [to_device(s, dev) for s in ws]
    lens = [75, 20, 0]
    kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    say(f"padded mha cross {dtype}")
    out = mha.mha_forward(to_device(xq, dev), to_device(mem, dev), to_device(mem, dev), *tw, h, kv_len=kv_len)
    torch.cuda.synchronize()
    want = oracle.mha_ref(xq.value, mem.value, mem.value, *[s.value for s in ws], h, kv_len=lens)
    assert_close(to_f64(out), want, dtype, "padded mha cross")
    assert float(out[2].abs().max()) == 0.0, "an item with no visible key gives 0 W^O = 0"
    say(f"padded mha causal self {dtype}")
    xs = workloads.random_tensor((B, nk, dm), dtype, seed=910)
    t = to_device(xs, dev)
    out = mha.mha_forward(t, t, t, *tw, h, causal=True, kv_len=kv_len)
    torch.cuda.synchronize()
    want = oracle.mha_ref(xs.value, xs.value, xs.value, *[s.value for s in ws], h, causal=True, kv_len=lens)
    assert_close(to_f64(out), want, dtype, "padded mha causal")


# ---------------------------------------------------------------- encoder sub-layer (NEXT-2)
def _oracle_params(ps):
    m = {"ln1_gamma": "ln1_g", "ln1_beta": "ln1_b", "ln2_gamma": "ln2_g", "ln2_beta": "ln2_b"}
    return {m.get(k, k): v.value for k, v in ps.items()}


ENCODER_CASES = [
    # (B, N, d_model, heads, d_ff, dtype, causal, lens)
    (2, 100, 512, 8, 2048, "bf16", False, None),
    (2, 300, 512, 8, 2048, "bf16", True, None),
    (3, 130, 512, 8, 2048, "bf16", False, [130, 45, 0]),
    (2, 70, 256, 4, 512, "f32", False, [70, 21]),
    (1, 65, 128, 2, 256, "f32", True, None),
    # rows wider than 512 columns: the LayerNorm wavefront holds 2, 4 or 8 chunks per row.
    # The big model's width (1024, 16 heads of 64; "The Transformer" (hoshank.vercel.app),
    # "The Mathematics"), and fp32 widths with 128- and 16-wide heads, one with a partial chunk
    (2, 130, 1024, 16, 4096, "bf16", False, [130, 77]),
    (1, 70, 1024, 16, 1024, "bf16", True, None),
    (1, 40, 2048, 16, 512, "f32", False, None),
    (1, 33, 1040, 65, 256, "f32", True, None),
    (1, 24, 4096, 32, 256, "f32", False, [17]),
]


@pytest.mark.parametrize("B,N,dm,h,ff,dtype,causal,lens", ENCODER_CASES)
def test_encoder_layer_parity(dev, B, N, dm, h, ff, dtype, causal, lens):
    import torch
    x = workloads.random_tensor((B, N, dm), dtype, seed=1100 + N)
    ps = workloads.encoder_params(dm, ff, dtype, seed=1200 + dm)
    kv_len = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=dev)
    say(f"encoder layer {B}x{N} d={dm} h={h} ff={ff} {dtype} causal={causal} lens={lens}")
    out = mha.encoder_layer_forward(to_device(x, dev), {k: to_device(v, dev) for k, v in ps.items()}, h,
                                    causal=causal, kv_len=kv_len)
    torch.cuda.synchronize()
    want = oracle.encoder_layer_ref(x.value, _oracle_params(ps), h, causal=causal, kv_len=lens)
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    err = np.abs(got - want)
    bound = ENC_TOL[dtype][0] + ENC_TOL[dtype][1] * np.abs(want)
    say(f"encoder layer max-abs {err.max():.3e}, worst ratio to bound {float((err / bound).max()):.3f}")
    assert np.all(err <= bound), f"max-abs {err.max():.3e}"


def test_encoder_layer_workload_parity(dev):
    """The encoder-layer bench workload at full size (B = 32, N = 512, d_model 512,
    d_ff 2048, bf16), in the launch configuration the bench times."""
    import torch
    w = workloads.get("layer")
    x = workloads.make_inputs(w)
    params = {k: to_device(v, dev) for k, v in x.items() if k != "x"}
    say(f"encoder_layer_forward {w.name}")
    out = mha.encoder_layer_forward(to_device(x["x"], dev), params, w.heads)
    torch.cuda.synchronize()
    want = oracle.encoder_layer_ref(x["x"].value, _oracle_params({k: v for k, v in x.items() if k != "x"}), w.heads)
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    err = np.abs(got - want)
    bound = ENC_TOL["bf16"][0] + ENC_TOL["bf16"][1] * np.abs(want)
    say(f"{w.name}: max-abs {err.max():.3e}, worst ratio to bound {float((err / bound).max()):.3f}")
    assert np.all(err <= bound), f"max-abs {err.max():.3e}"


def test_padded_mha_workload_parity(dev):
    """The padded encoder bench workload at full size (B = 32, N = 512, per-item key
    lengths in [64, 512]), in the launch configuration the bench times."""
    import torch
    w = workloads.get("padded")
    x = workloads.make_inputs(w)
    t = {k_: to_device(s, dev) for k_, s in x.items()}
    lens = w.kv_lengths()
    kv_len = torch.from_numpy(lens).to(dev)
    say(f"mha_forward_padded {w.name}")
    out = mha.mha_forward(t["x"], t["x"], t["x"], t["wq"], t["wk"], t["wv"], t["wo"], w.heads, kv_len=kv_len)
    torch.cuda.synchronize()
    xv = x["x"].value
    want = oracle.mha_ref(xv, xv, xv, x["wq"].value, x["wk"].value, x["wv"].value, x["wo"].value, w.heads,
                          kv_len=lens)
    err = assert_close(to_f64(out), want, "bf16", w.name)
    say(f"{w.name}: max-abs {err:.3e}")
