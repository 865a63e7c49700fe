"""Decoding against a K/V cache: the HIP path vs the fp64 oracle (GPU).

One query row per (batch, head) against the first kv_len[b] cached keys, with
the cache contiguous (both (B, N, H, d) and (B, H, N, d) layouts, passed by
strides) or paged through a shuffled page table. Bars: the attention bars,
max-abs 1e-4 (fp32) / 2e-2 (bf16) on unit-variance inputs, and the
log-sum-exp within 1e-5. Lengths cover 0, 1, split edges (256, 257, 512),
ragged tails and caches of up to 79 splits; the paged cases use page sizes
that do and do not divide the 256-key split.
"""
import numpy as np
import pytest

import oracle
import transformer_scaled_dot_mha_amd as mha
import workloads
from tests.gpu_util import assert_close, device, max_abs, say, to_device, to_f64

pytestmark = pytest.mark.gpu

# bf16 decode keeps the weights in fp32 (no rounding before the weighted sum):
# the log-sum-exp differs from the exact one by fp32 noise only
DEC_LSE_TOL = {"bf16": 1e-5, "f32": 1e-5}


@pytest.fixture(scope="module")
def dev():
    return device()


def _inputs(B, H, d, n, dtype, seed):
    q = workloads.random_tensor((B, H, d), dtype, seed=seed)
    k = workloads.random_tensor((B, H, n, d), dtype, seed=seed + 1)
    v = workloads.random_tensor((B, H, n, d), dtype, seed=seed + 2)
    return q, k, v


def _check(o, lse, q, k, v, lens, dtype, what):
    want, want_lse = oracle.decode_ref(q.value, k.value, v.value, lens)
    got = to_f64(o)
    assert_close(got, want, dtype, what)
    got_lse = to_f64(lse)
    dead = np.isneginf(want_lse)
    assert np.array_equal(np.isneginf(got_lse), dead), f"{what}: empty caches must report lse = -inf"
    assert np.all(got[dead] == 0.0), f"{what}: empty caches must give o = 0"
    if np.any(~dead):
        assert max_abs(got_lse[~dead], want_lse[~dead]) <= DEC_LSE_TOL[dtype], f"{what}: log-sum-exp"


CONTIGUOUS = [
    # (B, H, d, max_len, dtype, lengths, layout)
    (3, 4, 64, 700, "bf16", [1, 300, 700], "bnhd"),
    (3, 4, 64, 700, "bf16", [0, 257, 512], "bhnd"),
    (2, 2, 128, 1030, "bf16", [1030, 255], "bnhd"),
    (2, 3, 16, 300, "bf16", [256, 299], "bhnd"),
    (2, 3, 32, 300, "bf16", [17, 300], "bnhd"),
    (3, 2, 64, 513, "f32", [513, 256, 0], "bnhd"),
    (2, 2, 128, 600, "f32", [600, 1], "bhnd"),
    (2, 2, 16, 90, "f32", [90, 45], "bnhd"),
    (2, 2, 32, 90, "f32", [3, 90], "bhnd"),
    # more than 16 and more than 64 splits of 256 keys (the merge's later rounds)
    (3, 2, 64, 20000, "bf16", [20000, 4200, 16385], "bhnd"),
    (2, 1, 128, 17000, "f32", [17000, 5000], "bnhd"),
]


@pytest.mark.parametrize("B,H,d,n,dtype,lens,layout", CONTIGUOUS)
def test_decode_contiguous_parity(dev, B, H, d, n, dtype, lens, layout):
    import torch
    q, k, v = _inputs(B, H, d, n, dtype, seed=900 + n + d)
    qd, kd, vd = (to_device(t, dev) for t in (q, k, v))
    if layout == "bnhd":   # (B, N, H, d) storage, contiguous
        kc, vc = kd.transpose(1, 2).contiguous(), vd.transpose(1, 2).contiguous()
    else:                  # (B, H, N, d) storage, seen as (B, N, H, d) through strides
        kc, vc = kd.transpose(1, 2), vd.transpose(1, 2)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    say(f"decode contiguous {layout} B={B} H={H} d={d} max_len={n} {dtype} lens={lens}")
    o, lse = mha.attention_decode(qd, kc, vc, kv_len, return_lse=True)
    torch.cuda.synchronize()
    _check(o, lse, q, k, v, lens, dtype, f"decode {layout}")


PAGED = [
    # (B, H, d, page_size, max_pages, dtype, lengths, spare pages, page layout)
    (4, 2, 64, 16, 40, "bf16", [640, 1, 0, 333], 3, "nhd"),
    (4, 2, 64, 16, 40, "bf16", [640, 1, 0, 333], 3, "hnd"),
    (3, 4, 128, 32, 20, "bf16", [640, 257, 100], 0, "nhd"),
    (3, 2, 64, 7, 100, "bf16", [700, 256, 13], 5, "hnd"),
    (2, 2, 64, 300, 3, "f32", [900, 301], 1, "nhd"),
    (3, 2, 32, 16, 20, "f32", [320, 17, 0], 2, "hnd"),
]


def _paged(q, k, v, lens, page_size, max_pages, spare, seed, dev, layout="nhd"):
    """Pools as (pages, slots, H, d) views: "nhd" storage as is, "hnd" storage
    (pages, H, slots, d) through a transposed view."""
    import torch
    table, num_pages = workloads.page_table(lens, page_size, max_pages, seed=seed, spare=spare)
    kp = to_device(workloads.paged_pool(k, table, lens, page_size, num_pages, layout), dev)
    vp = to_device(workloads.paged_pool(v, table, lens, page_size, num_pages, layout), dev)
    if layout == "hnd":
        kp, vp = kp.transpose(1, 2), vp.transpose(1, 2)
    return kp, vp, torch.from_numpy(table).to(dev), table


@pytest.mark.parametrize("B,H,d,P,max_pages,dtype,lens,spare,layout", PAGED)
def test_decode_paged_parity(dev, B, H, d, P, max_pages, dtype, lens, spare, layout):
    import torch
    n = P * max_pages
    q, k, v = _inputs(B, H, d, n, dtype, seed=1000 + P + d)
    kp, vp, table, _ = _paged(q, k, v, lens, P, max_pages, spare, seed=77 + P, dev=dev, layout=layout)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    say(f"decode paged {layout} B={B} H={H} d={d} page={P} pages={max_pages} {dtype} lens={lens}")
    o, lse = mha.attention_decode(to_device(q, dev), kp, vp, kv_len, block_table=table, return_lse=True)
    torch.cuda.synchronize()
    _check(o, lse, q, k, v, lens, dtype, "decode paged")


def test_decode_paged_equals_contiguous(dev):
    """The same cache, contiguous and paged in a shuffled order, gives the same bits."""
    import torch
    B, H, d, P, max_pages = 3, 8, 64, 16, 64
    lens = [1024, 555, 16]
    q, k, v = _inputs(B, H, d, P * max_pages, "bf16", seed=1200)
    kp, vp, table, _ = _paged(q, k, v, lens, P, max_pages, 0, seed=5, dev=dev)
    qd = to_device(q, dev)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    say("decode paged == contiguous")
    a = mha.attention_decode(qd, to_device(k, dev).transpose(1, 2), to_device(v, dev).transpose(1, 2), kv_len)
    b = mha.attention_decode(qd, kp, vp, kv_len, block_table=table)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_unread_cache_is_never_read(dev):
    """Slots at or past kv_len[b] and table entries past a sequence's pages are
    never read: NaN there and a wild table entry leave the output unchanged."""
    import torch
    B, H, d, P, max_pages = 2, 2, 64, 16, 32
    lens = [300, 40]
    q, k, v = _inputs(B, H, d, P * max_pages, "bf16", seed=1300)
    kp, vp, table, table_np = _paged(q, k, v, lens, P, max_pages, 0, seed=9, dev=dev)
    qd = to_device(q, dev)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    say("decode unread slots")
    a = mha.attention_decode(qd, kp, vp, kv_len, block_table=table)
    # the last page of sequence 1 holds keys 32..47; keys 40..47 are past its length
    last = int(table_np[1, 2])
    kp2, vp2 = kp.clone(), vp.clone()
    kp2[last, 8:] = float("nan")
    vp2[last, 8:] = float("nan")
    t2 = table.clone()
    t2[1, 3:] = 10 ** 9           # entries past the owned pages: never read
    b = mha.attention_decode(qd, kp2, vp2, kv_len, block_table=t2)
    # the contiguous layout: NaN past the length
    kc = to_device(k, dev).transpose(1, 2).contiguous()
    vc = to_device(v, dev).transpose(1, 2).contiguous()
    c1 = mha.attention_decode(qd, kc, vc, kv_len)
    kc[0, 300:] = float("nan")
    vc[1, 40:] = float("nan")
    c2 = mha.attention_decode(qd, kc, vc, kv_len)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(c1, c2)


def test_decode_bad_page_entry_gives_nan(dev):
    """A table entry outside [0, num_pages) for a needed page is not followed:
    that sequence reports NaN (every head), the others are unaffected."""
    import torch
    B, H, d, P, max_pages = 3, 2, 64, 16, 32
    lens = [500, 200, 64]
    q, k, v = _inputs(B, H, d, P * max_pages, "bf16", seed=1400)
    kp, vp, table, _ = _paged(q, k, v, lens, P, max_pages, 0, seed=11, dev=dev)
    qd = to_device(q, dev)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    good = mha.attention_decode(qd, kp, vp, kv_len, block_table=table)
    t2 = table.clone()
    t2[0, 20] = kp.shape[0]        # one past the pool
    t2[2, 0] = -3
    say("decode bad page entries")
    o, lse = mha.attention_decode(qd, kp, vp, kv_len, block_table=t2, return_lse=True)
    torch.cuda.synchronize()
    assert torch.isnan(o[0]).all() and torch.isnan(lse[0]).all()
    assert torch.isnan(o[2]).all() and torch.isnan(lse[2]).all()
    assert torch.equal(o[1], good[1])


@pytest.mark.parametrize("scale", [0.0, -0.2, 1.5])
def test_decode_scale_values(dev, scale):
    import torch
    B, H, d, n = 2, 2, 64, 600
    lens = [600, 333]
    q, k, v = _inputs(B, H, d, n, "f32", seed=1500)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
    say(f"decode scale {scale}")
    o = mha.attention_decode(to_device(q, dev), to_device(k, dev).transpose(1, 2), to_device(v, dev).transpose(1, 2),
                             kv_len, scale=scale)
    torch.cuda.synchronize()
    want, _ = oracle.decode_ref(q.value, k.value, v.value, lens, scale=scale)
    assert_close(to_f64(o), want, "f32", f"decode scale {scale}")


def test_decode_workload_parity(dev):
    """The timed workload at full size, in the launch configuration the bench
    uses, against the oracle on every (batch, head)."""
    import torch
    w = workloads.get("decode")
    x = workloads.make_inputs(w)
    lens = w.kv_lengths()
    table_np, num_pages = w.pages()
    kp = to_device(workloads.paged_pool(x["k"], table_np, lens, w.page_size, num_pages, "hnd"), dev).transpose(1, 2)
    vp = to_device(workloads.paged_pool(x["v"], table_np, lens, w.page_size, num_pages, "hnd"), dev).transpose(1, 2)
    say(f"decode workload {w.name}")
    o, lse = mha.attention_decode(to_device(x["q"], dev), kp, vp, torch.from_numpy(lens).to(dev),
                                  block_table=torch.from_numpy(table_np).to(dev), return_lse=True)
    torch.cuda.synchronize()
    _check(o, lse, x["q"], x["k"], x["v"], lens, w.dtype, "decode workload")


def _first(t, B):
    """The first B batch items of a stored tensor."""
    return workloads.Stored(t.value[:B], t.dtype, t.raw[:B])


def test_decode_workspace_reuse(dev):
    """One workspace serves many calls in a row with changing lengths and
    shapes (its contents from one call never leak into the next)."""
    import torch
    B, H, d, n = 4, 3, 64, 3000
    q, k, v = _inputs(B, H, d, n, "bf16", seed=1600)
    qd, kc, vc = to_device(q, dev), to_device(k, dev).transpose(1, 2), to_device(v, dev).transpose(1, 2)
    ws = torch.full((mha.attention_decode_workspace_size(B, H, d, n),), 0x7F, dtype=torch.uint8, device=dev)
    for i, lens in enumerate(([3000, 257, 1, 700], [2999, 2048, 0, 256], [513, 3000, 3000, 12], [1, 1, 1, 1])):
        say(f"decode workspace reuse, call {i}: lens={lens}")
        kv_len = torch.tensor(lens, dtype=torch.int32, device=dev)
        o, lse = mha.attention_decode(qd, kc, vc, kv_len, workspace=ws, return_lse=True)
        torch.cuda.synchronize()
        _check(o, lse, q, k, v, lens, "bf16", f"workspace reuse call {i}")
    # a smaller problem on the same (larger) workspace
    kv_len = torch.tensor([600, 40], dtype=torch.int32, device=dev)
    o, lse = mha.attention_decode(qd[:2].contiguous(), kc[:2], vc[:2], kv_len, workspace=ws, return_lse=True)
    torch.cuda.synchronize()
    _check(o, lse, _first(q, 2), _first(k, 2), _first(v, 2), [600, 40], "bf16", "smaller call")
