"""mha_forward_noalloc against mha_forward (GPU), through the C ABI.

Named to be collected last: a failure here cannot hide the other GPU tests.

The allocation-free entry point runs mha_forward's launches on the library's
fixed per-GPU array instead of a caller workspace, so its output must equal
mha_forward's bit for bit. Two calls in a row, the second on a smaller
problem (the array keeps the first call's contents), and the first repeated
after it.
"""
import math

import numpy as np
import pytest

import oracle
import transformer_scaled_dot_mha_amd as mha
import workloads
from tests.gpu_util import TOL, assert_close, device, say, to_device, to_f64

pytestmark = pytest.mark.gpu


def _case(B, N, dm, seed, dtype="bf16"):
    x = workloads.random_tensor((B, N, dm), dtype, seed=seed)
    ws = [workloads.random_tensor((dm, dm), dtype, seed=seed + 1 + i, scale=1 / math.sqrt(dm)) for i in range(4)]
    return x, ws


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_mha_forward(causal):
    import torch
    dev = device()
    cases = [(32, 512, 512, 8, 1401), (3, 77, 512, 8, 1411), (32, 512, 512, 8, 1401)]
    for B, N, dm, h, seed in cases:
        x, ws = _case(B, N, dm, seed)
        t = to_device(x, dev)
        tw = [to_device(s, dev) for s in ws]
        say(f"mha_forward_noalloc {B}x{N} d_model={dm} h={h} causal={causal}")
        out_na = torch.full((B, N, dm), float("nan"), dtype=t.dtype, device=dev)
        mha.mha_forward_noalloc(t, t, t, *tw, h, causal=causal, out=out_na)
        want = mha.mha_forward(t, t, t, *tw, h, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(out_na, want), f"noalloc differs from mha_forward at {B}x{N}"
        if B * N <= 512:
            ref = oracle.mha_ref(x.value, x.value, x.value, *[s.value for s in ws], h, causal=causal)
            assert_close(to_f64(out_na), ref, "bf16", "noalloc vs oracle")


def test_noalloc_f32_and_cross():
    import torch
    dev = device()
    B, nq, nk, dm, h = 2, 50, 90, 256, 4
    xq = workloads.random_tensor((B, nq, dm), "f32", seed=1501)
    mem = workloads.random_tensor((B, nk, dm), "f32", seed=1502)
    ws = [workloads.random_tensor((dm, dm), "f32", seed=1503 + i, scale=1 / math.sqrt(dm)) for i in range(4)]
    tq, tm = to_device(xq, dev), to_device(mem, dev)
    tw = [to_device(s, dev) for s in ws]
    say("mha_forward_noalloc f32 cross")
    a = mha.mha_forward_noalloc(tq, tm, tm, *tw, h)
    b = mha.mha_forward(tq, tm, tm, *tw, h)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    ref = oracle.mha_ref(xq.value, mem.value, mem.value, *[s.value for s in ws], h)
    assert_close(to_f64(a), ref, "f32", "noalloc f32 cross")


def test_noalloc_rejects_oversized_problem():
    import torch
    dev = device()
    dm = 512
    x = torch.zeros((80, 512, dm), dtype=torch.bfloat16, device=dev)
    w = torch.zeros((dm, dm), dtype=torch.bfloat16, device=dev)
    with pytest.raises(mha.MHAError, match="MHA_ERR_UNSUPPORTED"):
        mha.mha_forward_noalloc(x, x, x, w, w, w, w, 8)
