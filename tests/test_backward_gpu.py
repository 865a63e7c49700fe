"""Attention backward: the HIP path vs the fp64 oracle (GPU).

Each case runs the library's own forward (attention_forward with
return_lse=True) for O and the log-sum-exp, draws a seeded dO, runs
attention_backward and compares dQ, dK, dV with oracle.attention_backward_ref
on the same stored q, k, v, dO. Bar (per gradient element):
|got - want| <= atol + rtol * E, E the absolute sum of the terms the element
adds up (the oracle's error_scale); see BWD_TOL in tests/gpu_util.py.
Shapes span several 64/128-row blocks with ragged tails, N_q != N_k, causal
and key-padding masks (lengths 0 and partial), strided (B, N, H, d) views and
every supported head width.
"""
import numpy as np
import pytest

import oracle
import transformer_scaled_dot_mha_amd as mha
import workloads
from tests.gpu_util import BWD_TOL, device, say, to_device, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _inputs(B, H, nq, nk, d, dtype, seed):
    q = workloads.random_tensor((B, H, nq, d), dtype, seed=seed)
    k = workloads.random_tensor((B, H, nk, d), dtype, seed=seed + 1)
    v = workloads.random_tensor((B, H, nk, d), dtype, seed=seed + 2)
    do = workloads.random_tensor((B, H, nq, d), dtype, seed=seed + 3)
    return q, k, v, do


def check_grads(got, want, dtype, what):
    """Each gradient element within atol + rtol * E, E its terms' absolute
    sum from the oracle (want = (dQ, dK, dV, (E_dQ, E_dK, E_dV)))."""
    atol, rtol = BWD_TOL[dtype]
    for name, g, w, e in zip(("dQ", "dK", "dV"), got, want[:3], want[3]):
        g = to_f64(g)
        assert np.all(np.isfinite(g)), f"{what}: non-finite {name}"
        excess = np.abs(g - w) - (atol + rtol * e)
        worst = np.unravel_index(np.argmax(excess), excess.shape)
        assert excess[worst] <= 0, (f"{what}: {name} off at {worst}: got {g[worst]:.5f}, want {w[worst]:.5f} "
                                    f"(|err| {abs(g[worst] - w[worst]):.3e}, term magnitude {e[worst]:.3f}, "
                                    f"bar atol {atol} + rtol {rtol} x magnitude)")


def run_backward(dev, q, k, v, do, *, causal=False, kv_len=None, scale=None, views=False):
    """Forward for O and lse, then the backward, through the C ABI."""
    import torch
    qd, kd, vd, dod = (to_device(t, dev) for t in (q, k, v, do))
    kvl = None if kv_len is None else torch.tensor(kv_len, dtype=torch.int32, device=dev)
    if views:
        # (B, N, H, d) storage seen as (B, H, N, d) through strides, outputs too
        qd, kd, vd, dod = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (qd, kd, vd, dod))
    o, lse = mha.attention_forward(qd, kd, vd, causal=causal, kv_len=kvl, scale=scale, return_lse=True)
    outs = {}
    if views:
        outs = {n: torch.empty(t.transpose(1, 2).shape, dtype=t.dtype, device=dev).transpose(1, 2)
                for n, t in (("dq", qd), ("dk", kd), ("dv", vd))}
    grads = mha.attention_backward(qd, kd, vd, o, dod, lse, causal=causal, kv_len=kvl, scale=scale, **outs)
    torch.cuda.synchronize()
    return grads


CASES = [
    # (B, H, n_q, n_k, d, dtype, causal, lens)
    (2, 2, 70, 90, 64, "f32", False, None),
    (2, 2, 100, 100, 64, "f32", True, None),
    (3, 2, 65, 65, 32, "f32", True, [65, 20, 0]),
    (2, 1, 40, 77, 16, "f32", False, [77, 5]),
    (2, 2, 50, 50, 128, "f32", True, None),
    (1, 3, 33, 140, 128, "f32", False, [100]),
    (2, 2, 70, 90, 64, "bf16", False, None),
    (2, 2, 200, 200, 64, "bf16", True, None),
    (3, 2, 129, 129, 64, "bf16", True, [129, 64, 0]),
    (2, 1, 300, 150, 64, "bf16", False, [150, 33]),
    (2, 1, 1, 1, 64, "bf16", True, None),
    (1, 2, 1000, 1000, 64, "bf16", True, None),
    (1, 2, 700, 2000, 64, "bf16", False, None),
]


@pytest.mark.parametrize("B,H,nq,nk,d,dtype,causal,lens", CASES)
def test_backward_parity(dev, B, H, nq, nk, d, dtype, causal, lens):
    q, k, v, do = _inputs(B, H, nq, nk, d, dtype, seed=3000 + nq + nk + d)
    say(f"backward {dtype} B={B} H={H} nq={nq} nk={nk} d={d} causal={causal} lens={lens}")
    got = run_backward(dev, q, k, v, do, causal=causal, kv_len=lens)
    want = oracle.attention_backward_ref(q.value, k.value, v.value, do.value, causal=causal, kv_len=lens,
                                          error_scale=True)
    check_grads(got, want, dtype, f"backward {dtype} {nq}x{nk} d={d} causal={causal} lens={lens}")
    if lens is not None:
        for b, L in enumerate(lens):
            assert float(got[1][b, :, L:].abs().max() if L < nk else 0.0) == 0.0, "padded keys: dK must be 0"
            assert float(got[2][b, :, L:].abs().max() if L < nk else 0.0) == 0.0, "padded keys: dV must be 0"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_strided_views(dev, dtype):
    B, H, n, d = 2, 3, 90, 64
    q, k, v, do = _inputs(B, H, n, n, d, dtype, seed=3100)
    say(f"backward strided views {dtype}")
    got = run_backward(dev, q, k, v, do, causal=True, views=True)
    want = oracle.attention_backward_ref(q.value, k.value, v.value, do.value, causal=True, error_scale=True)
    check_grads(got, want, dtype, "backward strided")


@pytest.mark.parametrize("dtype,scale", [("f32", -0.2), ("f32", 0.0), ("f32", 1.0), ("bf16", -0.2), ("bf16", 0.0),
                                         ("bf16", 0.4), ("bf16", 1.0)])
def test_backward_scale_values(dev, dtype, scale):
    B, H, n, d = 1, 2, 70, 64
    q, k, v, do = _inputs(B, H, n, n, d, dtype, seed=3200)
    say(f"backward scale {scale} {dtype}")
    got = run_backward(dev, q, k, v, do, causal=True, scale=scale)
    want = oracle.attention_backward_ref(q.value, k.value, v.value, do.value, causal=True, scale=scale,
                                         error_scale=True)
    check_grads(got, want, dtype, f"backward scale {scale}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_deterministic(dev, dtype):
    """No atomics: two runs give the same bits."""
    import torch
    q, k, v, do = _inputs(2, 2, 330, 330, 64, dtype, seed=3300)
    say(f"backward determinism {dtype}")
    a = run_backward(dev, q, k, v, do, causal=True)
    b = run_backward(dev, q, k, v, do, causal=True)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_backward_gradient_check_on_gpu(dev):
    """Directional derivative check through the library alone (fp32): the
    change of sum(dO * O) for a small step along a random direction of Q, K
    and V matches the gradients' inner product with that direction."""
    import torch
    B, H, n, d = 1, 2, 96, 64
    q, k, v, do = _inputs(B, H, n, n, d, "f32", seed=3400)
    qd, kd, vd, dod = (to_device(t, dev).double().float() for t in (q, k, v, do))
    say("backward directional derivative")
    o, lse = mha.attention_forward(qd, kd, vd, causal=True, return_lse=True)
    gq, gk, gv = mha.attention_backward(qd, kd, vd, o, dod, lse, causal=True)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    dirs = [torch.randn(t.shape, device=dev, generator=g) for t in (qd, kd, vd)]
    eps = 1e-3

    def loss(sign):
        oo = mha.attention_forward(*(t + sign * eps * u for t, u in zip((qd, kd, vd), dirs)), causal=True)
        return float((dod.double() * oo.double()).sum())
    fd = (loss(1.0) - loss(-1.0)) / (2 * eps)
    an = float(sum((gg.double() * u.double()).sum() for gg, u in zip((gq, gk, gv), dirs)))
    torch.cuda.synchronize()
    assert abs(fd - an) <= 1e-3 * max(1.0, abs(an)), f"directional derivative {fd} vs gradients {an}"


def test_backward_workload_parity(dev):
    """The timed backward workload (long causal, B=2, H=16, N=8192) at full size
    in the bench's launch configuration, against the oracle on 64 sampled query
    rows (dQ) and the same 64 key rows (dK, dV) of every (batch, head); the
    softmax statistics behind them cover all 8192 rows."""
    import torch
    w = workloads.get("bwd")
    x = workloads.make_inputs(w)
    q, k, v, do = (to_device(x[n], dev) for n in ("q", "k", "v", "do"))
    say(f"backward workload {w.name}")
    o, lse = mha.attention_forward(q, k, v, causal=True, return_lse=True)
    dq, dk, dv = mha.attention_backward(q, k, v, o, do, lse, causal=True)
    torch.cuda.synchronize()
    rows = workloads.sample_rows(w)
    want = oracle.attention_backward_sampled_ref(x["q"].value, x["k"].value, x["v"].value, x["do"].value, rows, rows,
                                                 causal=True, error_scale=True)
    idx = torch.from_numpy(rows).to(dev)
    got = tuple(t.index_select(2, idx) for t in (dq, dk, dv))
    check_grads(got, want, "bf16", "backward workload")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_padding_with_very_negative_scores(dev, dtype):
    """Every visible score near -128 (lse ~ -126): an unmasked weight of a
    padded key, exp(0 - lse), would overflow; padded keys must still get
    exactly zero gradients and everything else must stay finite."""
    import torch
    B, H, n, d, L = 1, 2, 96, 64, 10
    ones = np.ones((B, H, n, d))
    q = workloads.store(-ones, dtype)
    k = workloads.store(ones, dtype)
    v = workloads.random_tensor((B, H, n, d), dtype, seed=3500)
    do = workloads.random_tensor((B, H, n, d), dtype, seed=3501)
    say(f"backward very negative scores {dtype}")
    got = run_backward(dev, q, k, v, do, kv_len=[L], scale=2.0)
    want = oracle.attention_backward_ref(q.value, k.value, v.value, do.value, kv_len=[L], scale=2.0,
                                         error_scale=True)
    check_grads(got, want, dtype, "very negative scores")
    assert float(got[1][:, :, L:].abs().max()) == 0.0 and float(got[2][:, :, L:].abs().max()) == 0.0
