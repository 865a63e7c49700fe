"""Helpers shared by the GPU tests: device copies of stored inputs, comparisons."""
from __future__ import annotations

import math
import sys

import numpy as np

# Tolerances: max-abs error against the fp64 oracle on unit-variance inputs.
TOL = {"f32": 1e-4, "bf16": 2e-2}
ROWSUM_TOL = 1e-3
# The bf16 kernel sums the bf16-rounded weights it multiplies V with, so the
# applied weights sum to 1 to fp32 rounding. Each weight's rounding is at most
# 2^-8 relative (8-bit significand, half an ulp), so the kernel's normaliser,
# and with it the exported log-sum-exp, can differ from the exact one by at
# most log(1 + 2^-8), plus fp32 noise.
LSE_TOL = {"bf16": math.log1p(2.0 ** -8) + 1e-5, "f32": 1e-5}
# Encoder layer (LayerNorm outputs, magnitudes up to ~5): |got - ref| <= atol + rtol * |ref|.
# bf16: the attention bar (2e-2) for the mixing arithmetic, plus 2^-7 relative:
# the output's own rounding (half an ulp, 2^-9 relative) and the rounding of the
# stored h carried through the second residual (another 2^-9 relative after
# the norm), with a factor 2 of margin. fp32: the attention bar.
ENC_TOL = {"bf16": (2e-2, 2.0 ** -7), "f32": (1e-4, 0.0)}
# Attention backward: |got - want| <= atol + rtol * E per gradient element,
# with E the sum of the absolute values of the terms that element adds up
# (oracle error_scale): rounding a term leaves an error proportional to the
# term, not to the (possibly cancelling) sum. bf16: the lse the forward hands
# over is within 2^-8 relative in its weights, P and dS are rounded to bf16
# (2^-9) and so is the result (2^-9 <= 2^-9 E): 2^-7, times 2 for margin.
# fp32: fp32 accumulation over up to a few thousand terms (2^-14 of E).
BWD_TOL = {"f32": (1e-5, 2.0 ** -14), "bf16": (2e-3, 2.0 ** -6)}


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash still shows it."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def device():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda:0")


def to_device(stored, dev):
    import torch
    if stored.dtype == "bf16":
        t = torch.from_numpy(stored.raw.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(stored.raw, dtype=np.float32).copy())
    return t.to(dev)


def to_f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def assert_close(got, want, dtype: str, what: str = "") -> float:
    err = max_abs(got, want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= TOL[dtype], f"{what}: max-abs error {err:.3e} > {TOL[dtype]:.0e}"
    return err
