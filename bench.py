#!/usr/bin/env python3
"""Benchmark: multi-head attention forward on one MI355X (gfx950).

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch of synthetic input.
Default workload: the base-model encoder self-attention, bf16, batch 32,
N = 512, d_model = 512, h = 8, d_k = 64, no mask; a step is one mha_forward
(Q/K/V projections, attention, W^O). Attention-only workloads
(--workload decoder|cross|long) time one attention_forward per step;
--workload decode times one attention_decode (one query per (batch, head)
against a paged K/V cache), reported against the HBM roofline; --workload bwd
times one attention_backward of the long causal attention (FLOPs counted as
10*H*d per unmasked pair, 2.5x the forward's).

Prints ONE JSON line. `value` is algorithmic TFLOP/s of the step (FLOPs =
4*B*H*d*unmasked pairs for attention, 2*m*n*k per projection) with inputs
already resident in HBM; input and output buffers rotate over more than twice
the 256 MB Infinity Cache so each step reads its inputs from HBM.
`launches` lists every launch of the step (for the encoder step: the grouped
Q/K/V projection, the attention, W^O), each re-timed alone on its own rotating
inputs with HIP events on the stream it runs on; `roofline` belongs to the
longest of them. The other configurations (the tiny fp32 MHA, the decoder's
causal attention, cross-attention, the long causal attention) get a line each
(`tiny_mha`, `decoder_causal`, `cross_attention`, `long_causal`), timed the same
way. `cpu_baseline` times the fp64 CPU oracle on the host cores; `env` records
the ROCm and HIP versions and the device.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 vector
HBM_GBPS = 8000.0
ROTATE_BYTES = 512 << 20    # > 2x the 256 MB Infinity Cache
LEAD_SECONDS = 0.2          # back-to-back launches ahead of each timed pass
SCLK_PLAUSIBLE_MHZ = (500, 2400)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "attention": [os.path.join(ROOT, "transformer_scaled_dot_mha_amd", "csrc", "attn_bf16.hip"),
                  os.path.join(ROOT, "transformer_scaled_dot_mha_amd", "csrc", "attn_fwd_loop.inc")],
    "linear": os.path.join(ROOT, "transformer_scaled_dot_mha_amd", "csrc", "linear_bf16.hip"),
    "decode": os.path.join(ROOT, "transformer_scaled_dot_mha_amd", "csrc", "decode.hip"),
    "backward": os.path.join(ROOT, "transformer_scaled_dot_mha_amd", "csrc", "attn_bwd_bf16.hip"),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(path):
    """Hash of a kernel source's code (one file or a list of them): comments and
    blank lines do not count, so a comment edit keeps the recorded counters valid."""
    text = ""
    for p in ([path] if isinstance(path, str) else path):
        with open(p) as f:
            text += f.read() + "\n"
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def torch_tensor(stored, dev):
    import torch
    if stored.dtype == "bf16":
        t = torch.from_numpy(stored.raw.view(np.int16).copy()).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(stored.raw).copy())
    return t.to(dev)


def time_events(fn, iters, stream, per_step=None, lead_in=0, lead_seconds=0.0):
    """Average milliseconds per call, HIP events on `stream` around `iters` calls.

    Before the first event the stream is synchronised and then fed, without
    a host wait, `lead_in` calls, or as many as take `lead_seconds` on the GPU
    (from one call timed beforehand) if that is more: the timed calls continue
    a stream that is already running.
    (After a pause of a few milliseconds the clock dips for the next tens of
    launches -- the long causal launch went from 285 to 354 us and back -- so
    a timed pass that starts from an idle GPU would measure that transient.)
    per_step: optional list that receives each call's own duration (ms), from
    an event recorded after every call. Recording an event between launches
    leaves a gap of several microseconds on the stream, so a per-call pass is
    kept apart from the timed one (without per_step only the two bracketing
    events are recorded)."""
    import torch
    n_ev = iters + 1 if per_step is not None else 2
    events = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    if lead_seconds > 0:
        # size the lead-in from one call's duration (the host enqueues far faster
        # than the GPU runs, so a host-time bound would queue seconds of work)
        torch.cuda.synchronize()
        events[0].record(stream)
        fn(0)
        events[-1].record(stream)
        torch.cuda.synchronize()
        one_s = max(events[0].elapsed_time(events[-1]) * 1e-3, 1e-6)
        lead_in = max(lead_in, int(math.ceil(lead_seconds / one_s)))
    torch.cuda.synchronize()
    for j in range(lead_in):
        fn(j)
    j = lead_in
    events[0].record(stream)
    for i in range(iters):
        fn(j + i)
        if per_step is not None:
            events[i + 1].record(stream)
    if per_step is None:
        events[1].record(stream)
    torch.cuda.synchronize()
    if per_step is not None:
        per_step.extend(events[i].elapsed_time(events[i + 1]) for i in range(iters))
    return events[0].elapsed_time(events[-1]) / iters


def back_to_back(fn, seconds, start_hook=None):
    """Launch fn back to back (no synchronisation while launching) for about
    `seconds` of host time, then wait for the queue to drain. start_hook runs
    once the first launches are queued."""
    import torch
    for i in range(4):
        fn(i)
    torch.cuda.synchronize()
    t0, i = time.perf_counter(), 0
    while time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i == 16 and start_hook is not None:
            start_hook()
            start_hook = None
    if start_hook is not None:
        start_hook()
    torch.cuda.synchronize()


def sample_sclk(fn, stream, seconds=0.5):
    """Run fn back to back for `seconds` (a separate, untimed pass) and return
    the shader clock the GPU sustains meanwhile: amdsmi readings from a side
    thread. None where amdsmi cannot see this device."""
    import statistics
    import threading
    import torch
    handle, amdsmi = None, None
    try:
        import amdsmi
        props = torch.cuda.get_device_properties(0)
        want = (props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
        amdsmi.amdsmi_init()
        for h in amdsmi.amdsmi_get_processor_handles():
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)          # "dddd:bb:dd.f"
            dom, bus, rest = bdf.split(":")
            if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                handle = h
    except Exception:
        handle = None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                samples.append(amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.SYS)["clk"])
            except Exception:
                pass
            time.sleep(0.005)
    th = threading.Thread(target=poll) if handle is not None else None
    try:
        back_to_back(fn, seconds, th.start if th is not None else None)
    finally:
        if th is not None:
            stop.set()
            th.join()
        if amdsmi is not None:
            try:
                amdsmi.amdsmi_shut_down()
            except Exception:
                pass
    read = [x for x in samples if isinstance(x, (int, float))]
    # a busy MI355X runs between a few hundred MHz and its 2400 MHz maximum; a
    # reading outside that range is a misread of the sensor, not a clock
    busy = [x for x in read if SCLK_PLAUSIBLE_MHZ[0] <= x <= SCLK_PLAUSIBLE_MHZ[1]]
    if not busy:
        return None
    return {"median_mhz": statistics.median(busy), "min_mhz": min(busy), "max_mhz": max(busy),
            "samples": len(busy), "dropped_implausible": len(read) - len(busy),
            "how": "amdsmi SYS clock every ~5 ms while the step is launched back to back (separate untimed pass); "
                   f"readings outside {SCLK_PLAUSIBLE_MHZ[0]}-{SCLK_PLAUSIBLE_MHZ[1]} MHz dropped"}


def traffic_for(src_key, launch_desc):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    if that summary is missing or was taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(launch_desc)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != source_sha(KERNEL_SOURCES[src_key]):
        return None
    return rec.get("bytes_per_launch")


def linear_kernel_name(m, n, groups, dtype):
    """The projection kernel linear_forward(_grouped) runs for this shape: the
    bf16 tile kernel (every tile height), or the fp32 split-k form for grids
    of fewer than 256 64 x 64 tiles, else the fp32 tile kernel."""
    if dtype == "bf16":
        return "linear_bf16_kernel"
    return "linear_f32_splitk" if ((n + 63) // 64) * ((m + 63) // 64) * groups < 256 else "linear_f32_kernel"


def attention_kernel_name(n_q, causal, dtype):
    """The forward kernel attention_forward runs for this shape: the bf16 form
    with 64 query rows per wavefront or one with 32 (the library's
    attention_rows_per_wave rule; causal runs take the 32-row form with the
    LDS load ring), or the fp32 kernel."""
    if dtype != "bf16":
        return "attn_fwd_f32"
    pad = (n_q + 255) // 256 * 256 - n_q
    if (not causal and n_q >= 512 and pad == 0) or (n_q >= (4096 if causal else 2048) and pad * 16 <= n_q):
        return "attn_fwd_bf16_d64_r64"
    return "attn_fwd_bf16_d64_r32d" if causal else "attn_fwd_bf16_d64_r32"


def src_key_of(kernel):
    return ("linear" if kernel.startswith("linear") else "decode" if kernel.startswith("decode")
            else "backward" if kernel.startswith("attn_bwd") else "attention")


def cpu_baseline(w, inputs, min_seconds=10.0, max_seconds=30.0):
    """The fp64 oracle, untuned, on the host cores: repeat the sample until
    ~min_seconds of CPU work; report algorithmic TFLOP/s of what it computed."""
    import threadpoolctl
    import oracle
    info = threadpoolctl.threadpool_info()
    threads = max([d.get("num_threads", 1) for d in info if d.get("user_api") == "blas"] or [1])
    if w.kind == "bwd":
        # whole (batch, head) pairs at full length, one at a time, until ~min_seconds
        per_pair = 10 * w.d_k * (w.total_pairs() // w.batch)
        qv, kv, vv, dv = (inputs[n].value for n in ("q", "k", "v", "do"))
        done = []
        t0 = time.perf_counter()
        for b in range(w.batch):
            for h in range(w.heads):
                g = oracle.attention_backward_ref(qv[b:b + 1, h:h + 1], kv[b:b + 1, h:h + 1], vv[b:b + 1, h:h + 1],
                                                  dv[b:b + 1, h:h + 1], causal=w.causal)
                done.append(((b, h), g))
                el = time.perf_counter() - t0
                if el >= min_seconds or el + el / len(done) > max_seconds:
                    break
            else:
                continue
            break
        el = time.perf_counter() - t0
        return {"value": round(per_pair * len(done) / el / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
                "kind": "oracle",
                "sample": f"{len(done)} whole (batch, head) pair(s) of the workload at full length, "
                          f"oracle.attention_backward_ref in float64; {el:.1f} s",
                "host_cpus": os.cpu_count(),
                "blas": ",".join(sorted({d.get("internal_api", "?") for d in info}))}, done
    if w.kind == "decode":
        fn = lambda: oracle.decode_ref(inputs["q"].value, inputs["k"].value, inputs["v"].value, w.kv_lengths())
        flops = w.attention_flops()
        sample = (f"the full workload ({w.batch * w.heads} (batch, head) pairs against their cached keys), "
                  "oracle.decode_ref in float64 on the logical (unpaged) cache")
    elif w.kind == "layer":
        names = {"ln1_gamma": "ln1_g", "ln1_beta": "ln1_b", "ln2_gamma": "ln2_g", "ln2_beta": "ln2_b"}
        params = {names.get(k, k): v.value for k, v in inputs.items() if k != "x"}
        fn = lambda: oracle.encoder_layer_ref(inputs["x"].value, params, w.heads)
        flops = w.total_flops()
        sample = f"the full workload ({w.batch} batch elements), oracle.encoder_layer_ref in float64"
    elif w.kind == "mha":
        xv = inputs["x"].value
        args = (xv, xv, xv, inputs["wq"].value, inputs["wk"].value, inputs["wv"].value, inputs["wo"].value)
        fn = lambda: oracle.mha_ref(*args, w.heads, causal=w.causal, kv_len=w.kv_lengths())
        flops = w.total_flops()
        sample = f"the full workload ({w.batch} batch elements), oracle.mha_ref in float64"
    else:
        rows = workloads.sample_rows(w) if w.oracle_rows else None
        fn = lambda: oracle.attention_ref(inputs["q"].value, inputs["k"].value, inputs["v"].value,
                                          causal=w.causal, rows=rows)
        if rows is None:
            flops = w.attention_flops()
            sample = f"the full workload, oracle.attention_ref in float64"
        else:
            pairs = int(np.sum(rows + 1)) if w.causal else len(rows) * w.n_k
            flops = 4 * w.batch * w.heads * w.d_k * pairs
            sample = (f"{len(rows)} sampled query positions x {w.batch * w.heads} (batch, head) pairs, "
                      "each against all visible keys, oracle.attention_ref in float64")
    # three timed runs, each repeating the sample until a third of min_seconds has
    # passed (at least once); the median run's rate is reported
    rates, total_runs, t_all = [], 0, time.perf_counter()
    result = None
    for _ in range(3):
        runs, t0 = 0, time.perf_counter()
        while True:
            result = fn()
            runs += 1
            el = time.perf_counter() - t0
            if el >= min_seconds / 3 or time.perf_counter() - t_all + el / runs > max_seconds:
                break
        rates.append(flops * runs / el / 1e12)
        total_runs += runs
        if time.perf_counter() - t_all > max_seconds:
            break
    el_all = time.perf_counter() - t_all
    return {"value": round(float(np.median(rates)), 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{sample}; median of {len(rates)} timed run(s) ({total_runs} evaluations in {el_all:.1f} s)",
            "runs_tflops": [round(r, 6) for r in rates],
            "host_cpus": os.cpu_count(), "blas": ",".join(sorted({d.get("internal_api", "?") for d in info}))}, result


def env_info():
    """ROCm and HIP versions and the device, for the record."""
    import torch
    info = {"torch": torch.__version__, "torch_hip": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        info["rocm"] = None
    # the compiler that built libmha.so, as the build recorded it (no compiler is
    # run from this process: it has initialised the GPU)
    try:
        with open(os.path.join(ROOT, "transformer_scaled_dot_mha_amd", "libmha.build.json")) as f:
            out = "\n".join(json.load(f).get("hipcc_version", []))
        m = re.search(r"HIP version:\s*(\S+)", out)
        info["hipcc_hip_version"] = m.group(1) if m else None
        m = re.search(r"clang version\s*(\S+)", out)
        info["hipcc_clang"] = m.group(1) if m else None
    except (OSError, ValueError):
        info["hipcc_hip_version"] = None
    p = torch.cuda.get_device_properties(0)
    info["gpu"] = p.name
    info["arch"] = getattr(p, "gcnArchName", None)
    info["compute_units"] = p.multi_processor_count
    return info


def mha_step_launches(mha, w, x, ws, kv_len, lens, dev):
    """The three launches of one mha_forward step, each callable alone on its own
    rotating inputs (more than twice the Infinity Cache, so operands come from HBM):
    the grouped Q/K/V projection (linear_forward_grouped: the launch mha_forward
    makes), the attention over the head-split views, and W^O (linear_forward).
    Algorithmic bytes: each operand read once, each result written once."""
    import torch
    B, N, Nk, H, d, dm = w.batch, w.n_q, w.n_k, w.heads, w.d_k, w.d_model
    esz = x.element_size()
    rq, rk = B * N, B * Nk
    gen = torch.Generator(device=dev).manual_seed(77)
    rnd = lambda *shape: torch.randn(shape, device=dev, generator=gen).to(x.dtype)
    out = []

    # Q/K/V projection: X (shared by the three products of self-attention) and W^Q, W^K, W^V in; Q, K, V out
    per = (rq * dm + (rq + 2 * rk) * dm) * esz
    n_q = max(1, math.ceil(ROTATE_BYTES / per))
    qsets = [(x.view(rq, dm) if i == 0 else rnd(rq, dm),
              [torch.empty((r, dm), dtype=x.dtype, device=dev) for r in (rq, rk, rk)]) for i in range(n_q)]
    fq = lambda i: mha.linear_forward_grouped([qsets[i % n_q][0]] * 3, ws[:3], outs=qsets[i % n_q][1])
    out.append({"launch": "qkv_projection", "kernel": linear_kernel_name(max(rq, rk), dm, 3, w.dtype), "fn": fq,
                "flops": 2 * dm * dm * (rq + 2 * rk), "bytes": (rq * dm + 3 * dm * dm + (rq + 2 * rk) * dm) * esz,
                "sets": n_q})

    # attention over (B, N, H, d) buffers seen as (B, H, N, d): Q, K, V in (K, V over the visible keys), O out
    kv_rows = rk if lens is None else int(lens.astype(np.int64).sum())
    per = (2 * rq * dm + 2 * rk * dm) * esz
    n_a = max(1, math.ceil(ROTATE_BYTES / per))
    asets = [(rnd(B, N, H, d).transpose(1, 2), rnd(B, Nk, H, d).transpose(1, 2), rnd(B, Nk, H, d).transpose(1, 2),
              torch.empty((B, N, H, d), dtype=x.dtype, device=dev).transpose(1, 2)) for _ in range(n_a)]
    fa = lambda i: mha.attention_forward(*asets[i % n_a][:3], causal=w.causal, out=asets[i % n_a][3], kv_len=kv_len)
    out.append({"launch": "attention", "kernel": attention_kernel_name(N, w.causal, w.dtype),
                "fn": fa, "flops": w.attention_flops(), "bytes": (2 * rq * dm + 2 * H * kv_rows * d) * esz,
                "sets": n_a})

    # W^O: the concatenated heads (rq, dm) in, out (rq, dm)
    per = 2 * rq * dm * esz
    n_o = max(1, math.ceil(ROTATE_BYTES / per))
    osets = [(rnd(rq, dm), torch.empty((rq, dm), dtype=x.dtype, device=dev)) for _ in range(n_o)]
    fo = lambda i: mha.linear_forward(osets[i % n_o][0], ws[3], out=osets[i % n_o][1])
    out.append({"launch": "output_projection", "kernel": linear_kernel_name(rq, dm, 1, w.dtype), "fn": fo,
                "flops": 2 * rq * dm * dm, "bytes": (2 * rq * dm + dm * dm) * esz, "sets": n_o})
    return out


def time_secondary(mha, name, stream, dev, iters):
    """One of the other configurations, timed alone on rotating inputs: attention
    workloads run one attention_forward, the tiny fp32 one a whole mha_forward."""
    import torch
    w = workloads.get(name)
    x = workloads.make_inputs(w)
    if w.kind == "mha":
        t = {k: torch_tensor(v, dev) for k, v in x.items()}
        esz = t["x"].element_size()
        fn = lambda i: mha.mha_forward(t["x"], t["x"], t["x"], t["wq"], t["wk"], t["wv"], t["wo"], w.heads)
        flops, n_sets, kernel = w.total_flops(), 1, "mha_forward (3 launches)"
        nbytes = (2 * t["x"].numel() + 4 * w.d_model * w.d_model) * esz
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    else:
        q, k, v = (torch_tensor(x[n], dev) for n in ("q", "k", "v"))
        nbytes = (2 * q.numel() + k.numel() + v.numel()) * q.element_size()
        n_sets = max(1, math.ceil(ROTATE_BYTES / nbytes))
        sets = [(q, k, v)] + [(q.clone(), k.clone(), v.clone()) for _ in range(n_sets - 1)]
        outs = [torch.empty_like(q) for _ in range(n_sets)]
        fn = lambda i: mha.attention_forward(*sets[i % n_sets], causal=w.causal, out=outs[i % n_sets])
        flops, peak, kernel = w.attention_flops(), PEAK_BF16_TFLOPS, attention_kernel_name(w.n_q, w.causal, w.dtype)
    fn(0)
    torch.cuda.synchronize()
    ms = time_events(fn, iters, stream, lead_in=3, lead_seconds=LEAD_SECONDS)
    tf = flops / (ms * 1e-3) / 1e12
    gbps = nbytes / (ms * 1e-3) / 1e9
    rec = {"workload": w.name, "kernel": kernel, "us": round(ms * 1e3, 2), "tflops": round(tf, 2),
           "frac_of_peak": round(tf / peak, 4), "peak": peak, "algorithmic_bytes": nbytes, "gbps": round(gbps, 1),
           "frac_of_hbm": round(gbps / HBM_GBPS, 4), "rotating_sets": n_sets,
           "traffic": traffic_for("attention", f"attention:{w.name}") if w.kind == "attn" else None}
    log(f"{w.name}: {ms * 1e3:.1f} us, {tf:.1f} TFLOP/s ({100 * tf / peak:.1f} % of peak), {gbps:.0f} GB/s")
    return rec, fn, w


# the configurations besides the timed workload, each on one line of its own in the record
SECONDARY = {"tiny": "tiny_mha", "decoder": "decoder_causal", "cross": "cross_attention", "long": "long_causal"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="encoder",
                    help="encoder | tiny | decoder | cross | long | padded | layer | decode | bwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other configurations' lines")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding across GPUs is a design note, not an implemented path.", file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_scaled_dot_mha_amd as mha
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    mha.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    w = workloads.get(args.workload)
    log(f"workload {w.name}: generating seeded inputs")
    inputs = workloads.make_inputs(w)

    result = {}
    lens = w.kv_lengths()
    kv_len = None if lens is None else torch.from_numpy(lens).to(dev)
    # `launches`: the kernels of the step, each with a callable that runs it alone
    # (the step itself where the step is one launch or one fused pair of launches)
    if w.kind == "bwd":
        q, k, v, do = (torch_tensor(inputs[n], dev) for n in ("q", "k", "v", "do"))
        # the forward's output and log-sum-exp, saved once as training saves them
        o, lse = mha.attention_forward(q, k, v, causal=w.causal, return_lse=True)
        esz = q.element_size()
        per_set = 8 * q.numel() * esz
        n_sets = max(1, math.ceil(ROTATE_BYTES / per_set))
        sets = [(q, k, v, o, do)] + [tuple(t.clone() for t in (q, k, v, o, do)) for _ in range(n_sets - 1)]
        grads = [tuple(torch.empty_like(t) for t in (q, k, v)) for _ in range(n_sets)]
        work = torch.empty(mha.attention_backward_workspace_size(w.batch, w.heads, w.n_q), dtype=torch.uint8,
                           device=dev)

        def step(i):
            qi, ki, vi, oi, doi = sets[i % n_sets]
            dq, dk, dv = grads[i % n_sets]
            mha.attention_backward(qi, ki, vi, oi, doi, lse, causal=w.causal, dq=dq, dk=dk, dv=dv, workspace=work)

        step(0)
        torch.cuda.synchronize()
        flops_step = w.backward_flops()
        # the step is the backward itself: the dQ launch, then the dK/dV launch
        launches = [{"launch": "backward", "kernel": "attn_bwd_dq_bf16+attn_bwd_dkdv_bf16", "fn": step,
                     "flops": flops_step, "bytes": per_set, "sets": n_sets}]
        get_out = lambda: grads[0]
    elif w.kind == "decode":
        table_np, num_pages = w.pages()
        q = torch_tensor(inputs["q"], dev)
        # pages stored head-major, (num_pages, H, P, d), passed as a (pages, slots, H, d) view
        kp = torch_tensor(workloads.paged_pool(inputs["k"], table_np, lens, w.page_size, num_pages, "hnd"),
                          dev).transpose(1, 2)
        vp = torch_tensor(workloads.paged_pool(inputs["v"], table_np, lens, w.page_size, num_pages, "hnd"),
                          dev).transpose(1, 2)
        table = torch.from_numpy(table_np).to(dev)
        esz = q.element_size()
        pool_bytes = 2 * kp.numel() * esz
        n_sets = max(1, math.ceil(ROTATE_BYTES / pool_bytes))
        pools = [(kp, vp)] + [(kp.clone(memory_format=torch.preserve_format), vp.clone(memory_format=torch.preserve_format))
                              for _ in range(n_sets - 1)]
        outs = [torch.empty_like(q) for _ in range(n_sets)]
        need = mha.attention_decode_workspace_size(w.batch, w.heads, w.d_k, w.n_k)
        work = torch.empty(need, dtype=torch.uint8, device=dev)

        def step(i):
            ki, vi = pools[i % n_sets]
            mha.attention_decode(q, ki, vi, kv_len, block_table=table, out=outs[i % n_sets], workspace=work)

        step(0)
        torch.cuda.synchronize()
        flops_step = w.attention_flops()
        # the step is the decode itself: the split kernel and the merge of the splits;
        # algorithmic bytes: every visible cached key and value row, q in, o out
        launches = [{"launch": "decode", "kernel": "decode_split_kernel+decode_merge_kernel", "fn": step,
                     "flops": flops_step, "sets": n_sets,
                     "bytes": (2 * w.heads * int(lens.astype(np.int64).sum()) * w.d_k
                               + 2 * w.batch * w.heads * w.d_k) * esz}]
        get_out = lambda: outs[0]
    elif w.kind == "layer":
        dm, ff = w.d_model, w.d_ff
        x = torch_tensor(inputs["x"], dev)
        params = {k: torch_tensor(v, dev) for k, v in inputs.items() if k != "x"}
        per_set = x.numel() * x.element_size() * 2
        n_sets = max(1, math.ceil(ROTATE_BYTES / per_set))
        xs = [x] + [x.clone() for _ in range(n_sets - 1)]
        outs = [torch.empty_like(x) for _ in range(n_sets)]
        need = mha.encoder_layer_workspace_size(w.batch, w.n_q, dm, w.heads, ff, x.dtype)
        work = torch.empty(need, dtype=torch.uint8, device=dev)

        def step(i):
            mha.encoder_layer_forward(xs[i % n_sets], params, w.heads, kv_len=kv_len, out=outs[i % n_sets],
                                      workspace=work)

        step(0)
        torch.cuda.synchronize()
        flops_step = w.total_flops()
        # the FFN's first product (rows x d_model by d_model x d_ff, the longest launch of the
        # layer by the kernel trace), re-timed alone on rotating workspace-sized buffers
        rows = w.batch * w.n_q
        nf = max(1, math.ceil(ROTATE_BYTES / ((rows * dm + rows * ff) * x.element_size())))
        fsets = [(x.view(rows, dm).clone(), torch.empty((rows, ff), dtype=x.dtype, device=dev)) for _ in range(nf)]
        launches = [{"launch": "ffn_w1", "kernel": "linear_bf16_kernel", "sets": nf,
                     "fn": lambda i: mha.linear_forward(fsets[i % nf][0], params["w1"], out=fsets[i % nf][1]),
                     "flops": 2 * rows * dm * ff, "bytes": (rows * dm + dm * ff + rows * ff) * x.element_size()}]
        get_out = lambda: outs[0]
    elif w.kind == "mha":
        dm = w.d_model
        x = torch_tensor(inputs["x"], dev)
        ws = [torch_tensor(inputs[n], dev) for n in ("wq", "wk", "wv", "wo")]
        esz = x.element_size()
        per_set = x.numel() * esz * 2
        n_sets = max(1, math.ceil(ROTATE_BYTES / per_set))
        xs = [x] + [x.clone() for _ in range(n_sets - 1)]
        outs = [torch.empty_like(x) for _ in range(n_sets)]
        need = mha.mha_forward_workspace_size(w.batch, w.n_q, w.n_k, dm, w.heads, x.dtype)
        work = torch.empty(need, dtype=torch.uint8, device=dev)

        def step(i):
            xi = xs[i % n_sets]
            mha.mha_forward(xi, xi, xi, *ws, w.heads, causal=w.causal, out=outs[i % n_sets], workspace=work,
                            kv_len=kv_len)

        # parity on the exact launch configuration that is timed
        step(0)
        torch.cuda.synchronize()
        flops_step = w.total_flops()
        launches = mha_step_launches(mha, w, xs[0], ws, kv_len, lens, dev)
        get_out = lambda: outs[0]
    else:
        q, k, v = (torch_tensor(inputs[n], dev) for n in ("q", "k", "v"))
        per_set = (q.numel() + k.numel() + v.numel() + q.numel()) * q.element_size()
        n_sets = max(1, math.ceil(ROTATE_BYTES / per_set))
        sets = [(q, k, v)] + [(q.clone(), k.clone(), v.clone()) for _ in range(n_sets - 1)]
        outs = [torch.empty_like(q) for _ in range(n_sets)]

        def step(i):
            qi, ki, vi = sets[i % n_sets]
            mha.attention_forward(qi, ki, vi, causal=w.causal, out=outs[i % n_sets])

        step(0)
        torch.cuda.synchronize()
        flops_step = w.attention_flops()
        launches = [{"launch": "attention", "kernel": attention_kernel_name(w.n_q, w.causal, w.dtype),
                     "fn": step, "flops": flops_step, "bytes": per_set, "sets": n_sets}]
        get_out = lambda: outs[0]

    log(f"warmup {args.warmup}, timing {args.steps} steps ({n_sets} rotating input sets)")
    # single process on one GPU: the barrier is the device synchronisation itself.
    # The W warm-up steps close a 0.2 s lead-in of back-to-back steps, and the
    # timed steps follow them on the running stream.
    ms = time_events(step, args.steps, stream, lead_in=args.warmup, lead_seconds=LEAD_SECONDS)
    # per-step statistics from a second, untimed pass with an event after every step
    step_ms = []
    time_events(step, args.steps, stream, per_step=step_ms, lead_in=args.warmup, lead_seconds=LEAD_SECONDS)
    value = flops_step / (ms * 1e-3) / 1e12
    log(f"step {ms * 1e3:.1f} us, {value:.1f} TFLOP/s")
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS

    # each launch of the step: its own average duration (HIP events on the launch
    # stream around back-to-back launches); where the step is that launch, the step's
    per_launch = []
    for L in launches:
        L_ms = ms if L["fn"] is step else time_events(L["fn"], max(args.steps, 20), stream, lead_in=3,
                                                      lead_seconds=LEAD_SECONDS)
        tf = L["flops"] / (L_ms * 1e-3) / 1e12
        gbps = L["bytes"] / (L_ms * 1e-3) / 1e9
        traffic = traffic_for(src_key_of(L["kernel"]), f"{L['launch']}:{w.name}")
        rec = {"launch": L["launch"], "kernel": L["kernel"], "avg_launch_us": round(L_ms * 1e3, 2),
               "tflops": round(tf, 2), "frac_of_peak": round(tf / peak, 4), "algorithmic_bytes": L["bytes"],
               "gbps": round(gbps, 1), "traffic": traffic,
               "traffic_over_algorithmic": None if traffic is None else round(traffic / L["bytes"], 3),
               "rotating_sets": L["sets"]}
        per_launch.append(rec)
        log(f"launch {L['launch']} ({L['kernel']}): {L_ms * 1e3:.1f} us, {tf:.1f} TFLOP/s, {gbps:.0f} GB/s")

    # the roofline belongs to the launch that takes longest
    dom = max(per_launch, key=lambda r: r["avg_launch_us"])
    if w.kind == "decode":
        # one query row: 2 flops per byte-pair of K/V, far below the MFMA ridge -- HBM-bound
        roofline = {"bound": "hbm", "launch": dom["launch"], "kernel": dom["kernel"], "achieved": dom["gbps"],
                    "peak": HBM_GBPS, "unit": "GB/s", "frac": round(dom["gbps"] / HBM_GBPS, 4),
                    "traffic": dom["traffic"], "algorithmic_bytes": dom["algorithmic_bytes"],
                    "avg_launch_us": dom["avg_launch_us"], "achieved_tflops": dom["tflops"]}
    else:
        roofline = {"bound": "mfma", "launch": dom["launch"], "kernel": dom["kernel"], "achieved": dom["tflops"],
                    "peak": peak, "unit": "TFLOP/s", "frac": dom["frac_of_peak"], "traffic": dom["traffic"],
                    "algorithmic_bytes": dom["algorithmic_bytes"], "avg_launch_us": dom["avg_launch_us"],
                    "achieved_gbps": dom["gbps"]}
        if w.kind == "bwd":
            # the two launches recompute S and dP to avoid atomics: 7 products per pair, 5 counted
            roofline["executed_tflops"] = round(dom["tflops"] * 14 / 10, 2)
            roofline["launches_per_step"] = 2
    log(f"dominant launch {dom['launch']} ({dom['kernel']}): {dom['avg_launch_us']} us, frac {roofline['frac']}")

    secondary = {}
    if not args.no_secondary:
        for name, key in SECONDARY.items():
            if workloads.get(name).name == w.name:
                continue
            rec, fn, wl = time_secondary(mha, name, stream, dev, 20)
            if name == "long":
                rec["sclk"] = sample_sclk(fn, stream)
            secondary[key] = rec
            torch.cuda.synchronize()
            torch.cuda.empty_cache()

    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy: 3 x 256 MiB")

    sclk = sample_sclk(step, stream)
    if sclk:
        log(f"sustained shader clock: median {sclk['median_mhz']} MHz over {sclk['samples']} samples")

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host cores")
        cpu, ref = cpu_baseline(w, inputs)
        if w.kind == "bwd":
            outs = [t.float().cpu().numpy().astype(np.float64) for t in get_out()]
            err = max(float(np.max(np.abs(outs[i][b, h] - g[i][0, 0]))) for (b, h), g in ref for i in range(3))
        else:
            got = get_out().float().cpu().numpy().astype(np.float64)
            if w.kind == "attn" and w.oracle_rows:
                got = got[:, :, workloads.sample_rows(w)]
            ref_o = ref if w.kind in ("mha", "layer") else ref[0]
            err = float(np.max(np.abs(got - ref_o)))
        result["parity_max_abs"] = err
        log(f"parity vs oracle: max-abs {err:.3e}")

    cfg = {"workload": w.name, "batch": w.batch, "seq_len_q": w.n_q, "seq_len_k": w.n_k, "heads": w.heads,
           "d_k": w.d_k, "causal": w.causal,
           "step": {"mha": "mha_forward: QKV projections + attention + W^O",
                    "layer": "encoder_layer_forward: attention sub-layer + residual LayerNorm + FFN + residual "
                             "LayerNorm",
                    "decode": "attention_decode: one query per (batch, head) against the paged K/V cache "
                              "(two launches: the key splits, then their merge)",
                    "bwd": "attention_backward: dQ, dK, dV of causal attention for a given dO, from the "
                           "forward's saved O and log-sum-exp (two launches: dQ, then dK/dV)",
                    }.get(w.kind, "attention_forward")}
    if w.kind in ("mha", "layer"):
        cfg["d_model"] = w.d_model
    if w.kind == "layer":
        cfg["d_ff"] = w.d_ff
    if w.kind == "decode":
        cfg["page_size"] = w.page_size
        cfg["cache_capacity"] = w.n_k
    if lens is not None:
        cfg["kv_len"] = (f"per-batch key lengths uniform in [{w.kv_len_range[0]}, {w.kv_len_range[1]}] "
                         f"(seeded; mean {float(lens.mean()):.1f})")
    metric = "attention fwd TFLOP/s and % of bf16 MFMA peak at 1 GPU (h=8, d_k=64)"
    if w.kind == "bwd":
        metric = "attention bwd TFLOP/s (10*H*d per unmasked pair) and % of bf16 MFMA peak at 1 GPU"
    line = {"metric": metric,
            "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": w.dtype, "data": "synthetic", "config": cfg,
            "pct_of_peak": round(100 * value / peak, 2), "roofline": roofline, "cpu_baseline": cpu,
            "launches": per_launch,
            "step_ms_median": round(float(np.median(step_ms)), 5), "step_ms_min": round(float(np.min(step_ms)), 5),
            "sclk": sclk}
    line.update(secondary)
    line.update(result)
    line["env"] = env_info()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
