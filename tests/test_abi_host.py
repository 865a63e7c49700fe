"""The C ABI on the host: symbols, validation and bookkeeping (no GPU needed).

Every validation path returns before the library makes any HIP call, so these
tests pass fake, aligned, non-null addresses; nothing is ever dereferenced.
"""
import ctypes
import os
import re
import subprocess
import threading

import pytest

from transformer_scaled_dot_mha_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mha.h")

FAKE = 0x10000          # aligned, non-null; never dereferenced on these paths
MIS = 0x10002           # misaligned
S_BHND = (8 * 64 * 64, 64 * 64, 64)   # contiguous (B, H, N=64, d=64) strides


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_boundary():
    fns = header_functions()
    assert {"attention_forward", "attention_forward_padded", "mha_forward", "mha_forward_padded",
            "mha_forward_workspace_size", "mha_forward_noalloc", "linear_forward", "linear_forward_grouped", "encoder_layer_workspace_size",
            "encoder_layer_forward", "attention_decode_workspace_size", "attention_decode",
            "attention_backward_workspace_size", "attention_backward",
            "mha_status_string", "mha_last_error", "mha_version"} == set(fns)
    assert set(fns) == set(_lib.SIGNATURES), "binding signatures out of sync with include/mha.h"


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert set(header_functions()) <= exported


def test_status_strings_and_version(lib):
    assert lib.mha_status_string(0) == b"MHA_OK"
    assert lib.mha_status_string(3) == b"MHA_ERR_WORKSPACE"
    assert lib.mha_status_string(99) == b"MHA_ERR_UNKNOWN"
    assert lib.mha_version() >= 100


def attn(lib, q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=2, H=8, nq=64, nk=64, dk=64, dv=64, qs=S_BHND, ks=S_BHND,
         vs=S_BHND, os_=S_BHND, dtype=_lib.MHA_BF16, causal=0, scale=0.125, lse=None):
    return lib.attention_forward(q, k, v, o, B, H, nq, nk, dk, dv, _lib.strides3(qs), _lib.strides3(ks),
                                 _lib.strides3(vs), _lib.strides3(os_), dtype, causal, scale, lse, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(o=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(B=0), _lib.MHA_ERR_INVALID_ARG, ">= 1"),
    (dict(nk=0), _lib.MHA_ERR_INVALID_ARG, ">= 1"),
    (dict(dtype=7), _lib.MHA_ERR_INVALID_ARG, "dtype"),
    (dict(causal=1, nq=64, nk=65), _lib.MHA_ERR_INVALID_ARG, "n_q == n_k"),
    (dict(causal=2), _lib.MHA_ERR_INVALID_ARG, "causal"),
    (dict(scale=float("inf")), _lib.MHA_ERR_INVALID_ARG, "finite"),
    (dict(scale=float("nan")), _lib.MHA_ERR_INVALID_ARG, "finite"),
    (dict(dk=32, dv=32), _lib.MHA_ERR_UNSUPPORTED, "d_k = 64"),
    (dict(dk=64, dv=32), _lib.MHA_ERR_UNSUPPORTED, "d_v"),
    (dict(dtype=_lib.MHA_F32, dk=48, dv=48), _lib.MHA_ERR_UNSUPPORTED, "{16, 32, 64, 128}"),
    (dict(k=MIS), _lib.MHA_ERR_INVALID_ARG, "aligned"),
    (dict(qs=(4096, 64, 68)), _lib.MHA_ERR_INVALID_ARG, "multiple of 8"),
    (dict(dtype=_lib.MHA_F32, vs=(4096, 64, 66)), _lib.MHA_ERR_INVALID_ARG, "multiple of 4"),
    (dict(os_=(4096, -64, 64)), _lib.MHA_ERR_INVALID_ARG, "negative"),
])
def test_attention_validation(lib, kw, status, needle):
    assert attn(lib, **kw) == status
    assert needle in lib.mha_last_error().decode()


def test_misaligned_lse_rejected(lib):
    assert attn(lib, lse=MIS) == _lib.MHA_ERR_INVALID_ARG


def attn_padded(lib, kv_len=FAKE, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=2, H=8, nq=64, nk=64, dk=64, dv=64, qs=S_BHND, ks=S_BHND,
             vs=S_BHND, os_=S_BHND, dtype=_lib.MHA_BF16, causal=0, scale=0.125, lse=None)
    a.update(kw)
    return lib.attention_forward_padded(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["nq"], a["nk"], a["dk"],
                                        a["dv"], _lib.strides3(a["qs"]), _lib.strides3(a["ks"]),
                                        _lib.strides3(a["vs"]), _lib.strides3(a["os_"]), a["dtype"], a["causal"],
                                        a["scale"], kv_len, a["lse"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(kv_len=None), _lib.MHA_ERR_INVALID_ARG, "kv_len"),
    (dict(kv_len=FAKE + 2), _lib.MHA_ERR_INVALID_ARG, "kv_len"),
    (dict(q=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(causal=1, nq=64, nk=65), _lib.MHA_ERR_INVALID_ARG, "n_q == n_k"),
    (dict(dk=32, dv=32), _lib.MHA_ERR_UNSUPPORTED, "d_k = 64"),
])
def test_padded_attention_validation(lib, kw, status, needle):
    """The padded entry point checks its own argument, then applies every
    rule of attention_forward."""
    assert attn_padded(lib, **kw) == status
    assert needle in lib.mha_last_error().decode()


def test_padded_mha_validation(lib):
    assert lib.mha_forward_padded(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, 2, 16, 16, 512, 8,
                                  _lib.MHA_BF16, 0, None, None) == _lib.MHA_ERR_INVALID_ARG
    assert "kv_len" in lib.mha_last_error().decode()
    assert lib.mha_forward_padded(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1000, 2, 16, 16, 512, 8,
                                  _lib.MHA_BF16, 0, FAKE, None) == _lib.MHA_ERR_WORKSPACE


def test_null_stride_array_rejected(lib):
    st = lib.attention_forward(FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 8, 64, 64, None, _lib.strides3(S_BHND),
                               _lib.strides3(S_BHND), _lib.strides3(S_BHND), 1, 0, 0.125, None, None)
    assert st == _lib.MHA_ERR_INVALID_ARG


def mha(lib, ws=FAKE, ws_bytes=1 << 40, B=2, nq=16, nk=16, dm=512, h=8, dtype=_lib.MHA_BF16, causal=0,
        ptr=FAKE):
    return lib.mha_forward(ptr, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, ws_bytes, B, nq, nk, dm, h,
                           dtype, causal, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(ws=None), _lib.MHA_ERR_INVALID_ARG, "workspace"),
    (dict(ptr=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(dm=500, h=8), _lib.MHA_ERR_INVALID_ARG, "divisible"),
    (dict(h=0), _lib.MHA_ERR_INVALID_ARG, ">= 1"),
    (dict(causal=1, nq=16, nk=32), _lib.MHA_ERR_INVALID_ARG, "n_q == n_k"),
    (dict(dm=256, h=8), _lib.MHA_ERR_UNSUPPORTED, "d_k = 64"),
    (dict(dtype=_lib.MHA_F32, dm=480, h=8), _lib.MHA_ERR_UNSUPPORTED, "{16, 32, 64, 128}"),
    (dict(ws_bytes=1000), _lib.MHA_ERR_WORKSPACE, "too small"),
    (dict(ws=MIS), _lib.MHA_ERR_INVALID_ARG, "aligned"),
])
def test_mha_validation(lib, kw, status, needle):
    assert mha(lib, **kw) == status
    assert needle in lib.mha_last_error().decode()


def test_workspace_size_arithmetic(lib):
    def r(x):
        return (x + 255) // 256 * 256
    for (B, nq, nk, dm, h, dt, e) in [(32, 512, 512, 512, 8, 1, 2), (1, 128, 128, 512, 8, 0, 4),
                                      (3, 7, 13, 64, 1, 1, 2)]:
        want = 2 * r(B * nq * dm * e) + 2 * r(B * nk * dm * e)
        assert lib.mha_forward_workspace_size(B, nq, nk, dm, h, dt) == want
    assert lib.mha_forward_workspace_size(0, 1, 1, 64, 1, 1) == 0
    assert lib.mha_forward_workspace_size(1, 1, 1, 64, 1, 5) == 0
    # exactly the required size passes the workspace check (fails later only on the missing device)
    need = lib.mha_forward_workspace_size(2, 16, 16, 512, 8, 1)
    assert mha(lib, ws_bytes=need - 1) == _lib.MHA_ERR_WORKSPACE


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), _lib.MHA_ERR_INVALID_ARG),
    (dict(m=0), _lib.MHA_ERR_INVALID_ARG),
    (dict(k=12), _lib.MHA_ERR_INVALID_ARG),
    (dict(ldx=8), _lib.MHA_ERR_INVALID_ARG),
    (dict(y=MIS), _lib.MHA_ERR_INVALID_ARG),
    (dict(dtype=3), _lib.MHA_ERR_INVALID_ARG),
    (dict(ldx=(1 << 21) + 8), _lib.MHA_ERR_UNSUPPORTED),
    (dict(ldw=(1 << 23) + 8), _lib.MHA_ERR_UNSUPPORTED),
])
def test_linear_validation(lib, kw, status):
    a = dict(x=FAKE, w=FAKE, y=FAKE, m=64, n=64, k=64, ldx=64, ldw=64, ldy=64, dtype=_lib.MHA_BF16)
    a.update(kw)
    assert lib.linear_forward(a["x"], a["w"], a["y"], a["m"], a["n"], a["k"], a["ldx"], a["ldw"], a["ldy"],
                              a["dtype"], None) == status


def grouped(lib, groups=3, n=64, k=64, dtype=_lib.MHA_BF16, **over):
    vp = lambda v: (ctypes.c_void_p * 3)(*v)
    a = dict(x=[FAKE] * 3, w=[FAKE] * 3, y=[FAKE] * 3, m=[64, 64, 64], ldx=[64] * 3, ldw=[64] * 3, ldy=[64] * 3)
    a.update(over)
    return lib.linear_forward_grouped(vp(a["x"]), vp(a["w"]), vp(a["y"]), (ctypes.c_int * 3)(*a["m"]), groups, n, k,
                                      (ctypes.c_int64 * 3)(*a["ldx"]), (ctypes.c_int64 * 3)(*a["ldw"]),
                                      (ctypes.c_int64 * 3)(*a["ldy"]), dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(groups=0), _lib.MHA_ERR_INVALID_ARG, "groups"),
    (dict(groups=4), _lib.MHA_ERR_INVALID_ARG, "groups"),
    (dict(x=[FAKE, FAKE, None]), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(m=[64, 0, 64]), _lib.MHA_ERR_INVALID_ARG, "sizes"),
    (dict(y=[FAKE, MIS, FAKE]), _lib.MHA_ERR_INVALID_ARG, "aligned"),
    (dict(ldw=[64, 64, 32]), _lib.MHA_ERR_INVALID_ARG, "leading"),
    (dict(k=12), _lib.MHA_ERR_INVALID_ARG, "multiples"),
    (dict(dtype=7), _lib.MHA_ERR_INVALID_ARG, "dtype"),
    (dict(ldx=[64, (1 << 21) + 8, 64]), _lib.MHA_ERR_UNSUPPORTED, "leading dimension too large"),
])
def test_linear_grouped_validation(lib, kw, status, needle):
    assert grouped(lib, **kw) == status
    assert needle in lib.mha_last_error().decode()


def test_linear_grouped_null_arrays(lib):
    i64 = (ctypes.c_int64 * 3)(64, 64, 64)
    assert lib.linear_forward_grouped(None, None, None, None, 1, 64, 64, i64, i64, i64, 1, None) == \
        _lib.MHA_ERR_INVALID_ARG


def test_last_error_is_thread_local(lib):
    assert attn(lib, B=0) == _lib.MHA_ERR_INVALID_ARG
    mine = lib.mha_last_error().decode()
    seen = {}

    def other():
        seen["before"] = lib.mha_last_error().decode()
        attn(lib, dtype=9)
        seen["after"] = lib.mha_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["before"] == ""
    assert "dtype" in seen["after"]
    assert lib.mha_last_error().decode() == mine


def test_binding_rejects_cpu_tensors():
    import torch
    import transformer_scaled_dot_mha_amd as m
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        m.attention_forward(x, x, x)


def enc(lib, weights=None, ws=FAKE, ws_bytes=1 << 40, B=2, n=16, dm=512, h=8, ff=2048, eps=1e-5,
        dtype=_lib.MHA_BF16, causal=0, kv_len=None, x=FAKE):
    if weights is None:
        weights = _lib.EncoderWeights(*([FAKE] * 16))
    return lib.encoder_layer_forward(x, ctypes.byref(weights) if weights is not False else None, FAKE, ws,
                                     ws_bytes, B, n, dm, h, ff, eps, dtype, causal, kv_len, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(weights=False), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(weights=_lib.EncoderWeights(*([FAKE] * 15 + [None]))), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(weights=_lib.EncoderWeights(*([FAKE] * 10 + [MIS] + [FAKE] * 5))), _lib.MHA_ERR_INVALID_ARG, "aligned"),
    (dict(eps=float("nan")), _lib.MHA_ERR_INVALID_ARG, "eps"),
    (dict(eps=-1.0), _lib.MHA_ERR_INVALID_ARG, "eps"),
    (dict(ff=2044), _lib.MHA_ERR_INVALID_ARG, "multiples of 8"),
    (dict(dm=8192, h=128), _lib.MHA_ERR_UNSUPPORTED, "LayerNorm"),
    (dict(ws=None), _lib.MHA_ERR_INVALID_ARG, "workspace"),
    (dict(ws_bytes=1000), _lib.MHA_ERR_WORKSPACE, "too small"),
    (dict(dm=256, h=8), _lib.MHA_ERR_UNSUPPORTED, "d_k = 64"),
    (dict(kv_len=FAKE + 2), _lib.MHA_ERR_INVALID_ARG, "kv_len"),
])
def test_encoder_layer_validation(lib, kw, status, needle):
    assert enc(lib, **kw) == status
    assert needle in lib.mha_last_error().decode()


def test_encoder_layer_workspace_size(lib):
    def r(x):
        return (x + 255) // 256 * 256
    B, n, dm, ff = 32, 512, 512, 2048
    assert lib.encoder_layer_workspace_size(B, n, dm, 8, ff, 1) == 4 * r(B * n * dm * 2) + r(B * n * ff * 2)
    assert lib.encoder_layer_workspace_size(B, n, dm, 8, 0, 1) == 0


def cache(k=FAKE, v=FAKE, table=None, ps=8 * 64, rs=64, hs=4096 * 8 * 64 // 8, page_size=0, max_pages=0, num_pages=0,
          max_len=4096):
    return _lib.KVCache(k, v, table, ps, rs, hs, page_size, max_pages, num_pages, max_len)


def dec(lib, c=None, q=FAKE, kv_len=FAKE, o=FAKE, lse=None, ws=FAKE, ws_bytes=1 << 40, B=2, H=8, d=64,
        dtype=_lib.MHA_BF16, scale=0.125):
    c = cache() if c is None else c
    return lib.attention_decode(q, ctypes.byref(c) if c is not False else None, kv_len, o, lse, ws, ws_bytes, B, H,
                                d, dtype, scale, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(c=False), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(kv_len=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(ws=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(c=cache(v=None)), _lib.MHA_ERR_INVALID_ARG, "cache->v"),
    (dict(B=0), _lib.MHA_ERR_INVALID_ARG, ">= 1"),
    (dict(c=cache(max_len=0)), _lib.MHA_ERR_INVALID_ARG, ">= 1"),
    (dict(dtype=7), _lib.MHA_ERR_INVALID_ARG, "dtype"),
    (dict(scale=float("inf")), _lib.MHA_ERR_INVALID_ARG, "scale"),
    (dict(d=48), _lib.MHA_ERR_UNSUPPORTED, "decode supports d"),
    (dict(c=cache(rs=-64)), _lib.MHA_ERR_INVALID_ARG, "negative"),
    (dict(c=cache(hs=12)), _lib.MHA_ERR_INVALID_ARG, "multiple of 8"),
    (dict(c=cache(k=MIS)), _lib.MHA_ERR_INVALID_ARG, "16-byte"),
    (dict(o=MIS), _lib.MHA_ERR_INVALID_ARG, "16-byte"),
    (dict(kv_len=FAKE + 2), _lib.MHA_ERR_INVALID_ARG, "4-byte"),
    (dict(lse=FAKE + 2), _lib.MHA_ERR_INVALID_ARG, "4-byte"),
    (dict(c=cache(table=FAKE + 2, page_size=16, max_pages=256, num_pages=10)), _lib.MHA_ERR_INVALID_ARG, "4-byte"),
    (dict(c=cache(table=FAKE, page_size=0, max_pages=256, num_pages=10)), _lib.MHA_ERR_INVALID_ARG, "page_size"),
    (dict(c=cache(table=FAKE, page_size=16, max_pages=256, num_pages=0)), _lib.MHA_ERR_INVALID_ARG, "num_pages"),
    (dict(c=cache(table=FAKE, page_size=16, max_pages=255, num_pages=10)), _lib.MHA_ERR_INVALID_ARG, "exceeds"),
    (dict(c=cache(max_len=65536 * 256)), _lib.MHA_ERR_UNSUPPORTED, "max_len"),
    (dict(ws_bytes=1000), _lib.MHA_ERR_WORKSPACE, "required"),
])
def test_decode_validation(lib, kw, status, needle):
    assert dec(lib, **kw) == status
    assert needle in lib.mha_last_error().decode()


def test_decode_workspace_size(lib):
    def r(x):
        return (x + 255) // 256 * 256
    for B, H, d, n in ((64, 8, 64, 4096), (3, 5, 128, 257), (1, 1, 16, 1)):
        parts = B * H * ((n + 255) // 256)
        assert lib.attention_decode_workspace_size(B, H, d, n) == r(parts * 8) + r(parts * d * 4)
    assert lib.attention_decode_workspace_size(1, 1, 64, 0) == 0


def bwd(lib, q=FAKE, lse=FAKE, dq=FAKE, ws=FAKE, ws_bytes=1 << 30, B=2, H=8, nq=64, nk=64, d=64, strides=None,
        dtype=_lib.MHA_BF16, causal=0, scale=0.125, kv_len=None):
    st = [S_BHND] * 8 if strides is None else strides
    return lib.attention_backward(q, FAKE, FAKE, FAKE, FAKE, lse, dq, FAKE, FAKE, B, H, nq, nk, d,
                                  *[_lib.strides3(x) for x in st], dtype, causal, scale, kv_len, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(lse=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(dq=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(ws=None), _lib.MHA_ERR_INVALID_ARG, "non-null"),
    (dict(dq=MIS), _lib.MHA_ERR_INVALID_ARG, "aligned"),
    (dict(lse=FAKE + 4), _lib.MHA_ERR_INVALID_ARG, "aligned"),
    (dict(d=32), _lib.MHA_ERR_UNSUPPORTED, "d_k = 64"),
    (dict(causal=1, nk=65), _lib.MHA_ERR_INVALID_ARG, "causal"),
    (dict(ws_bytes=100), _lib.MHA_ERR_WORKSPACE, "required"),
    (dict(kv_len=FAKE + 2), _lib.MHA_ERR_INVALID_ARG, "kv_len"),
    (dict(strides=[S_BHND] * 5 + [(8 * 64 * 64, 64 * 64, 12)] + [S_BHND] * 2), _lib.MHA_ERR_INVALID_ARG, "dq stride"),
    (dict(strides=[(8 * 64 * 64, 64 * 64, 1 << 25)] + [S_BHND] * 7), _lib.MHA_ERR_UNSUPPORTED, "row stride"),
    (dict(strides=[S_BHND] * 4 + [(8 * 64 * 64, 64 * 64, 1 << 25)] + [S_BHND] * 3), _lib.MHA_ERR_UNSUPPORTED,
     "d_o row stride"),
])
def test_backward_validation(lib, kw, status, needle):
    assert bwd(lib, **kw) == status
    assert needle in lib.mha_last_error().decode()


def test_backward_workspace_size(lib):
    assert lib.attention_backward_workspace_size(2, 8, 100) == (2 * 8 * 100 * 8 + 255) // 256 * 256
    assert lib.attention_backward_workspace_size(0, 8, 100) == 0


def test_noalloc_rejects_oversized_problems_before_any_device_call(lib):
    """mha_forward_noalloc serves workspaces up to MHA_NOALLOC_MAX_WORKSPACE bytes
    (its fixed per-GPU array); a larger problem is refused on the host."""
    header = open(HEADER).read()
    assert "#define MHA_NOALLOC_MAX_WORKSPACE ((size_t)128 << 20)" in header
    assert _lib.NOALLOC_MAX_WORKSPACE == 128 << 20
    args = lambda B, n, dm, h, dt=1: (FAKE,) * 8 + (B, n, n, dm, h, dt, 0, None)
    # the encoder workload (B=32, N=512, d_model 512, bf16) needs exactly 64 MiB: served
    assert lib.mha_forward_workspace_size(32, 512, 512, 512, 8, 1) == 64 << 20
    # 2.5x that is refused
    assert lib.mha_forward_noalloc(*args(80, 512, 512, 8)) == _lib.MHA_ERR_UNSUPPORTED
    assert "128 MiB" in lib.mha_last_error().decode()
    assert lib.mha_forward_noalloc(*args(0, 512, 512, 8)) == _lib.MHA_ERR_INVALID_ARG
    assert lib.mha_forward_noalloc(*args(1, 16, 512, 8, dt=9)) == _lib.MHA_ERR_INVALID_ARG
    null_out = (FAKE,) * 7 + (None, 1, 16, 16, 512, 8, 1, 0, None)
    assert lib.mha_forward_noalloc(*null_out) == _lib.MHA_ERR_INVALID_ARG
