"""Multi-head scaled dot-product attention forward for AMD MI355X (gfx950).

Thin Python binding over libmha.so's C ABI (include/mha.h): each function
checks and marshals torch tensors (device pointers, element strides, the
current HIP stream) and calls the C entry point of the same name. Every step
of the computation runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and calling with CPU tensors raises.
"""
from __future__ import annotations

import ctypes
import math

from ._lib import (ENCODER_WEIGHT_NAMES, EncoderWeights, KVCache, MHA_BF16, MHA_ERR_HIP, MHA_ERR_INVALID_ARG,
                   MHA_ERR_UNSUPPORTED, NOALLOC_MAX_WORKSPACE,
                   MHA_ERR_WORKSPACE, MHA_F32, MHA_OK, LIB_PATH, MHAError, check, load, strides3)

__all__ = ["attention_backward", "attention_backward_workspace_size", "attention_decode",
           "attention_decode_workspace_size", "attention_forward", "encoder_layer_forward", "encoder_layer_workspace_size",
           "linear_forward", "linear_forward_grouped",
           "mha_forward", "mha_forward_noalloc", "mha_forward_workspace_size",
           "MHAError", "MHA_F32", "MHA_BF16", "LIB_PATH", "load"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MHA_F32
    if t.dtype == torch.bfloat16:
        return MHA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.float32 or torch.bfloat16")


def _require_device(*ts):
    dev = ts[0].device
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU (no CPU path exists)")
        if t.device != dev:
            raise ValueError("all tensors must be on the same device")
        if t.dtype != ts[0].dtype:
            raise TypeError("all tensors must share one dtype")
    return dev


def _stream_handle(dev, stream):
    torch = _torch()
    s = torch.cuda.current_stream(dev) if stream is None else stream
    return s.cuda_stream


class _on_device:
    """Make `dev` the current device for a library call; free when it already is
    (the usual case), since a device switch costs more than the call itself."""
    __slots__ = ("dev", "prev")

    def __init__(self, dev):
        self.dev = dev
        self.prev = None

    def __enter__(self):
        torch = _torch()
        cur = torch.cuda.current_device()
        if cur != self.dev.index:
            self.prev = cur
            torch.cuda.set_device(self.dev)

    def __exit__(self, *exc):
        if self.prev is not None:
            _torch().cuda.set_device(self.prev)
        return False


def _kv_len_arg(kv_len, B, dev):
    """Check a key-length tensor: int32, on the device, (B,) contiguous."""
    torch = _torch()
    if not isinstance(kv_len, torch.Tensor) or kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be an int32 tensor of per-batch key lengths")
    if not kv_len.is_cuda or kv_len.device != dev:
        raise ValueError("kv_len must live on the same GPU as the inputs")
    if tuple(kv_len.shape) != (B,) or not kv_len.is_contiguous():
        raise ValueError(f"kv_len must be a contiguous ({B},) tensor")
    return kv_len.data_ptr()


def attention_forward(q, k, v, *, causal: bool = False, scale: float | None = None, out=None,
                      return_lse: bool = False, kv_len=None, stream=None):
    """O = softmax(scale * Q K^T (+ causal mask)) V for (batch, heads, n, d) tensors.

    q: (B, H, N_q, d), k: (B, H, N_k, d), v: (B, H, N_k, d); any strides with a
    contiguous last dimension (so (B, N, H, d) buffers can be passed through
    .transpose(1, 2) without a copy). Returns out (B, H, N_q, d), and the fp32
    log-sum-exp (B, H, N_q) when return_lse is set.
    kv_len: optional int32 device tensor (B,) of key lengths (a key-padding
    mask): keys at or past kv_len[b] are blocked for batch item b; a row with
    no visible key returns 0 (lse -inf). Calls attention_forward_padded.
    """
    torch = _torch()
    dev = _require_device(q, k, v)
    B, H, n_q, d_k = q.shape
    n_k, d_v = k.shape[2], v.shape[3]
    if k.shape[:2] != (B, H) or v.shape[:3] != (B, H, n_k) or k.shape[3] != d_k:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
    if out is None:
        out = torch.empty((B, H, n_q, d_v), dtype=q.dtype, device=dev)
    _require_device(q, out)
    if tuple(out.shape) != (B, H, n_q, d_v) or out.stride(3) != 1:
        raise ValueError("out must be (B, H, N_q, d_v) with a contiguous last dimension")
    lse = torch.empty((B, H, n_q), dtype=torch.float32, device=dev) if return_lse else None
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    lib = load()
    with _on_device(dev):
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, n_q, n_k, d_k, d_v,
                strides3(q.stride()[:3]), strides3(k.stride()[:3]), strides3(v.stride()[:3]),
                strides3(out.stride()[:3]), _dtype_code(q), int(bool(causal)), float(scale))
        lse_p = lse.data_ptr() if lse is not None else None
        if kv_len is None:
            st = lib.attention_forward(*args, lse_p, _stream_handle(dev, stream))
        else:
            st = lib.attention_forward_padded(*args, _kv_len_arg(kv_len, B, dev), lse_p,
                                              _stream_handle(dev, stream))
    check(st)
    return (out, lse) if return_lse else out


def attention_backward_workspace_size(batch: int, heads: int, n_q: int) -> int:
    """Bytes of device workspace attention_backward needs (0 for invalid sizes)."""
    return int(load().attention_backward_workspace_size(batch, heads, n_q))


def attention_backward(q, k, v, o, d_o, lse, *, causal: bool = False, scale: float | None = None, kv_len=None,
                       dq=None, dk=None, dv=None, workspace=None, stream=None):
    """dQ, dK, dV of attention_forward for the output gradient d_o.

    q, k, v, o, d_o: (B, H, N, d) tensors as in attention_forward (any strides
    with a contiguous last dimension); o and lse (fp32 (B, H, N_q), contiguous)
    are what attention_forward returned for these inputs with return_lse=True,
    the same causal flag, scale and kv_len. Returns (dq, dk, dv).
    """
    torch = _torch()
    dev = _require_device(q, k, v, o, d_o)
    B, H, n_q, d = q.shape
    n_k = k.shape[2]
    if k.shape != (B, H, n_k, d) or v.shape != (B, H, n_k, d) or o.shape != q.shape or d_o.shape != q.shape:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}, "
                         f"o {tuple(o.shape)}, d_o {tuple(d_o.shape)}")
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, n_q) \
            or not lse.is_contiguous() or lse.device != dev:
        raise ValueError("lse must be a contiguous float32 (B, H, N_q) tensor on the inputs' device")
    outs = []
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t is None:
            t = torch.empty(like.shape, dtype=like.dtype, device=dev)
        _require_device(q, t)
        if tuple(t.shape) != tuple(like.shape):
            raise ValueError(f"{name} must have shape {tuple(like.shape)}")
        outs.append(t)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("d_o", d_o), ("dq", outs[0]), ("dk", outs[1]),
                    ("dv", outs[2])):
        if t.stride(3) != 1:
            raise ValueError(f"{name} must have a contiguous last dimension")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lib = load()
    if workspace is None:
        workspace = torch.empty(max(int(lib.attention_backward_workspace_size(B, H, n_q)), 16), dtype=torch.uint8,
                                device=dev)
    kvp = None if kv_len is None else _kv_len_arg(kv_len, B, dev)
    st3 = [strides3(t.stride()[:3]) for t in (q, k, v, o, d_o, *outs)]
    with _on_device(dev):
        st = lib.attention_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), d_o.data_ptr(),
                                    lse.data_ptr(), outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
                                    B, H, n_q, n_k, d, *st3, _dtype_code(q), int(bool(causal)), float(scale), kvp,
                                    workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                    _stream_handle(dev, stream))
    check(st)
    return tuple(outs)


def linear_forward(x, w, *, out=None, stream=None):
    """Y = X W for X (m, k) and W (k, n) row-major (leading dimension = row stride)."""
    torch = _torch()
    dev = _require_device(x, w)
    m, k = x.shape
    k2, n = w.shape
    if k2 != k:
        raise ValueError(f"inner sizes differ: {k} vs {k2}")
    if x.stride(1) != 1 or w.stride(1) != 1:
        raise ValueError("x and w must be row-major with contiguous rows")
    if out is None:
        out = torch.empty((m, n), dtype=x.dtype, device=dev)
    _require_device(x, out)
    if tuple(out.shape) != (m, n) or out.stride(1) != 1:
        raise ValueError("out must be (m, n) row-major")
    lib = load()
    with _on_device(dev):
        st = lib.linear_forward(x.data_ptr(), w.data_ptr(), out.data_ptr(), m, n, k, x.stride(0),
                                w.stride(0), out.stride(0), _dtype_code(x), _stream_handle(dev, stream))
    check(st)
    return out


def linear_forward_grouped(xs, ws, *, outs=None, stream=None):
    """Y_g = X_g W_g for up to three problems sharing n and k, in one launch
    (the launch mha_forward makes for its Q, K and V projections)."""
    torch = _torch()
    if not 1 <= len(xs) <= 3 or len(ws) != len(xs):
        raise ValueError("one to three (x, w) pairs are needed")
    dev = _require_device(*xs, *ws)
    k, n = ws[0].shape
    for x, w in zip(xs, ws):
        if x.shape[1] != k or tuple(w.shape) != (k, n):
            raise ValueError("every problem must share n and k")
        if x.stride(1) != 1 or w.stride(1) != 1:
            raise ValueError("x and w must be row-major with contiguous rows")
    if outs is None:
        outs = [torch.empty((x.shape[0], n), dtype=x.dtype, device=dev) for x in xs]
    for x, y in zip(xs, outs):
        _require_device(x, y)
        if tuple(y.shape) != (x.shape[0], n) or y.stride(1) != 1:
            raise ValueError("each out must be (m, n) row-major")
    g = len(xs)
    ptrs = lambda ts: (ctypes.c_void_p * g)(*[t.data_ptr() for t in ts])
    lds = lambda ts: (ctypes.c_int64 * g)(*[t.stride(0) for t in ts])
    lib = load()
    with _on_device(dev):
        st = lib.linear_forward_grouped(ptrs(xs), ptrs(ws), ptrs(outs), (ctypes.c_int * g)(*[x.shape[0] for x in xs]),
                                        g, n, k, lds(xs), lds(ws), lds(outs), _dtype_code(xs[0]),
                                        _stream_handle(dev, stream))
    check(st)
    return outs


def mha_forward_workspace_size(batch: int, n_q: int, n_k: int, d_model: int, heads: int, dtype) -> int:
    """Bytes of workspace mha_forward needs (dtype: torch dtype or MHA_F32/MHA_BF16)."""
    code = dtype if isinstance(dtype, int) else (MHA_BF16 if str(dtype).endswith("bfloat16") else MHA_F32)
    return int(load().mha_forward_workspace_size(batch, n_q, n_k, d_model, heads, code))


def mha_forward(xq, xk, xv, wq, wk, wv, wo, heads: int, *, causal: bool = False, out=None,
                workspace=None, kv_len=None, stream=None):
    """MultiHead(xq, xk, xv) = Concat(head_1..head_h) W^O, bias-free.

    xq (B, N_q, d_model); xk, xv (B, N_k, d_model); w* (d_model, d_model) stored
    (in, out). Pass the same tensor three times for self-attention. workspace,
    if given, is a uint8 device tensor of at least mha_forward_workspace_size bytes.
    kv_len: optional int32 device tensor (B,) of key lengths of the xk/xv
    sequence (a key-padding mask); calls mha_forward_padded.
    """
    torch = _torch()
    dev = _require_device(xq, xk, xv, wq, wk, wv, wo)
    B, n_q, d_model = xq.shape
    n_k = xk.shape[1]
    if xk.shape != (B, n_k, d_model) or xv.shape != xk.shape:
        raise ValueError("xk and xv must be (B, N_k, d_model)")
    for w in (wq, wk, wv, wo):
        if tuple(w.shape) != (d_model, d_model):
            raise ValueError("weights must be (d_model, d_model)")
    for t in (xq, xk, xv, wq, wk, wv, wo):
        if not t.is_contiguous():
            raise ValueError("mha_forward takes contiguous tensors")
    code = _dtype_code(xq)
    lib = load()
    need = int(lib.mha_forward_workspace_size(B, n_q, n_k, d_model, heads, code))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((B, n_q, d_model), dtype=xq.dtype, device=dev)
    if tuple(out.shape) != (B, n_q, d_model) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B, N_q, d_model) tensor")
    with _on_device(dev):
        args = (xq.data_ptr(), xk.data_ptr(), xv.data_ptr(), wq.data_ptr(), wk.data_ptr(),
                wv.data_ptr(), wo.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                workspace.numel() * workspace.element_size(), B, n_q, n_k, d_model, heads,
                code, int(bool(causal)))
        if kv_len is None:
            st = lib.mha_forward(*args, _stream_handle(dev, stream))
        else:
            st = lib.mha_forward_padded(*args, _kv_len_arg(kv_len, B, dev), _stream_handle(dev, stream))
    check(st)
    return out


def mha_forward_noalloc(xq, xk, xv, wq, wk, wv, wo, heads: int, *, causal: bool = False, out=None, stream=None):
    """mha_forward without a workspace: the library keeps the intermediates in its
    own fixed per-GPU device array (NOALLOC_MAX_WORKSPACE bytes), so the call
    allocates nothing on the device when `out` is given. Calls that overlap on
    one GPU race on that array."""
    torch = _torch()
    dev = _require_device(xq, xk, xv, wq, wk, wv, wo)
    B, n_q, d_model = xq.shape
    n_k = xk.shape[1]
    if xk.shape != (B, n_k, d_model) or xv.shape != xk.shape:
        raise ValueError("xk and xv must be (B, N_k, d_model)")
    for w in (wq, wk, wv, wo):
        if tuple(w.shape) != (d_model, d_model):
            raise ValueError("weights must be (d_model, d_model)")
    for t in (xq, xk, xv, wq, wk, wv, wo):
        if not t.is_contiguous():
            raise ValueError("mha_forward_noalloc takes contiguous tensors")
    if out is None:
        out = torch.empty((B, n_q, d_model), dtype=xq.dtype, device=dev)
    if tuple(out.shape) != (B, n_q, d_model) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B, N_q, d_model) tensor")
    lib = load()
    with _on_device(dev):
        st = lib.mha_forward_noalloc(xq.data_ptr(), xk.data_ptr(), xv.data_ptr(), wq.data_ptr(), wk.data_ptr(),
                                     wv.data_ptr(), wo.data_ptr(), out.data_ptr(), B, n_q, n_k, d_model, heads,
                                     _dtype_code(xq), int(bool(causal)), _stream_handle(dev, stream))
    check(st)
    return out


def encoder_layer_workspace_size(batch: int, n: int, d_model: int, heads: int, d_ff: int, dtype) -> int:
    """Bytes of workspace encoder_layer_forward needs (dtype: torch dtype or MHA_F32/MHA_BF16)."""
    code = dtype if isinstance(dtype, int) else (MHA_BF16 if str(dtype).endswith("bfloat16") else MHA_F32)
    return int(load().encoder_layer_workspace_size(batch, n, d_model, heads, d_ff, code))


def encoder_layer_forward(x, weights: dict, heads: int, *, eps: float = 1e-5, causal: bool = False, kv_len=None,
                          out=None, workspace=None, stream=None):
    """One post-norm encoder layer: LayerNorm(h + FFN(h)) with h = LayerNorm(x + MHA(x)).

    x (B, N, d_model). weights: dict of device tensors named wq, wk, wv, wo,
    bq, bk, bv, bo, ln1_gamma, ln1_beta, w1, b1, w2, b2, ln2_gamma, ln2_beta,
    matrices stored (in, out): w1 (d_model, d_ff), w2 (d_ff, d_model).
    kv_len: optional int32 device tensor (B,) of key lengths (padding mask).
    """
    torch = _torch()
    missing = [n for n in ENCODER_WEIGHT_NAMES if n not in weights]
    if missing:
        raise KeyError(f"missing encoder weights: {missing}")
    ts = [weights[n] for n in ENCODER_WEIGHT_NAMES]
    dev = _require_device(x, *ts)
    B, N, d_model = x.shape
    d_ff = weights["w1"].shape[1]
    shapes = {"wq": (d_model, d_model), "wk": (d_model, d_model), "wv": (d_model, d_model),
              "wo": (d_model, d_model), "w1": (d_model, d_ff), "w2": (d_ff, d_model), "b1": (d_ff,)}
    for n in ENCODER_WEIGHT_NAMES:
        want = shapes.get(n, (d_model,))
        if tuple(weights[n].shape) != want or not weights[n].is_contiguous():
            raise ValueError(f"{n} must be a contiguous {want} tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    code = _dtype_code(x)
    lib = load()
    need = int(lib.encoder_layer_workspace_size(B, N, d_model, heads, d_ff, code))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty_like(x)
    if tuple(out.shape) != (B, N, d_model) or not out.is_contiguous() or out.dtype != x.dtype:
        raise ValueError("out must be a contiguous (B, N, d_model) tensor of x's dtype")
    w = EncoderWeights(*[t.data_ptr() for t in ts])
    kvp = None if kv_len is None else _kv_len_arg(kv_len, B, dev)
    with _on_device(dev):
        st = lib.encoder_layer_forward(x.data_ptr(), ctypes.byref(w), out.data_ptr(), workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), B, N, d_model, heads, d_ff,
                                       float(eps), code, int(bool(causal)), kvp, _stream_handle(dev, stream))
    check(st)
    return out


def attention_decode_workspace_size(batch: int, heads: int, d: int, max_len: int) -> int:
    """Bytes of device workspace attention_decode needs (0 for invalid sizes)."""
    return int(load().attention_decode_workspace_size(batch, heads, d, max_len))


def attention_decode(q, k_cache, v_cache, kv_len, *, block_table=None, scale: float | None = None, out=None,
                     return_lse: bool = False, workspace=None, stream=None):
    """One decoding step: q (B, H, d) attends to the first kv_len[b] cached keys.

    k_cache, v_cache: 4-D tensors (pages, slots, H, d) with a contiguous last
    dimension and identical shape and strides; their strides are the cache
    geometry passed to the library.
      - block_table None: page b is sequence b (pages == B) and slot j is its
        key j, so a (B, max_len, H, d) cache is passed as is and a
        (B, H, max_len, d) one as .transpose(1, 2).
      - block_table: int32 device tensor (B, max_pages); key j of sequence b
        is in page block_table[b, j // slots] at slot j % slots.
    kv_len: int32 device tensor (B,). Returns out (B, H, d), and the fp32
    log-sum-exp (B, H) when return_lse is set.
    workspace: optional uint8 device tensor of attention_decode_workspace_size
    bytes (scratch; one call at a time per workspace), allocated per call if
    omitted.
    """
    torch = _torch()
    dev = _require_device(q, k_cache, v_cache)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous (B, H, d) tensor")
    B, H, d = q.shape
    if k_cache.dim() != 4 or tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.stride() != v_cache.stride():
        raise ValueError("k_cache and v_cache must be 4-D (pages, slots, H, d) with equal shapes and strides")
    pages, slots, hc, dc = k_cache.shape
    if (hc, dc) != (H, d) or k_cache.stride(3) != 1:
        raise ValueError(f"cache heads/width {(hc, dc)} must match q's {(H, d)} with a contiguous last dimension")
    table_p = None
    page_size = max_pages = num_pages = 0
    if block_table is None:
        if pages != B:
            raise ValueError(f"without a block table the cache's first dimension must be the batch ({B})")
        max_len = slots
    else:
        if not isinstance(block_table, torch.Tensor) or block_table.dtype != torch.int32:
            raise TypeError("block_table must be an int32 tensor")
        if not block_table.is_cuda or block_table.device != dev:
            raise ValueError("block_table must live on the same GPU as the inputs")
        if block_table.dim() != 2 or block_table.shape[0] != B or not block_table.is_contiguous():
            raise ValueError(f"block_table must be a contiguous ({B}, max_pages) tensor")
        page_size, max_pages, num_pages = slots, block_table.shape[1], pages
        max_len = page_size * max_pages
        table_p = block_table.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, d), dtype=q.dtype, device=dev)
    _require_device(q, out)
    if tuple(out.shape) != (B, H, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous (B, H, d) tensor")
    lse = torch.empty((B, H), dtype=torch.float32, device=dev) if return_lse else None
    lib = load()
    if workspace is None:   # the library checks a caller's workspace size itself
        need = int(lib.attention_decode_workspace_size(B, H, d, max_len))
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ks = k_cache.stride()
    cache = KVCache(k_cache.data_ptr(), v_cache.data_ptr(), table_p, ks[0], ks[1], ks[2], page_size, max_pages,
                    num_pages, max_len)
    with _on_device(dev):
        st = lib.attention_decode(q.data_ptr(), ctypes.byref(cache), _kv_len_arg(kv_len, B, dev), out.data_ptr(),
                                  lse.data_ptr() if lse is not None else None, workspace.data_ptr(),
                                  workspace.numel() * workspace.element_size(), B, H, d, _dtype_code(q),
                                  float(scale), _stream_handle(dev, stream))
    check(st)
    return (out, lse) if return_lse else out
