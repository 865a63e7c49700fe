"""ctypes loader for libmha.so (built in-tree by build.py).

This module imports nothing but the standard library, so the C ABI can be
loaded and inspected on a machine without a GPU. There is no fallback: if the
library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

# MHA_LIBRARY points the binding at another build of the same C ABI (the
# host AddressSanitizer build of the front end used by the CPU tests)
LIB_PATH = os.environ.get("MHA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmha.so")

MHA_OK, MHA_ERR_INVALID_ARG, MHA_ERR_UNSUPPORTED, MHA_ERR_WORKSPACE, MHA_ERR_HIP = range(5)
MHA_F32, MHA_BF16 = 0, 1
NOALLOC_MAX_WORKSPACE = 128 << 20  # MHA_NOALLOC_MAX_WORKSPACE of include/mha.h

_i64x3 = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p
_int = ctypes.c_int

ENCODER_WEIGHT_NAMES = ("wq", "wk", "wv", "wo", "bq", "bk", "bv", "bo", "ln1_gamma", "ln1_beta",
                        "w1", "b1", "w2", "b2", "ln2_gamma", "ln2_beta")


class EncoderWeights(ctypes.Structure):
    """mha_encoder_weights of include/mha.h: sixteen device pointers."""
    _fields_ = [(n, ctypes.c_void_p) for n in ENCODER_WEIGHT_NAMES]


class KVCache(ctypes.Structure):
    """mha_kv_cache of include/mha.h: the cache pools and their geometry."""
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("page_stride", ctypes.c_int64), ("row_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_len", ctypes.c_int32)]


# name -> (restype, argtypes); must match include/mha.h
SIGNATURES = {
    "attention_forward": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _int,
                                 _i64x3, _i64x3, _i64x3, _i64x3, _int, _int, ctypes.c_float,
                                 _vp, _vp]),
    "attention_forward_padded": (_int, [_vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _int,
                                        _i64x3, _i64x3, _i64x3, _i64x3, _int, _int, ctypes.c_float,
                                        _vp, _vp, _vp]),
    "linear_forward": (_int, [_vp, _vp, _vp, _int, _int, _int, ctypes.c_int64, ctypes.c_int64,
                              ctypes.c_int64, _int, _vp]),
    "linear_forward_grouped": (_int, [ctypes.POINTER(_vp), ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                      ctypes.POINTER(_int), _int, _int, _int, _i64x3, _i64x3, _i64x3, _int, _vp]),
    "mha_forward_workspace_size": (ctypes.c_size_t, [_int, _int, _int, _int, _int, _int]),
    "mha_forward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                           _int, _int, _int, _int, _int, _int, _int, _vp]),
    "mha_forward_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _int,
                                   _int, _vp]),
    "mha_forward_padded": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                  _int, _int, _int, _int, _int, _int, _int, _vp, _vp]),
    "encoder_layer_workspace_size": (ctypes.c_size_t, [_int, _int, _int, _int, _int, _int]),
    "encoder_layer_forward": (_int, [_vp, ctypes.POINTER(EncoderWeights), _vp, _vp, ctypes.c_size_t, _int, _int,
                                     _int, _int, _int, ctypes.c_float, _int, _int, _vp, _vp]),
    "attention_backward_workspace_size": (ctypes.c_size_t, [_int, _int, _int]),
    "attention_backward": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int,
                                  _i64x3, _i64x3, _i64x3, _i64x3, _i64x3, _i64x3, _i64x3, _i64x3, _int, _int,
                                  ctypes.c_float, _vp, _vp, ctypes.c_size_t, _vp]),
    "attention_decode_workspace_size": (ctypes.c_size_t, [_int, _int, _int, _int]),
    "attention_decode": (_int, [_vp, ctypes.POINTER(KVCache), _vp, _vp, _vp, _vp, ctypes.c_size_t, _int, _int,
                                _int, _int, ctypes.c_float, _vp]),
    "mha_status_string": (ctypes.c_char_p, [_int]),
    "mha_last_error": (ctypes.c_char_p, []),
    "mha_version": (_int, []),
}


class MHAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{_status_name(status)}: {detail}")


_lib = None


def _status_name(status: int) -> str:
    names = ["MHA_OK", "MHA_ERR_INVALID_ARG", "MHA_ERR_UNSUPPORTED", "MHA_ERR_WORKSPACE", "MHA_ERR_HIP"]
    return names[status] if 0 <= status < len(names) else f"status {status}"


def load() -> ctypes.CDLL:
    """Load libmha.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m transformer_scaled_dot_mha_amd.build` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def strides3(s) -> ctypes.Array:
    return (ctypes.c_int64 * 3)(*[int(x) for x in s])


def check(status: int) -> None:
    if status != MHA_OK:
        raise MHAError(status, load().mha_last_error().decode())
