"""ctypes loader for ``libnvfp4.so`` — argument marshalling only.

The library is the in-tree build product of :mod:`bit_block_scaled_amd.build`.
There is no fallback: if the library is missing or does not load, every call
raises.
"""

from __future__ import annotations

import ctypes as C
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libnvfp4.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")
HEADERS = [os.path.join(INCLUDE, h) for h in ("nvfp4.h", "nvfp4_testing.h")]

NVFP4_OK = 0
NVFP4_EINVAL = 1
NVFP4_EWORKSPACE = 2
NVFP4_ECAPACITY = 3
NVFP4_EHIP = 4
NVFP4_EPI_GELU_TANH = 0x1
NVFP4_NOALLOC_MAX_ELEMENTS = 1 << 26
NVFP4_Q_ADAPTIVE_4_6 = 0x10
NVFP4_Q_BLOCK_2D = 0x20
NVFP4_TILES = {(256, 256): 0x100, (256, 192): 0x200, (192, 256): 0x300, (256, 128): 0x400,
               (128, 256): 0x500, (128, 128): 0x600}

_i64 = C.c_int64
_p = C.c_void_p
_sz = C.c_size_t


class KVCacheDesc(C.Structure):
    """Mirror of ``nvfp4_kv_cache`` in include/nvfp4.h (same field order)."""

    _fields_ = [
        ("capacity", _i64), ("heads", _i64), ("head_dim", _i64), ("max_chunks", _i64),
        ("k_codes", _p), ("k_scales", _p), ("v_codes", _p), ("v_scales", _p),
        ("gscale", _p), ("chunk_start", _p),
        ("n_tokens", _i64), ("n_chunks", _i64),
        ("k_center", _p),
    ]


_SIGS = {
    "nvfp4_quantize_workspace": ([_i64, _i64, C.POINTER(_sz)], C.c_int),
    "nvfp4_quantize": ([_p, _i64, _i64, _p, _p, _p, _p, _sz, _p], C.c_int),
    "nvfp4_quantize_ex": ([_p, _i64, _i64, C.c_uint32, _p, _p, _p, _p, _sz, _p], C.c_int),
    "nvfp4_gemm": ([_p, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, C.c_uint32, _p], C.c_int),
    "nvfp4_gemm_tile": ([_i64, _i64, _i64, C.POINTER(C.c_int), C.POINTER(C.c_int)], C.c_int),
    "nvfp4_linear_workspace": ([_i64, _i64, C.POINTER(_sz)], C.c_int),
    "nvfp4_linear": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, C.c_uint32, _p, _sz, _p], C.c_int),
    "nvfp4_linear_noalloc": ([_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, C.c_uint32, _p], C.c_int),
    "nvfp4_linear_q_workspace": ([_i64, _i64, _i64, C.POINTER(_sz)], C.c_int),
    "nvfp4_linear_q": ([_p, _p, _p, _p, _p, _i64, _i64, _i64, C.c_uint32, _p, _p, _p, _p, _sz, _p],
                       C.c_int),
    "nvfp4_kv_init": ([C.POINTER(KVCacheDesc)], C.c_int),
    "nvfp4_kv_append_workspace": ([_i64, _i64, _i64, C.POINTER(_sz)], C.c_int),
    "nvfp4_kv_smooth_workspace": ([_i64, _i64, _i64, C.POINTER(_sz)], C.c_int),
    "nvfp4_kv_append": ([C.POINTER(KVCacheDesc), _p, _p, _i64, _i64, _p, _sz, _p], C.c_int),
    "nvfp4_kv_append_ex": ([C.POINTER(KVCacheDesc), _p, _p, _i64, _i64, C.c_uint32, _p, _sz, _p],
                           C.c_int),
    "nvfp4_kv_dequant": ([C.POINTER(KVCacheDesc), _i64, _i64, _p, _p, _p], C.c_int),
    "nvfp4_kv_attention_workspace": ([_i64, _i64, _i64, C.POINTER(_sz)], C.c_int),
    "nvfp4_kv_attention": ([C.POINTER(KVCacheDesc), _p, _i64, _i64, C.POINTER(_i64), C.c_int, C.c_float,
                            _p, _i64, _p, _sz, _p], C.c_int),
    "nvfp4_attention_bf16": ([_p, _i64, _i64, _p, _p, _i64, _i64, _i64, C.c_float, _p, _i64, _p, _sz, _p],
                             C.c_int),
    "nvfp4_qkv_append_workspace": ([_i64, _i64, _i64, _i64, C.POINTER(_sz)], C.c_int),
    "nvfp4_qkv_append": ([C.POINTER(KVCacheDesc), _p, _i64, _i64, _p, _p, _p, _p, _p, C.c_uint32, _p, _sz, _p],
                         C.c_int),
    "nvfp4_quantize_rht_workspace": ([_i64, _i64, C.POINTER(_sz)], C.c_int),
    "nvfp4_quantize_rht": ([_p, _i64, _i64, _i64, C.c_uint32, _p, _p, _p, _p, _sz, _p], C.c_int),
    "nvfp4_testing_set_quantize_wait": ([C.c_uint64], C.c_uint64),
    "nvfp4_testing_set_launch_events": ([C.POINTER(C.c_void_p), C.c_int], C.c_int),
    "nvfp4_strerror": ([C.c_int], C.c_char_p),
    "nvfp4_last_error": ([], C.c_char_p),
}

_lib = None


class NVFP4Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


def header_symbols(paths=None):
    """Function names declared in the public headers under include/."""
    names = set()
    for path in paths or HEADERS:
        names |= set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", open(path).read()))
    return sorted(names)


def lib():
    """The loaded library (ctypes.CDLL); raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m bit_block_scaled_amd.build` "
                "(there is no CPU fallback)")
        h = C.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(h, name)
            f.argtypes = args
            f.restype = res
        _lib = h
    return _lib


def check(status: int):
    if status != NVFP4_OK:
        msg = lib().nvfp4_last_error().decode()
        raise NVFP4Error(status, msg or lib().nvfp4_strerror(status).decode())
