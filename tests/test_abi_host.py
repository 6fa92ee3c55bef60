"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function include/nvfp4.h declares, and
reject every invalid argument on the host — with the documented status code,
before anything is enqueued.  No call here passes validation: pointers are
fake addresses that are never dereferenced.
"""

import ctypes as C
import os
import subprocess

import pytest

import bit_block_scaled_amd as nv
from bit_block_scaled_amd import _lib

EINVAL, EWS, ECAP = _lib.NVFP4_EINVAL, _lib.NVFP4_EWORKSPACE, _lib.NVFP4_ECAPACITY

FAKE = 0x100000           # 16-byte aligned, never dereferenced
MIS = FAKE + 8            # misaligned


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail(f"{_lib.LIB_PATH} not built (run __graft_entry__.build())")
    return nv.lib()


def test_exports_every_declared_symbol(L):
    declared = _lib.header_symbols()
    assert len(declared) >= 12
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    for s in declared:
        assert getattr(L, s) is not None


def test_strerror(L):
    assert L.nvfp4_strerror(0) == b"ok"
    assert b"invalid" in L.nvfp4_strerror(EINVAL)
    assert b"workspace" in L.nvfp4_strerror(EWS)
    assert b"capacity" in L.nvfp4_strerror(ECAP)
    assert L.nvfp4_strerror(99) == b"unknown status"


def _ws(L, M, K):
    n = C.c_size_t()
    return L.nvfp4_quantize_workspace(M, K, C.byref(n)), n.value


def test_workspace_queries(L):
    s, n = _ws(L, 4096, 3072)
    assert s == 0 and n >= 4096
    assert _ws(L, 4096, 48)[0] == EINVAL
    assert _ws(L, 0, 64)[0] == EINVAL
    assert L.nvfp4_quantize_workspace(4, 64, None) == EINVAL
    n = C.c_size_t()
    assert L.nvfp4_linear_workspace(4096, 3072, C.byref(n)) == 0
    assert n.value >= 4096 * 3072 // 2 + 4096 * 3072 // 16
    assert L.nvfp4_kv_append_workspace(880, 24, 128, C.byref(n)) == 0 and n.value > 0
    assert L.nvfp4_kv_append_workspace(880, 24, 100, C.byref(n)) == EINVAL
    bm, bn = C.c_int(), C.c_int()
    assert L.nvfp4_gemm_tile(4096, 9216, 3072, C.byref(bm), C.byref(bn)) == 0
    assert bm.value % 64 == 0 and bn.value % 64 == 0


def _q(L, x=FAKE, M=64, K=64, codes=FAKE, scales=FAKE, g=FAKE, ws=FAKE, wsb=1 << 20):
    return L.nvfp4_quantize(x, M, K, codes, scales, g, ws, wsb, None)


def test_quantize_rejects(L):
    assert _q(L, x=None) == EINVAL
    assert _q(L, codes=None) == EINVAL
    assert _q(L, x=MIS) == EINVAL
    assert _q(L, scales=MIS) == EINVAL
    assert _q(L, K=48) == EINVAL            # K % 32
    assert _q(L, K=16) == EINVAL
    assert _q(L, M=0) == EINVAL
    assert _q(L, M=-5) == EINVAL
    assert _q(L, M=1 << 30, K=1 << 10) == EINVAL          # more than 2^36 elements
    assert _q(L, ws=None) == EWS
    assert _q(L, wsb=16) == EWS
    assert b"workspace" in L.nvfp4_last_error()


def _g(L, Aq=FAKE, As=FAKE, Ag=FAKE, Wq=FAKE, Ws=FAKE, Wg=FAKE, bias=None, Cp=FAKE, M=64, N=64,
       K=64, flags=0):
    return L.nvfp4_gemm(Aq, As, Ag, Wq, Ws, Wg, bias, Cp, M, N, K, flags, None)


def test_gemm_rejects(L):
    assert _g(L, Aq=None) == EINVAL
    assert _g(L, Ws=None) == EINVAL
    assert _g(L, Wg=None) == EINVAL
    assert _g(L, Cp=None) == EINVAL
    assert _g(L, Cp=MIS) == EINVAL
    assert _g(L, Wq=MIS) == EINVAL
    assert _g(L, bias=MIS) == EINVAL
    assert _g(L, K=80) == EINVAL
    assert _g(L, N=0) == EINVAL
    assert _g(L, M=0) == EINVAL
    assert _g(L, flags=0x10) == EINVAL
    assert b"flag" in L.nvfp4_last_error()


def test_linear_rejects(L):
    f = L.nvfp4_linear
    assert f(None, FAKE, FAKE, FAKE, None, FAKE, 64, 64, 64, 0, FAKE, 1 << 20, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 64, 64, 0, FAKE, 16, None) == EWS
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 64, 64, 0, None, 1 << 20, None) == EWS
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 64, 40, 0, FAKE, 1 << 20, None) == EINVAL


def _desc(**kw):
    d = _lib.KVCacheDesc(100, 24, 128, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 7, 7)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_kv_init_and_rejects(L):
    d = _desc()
    assert L.nvfp4_kv_init(C.byref(d)) == 0
    assert d.n_tokens == 0 and d.n_chunks == 0
    assert L.nvfp4_kv_init(None) == EINVAL
    assert L.nvfp4_kv_init(C.byref(_desc(head_dim=100))) == EINVAL
    assert L.nvfp4_kv_init(C.byref(_desc(capacity=0))) == EINVAL
    assert L.nvfp4_kv_init(C.byref(_desc(max_chunks=0))) == EINVAL
    assert L.nvfp4_kv_init(C.byref(_desc(k_codes=None))) == EINVAL
    assert L.nvfp4_kv_init(C.byref(_desc(v_scales=MIS))) == EINVAL


def test_kv_append_capacity_and_args(L):
    d = _desc()
    assert L.nvfp4_kv_init(C.byref(d)) == 0
    ws, wsb = FAKE, 1 << 20
    # token capacity
    assert L.nvfp4_kv_append(C.byref(d), FAKE, FAKE, 101, 3072, ws, wsb, None) == ECAP
    assert d.n_tokens == 0 and d.n_chunks == 0
    # chunk slots
    d.n_tokens, d.n_chunks = 10, 4
    assert L.nvfp4_kv_append(C.byref(d), FAKE, FAKE, 1, 3072, ws, wsb, None) == ECAP
    assert d.n_tokens == 10 and d.n_chunks == 4
    d.n_tokens, d.n_chunks = 0, 0
    assert L.nvfp4_kv_append(C.byref(d), FAKE, FAKE, 0, 3072, ws, wsb, None) == EINVAL
    assert L.nvfp4_kv_append(C.byref(d), None, FAKE, 1, 3072, ws, wsb, None) == EINVAL
    assert L.nvfp4_kv_append(C.byref(d), FAKE, MIS, 1, 3072, ws, wsb, None) == EINVAL
    assert L.nvfp4_kv_append(C.byref(d), FAKE, FAKE, 1, 3072, ws, 8, None) == EWS
    assert L.nvfp4_kv_append(None, FAKE, FAKE, 1, 3072, ws, wsb, None) == EINVAL
    assert L.nvfp4_kv_append(C.byref(d), FAKE, FAKE, 1, 3000, ws, wsb, None) == EINVAL   # ld < H*D
    assert L.nvfp4_kv_append(C.byref(d), FAKE, FAKE, 1, 3076, ws, wsb, None) == EINVAL   # ld % 8
    # a corrupted descriptor
    assert L.nvfp4_kv_append(C.byref(_desc(n_tokens=500)), FAKE, FAKE, 1, 3072, ws, wsb, None) == EINVAL


def test_kv_smoothing_host_checks(L):
    # the centre table is optional (NULL: no K-smoothing) and must be aligned
    assert L.nvfp4_kv_init(C.byref(_desc(k_center=MIS))) == EINVAL
    assert L.nvfp4_kv_init(C.byref(_desc(k_center=None))) == 0
    d = _desc(k_center=FAKE)
    assert L.nvfp4_kv_init(C.byref(d)) == 0
    n, m = C.c_size_t(), C.c_size_t()
    assert L.nvfp4_kv_append_workspace(880, 24, 128, C.byref(n)) == 0
    assert L.nvfp4_kv_smooth_workspace(880, 24, 128, C.byref(m)) == 0
    assert 3072 * 8 <= m.value < 880 * 3072                         # channel sums, no copy of the keys
    assert L.nvfp4_kv_smooth_workspace(880, 24, 100, C.byref(m)) == EINVAL
    assert L.nvfp4_kv_smooth_workspace(0, 24, 128, C.byref(m)) == EINVAL
    assert L.nvfp4_kv_smooth_workspace(880, 24, 128, None) == EINVAL
    # an append to a smoothed cache needs both parts; with only the plain
    # workspace it is refused before anything is enqueued
    assert L.nvfp4_kv_append_workspace(10, 24, 128, C.byref(n)) == 0
    assert L.nvfp4_kv_append(C.byref(d), FAKE, FAKE, 10, 3072, FAKE, n.value, None) == EWS
    assert d.n_tokens == 0 and d.n_chunks == 0
    need = C.c_size_t()
    assert L.nvfp4_qkv_append_workspace(10, 24, 128, 3072, C.byref(need)) == 0
    assert L.nvfp4_qkv_append(C.byref(d), FAKE, 10, 3072, FAKE, FAKE, FAKE, None, FAKE, 0, FAKE,
                              need.value, None) == EWS
    assert d.n_tokens == 0 and d.n_chunks == 0


def test_kv_dequant_range(L):
    d = _desc()
    assert L.nvfp4_kv_init(C.byref(d)) == 0
    d.n_tokens, d.n_chunks = 20, 1
    assert L.nvfp4_kv_dequant(C.byref(d), 0, 21, FAKE, FAKE, None) == EINVAL
    assert L.nvfp4_kv_dequant(C.byref(d), 5, 4, FAKE, FAKE, None) == EINVAL
    assert L.nvfp4_kv_dequant(C.byref(d), -1, 4, FAKE, FAKE, None) == EINVAL
    assert L.nvfp4_kv_dequant(C.byref(d), 0, 4, None, FAKE, None) == EINVAL
    assert L.nvfp4_kv_dequant(C.byref(d), 0, 4, FAKE, MIS, None) == EINVAL
    # an empty range is a valid no-op that enqueues nothing
    assert L.nvfp4_kv_dequant(C.byref(d), 3, 3, FAKE, FAKE, None) == 0
    assert L.nvfp4_kv_dequant(C.byref(d), 3, 3, None, None, None) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        nv.quantize(x)


def test_quantizer_flags_rejected(L):
    # unknown quantiser flags are argument errors, found before any launch
    assert L.nvfp4_quantize_ex(FAKE, 64, 64, 0x40, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == EINVAL
    assert L.nvfp4_quantize_ex(FAKE, 64, 64, 0x1, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == EINVAL
    # the adaptive {4, 6} scales and the 2-D blocks exclude each other
    both = _lib.NVFP4_Q_ADAPTIVE_4_6 | _lib.NVFP4_Q_BLOCK_2D
    assert L.nvfp4_quantize_ex(FAKE, 64, 64, both, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == EINVAL
    assert b"exclude" in L.nvfp4_last_error()
    d = _lib.KVCacheDesc(100, 24, 128, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0)
    assert L.nvfp4_kv_init(C.byref(d)) == 0
    # 2-D blocks are for weights; the KV cache keeps 1-D blocks along head_dim
    for f in (0x30, _lib.NVFP4_Q_BLOCK_2D):
        assert L.nvfp4_kv_append_ex(C.byref(d), FAKE, FAKE, 1, 3072, f, FAKE, 1 << 20, None) == EINVAL
        assert d.n_tokens == 0 and d.n_chunks == 0
        assert b"flags" in L.nvfp4_last_error()


def test_linear_q_rejects(L):
    n = C.c_size_t()
    assert L.nvfp4_linear_q_workspace(8192, 14336, 3072, C.byref(n)) == 0
    assert n.value >= 8192 * 14336 * 2                       # holds the bf16 output
    assert L.nvfp4_linear_q_workspace(64, 48, 64, C.byref(n)) == EINVAL      # N % 32
    args = (FAKE, FAKE, FAKE, FAKE, None)
    assert L.nvfp4_linear_q(*args, 64, 48, 64, 0, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == EINVAL
    assert L.nvfp4_linear_q(*args, 64, 64, 64, 0, FAKE, FAKE, FAKE, FAKE, 16, None) == EWS
    assert L.nvfp4_linear_q(*args, 64, 64, 64, 0x80, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == EINVAL
    assert L.nvfp4_linear_q(*args, 64, 64, 64, 0, MIS, FAKE, FAKE, FAKE, 1 << 30, None) == EINVAL


def test_linear_noalloc_rejects(L):
    # argument errors and the size limit of the built-in workspace are found on
    # the host, before the device array is looked up or anything is enqueued
    f = L.nvfp4_linear_noalloc
    lim = _lib.NVFP4_NOALLOC_MAX_ELEMENTS
    assert f(None, FAKE, FAKE, FAKE, None, FAKE, 64, 64, 64, 0, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, MIS, FAKE, 64, 64, 64, 0, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, 64, 64, 40, 0, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, None, FAKE, lim // 3072 + 1, 64, 3072, 0, None) == EINVAL
    msg = L.nvfp4_last_error()
    assert b"NVFP4_NOALLOC_MAX_ELEMENTS" in msg and str(lim).encode() in msg


def test_launch_event_hook_rejects(L):
    assert L.nvfp4_testing_set_launch_events(None, 2) == EINVAL
    assert L.nvfp4_testing_set_launch_events(None, -1) == EINVAL
    assert L.nvfp4_testing_set_launch_events(None, 0) == 0


def test_quantize_rht_rejects(L):
    n = C.c_size_t()
    assert L.nvfp4_quantize_rht_workspace(8192, 14336, C.byref(n)) == 0 and n.value >= 4
    assert L.nvfp4_quantize_rht_workspace(48, 64, C.byref(n)) == EINVAL            # T % 32
    assert L.nvfp4_quantize_rht_workspace(64, 0, C.byref(n)) == EINVAL
    f = L.nvfp4_quantize_rht
    ok = (FAKE, 64, 40, 40, 0x1234, FAKE, FAKE, FAKE, FAKE, 1 << 20, None)
    def call(**kw):
        a = list(ok)
        for k, v in kw.items():
            a[["x", "T", "N", "ldx", "mask", "codes", "scales", "g", "ws", "wsb", "st"].index(k)] = v
        return f(*a)
    assert call(T=48) == EINVAL                  # not a multiple of 32
    assert call(ldx=36) == EINVAL                # below N
    assert call(ldx=44) == EINVAL                # not a multiple of 8
    assert call(mask=1 << 16) == EINVAL          # 17-bit sign mask
    assert call(x=MIS) == EINVAL
    assert call(codes=None) == EINVAL
    assert call(scales=MIS) == EINVAL
    assert call(g=FAKE + 2) == EINVAL
    assert call(wsb=16) == EWS
    assert call(ws=None) == EWS
    assert b"quantize_rht" in L.nvfp4_last_error()


def test_qkv_append_rejects(L):
    d = _desc()
    assert L.nvfp4_kv_init(C.byref(d)) == 0
    n = C.c_size_t()
    assert L.nvfp4_qkv_append_workspace(880, 24, 128, 3072, C.byref(n)) == 0
    need = n.value
    assert need >= 880 * 3072 // 2                          # holds the quantised activations
    assert L.nvfp4_qkv_append_workspace(880, 24, 100, 3072, C.byref(n)) == EINVAL
    assert L.nvfp4_qkv_append_workspace(880, 24, 128, 3000, C.byref(n)) == EINVAL
    f = L.nvfp4_qkv_append
    args = [C.byref(d), FAKE, 10, 3072, FAKE, FAKE, FAKE, None, FAKE, 0, FAKE, need, None]
    def call(i, v):
        a = list(args)
        a[i] = v
        return f(*a)
    assert call(9, 0x80) == EINVAL                           # unknown flag
    assert call(1, MIS) == EINVAL                            # x misaligned
    assert call(8, None) == EINVAL                           # no output
    assert call(3, 3000) == EINVAL                           # D % 32
    assert call(11, 64) == EWS                               # workspace too small
    assert call(2, 101) == ECAP                              # 101 tokens into a 100-token cache
    d.n_chunks = 4
    assert f(*args) == ECAP                                  # no chunk slot
    assert d.n_tokens == 0 and d.n_chunks == 4               # unchanged on error


def test_every_workspace_starts_with_the_quantiser_head(L):
    # Every workspace reserves the same 24 KiB head (the quantiser scratch of
    # two tensors) before its other buffers, so the sizes of the calls that
    # keep more than the quantiser scratch are at least the head plus those
    # buffers; a call without split results (one key split) needs none.
    HEAD = 2 * (8 * 1024 + 4 * 1024)
    n = C.c_size_t()
    assert L.nvfp4_quantize_workspace(4096, 3072, C.byref(n)) == 0 and n.value == HEAD // 2
    assert L.nvfp4_kv_append_workspace(880, 24, 128, C.byref(n)) == 0 and n.value == HEAD
    assert L.nvfp4_linear_workspace(4096, 3072, C.byref(n)) == 0
    assert n.value >= HEAD + 4096 * 3072 // 2 + 4096 * 3072 // 16
    assert L.nvfp4_linear_q_workspace(4096, 9216, 3072, C.byref(n)) == 0
    assert n.value >= HEAD + 4096 * 3072 * 9 // 16 + 4096 * 9216 * 2
    assert L.nvfp4_qkv_append_workspace(880, 24, 128, 3072, C.byref(n)) == 0
    assert n.value >= HEAD + 880 * 3072 * 9 // 16
    assert L.nvfp4_quantize_rht_workspace(8192, 3072, C.byref(n)) == 0 and n.value > HEAD
    assert L.nvfp4_kv_attention_workspace(880, 24, 65536, C.byref(n)) == 0
    assert n.value >= HEAD + 2 * 880 * 24 * 128 * 4                 # several key splits
    assert L.nvfp4_kv_attention_workspace(1, 1, 64, C.byref(n)) == 0 and n.value == 0   # one split
