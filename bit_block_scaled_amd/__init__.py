"""NVFP4 W4A4 linear layer and NVFP4 KV cache for one MI355X (gfx950).

Thin torch-facing binding over the C ABI in ``include/nvfp4.h`` (``libnvfp4.so``):
the functions here only check tensor shapes / dtypes / devices, allocate
outputs as torch tensors and pass raw pointers plus the current HIP stream.
Every step of the computation runs in the library's HIP kernels.

Method: "LongLive-2.0：用 NVFP4 并行底座做长视频生成" (yingwang.github.io), 二、方法 /
NVFP4 量化格式 (E2M1 elements, E4M3 per-16 block scales, FP32 tensor scale) and
二、方法 / 推理底座 (W4A4 inference, NVFP4 KV cache).
"""

from __future__ import annotations

import ctypes as C

import torch

from ._lib import (  # noqa: F401
    LIB_PATH,
    NVFP4_EPI_GELU_TANH,
    NVFP4_NOALLOC_MAX_ELEMENTS,
    NVFP4_Q_ADAPTIVE_4_6,
    NVFP4_Q_BLOCK_2D,
    NVFP4_TILES,
    KVCacheDesc,
    NVFP4Error,
    check,
    header_symbols,
    lib,
)

__all__ = ["quantize", "quantize_into", "gemm", "linear", "linear_noalloc", "linear_q", "KVCache", "NVFP4Error", "lib",
           "gemm_tile", "workspace", "attention_bf16", "attention_workspace_bytes", "quantize_workspace_bytes", "linear_workspace_bytes",
           "linear_q_workspace_bytes", "quantize_rht", "quantize_rht_workspace_bytes", "weight_grad"]


def _stream(device=None):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _need(t, dtype, name, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the NVFP4 kernels run only on the GPU)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A workspace of ``nbytes`` bytes in the state the library requires before
    its first use: all zero.  Reuse it for later calls on the same stream."""
    return torch.zeros((nbytes,), dtype=torch.uint8, device=device)


def quantize_workspace_bytes(M: int, K: int) -> int:
    n = C.c_size_t()
    check(lib().nvfp4_quantize_workspace(M, K, C.byref(n)))
    return n.value


def linear_workspace_bytes(M: int, K: int) -> int:
    n = C.c_size_t()
    check(lib().nvfp4_linear_workspace(M, K, C.byref(n)))
    return n.value


def quantize_into(x, codes, scales, gscale, ws, adaptive46=False, blocks2d=False):
    """nvfp4_quantize (nvfp4_quantize_ex with NVFP4_Q_ADAPTIVE_4_6 when
    ``adaptive46``, NVFP4_Q_BLOCK_2D when ``blocks2d``) into caller-provided
    tensors (no allocation)."""
    M, K = x.shape
    _need(x, torch.bfloat16, "x")
    _need(codes, torch.uint8, "codes", (M, K // 2))
    _need(scales, torch.uint8, "scales", (M, K // 16))
    _need(gscale, torch.float32, "gscale", (1,))
    _need(ws, torch.uint8, "ws")
    qflags = (NVFP4_Q_ADAPTIVE_4_6 if adaptive46 else 0) | (NVFP4_Q_BLOCK_2D if blocks2d else 0)
    check(lib().nvfp4_quantize_ex(_ptr(x), M, K, qflags, _ptr(codes), _ptr(scales), _ptr(gscale),
                                  _ptr(ws), ws.numel(), _stream(x.device)))


def quantize(x: torch.Tensor, adaptive46=False, blocks2d=False):
    """bf16 [M, K] → (codes u8 [M, K/2], scales u8 [M, K/16], gscale f32 [1]);
    ``adaptive46`` selects the adaptive {4, 6} block scales, ``blocks2d`` the
    16x16 two-dimensional blocks (for weights)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    dev = x.device
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    gscale = torch.empty((1,), dtype=torch.float32, device=dev)
    ws = workspace(quantize_workspace_bytes(M, K), dev)
    quantize_into(x, codes, scales, gscale, ws, adaptive46, blocks2d)
    return codes, scales, gscale


def _flags(gelu, tile):
    f = NVFP4_EPI_GELU_TANH if gelu else 0
    if tile is not None:
        f |= NVFP4_TILES[tuple(tile)]
    return f


def gemm(Aq, As, Ag, Wq, Ws, Wg, bias=None, gelu=False, out=None, tile=None):
    """W4A4 GEMM: NVFP4 A [M, K] times NVFP4 Wᵀ ([N, K]) → bf16 [M, N].

    ``tile`` optionally forces the workgroup tile, e.g. (256, 192)."""
    M, K2 = Aq.shape
    N = Wq.shape[0]
    K = 2 * K2
    _need(Aq, torch.uint8, "Aq")
    _need(As, torch.uint8, "As", (M, K // 16))
    _need(Ag, torch.float32, "Ag", (1,))
    _need(Wq, torch.uint8, "Wq", (N, K // 2))
    _need(Ws, torch.uint8, "Ws", (N, K // 16))
    _need(Wg, torch.float32, "Wg", (1,))
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", (N,))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=Aq.device)
    _need(out, torch.bfloat16, "out", (M, N))
    flags = _flags(gelu, tile)
    check(lib().nvfp4_gemm(_ptr(Aq), _ptr(As), _ptr(Ag), _ptr(Wq), _ptr(Ws), _ptr(Wg), _ptr(bias),
                           _ptr(out), M, N, K, flags, _stream(Aq.device)))
    return out


def linear(x, Wq, Ws, Wg, bias=None, gelu=False, out=None, ws=None, tile=None):
    """The W4A4 linear layer: quantise bf16 x [M, K] per call, then GEMM with
    pre-quantised weights.  ``ws`` (uint8, ≥ linear_workspace_bytes, zero
    before its first use: see :func:`workspace`) may be passed to avoid an
    allocation per call."""
    M, K = x.shape
    N = Wq.shape[0]
    _need(x, torch.bfloat16, "x")
    _need(Wq, torch.uint8, "Wq", (N, K // 2))
    _need(Ws, torch.uint8, "Ws", (N, K // 16))
    _need(Wg, torch.float32, "Wg", (1,))
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", (N,))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out", (M, N))
    if ws is None:
        ws = workspace(linear_workspace_bytes(M, K), x.device)
    _need(ws, torch.uint8, "ws")
    flags = _flags(gelu, tile)
    check(lib().nvfp4_linear(_ptr(x), _ptr(Wq), _ptr(Ws), _ptr(Wg), _ptr(bias), _ptr(out),
                             M, N, K, flags, _ptr(ws), ws.numel(), _stream(x.device)))
    return out


def linear_noalloc(x, Wq, Ws, Wg, bias=None, gelu=False, out=None, tile=None):
    """nvfp4_linear_noalloc: the W4A4 linear layer with the library's built-in
    device workspace (no workspace argument, nothing allocated by the library;
    ``out`` may be passed so that this call allocates nothing either).  Calls
    that may overlap on one device race; M·K <= NVFP4_NOALLOC_MAX_ELEMENTS."""
    M, K = x.shape
    N = Wq.shape[0]
    _need(x, torch.bfloat16, "x")
    _need(Wq, torch.uint8, "Wq", (N, K // 2))
    _need(Ws, torch.uint8, "Ws", (N, K // 16))
    _need(Wg, torch.float32, "Wg", (1,))
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", (N,))
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out", (M, N))
    flags = _flags(gelu, tile)
    check(lib().nvfp4_linear_noalloc(_ptr(x), _ptr(Wq), _ptr(Ws), _ptr(Wg), _ptr(bias), _ptr(out),
                                     M, N, K, flags, _stream(x.device)))
    return out


def linear_q_workspace_bytes(M: int, N: int, K: int) -> int:
    n = C.c_size_t()
    check(lib().nvfp4_linear_q_workspace(M, N, K, C.byref(n)))
    return n.value


def linear_q(x, Wq, Ws, Wg, bias=None, gelu=False, out=None, ws=None, tile=None):
    """nvfp4_linear_q: the linear layer's bf16 output handed on in NVFP4.
    Returns (Hq u8 [M, N/2], Hs u8 [M, N/16], Hg f32 [1]); ``out`` may pass
    that triple to write into."""
    M, K = x.shape
    N = Wq.shape[0]
    _need(x, torch.bfloat16, "x")
    _need(Wq, torch.uint8, "Wq", (N, K // 2))
    _need(Ws, torch.uint8, "Ws", (N, K // 16))
    _need(Wg, torch.float32, "Wg", (1,))
    if bias is not None:
        _need(bias, torch.bfloat16, "bias", (N,))
    if out is None:
        out = (torch.empty((M, N // 2), dtype=torch.uint8, device=x.device),
               torch.empty((M, N // 16), dtype=torch.uint8, device=x.device),
               torch.empty((1,), dtype=torch.float32, device=x.device))
    Hq, Hs, Hg = out
    _need(Hq, torch.uint8, "Hq", (M, N // 2))
    _need(Hs, torch.uint8, "Hs", (M, N // 16))
    _need(Hg, torch.float32, "Hg", (1,))
    if ws is None:
        ws = workspace(linear_q_workspace_bytes(M, N, K), x.device)
    _need(ws, torch.uint8, "ws")
    flags = _flags(gelu, tile)
    check(lib().nvfp4_linear_q(_ptr(x), _ptr(Wq), _ptr(Ws), _ptr(Wg), _ptr(bias), M, N, K, flags,
                               _ptr(Hq), _ptr(Hs), _ptr(Hg), _ptr(ws), ws.numel(), _stream(x.device)))
    return Hq, Hs, Hg


class KVCache:
    """NVFP4 KV cache with device buffers held as torch tensors.

    ``append(K, V)`` quantises a chunk of bf16 [T, heads, head_dim] keys and
    values into the cache (one pair of tensor scales per append);
    ``qkv_append(x, W…)`` runs the QKV projection and appends its K and V;
    ``dequant(t0, t1)`` returns bf16 K and V for tokens [t0, t1);
    ``attention(Q, ranges)`` attends over the cache in NVFP4.
    With ``smooth_k`` every append centres each key channel first (the
    centres are kept in ``k_center``, [max_chunks, heads, head_dim] bf16).
    """

    def __init__(self, capacity: int, heads: int, head_dim: int, max_chunks: int, device="cuda",
                 smooth_k: bool = False):
        dev = torch.device(device)
        self.smooth_k = bool(smooth_k)
        self.k_center = (torch.zeros((max_chunks, heads, head_dim), dtype=torch.bfloat16, device=dev)
                         if self.smooth_k else None)
        self.k_codes = torch.zeros((capacity, heads, head_dim // 2), dtype=torch.uint8, device=dev)
        self.v_codes = torch.zeros_like(self.k_codes)
        self.k_scales = torch.zeros((capacity, heads, head_dim // 16), dtype=torch.uint8, device=dev)
        self.v_scales = torch.zeros_like(self.k_scales)
        self.gscale = torch.zeros((max_chunks, 2), dtype=torch.float32, device=dev)
        self.chunk_start = torch.zeros((max_chunks + 1,), dtype=torch.int64, device=dev)
        self.desc = KVCacheDesc(capacity, heads, head_dim, max_chunks,
                                self.k_codes.data_ptr(), self.k_scales.data_ptr(),
                                self.v_codes.data_ptr(), self.v_scales.data_ptr(),
                                self.gscale.data_ptr(), self.chunk_start.data_ptr(), 0, 0,
                                self.k_center.data_ptr() if self.smooth_k else None)
        check(lib().nvfp4_kv_init(C.byref(self.desc)))
        self.device = dev
        self._ws = None

    @property
    def n_tokens(self):
        return self.desc.n_tokens

    @property
    def n_chunks(self):
        return self.desc.n_chunks

    def _smooth_bytes(self, T: int) -> int:
        if not self.smooth_k:
            return 0
        n = C.c_size_t()
        check(lib().nvfp4_kv_smooth_workspace(T, self.desc.heads, self.desc.head_dim, C.byref(n)))
        return n.value

    def workspace_bytes(self, T: int) -> int:
        n = C.c_size_t()
        check(lib().nvfp4_kv_append_workspace(T, self.desc.heads, self.desc.head_dim, C.byref(n)))
        return n.value + self._smooth_bytes(T)

    def append(self, K, V, ws=None, adaptive46=False):
        """Append K, V: bf16 [T, heads, head_dim] tensors, or [T, ld] row views
        (e.g. column slices of a fused QKV output) whose rows hold
        heads·head_dim contiguous values.  ``adaptive46`` selects the adaptive
        {4, 6} block scales for this append."""
        T = K.shape[0]
        HD = self.desc.heads * self.desc.head_dim
        for t, name in ((K, "K"), (V, "V")):
            if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16:
                raise TypeError(f"{name} must be a bf16 GPU tensor")
        if K.dim() == 3:
            _need(K, torch.bfloat16, "K", (T, self.desc.heads, self.desc.head_dim))
            _need(V, torch.bfloat16, "V", (T, self.desc.heads, self.desc.head_dim))
            ld = HD
        else:
            if K.dim() != 2 or tuple(K.shape) != (T, HD) or tuple(V.shape) != (T, HD):
                raise ValueError(f"K/V must be [T, heads, head_dim] or 2-D [T, {HD}] row views")
            if K.stride(1) != 1 or V.stride(1) != 1 or K.stride(0) != V.stride(0):
                raise ValueError("K/V row views need unit column stride and equal row strides")
            ld = K.stride(0) if T > 1 else max(K.stride(0), HD)
        if ws is None:
            if self._ws is None or self._ws.numel() < self.workspace_bytes(T):
                self._ws = workspace(self.workspace_bytes(T), self.device)
            ws = self._ws
        qflags = NVFP4_Q_ADAPTIVE_4_6 if adaptive46 else 0
        check(lib().nvfp4_kv_append_ex(C.byref(self.desc), _ptr(K), _ptr(V), T, ld, qflags, _ptr(ws),
                                       ws.numel(), _stream(self.device)))

    def qkv_workspace_bytes(self, T: int, D: int) -> int:
        n = C.c_size_t()
        check(lib().nvfp4_qkv_append_workspace(T, self.desc.heads, self.desc.head_dim, D, C.byref(n)))
        return n.value + self._smooth_bytes(T)

    def qkv_append(self, x, Wq, Ws, Wg, bias=None, out=None, ws=None, adaptive46=False):
        """nvfp4_qkv_append: the QKV projection of x (bf16 [T, D]) with NVFP4
        weights [3·heads·head_dim, D] (Q, K, V rows stacked), its K and V
        slices appended to the cache as one chunk.  Returns QKV bf16
        [T, 3·heads·head_dim] (or writes ``out``)."""
        _need(x, torch.bfloat16, "x")
        if x.dim() != 2:
            raise ValueError("x must be 2-D [T, D]")
        T, D = x.shape
        N = 3 * self.desc.heads * self.desc.head_dim
        _need(Wq, torch.uint8, "Wq", (N, D // 2))
        _need(Ws, torch.uint8, "Ws", (N, D // 16))
        _need(Wg, torch.float32, "Wg", (1,))
        if bias is not None:
            _need(bias, torch.bfloat16, "bias", (N,))
        if out is None:
            out = torch.empty((T, N), dtype=torch.bfloat16, device=x.device)
        _need(out, torch.bfloat16, "out", (T, N))
        need = self.qkv_workspace_bytes(T, D)
        if ws is None:
            if getattr(self, "_qkv_ws", None) is None or self._qkv_ws.numel() < need:
                self._qkv_ws = workspace(need, self.device)
            ws = self._qkv_ws
        qflags = NVFP4_Q_ADAPTIVE_4_6 if adaptive46 else 0
        check(lib().nvfp4_qkv_append(C.byref(self.desc), _ptr(x), T, D, _ptr(Wq), _ptr(Ws), _ptr(Wg), _ptr(bias),
                                     _ptr(out), qflags, _ptr(ws), ws.numel(), _stream(self.device)))
        return out

    def attention(self, Q, ranges, scale=0.0, out=None, ws=None):
        """nvfp4_kv_attention: softmax(Q·Kᵀ·scale)·V over the cache tokens of
        ``ranges`` (a list of disjoint (start, end) pairs), K/V dequantised in
        the kernel.  ``Q`` is bf16 [Tq, heads, 128] or a [Tq, heads·128] row
        view (e.g. the query slice of a fused QKV output).  Returns O bf16
        [Tq, heads, 128] (or writes ``out``)."""
        Tq, ldq = _rows_view(Q, self.desc.heads, "Q")
        if out is None:
            out = torch.empty((Tq, self.desc.heads, 128), dtype=torch.bfloat16, device=Q.device)
        To, ldo = _rows_view(out, self.desc.heads, "out")
        if To != Tq:
            raise ValueError("out must have Tq rows")
        rng = [(int(a), int(b)) for a, b in ranges]
        Tk = sum(b - a for a, b in rng)
        arr = (C.c_int64 * (2 * len(rng)))(*[v for ab in rng for v in ab])
        if ws is None:
            ws = _attention_ws(Tq, self.desc.heads, max(Tk, 1), Q.device)
        check(lib().nvfp4_kv_attention(C.byref(self.desc), _ptr(Q), Tq, ldq, arr, len(rng), float(scale),
                                       _ptr(out), ldo, _ptr(ws), 0 if ws is None else ws.numel(),
                                       _stream(Q.device)))
        return out

    def reset(self):
        """Forget every token (host counters only; enqueues nothing)."""
        check(lib().nvfp4_kv_init(C.byref(self.desc)))

    def dequant(self, t0: int, t1: int, k_out=None, v_out=None):
        shape = (t1 - t0, self.desc.heads, self.desc.head_dim)
        if k_out is None:
            k_out = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
        if v_out is None:
            v_out = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
        _need(k_out, torch.bfloat16, "k_out", shape)
        _need(v_out, torch.bfloat16, "v_out", shape)
        check(lib().nvfp4_kv_dequant(C.byref(self.desc), t0, t1, _ptr(k_out), _ptr(v_out),
                                     _stream(self.device)))
        return k_out, v_out


def _rows_view(t, heads, name):
    """(rows, row stride) of a bf16 [T, heads, 128] tensor or [T, heads·128] row view."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a bf16 GPU tensor")
    if t.dim() == 3:
        if tuple(t.shape[1:]) != (heads, 128) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [T, {heads}, 128]")
        return t.shape[0], heads * 128
    if t.dim() == 2 and t.shape[1] == heads * 128 and t.stride(1) == 1:
        return t.shape[0], t.stride(0)
    raise ValueError(f"{name} must be [T, {heads}, 128] or a [T, {heads * 128}] row view")


def attention_workspace_bytes(Tq: int, heads: int, Tk: int) -> int:
    n = C.c_size_t()
    check(lib().nvfp4_kv_attention_workspace(Tq, heads, Tk, C.byref(n)))
    return n.value


def _attention_ws(Tq, heads, Tk, device):
    nb = attention_workspace_bytes(Tq, heads, Tk)
    return torch.empty((nb,), dtype=torch.uint8, device=device) if nb else None


def attention_bf16(Q, K, V, scale=0.0, out=None, ws=None):
    """nvfp4_attention_bf16: the same attention with bf16 K and V [Tk, heads,
    128] (or row views): the baseline of the fused NVFP4 read."""
    Tk, ldk = _rows_view(K, K.shape[1] if K.dim() == 3 else K.shape[1] // 128, "K")
    heads = K.shape[1] if K.dim() == 3 else K.shape[1] // 128
    Tv, ldv = _rows_view(V, heads, "V")
    if Tv != Tk or ldv != ldk:
        raise ValueError("K and V must have the same rows and row stride")
    Tq, ldq = _rows_view(Q, heads, "Q")
    if out is None:
        out = torch.empty((Tq, heads, 128), dtype=torch.bfloat16, device=Q.device)
    To, ldo = _rows_view(out, heads, "out")
    if To != Tq:
        raise ValueError("out must have Tq rows")
    if ws is None:
        ws = _attention_ws(Tq, heads, Tk, Q.device)
    check(lib().nvfp4_attention_bf16(_ptr(Q), Tq, ldq, _ptr(K), _ptr(V), Tk, ldk, heads, float(scale),
                                     _ptr(out), ldo, _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream(Q.device)))
    return out


def quantize_rht_workspace_bytes(T: int, N: int) -> int:
    n = C.c_size_t()
    check(lib().nvfp4_quantize_rht_workspace(T, N, C.byref(n)))
    return n.value


def quantize_rht(x, sign_mask: int, codes=None, scales=None, gscale=None, ws=None):
    """nvfp4_quantize_rht: bf16 x [T, N] (rows may be strided, features
    contiguous) → the NVFP4 transpose of its random Hadamard transform along T:
    (codes u8 [N, T/2], scales u8 [N, T/16], gscale f32 [1]).  ``sign_mask``
    holds the 16 random signs (bit k set: s_k = −1); use the same mask for both
    operands of a weight gradient."""
    if not isinstance(x, torch.Tensor) or x.dim() != 2:
        raise ValueError("x must be a 2-D tensor [T, N]")
    T, N = x.shape
    if not x.is_cuda or x.dtype != torch.bfloat16:
        raise TypeError("x must be a bf16 GPU tensor")
    if x.stride(1) != 1:
        raise ValueError("x must have contiguous rows")
    dev = x.device
    if codes is None:
        codes = torch.empty((N, T // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((N, T // 16), dtype=torch.uint8, device=dev)
    if gscale is None:
        gscale = torch.empty((1,), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty((quantize_rht_workspace_bytes(T, N),), dtype=torch.uint8, device=dev)
    _need(codes, torch.uint8, "codes", (N, T // 2))
    _need(scales, torch.uint8, "scales", (N, T // 16))
    _need(gscale, torch.float32, "gscale", (1,))
    _need(ws, torch.uint8, "ws")
    check(lib().nvfp4_quantize_rht(_ptr(x), T, N, x.stride(0), int(sign_mask), _ptr(codes), _ptr(scales),
                                   _ptr(gscale), _ptr(ws), ws.numel(), _stream(dev)))
    return codes, scales, gscale


def weight_grad(dy, x, sign_mask: int, out=None, tile=None):
    """dW = dyᵀ·x for dy [T, O] and x [T, I] (bf16): both operands through
    quantize_rht with the same signs, then the W4A4 GEMM → bf16 [O, I]."""
    return gemm(*quantize_rht(dy, sign_mask), *quantize_rht(x, sign_mask), out=out, tile=tile)


def gemm_tile(M: int, N: int, K: int) -> tuple:
    """Workgroup tile (BM, BN) the library uses for an M x N x K GEMM."""
    bm, bn = C.c_int(), C.c_int()
    check(lib().nvfp4_gemm_tile(M, N, K, C.byref(bm), C.byref(bn)))
    return bm.value, bn.value
