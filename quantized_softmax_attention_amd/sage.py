"""Thin Python binding of libsage_mi355x.so (C ABI in include/sage_mi355x.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  torch supplies device memory and the current stream.  The
library must have been built (``python -m quantized_softmax_attention_amd.build``);
there is no fallback of any kind, and every non-zero status raises SageError.

The functions carry the C names.  Tensor arguments are torch tensors on the GPU:
bf16 inputs are [B, N, H, D] views with unit last stride (any batch/token/head
strides, e.g. column slices of a packed [B, N, 3*H*D] projection buffer).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsage_mi355x.so")

HEAD_DIM = 128
Q_BLOCK = 32
K_BLOCK = 64
P_TILE = 64
N_ALIGN = 256

STATUS = {0: "SAGE_OK", 1: "SAGE_ERR_NULL", 2: "SAGE_ERR_SHAPE", 3: "SAGE_ERR_STRIDE", 4: "SAGE_ERR_ALIGN",
          5: "SAGE_ERR_WORKSPACE", 6: "SAGE_ERR_HIP", 7: "SAGE_ERR_VALUE"}


class SageError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (fn, STATUS.get(status, status), sage_status_str(status)))


class BF16In(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_n", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


class BF16Out(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_n", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libsage_mi355x.so is not built (run python -m quantized_softmax_attention_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        pin, pout = ctypes.POINTER(BF16In), ctypes.POINTER(BF16Out)
        L.sage_npad.argtypes, L.sage_npad.restype = [i], ctypes.c_int64
        L.sage_qk_workspace_bytes.argtypes, L.sage_qk_workspace_bytes.restype = [i, i, i, i], sz
        L.sage_v_workspace_bytes.argtypes, L.sage_v_workspace_bytes.restype = [i, i, i, i], sz
        L.sage_qkv_workspace_bytes.argtypes, L.sage_qkv_workspace_bytes.restype = [i, i, i, i], sz
        L.sage_qkv_rope_workspace_bytes.argtypes, L.sage_qkv_rope_workspace_bytes.restype = [i, i, i, i], sz
        L.sage_quantize_qkv.argtypes = [pin, pin, pin, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sage_quantize_qkv_noalloc.argtypes = [pin, pin, pin, i, i, i, i, vp, vp, vp, vp, vp, vp, vp, vp]
        L.sage_qkv_noalloc_max_bytes.argtypes, L.sage_qkv_noalloc_max_bytes.restype = [], sz
        L.sage_quantize_qk.argtypes = [pin, pin, i, i, i, i, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sage_quantize_v.argtypes = [pin, i, i, i, i, vp, vp, vp, sz, vp]
        L.sage_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, pout, vp]
        L.sage_attn_fwd_bf16.argtypes = [pin, pin, pin, i, i, i, i, f, pout, vp]
        L.sage_attn_fwd_int8qk.argtypes = [vp, vp, vp, vp, pin, i, i, i, i, f, pout, vp]
        L.sage_qk_norm_rope.argtypes = [pout, pout, i, i, i, i, vp, vp, vp, f, vp]
        L.sage_quantize_qkv_rope.argtypes = [pin, pin, pin, i, i, i, i, vp, vp, vp, f,
                                             vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.sage_mx_quantize.argtypes = [pin, i, i, i, i, i, vp, vp, vp]
        L.sage_attn_fwd_mx.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, vp, vp]
        for fn in ("sage_quantize_qk", "sage_quantize_v", "sage_quantize_qkv", "sage_quantize_qkv_noalloc",
                   "sage_attn_fwd", "sage_attn_fwd_bf16",
                   "sage_attn_fwd_int8qk", "sage_mx_quantize", "sage_attn_fwd_mx", "sage_qk_norm_rope",
                   "sage_quantize_qkv_rope"):
            getattr(L, fn).restype = i
        L.sage_status_str.argtypes, L.sage_status_str.restype = [i], ctypes.c_char_p
        _lib = L
    return _lib


def sage_status_str(status: int) -> str:
    return lib().sage_status_str(int(status)).decode()


def _check(status: int, fn: str) -> None:
    if status != 0:
        raise SageError(status, fn)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _shape(t: torch.Tensor):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, N, H, D] view with unit last stride")
    return tuple(t.shape)


def bf16_in(t: torch.Tensor) -> BF16In:
    _shape(t)
    if t.dtype != torch.bfloat16:
        raise TypeError("expected bfloat16")
    return BF16In(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def bf16_out(t: torch.Tensor) -> BF16Out:
    _shape(t)
    if t.dtype != torch.bfloat16:
        raise TypeError("expected bfloat16")
    return BF16Out(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _on_gpu(name: str, t) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: expected a torch tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s: the library takes device memory; got a tensor on %s" % (name, t.device))


def _need(name: str, t, dtype, count: int) -> None:
    """A library-layout buffer: on the GPU, of `dtype`, contiguous, with at
    least `count` elements (the kernels write every one of them)."""
    _on_gpu(name, t)
    if t.dtype != dtype:
        raise TypeError("%s: expected %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s: expected a contiguous buffer" % name)
    if t.numel() < count:
        raise ValueError("%s: holds %d elements, %d needed" % (name, t.numel(), count))


def _same_device(*tensors) -> None:
    devs = {t.device for t in tensors if isinstance(t, torch.Tensor)}
    if len(devs) > 1:
        raise ValueError("all tensors of one call must be on one GPU; got %s" % sorted(map(str, devs)))


def _views(shape, **views) -> None:
    for name, t in views.items():
        _on_gpu(name, t)
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _codes(B: int, N: int, H: int, D: int, q_codes=None, q_scale=None, k_codes=None, k_scale=None, k_mean=None,
           v_codes=None, v_scale=None) -> None:
    """Size, type and placement checks of the code and scale buffers (the C ABI
    takes their pointers as given, so an undersized buffer would be overrun)."""
    npad = (N + N_ALIGN - 1) // N_ALIGN * N_ALIGN
    spec = {"q_codes": (q_codes, torch.int8, B * H * npad * D), "q_scale": (q_scale, torch.float32,
            B * H * npad // Q_BLOCK), "k_codes": (k_codes, torch.int8, B * H * npad * D),
            "k_scale": (k_scale, torch.float32, B * H * npad // K_BLOCK), "k_mean": (k_mean, torch.float32, B * H * D),
            "v_codes": (v_codes, torch.uint8, B * H * npad * D), "v_scale": (v_scale, torch.float32, B * H * D)}
    for name, (t, dtype, count) in spec.items():
        if t is not None:
            _need(name, t, dtype, count)


def _workspace(t) -> int:
    _on_gpu("workspace", t)
    if not t.is_contiguous():
        raise ValueError("workspace: expected a contiguous buffer")
    return t.numel() * t.element_size()


def sage_npad(N: int) -> int:
    return int(lib().sage_npad(N))


def sage_qk_workspace_bytes(B: int, N: int, H: int, D: int = HEAD_DIM) -> int:
    return int(lib().sage_qk_workspace_bytes(B, N, H, D))


def sage_v_workspace_bytes(B: int, N: int, H: int, D: int = HEAD_DIM) -> int:
    return int(lib().sage_v_workspace_bytes(B, N, H, D))


def sage_quantize_qk(q, k, q_codes, q_scale, k_codes, k_scale, k_mean, workspace, stream=None) -> None:
    B, N, H, D = _shape(q)
    _views((B, N, H, D), q=q, k=k)
    _codes(B, N, H, D, q_codes=q_codes, q_scale=q_scale, k_codes=k_codes, k_scale=k_scale, k_mean=k_mean)
    ws = _workspace(workspace)
    _same_device(q, k, q_codes, q_scale, k_codes, k_scale, k_mean, workspace)
    qi, ki = bf16_in(q), bf16_in(k)
    st = lib().sage_quantize_qk(ctypes.byref(qi), ctypes.byref(ki), B, N, H, D, _ptr(q_codes), _ptr(q_scale),
                                _ptr(k_codes), _ptr(k_scale), _ptr(k_mean), _ptr(workspace), ws, _stream(stream))
    _check(st, "sage_quantize_qk")


def sage_quantize_v(v, v_codes, v_scale, workspace, stream=None) -> None:
    B, N, H, D = _shape(v)
    _views((B, N, H, D), v=v)
    _codes(B, N, H, D, v_codes=v_codes, v_scale=v_scale)
    ws = _workspace(workspace)
    _same_device(v, v_codes, v_scale, workspace)
    vi = bf16_in(v)
    st = lib().sage_quantize_v(ctypes.byref(vi), B, N, H, D, _ptr(v_codes), _ptr(v_scale), _ptr(workspace), ws,
                               _stream(stream))
    _check(st, "sage_quantize_v")


def sage_qkv_workspace_bytes(B: int, N: int, H: int, D: int = HEAD_DIM) -> int:
    return lib().sage_qkv_workspace_bytes(B, N, H, D)


def sage_qkv_rope_workspace_bytes(B: int, N: int, H: int, D: int = HEAD_DIM) -> int:
    return lib().sage_qkv_rope_workspace_bytes(B, N, H, D)


def sage_quantize_qkv(q, k, v, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale, workspace,
                      stream=None) -> None:
    B, N, H, D = _shape(q)
    _views((B, N, H, D), q=q, k=k, v=v)
    _codes(B, N, H, D, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale)
    ws = _workspace(workspace)
    _same_device(q, k, v, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale, workspace)
    qi, ki, vi = bf16_in(q), bf16_in(k), bf16_in(v)
    st = lib().sage_quantize_qkv(ctypes.byref(qi), ctypes.byref(ki), ctypes.byref(vi), B, N, H, D, _ptr(q_codes),
                                 _ptr(q_scale), _ptr(k_codes), _ptr(k_scale), _ptr(k_mean), _ptr(v_codes),
                                 _ptr(v_scale), _ptr(workspace), ws, _stream(stream))
    _check(st, "sage_quantize_qkv")


def sage_qkv_noalloc_max_bytes() -> int:
    return int(lib().sage_qkv_noalloc_max_bytes())


def sage_quantize_qkv_noalloc(q, k, v, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale,
                              stream=None) -> None:
    """sage_quantize_qkv without a workspace: its scratch is the library's own device array (see the header)."""
    B, N, H, D = _shape(q)
    _views((B, N, H, D), q=q, k=k, v=v)
    _codes(B, N, H, D, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale)
    _same_device(q, k, v, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale)
    qi, ki, vi = bf16_in(q), bf16_in(k), bf16_in(v)
    st = lib().sage_quantize_qkv_noalloc(ctypes.byref(qi), ctypes.byref(ki), ctypes.byref(vi), B, N, H, D,
                                         _ptr(q_codes), _ptr(q_scale), _ptr(k_codes), _ptr(k_scale), _ptr(k_mean),
                                         _ptr(v_codes), _ptr(v_scale), _stream(stream))
    _check(st, "sage_quantize_qkv_noalloc")


def _norm_rope_params(N: int, D: int, gamma_q, gamma_k, rope) -> None:
    _need("gamma_q", gamma_q, torch.float32, D)
    _need("gamma_k", gamma_k, torch.float32, D)
    _need("rope", rope, torch.float32, N * D)
    if tuple(rope.shape) != (N, D // 2, 2):
        raise ValueError("rope: shape %s, expected %s" % (tuple(rope.shape), (N, D // 2, 2)))


def sage_qk_norm_rope(q, k, gamma_q, gamma_k, rope, eps: float, stream=None) -> None:
    """RMSNorm + RoPE of the Q and K views, in place."""
    B, N, H, D = _shape(q)
    _views((B, N, H, D), q=q, k=k)
    _norm_rope_params(N, D, gamma_q, gamma_k, rope)
    _same_device(q, k, gamma_q, gamma_k, rope)
    qo, ko = bf16_out(q), bf16_out(k)
    st = lib().sage_qk_norm_rope(ctypes.byref(qo), ctypes.byref(ko), B, N, H, D, _ptr(gamma_q), _ptr(gamma_k),
                                 _ptr(rope), float(eps), _stream(stream))
    _check(st, "sage_qk_norm_rope")


def sage_quantize_qkv_rope(q, k, v, gamma_q, gamma_k, rope, eps: float, q_codes, q_scale, k_codes, k_scale, k_mean,
                           v_codes, v_scale, workspace, stream=None) -> None:
    B, N, H, D = _shape(q)
    _views((B, N, H, D), q=q, k=k, v=v)
    _norm_rope_params(N, D, gamma_q, gamma_k, rope)
    _codes(B, N, H, D, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale)
    ws = _workspace(workspace)
    _same_device(q, k, v, gamma_q, gamma_k, rope, q_codes, q_scale, k_codes, k_scale, k_mean, v_codes, v_scale,
                 workspace)
    qi, ki, vi = bf16_in(q), bf16_in(k), bf16_in(v)
    st = lib().sage_quantize_qkv_rope(ctypes.byref(qi), ctypes.byref(ki), ctypes.byref(vi), B, N, H, D, _ptr(gamma_q),
                                      _ptr(gamma_k), _ptr(rope), float(eps), _ptr(q_codes), _ptr(q_scale),
                                      _ptr(k_codes), _ptr(k_scale), _ptr(k_mean), _ptr(v_codes), _ptr(v_scale),
                                      _ptr(workspace), ws, _stream(stream))
    _check(st, "sage_quantize_qkv_rope")


def sage_attn_fwd(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, out, sm_scale=None, stream=None) -> None:
    B, N, H, D = _shape(out)
    _views((B, N, H, D), out=out)
    _codes(B, N, H, D, q_codes, q_scale, k_codes, k_scale, None, v_codes, v_scale)
    _same_device(out, q_codes, q_scale, k_codes, k_scale, v_codes, v_scale)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    o = bf16_out(out)
    st = lib().sage_attn_fwd(_ptr(q_codes), _ptr(q_scale), _ptr(k_codes), _ptr(k_scale), _ptr(v_codes),
                             _ptr(v_scale), B, N, H, D, float(sm_scale), ctypes.byref(o), _stream(stream))
    _check(st, "sage_attn_fwd")


def sage_attn_fwd_bf16(q, k, v, out, sm_scale=None, stream=None) -> None:
    B, N, H, D = _shape(q)
    _views((B, N, H, D), q=q, k=k, v=v, out=out)
    _same_device(q, k, v, out)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    qi, ki, vi, o = bf16_in(q), bf16_in(k), bf16_in(v), bf16_out(out)
    st = lib().sage_attn_fwd_bf16(ctypes.byref(qi), ctypes.byref(ki), ctypes.byref(vi), B, N, H, D,
                                  float(sm_scale), ctypes.byref(o), _stream(stream))
    _check(st, "sage_attn_fwd_bf16")


def sage_attn_fwd_int8qk(q_codes, q_scale, k_codes, k_scale, v, out, sm_scale=None, stream=None) -> None:
    B, N, H, D = _shape(out)
    _views((B, N, H, D), v=v, out=out)
    _codes(B, N, H, D, q_codes, q_scale, k_codes, k_scale)
    _same_device(v, out, q_codes, q_scale, k_codes, k_scale)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    vi, o = bf16_in(v), bf16_out(out)
    st = lib().sage_attn_fwd_int8qk(_ptr(q_codes), _ptr(q_scale), _ptr(k_codes), _ptr(k_scale), ctypes.byref(vi),
                                    B, N, H, D, float(sm_scale), ctypes.byref(o), _stream(stream))
    _check(st, "sage_attn_fwd_int8qk")


MX_E4M3, MX_E2M1 = 0, 1


def mx_out(B: int, N: int, H: int, fmt: int, device="cuda", D: int = HEAD_DIM):
    """Token-major MX output buffers: codes [B, N, H*D] (E4M3) or [B, N, H*D/2]
    (E2M1 pairs) and E8M0 scales [B, N, H*D/32]."""
    per = H * D if fmt == MX_E4M3 else H * D // 2
    dev = torch.device(device)
    return (torch.empty(B, N, per, dtype=torch.uint8, device=dev),
            torch.empty(B, N, H * D // 32, dtype=torch.uint8, device=dev))


def _mx_shape(codes, scales, fmt):
    """(B, N, H) of token-major MX buffers: codes [B, N, H*D] (E4M3) or
    [B, N, H*D/2] (E2M1), scales [B, N, H*D/32], uint8, contiguous, on the GPU."""
    if fmt not in (MX_E4M3, MX_E2M1):
        raise ValueError("unknown MX format %r" % (fmt,))
    for name, t in (("codes", codes), ("scales", scales)):
        _on_gpu(name, t)
        if t.dtype != torch.uint8 or t.dim() != 3 or not t.is_contiguous():
            raise ValueError("MX %s: a contiguous uint8 [B, N, *] token-major buffer" % name)
    B, N, per = codes.shape
    if tuple(scales.shape[:2]) != (B, N) or (scales.shape[2] * 32) % HEAD_DIM:
        raise ValueError("MX scales: shape %s does not match codes %s" % (tuple(scales.shape), tuple(codes.shape)))
    H = scales.shape[2] * 32 // HEAD_DIM
    if per != (H * HEAD_DIM if fmt == MX_E4M3 else H * HEAD_DIM // 2):
        raise ValueError("MX codes: shape %s does not match scales %s" % (tuple(codes.shape), tuple(scales.shape)))
    return B, N, H


def sage_mx_quantize(x, fmt: int, codes, scales, stream=None) -> None:
    B, N, H, D = _shape(x)
    _views((B, N, H, D), x=x)
    if _mx_shape(codes, scales, fmt) != (B, N, H):
        raise ValueError("MX buffers do not match x of shape %s" % ((B, N, H, D),))
    _same_device(x, codes, scales)
    xi = bf16_in(x)
    st = lib().sage_mx_quantize(ctypes.byref(xi), B, N, H, D, int(fmt), _ptr(codes), _ptr(scales), _stream(stream))
    _check(st, "sage_mx_quantize")


def sage_attn_fwd_mx(q_codes, q_scale, k_codes, k_scale, v_codes, v_scale, fmt: int, codes, scales, sm_scale=None,
                     stream=None) -> None:
    B, N, H = _mx_shape(codes, scales, fmt)
    _codes(B, N, H, HEAD_DIM, q_codes, q_scale, k_codes, k_scale, None, v_codes, v_scale)
    _same_device(codes, scales, q_codes, q_scale, k_codes, k_scale, v_codes, v_scale)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(HEAD_DIM)
    st = lib().sage_attn_fwd_mx(_ptr(q_codes), _ptr(q_scale), _ptr(k_codes), _ptr(k_scale), _ptr(v_codes),
                                _ptr(v_scale), B, N, H, HEAD_DIM, float(sm_scale), int(fmt), _ptr(codes),
                                _ptr(scales), _stream(stream))
    _check(st, "sage_attn_fwd_mx")


class Buffers:
    """Device buffers one quantised forward needs, allocated once with torch
    (library-defined layouts: see the public header)."""

    def __init__(self, B: int, N: int, H: int, device="cuda", D: int = HEAD_DIM):
        npad = sage_npad(N)
        self.B, self.N, self.H, self.D, self.npad = B, N, H, D, npad
        dev = torch.device(device)
        self.q_codes = torch.empty(B, H, npad, D, dtype=torch.int8, device=dev)
        self.k_codes = torch.empty(B, H, npad, D, dtype=torch.int8, device=dev)
        self.q_scale = torch.empty(B, H, npad // Q_BLOCK, dtype=torch.float32, device=dev)
        self.k_scale = torch.empty(B, H, npad // K_BLOCK, dtype=torch.float32, device=dev)
        self.k_mean = torch.empty(B, H, D, dtype=torch.float32, device=dev)
        self.v_codes = torch.empty(B, H, npad // P_TILE, D, P_TILE, dtype=torch.uint8, device=dev)
        self.v_scale = torch.empty(B, H, D, dtype=torch.float32, device=dev)
        self.ws_qk = torch.empty(max(1, sage_qk_workspace_bytes(B, N, H, D) // 8), dtype=torch.float64, device=dev)
        self.ws_v = torch.empty(max(1, sage_v_workspace_bytes(B, N, H, D) // 4), dtype=torch.float32, device=dev)
        # sized for sage_quantize_qkv_rope, which needs more than sage_quantize_qkv
        self.ws_qkv = torch.empty(max(1, -(-sage_qkv_rope_workspace_bytes(B, N, H, D) // 8)), dtype=torch.float64,
                                  device=dev)


def quantize(q, k, v, buf: Buffers, stream=None) -> None:
    """qk_quantize (with K smoothing) then v_quantize into `buf`."""
    sage_quantize_qk(q, k, buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.k_mean, buf.ws_qk, stream)
    sage_quantize_v(v, buf.v_codes, buf.v_scale, buf.ws_v, stream)


def quantize_qkv(q, k, v, buf: Buffers, stream=None) -> None:
    """The same codes and scales as quantize(), from the single three-pass call."""
    sage_quantize_qkv(q, k, v, buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.k_mean, buf.v_codes,
                      buf.v_scale, buf.ws_qkv, stream)


def quantize_qkv_rope(q, k, v, nr, buf: Buffers, stream=None) -> None:
    """quantize_qkv of the RMSNorm + RoPE transform of Q and K; nr carries
    gamma_q, gamma_k, rope (device tensors) and eps."""
    sage_quantize_qkv_rope(q, k, v, nr.gamma_q, nr.gamma_k, nr.rope, nr.eps, buf.q_codes, buf.q_scale, buf.k_codes,
                           buf.k_scale, buf.k_mean, buf.v_codes, buf.v_scale, buf.ws_qkv, stream)


def forward(q, k, v, out, buf: Buffers, sm_scale=None, stream=None) -> None:
    """The quantised forward: quantize Q/K/V (one three-pass call), then the fused
    attention into `out`."""
    quantize_qkv(q, k, v, buf, stream)
    sage_attn_fwd(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.v_codes, buf.v_scale, out, sm_scale, stream)


def token_major_out(B: int, N: int, H: int, device="cuda", D: int = HEAD_DIM) -> torch.Tensor:
    """A [B, N, H*D] bf16 output viewed as [B, N, H, D]."""
    return torch.empty(B, N, H * D, dtype=torch.bfloat16, device=device).view(B, N, H, D)


def v_token_order() -> torch.Tensor:
    """kappa: the token (within a 64-key tile) held at byte p of a V-code row."""
    p = torch.arange(P_TILE)
    u, j = p // 32, p % 32
    return 32 * (j // 16) + 8 * ((j % 16) // 4) + 4 * u + (j % 4)
