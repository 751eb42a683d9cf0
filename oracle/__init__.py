"""CPU oracle for the quantized softmax attention forward -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and shares no code with it.

This module is argument marshalling around ``sage_oracle.c`` (plain C, fp64,
OpenMP over independent rows).  Every function documents which part of the
method it computes; the arithmetic lives in the C file.

Arrays are numpy.  bf16 tensors are passed as ``numpy.uint16`` bit patterns with
element strides ``(sb, sn, sh)`` of a ``[B, N, H, D]`` view whose d-stride is 1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage_oracle.c")
_LIB = os.path.join(_HERE, "libsage_oracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra"]


# Opt-in sanitizer builds (the tests' sanitizer runs): libsage_oracle_<name>.so beside the normal one.
SANITIZERS = {"ubsan": ["-fsanitize=undefined", "-fno-sanitize-recover=all", "-g"],
              "asan": ["-fsanitize=address", "-fno-omit-frame-pointer", "-g"]}


def build(force: bool = True, sanitize: str | None = None) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction); with sanitize="ubsan" or "asan" a
    separately named library built under that sanitizer (load it by setting oracle._LIB to the path)."""
    out = _LIB if sanitize is None else os.path.join(_HERE, "libsage_oracle_%s.so" % sanitize)
    extra = [] if sanitize is None else SANITIZERS[sanitize]
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *GCC_FLAGS, *extra, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, out)
    return out


_lib = None

_i64 = ctypes.c_longlong
_int = ctypes.c_int
_dbl = ctypes.c_double
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        lib.sage_oracle_num_threads.restype = _int
        lib.sage_oracle_num_threads.argtypes = []
        lib.sage_oracle_e4m3_decode.restype = _dbl
        lib.sage_oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.sage_oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.sage_oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.sage_oracle_e4m3_encode_array.argtypes = [_p, _i64, _p]
        lib.sage_oracle_e4m3_decode_array.argtypes = [_p, _i64, _p]
        lib.sage_oracle_kmean.argtypes = [_p, _i64, _i64, _i64, _int, _int, _int, _int, _int, _p]
        lib.sage_oracle_quant_q.argtypes = [_p, _i64, _i64, _i64, _int, _int, _int, _int, _int, _p, _p]
        lib.sage_oracle_quant_k.argtypes = [_p, _i64, _i64, _i64, _int, _int, _int, _int, _p, _int, _p, _p]
        lib.sage_oracle_quant_v.argtypes = [_p, _i64, _i64, _i64, _int, _int, _int, _int, _p, _p]
        lib.sage_oracle_softmax_row.argtypes = ([_p, _i64, _i64, _i64] * 2 +
                                                [_int, _int, _int, _int, _int, _dbl, _p])
        lib.sage_oracle_attn_exact.argtypes = ([_p, _i64, _i64, _i64] * 3 +
                                               [_int, _int, _int, _int, _dbl, _p, _int, _p])
        lib.sage_oracle_attn_method.argtypes = ([_p] * 6 + [_int] * 7 + [_dbl, _dbl, _int, _p, _int, _p])
        lib.sage_oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        lib.sage_oracle_e2m1_decode.restype = ctypes.c_double
        lib.sage_oracle_e2m1_encode.argtypes = [ctypes.c_double]
        lib.sage_oracle_e2m1_encode.restype = ctypes.c_uint8
        lib.sage_oracle_mx_quantize.argtypes = [_p, _i64, _int, _int, _p, _p]
        lib.sage_oracle_mx_quantize.restype = None
        lib.sage_oracle_norm_rope.argtypes = [_p, _i64, _i64, _i64, _int, _int, _int, _int, _p, _p,
                                              ctypes.c_float, _p]
        lib.sage_oracle_sum_squares.argtypes = [_p, _i64, _int, _p]
        lib.sage_oracle_sum_squares.restype = None
        lib.sage_oracle_norm_rope.restype = None
        lib.sage_oracle_norm_rope_f64.argtypes = [_p, _i64, _i64, _i64, _int, _int, _int, _int, _p, _p, _dbl, _p]
        lib.sage_oracle_norm_rope_f64.restype = None
        lib.sage_oracle_attn_int8qk.argtypes = ([_p] * 4 + [_p, _i64, _i64, _i64] + [_int] * 7 +
                                                [_dbl, _int, _p, _int, _p])
        lib.sage_oracle_set_num_threads.argtypes = [_int]
        lib.sage_oracle_set_num_threads.restype = None
        for f in ("sage_oracle_kmean", "sage_oracle_quant_q", "sage_oracle_quant_k", "sage_oracle_quant_v",
                  "sage_oracle_softmax_row", "sage_oracle_attn_exact", "sage_oracle_attn_method",
                  "sage_oracle_attn_int8qk",
                  "sage_oracle_e4m3_encode_array", "sage_oracle_e4m3_decode_array"):
            getattr(lib, f).restype = None
        _lib = lib
    return _lib


class View:
    """A strided ``[B, N, H, D]`` bf16 view: a flat uint16 buffer plus element
    strides.  ``base`` must stay alive while the view is used."""

    def __init__(self, base: np.ndarray, offset: int, sb: int, sn: int, sh: int,
                 B: int, N: int, H: int, D: int):
        assert base.dtype == np.uint16 and base.flags["C_CONTIGUOUS"]
        last = offset + (B - 1) * sb + (N - 1) * sn + (H - 1) * sh + (D - 1)
        assert offset >= 0 and last < base.size, "view exceeds its buffer"
        self.base, self.offset = base, offset
        self.sb, self.sn, self.sh = sb, sn, sh
        self.B, self.N, self.H, self.D = B, N, H, D

    def ptr(self) -> int:
        return self.base.ctypes.data + 2 * self.offset

    def args(self):
        return (self.ptr(), self.sb, self.sn, self.sh)

    @staticmethod
    def from_bnhd(a: np.ndarray) -> "View":
        """A contiguous [B, N, H, D] uint16 array."""
        B, N, H, D = a.shape
        a = np.ascontiguousarray(a)
        return View(a.reshape(-1), 0, N * H * D, H * D, D, B, N, H, D)

    @staticmethod
    def from_bhnd(a: np.ndarray) -> "View":
        """A contiguous [B, H, N, D] (HND) uint16 array."""
        B, H, N, D = a.shape
        a = np.ascontiguousarray(a)
        return View(a.reshape(-1), 0, H * N * D, D, N * D, B, N, H, D)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return int(_load().sage_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Set the OpenMP threads of the following oracle calls."""
    _load().sage_oracle_set_num_threads(int(n))


# ------------------------------------------------------------------ codec
def e4m3_encode(x) -> np.ndarray:
    """OCP E4M3FN, round to nearest even, saturating at 448, signed zero."""
    x, px = _c(np.asarray(x, dtype=np.float32).reshape(-1), np.float32)
    out = np.empty(x.size, dtype=np.uint8)
    _load().sage_oracle_e4m3_encode_array(px, x.size, out.ctypes.data)
    return out


def e4m3_decode(c) -> np.ndarray:
    c, pc = _c(np.asarray(c, dtype=np.uint8).reshape(-1), np.uint8)
    out = np.empty(c.size, dtype=np.float64)
    _load().sage_oracle_e4m3_decode_array(pc, c.size, out.ctypes.data)
    return out


# -------------------------------------------------------------- quantizers
def kmean(k: View, chunk: int = 64) -> np.ndarray:
    """Per-(b, h, d) token mean of K in fp64 chunk order, rounded to fp32. [B, H, D]"""
    km = np.empty((k.B, k.H, k.D), dtype=np.float32)
    _load().sage_oracle_kmean(*k.args(), k.B, k.N, k.H, k.D, chunk, km.ctypes.data)
    return km


def quant_q(q: View, blk: int = 32):
    """INT8 codes [B, H, N, D] and fp32 scales [B, H, ceil(N/blk)]."""
    nblk = -(-q.N // blk)
    codes = np.empty((q.B, q.H, q.N, q.D), dtype=np.int8)
    scales = np.empty((q.B, q.H, nblk), dtype=np.float32)
    _load().sage_oracle_quant_q(*q.args(), q.B, q.N, q.H, q.D, blk, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def quant_k(k: View, km: np.ndarray, blk: int = 64):
    """K smoothed by km [B, H, D], then INT8 codes [B, H, N, D] and scales [B, H, ceil(N/blk)]."""
    nblk = -(-k.N // blk)
    km, pkm = _c(km, np.float32)
    assert km.shape == (k.B, k.H, k.D)
    codes = np.empty((k.B, k.H, k.N, k.D), dtype=np.int8)
    scales = np.empty((k.B, k.H, nblk), dtype=np.float32)
    _load().sage_oracle_quant_k(*k.args(), k.B, k.N, k.H, k.D, pkm, blk, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def quant_v(v: View):
    """E4M3FN codes [B, H, N, D] and per-channel fp32 scales [B, H, D]."""
    codes = np.empty((v.B, v.H, v.N, v.D), dtype=np.uint8)
    scales = np.empty((v.B, v.H, v.D), dtype=np.float32)
    _load().sage_oracle_quant_v(*v.args(), v.B, v.N, v.H, v.D, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


# --------------------------------------------------------------- attention
def all_rows(B: int, H: int, N: int) -> np.ndarray:
    return np.broadcast_to(np.arange(N, dtype=np.int32), (B, H, N)).copy()


def _rows(rows, B, H):
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    assert rows.ndim == 3 and rows.shape[:2] == (B, H)
    return rows, rows.shape[2]


def softmax_row(q: View, k: View, b: int, h: int, i: int, sm_scale: float) -> np.ndarray:
    p = np.empty(k.N, dtype=np.float64)
    _load().sage_oracle_softmax_row(*q.args(), *k.args(), k.N, q.D, b, h, i, sm_scale, p.ctypes.data)
    return p


def attn_exact(q: View, k: View, v: View, sm_scale: float, rows=None) -> np.ndarray:
    """fp64 softmax(Q K^T sm_scale) V on the rows [B, H, R]; returns [B, H, R, D]."""
    B, N, H, D = q.B, q.N, q.H, q.D
    assert (k.B, k.N, k.H, k.D) == (B, N, H, D) == (v.B, v.N, v.H, v.D)
    rows, R = _rows(all_rows(B, H, N) if rows is None else rows, B, H)
    out = np.empty((B, H, R, D), dtype=np.float64)
    _load().sage_oracle_attn_exact(*q.args(), *k.args(), *v.args(), B, N, H, D, sm_scale,
                                   rows.ctypes.data, R, out.ctypes.data)
    return out


def attn_method(qc, qs, kc, ks, vc, vs, sm_scale: float, rows=None, qblk: int = 32, kblk: int = 64,
                ptile: int = 64, pscale: float = 448.0, round_p: bool = True) -> np.ndarray:
    """Step-by-step quantised forward from logical codes/scales; returns [B, H, R, D]."""
    B, H, N, D = qc.shape
    qc, pqc = _c(qc, np.int8)
    kc, pkc = _c(kc, np.int8)
    vc, pvc = _c(vc, np.uint8)
    qs, pqs = _c(qs, np.float32)
    ks, pks = _c(ks, np.float32)
    vs, pvs = _c(vs, np.float32)
    assert kc.shape == vc.shape == (B, H, N, D)
    assert qs.shape == (B, H, -(-N // qblk)) and ks.shape == (B, H, -(-N // kblk)) and vs.shape == (B, H, D)
    rows, R = _rows(all_rows(B, H, N) if rows is None else rows, B, H)
    out = np.empty((B, H, R, D), dtype=np.float64)
    _load().sage_oracle_attn_method(pqc, pqs, pkc, pks, pvc, pvs, B, N, H, D, qblk, kblk, ptile,
                                    sm_scale, pscale, int(round_p), rows.ctypes.data, R, out.ctypes.data)
    return out


def attn_int8qk(qc, qs, kc, ks, v: View, sm_scale: float, rows=None, qblk: int = 32, kblk: int = 64,
                ptile: int = 64, round_p: bool = True) -> np.ndarray:
    """INT8 Q K^T from logical codes/scales with the bf16 V view unquantised and
    P rounded to bf16 for the product; returns [B, H, R, D]."""
    B, H, N, D = qc.shape
    qc, pqc = _c(qc, np.int8)
    kc, pkc = _c(kc, np.int8)
    qs, pqs = _c(qs, np.float32)
    ks, pks = _c(ks, np.float32)
    assert kc.shape == (B, H, N, D) and (v.B, v.N, v.H, v.D) == (B, N, H, D)
    assert qs.shape == (B, H, -(-N // qblk)) and ks.shape == (B, H, -(-N // kblk))
    rows, R = _rows(all_rows(B, H, N) if rows is None else rows, B, H)
    out = np.empty((B, H, R, D), dtype=np.float64)
    _load().sage_oracle_attn_int8qk(pqc, pqs, pkc, pks, *v.args(), B, N, H, D, qblk, kblk, ptile, sm_scale,
                                    int(round_p), rows.ctypes.data, R, out.ctypes.data)
    return out


MX_E4M3, MX_E2M1 = 0, 1


def e2m1_decode(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([_load().sage_oracle_e2m1_decode(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e2m1_encode(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return np.array([_load().sage_oracle_e2m1_encode(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)


def mx_quantize(x, fmt: int):
    """OCP MX blocks of 32 along the last axis of x (values taken exactly as fp64).
    Returns (codes, scales): codes [..., C] (E4M3) or [..., C/2] (E2M1 pairs),
    scales [..., C/32] E8M0 bytes."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    C = x.shape[-1]
    assert C % 32 == 0
    rows = x.size // C
    codes = np.zeros(x.shape[:-1] + (C if fmt == MX_E4M3 else C // 2,), np.uint8)
    scales = np.zeros(x.shape[:-1] + (C // 32,), np.uint8)
    _load().sage_oracle_mx_quantize(x.ctypes.data, rows, C, fmt, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def mx_dequantize(codes, scales, fmt: int) -> np.ndarray:
    """Values of MX blocks: element * 2^(scale - 127)."""
    codes = np.asarray(codes, np.uint8)
    if fmt == MX_E4M3:
        el = e4m3_decode(codes).reshape(codes.shape)
    else:
        table = e2m1_decode(np.arange(16))
        el = np.stack([table[codes & 0xF], table[codes >> 4]], axis=-1).reshape(codes.shape[:-1] + (2 * codes.shape[-1],))
    sc = np.ldexp(1.0, np.asarray(scales, np.int64) - 127)
    return el * np.repeat(sc, 32, axis=-1)


def norm_rope(x: View, gamma, rope, eps: float) -> np.ndarray:
    """RMSNorm over each head row's D channels (weight gamma[D]) then RoPE on
    channel pairs (2i, 2i+1) with rope[n, i] = (cos, sin): the sum of squares
    exact and rounded once to fp32, the rest in the fp32 steps written out in
    sage_oracle.c; bf16 result bits, [B, N, H, D] uint16."""
    g, pg = _c(np.asarray(gamma, np.float32).reshape(-1), np.float32)
    r, pr = _c(np.asarray(rope, np.float32), np.float32)
    assert g.size == x.D and r.shape == (x.N, x.D // 2, 2)
    out = np.empty((x.B, x.N, x.H, x.D), np.uint16)
    _load().sage_oracle_norm_rope(*x.args(), x.B, x.N, x.H, x.D, pg, pr, float(np.float32(eps)), out.ctypes.data)
    return out


def sum_squares(bits) -> np.ndarray:
    """The exact sum of the squares of each row of bf16 values (uint16 bit patterns, [..., n]), rounded once
    to fp32 (nearest even): the norm's ss."""
    b, pb = _c(np.asarray(bits, np.uint16), np.uint16)
    n = b.shape[-1]
    rows = b.size // n
    out = np.empty(b.shape[:-1], np.float32)
    _load().sage_oracle_sum_squares(pb, rows, n, out.ctypes.data)
    return out


def norm_rope_f64(x: View, gamma, rope, eps: float) -> np.ndarray:
    """The same transform in fp64, unrounded: [B, N, H, D] float64."""
    g, pg = _c(np.asarray(gamma, np.float32).reshape(-1), np.float32)
    r, pr = _c(np.asarray(rope, np.float32), np.float32)
    assert g.size == x.D and r.shape == (x.N, x.D // 2, 2)
    out = np.empty((x.B, x.N, x.H, x.D), np.float64)
    _load().sage_oracle_norm_rope_f64(*x.args(), x.B, x.N, x.H, x.D, pg, pr, float(eps), out.ctypes.data)
    return out


def rel_l2(a, ref) -> float:
    """Whole-tensor ||a - ref||_2 / ||ref||_2 in fp64."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((a - ref).ravel()) / np.linalg.norm(ref.ravel()))
