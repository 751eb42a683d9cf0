"""The C ABI without a GPU: the library loads, exports every function the public
header declares, and its host-side validation rejects bad arguments with the
documented status before anything is launched (fake, never-dereferenced device
addresses are used)."""
import ctypes
import os
import re

import pytest

from quantized_softmax_attention_amd import sage

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sage_mi355x.h")

pytestmark = pytest.mark.skipif(not os.path.exists(sage.LIB_PATH), reason="library not built")

OK, NULL, SHAPE, STRIDE, ALIGN, WORKSPACE, HIP, VALUE = range(8)
A = 0x10000          # a fake 16-byte-aligned "device" address, never dereferenced
N, H, B, D = 100, 3, 2, 128


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_\w+)\s*\(", text)))


def test_header_symbols_are_exported():
    names = declared_functions()
    assert set(names) >= {"sage_quantize_qk", "sage_quantize_v", "sage_attn_fwd", "sage_attn_fwd_bf16", "sage_attn_fwd_int8qk",
                          "sage_status_str", "sage_npad", "sage_qk_workspace_bytes", "sage_v_workspace_bytes"}
    L = ctypes.CDLL(sage.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_sizes():
    for s in range(8):
        assert sage.sage_status_str(s) and sage.sage_status_str(s) != "unknown status"
    assert sage.sage_status_str(99) == "unknown status"
    assert sage.sage_npad(1) == 256 and sage.sage_npad(256) == 256 and sage.sage_npad(37810) == 37888
    assert sage.sage_npad(0) == 0
    assert sage.sage_qk_workspace_bytes(1, 37810, 56, 128) == 591 * 56 * 128 * 8
    assert sage.sage_v_workspace_bytes(1, 37810, 56, 128) == (148 + 1) * 56 * 128 * 4
    assert sage.sage_qk_workspace_bytes(1, 10, 2, 64) == 0
    assert sage.sage_qkv_workspace_bytes(1, 37810, 56, 128) == 591 * 56 * 128 * 12 + 56 * 128 * 4


def view(data=A, sb=N * 3 * H * D, sn=3 * H * D, sh=D):
    return sage.BF16In(data, sb, sn, sh)


def out(data=A, sb=N * H * D, sn=H * D, sh=D):
    return sage.BF16Out(data, sb, sn, sh)


def qk(q=None, k=None, Bv=B, Nv=N, Hv=H, Dv=D, ptrs=(A, A, A, A, A), ws=A, wsb=None):
    L = sage.lib()
    q = q or view()
    k = k or view(A + 2 * H * D)
    wsb = sage.sage_qk_workspace_bytes(B, N, H, D) if wsb is None else wsb
    return L.sage_quantize_qk(ctypes.byref(q), ctypes.byref(k), Bv, Nv, Hv, Dv, *ptrs, ws, wsb, None)


def test_quantize_qk_validation():
    assert qk(ptrs=(None, A, A, A, A)) == NULL
    assert qk(ws=None) == NULL
    assert qk(q=view(data=None)) == NULL
    assert qk(Dv=64) == SHAPE and qk(Nv=0) == SHAPE and qk(Bv=0) == SHAPE and qk(Hv=0) == SHAPE
    assert qk(Hv=70000) == SHAPE
    # every launch's work-items (at most 8 B H Npad) fit 32 bits: B H Npad <= 2^29 - 1
    assert sage.sage_qkv_workspace_bytes(1, (1 << 28) - 256, 2, D) > 0     # Npad = 2^28 - 256: fits
    assert sage.sage_qkv_workspace_bytes(1, (1 << 28) - 255, 2, D) == 0    # Npad = 2^28: 8 B H Npad = 2^32
    assert qk(Bv=1, Hv=2, Nv=(1 << 28) - 255) == SHAPE
    assert qk(q=view(data=A + 8)) == ALIGN
    assert qk(q=view(sn=3 * H * D + 4)) == ALIGN
    assert qk(ptrs=(A + 4, A, A, A, A)) == ALIGN
    assert qk(ptrs=(A, A, A, A + 2, A)) == ALIGN
    assert qk(ws=A + 4) == ALIGN
    assert qk(q=view(sn=-8)) == STRIDE
    assert qk(wsb=100) == WORKSPACE


def test_quantize_v_validation():
    L = sage.lib()
    wsb = sage.sage_v_workspace_bytes(B, N, H, D)
    call = lambda v, vc=A, vs=A, ws=A, w=wsb, Dv=D: L.sage_quantize_v(ctypes.byref(v), B, N, H, Dv, vc, vs, ws, w,
                                                                        None)
    assert call(view(), vc=None) == NULL
    assert call(view(), ws=None) == NULL
    assert call(view(), Dv=256) == SHAPE
    assert call(view(), vc=A + 8) == ALIGN
    assert call(view(), w=wsb - 4) == WORKSPACE
    assert call(view(sh=-D)) == STRIDE


def test_attn_fwd_validation():
    L = sage.lib()
    call = lambda o, ptrs=(A,) * 6, sm=0.088, Nv=N: L.sage_attn_fwd(*ptrs, B, Nv, H, D, sm, ctypes.byref(o), None)
    assert call(out(), ptrs=(A, A, None, A, A, A)) == NULL
    assert call(out(data=None)) == NULL
    assert call(out(), Nv=-1) == SHAPE
    assert call(out(data=A + 4)) == ALIGN
    assert call(out(), ptrs=(A, A, A, A, A + 8, A)) == ALIGN
    assert call(out(sn=H * D + 2)) == ALIGN
    assert call(out(sh=64)) == STRIDE                  # heads overlap
    assert call(out(sn=D, sh=D)) == STRIDE             # tokens overlap heads
    assert call(out(sb=D)) == STRIDE                   # batches overlap
    assert call(out(), sm=0.0) == VALUE
    assert call(out(), sm=float("nan")) == VALUE
    assert call(out(), sm=-1.0) == VALUE
    # HND-style output (heads outermost) is a valid non-overlapping layout
    # (checked by not returning a stride error; the NULL check fires first here)
    assert call(out(sb=H * N * D, sn=D, sh=N * D), ptrs=(None,) * 6) == NULL


def test_attn_fwd_bf16_validation():
    L = sage.lib()
    call = lambda q, o=None, sm=0.1, Dv=D: L.sage_attn_fwd_bf16(ctypes.byref(q), ctypes.byref(view()),
                                                                ctypes.byref(view()), B, N, H, Dv, sm,
                                                                ctypes.byref(o or out()), None)
    assert call(view(data=None)) == NULL
    assert call(view(), Dv=127) == SHAPE
    assert call(view(data=A + 2)) == ALIGN
    assert call(view(), o=out(sh=0)) == STRIDE
    assert call(view(), sm=float("inf")) == VALUE
    # K/V token rows must not overlap on this path
    L2 = sage.lib()
    k_bad = sage.BF16In(A, N * 3 * H * D, 64, D)
    assert L2.sage_attn_fwd_bf16(ctypes.byref(view()), ctypes.byref(k_bad), ctypes.byref(view()), B, N, H, D, 0.1,
                                 ctypes.byref(out()), None) == STRIDE


def test_attn_fwd_int8qk_validation():
    L = sage.lib()
    call = lambda v=None, o=None, ptrs=(A,) * 4, sm=0.088, Dv=D: L.sage_attn_fwd_int8qk(
        *ptrs, ctypes.byref(v or view()), B, N, H, Dv, sm, ctypes.byref(o or out()), None)
    assert call(ptrs=(A, None, A, A)) == NULL
    assert call(v=view(data=None)) == NULL
    assert call(Dv=64) == SHAPE
    assert call(ptrs=(A + 8, A, A, A)) == ALIGN
    assert call(v=view(data=A + 2)) == ALIGN
    assert call(v=sage.BF16In(A, N * 3 * H * D, 64, D)) == STRIDE    # V token rows overlap
    assert call(o=out(sh=0)) == STRIDE
    assert call(sm=float("nan")) == VALUE


def test_quantize_qkv_validation():
    L = sage.lib()
    wsb = sage.sage_qkv_workspace_bytes(B, N, H, D)
    call = lambda q=None, ptrs=(A,) * 7, ws=A, w=wsb, Dv=D: L.sage_quantize_qkv(
        ctypes.byref(q or view()), ctypes.byref(view(A + 2 * H * D)), ctypes.byref(view(A + 4 * H * D)), B, N, H, Dv,
        *ptrs, ws, w, None)
    assert call(ptrs=(A, A, A, A, A, None, A)) == NULL
    assert call(ws=None) == NULL
    assert call(Dv=96) == SHAPE
    assert call(ptrs=(A, A, A, A, A, A + 8, A)) == ALIGN
    assert call(ws=A + 4) == ALIGN
    assert call(q=view(sn=-8)) == STRIDE
    assert call(w=wsb - 8) == WORKSPACE


def test_quantize_qkv_noalloc_validation():
    """The allocation-free quantiser validates like sage_quantize_qkv and refuses sizes whose scratch
    exceeds its fixed array, all before any HIP call."""
    L = sage.lib()
    assert sage.sage_qkv_noalloc_max_bytes() == 64 << 20
    call = lambda q=None, ptrs=(A,) * 7, Bv=B, Nv=N, Hv=H, Dv=D: L.sage_quantize_qkv_noalloc(
        ctypes.byref(q or view()), ctypes.byref(view(A + 2 * H * D)), ctypes.byref(view(A + 4 * H * D)), Bv, Nv, Hv,
        Dv, *ptrs, None)
    assert call(ptrs=(A, A, A, A, A, None, A)) == NULL
    assert call(Dv=96) == SHAPE
    assert call(ptrs=(A, A, A, A, A, A + 8, A)) == ALIGN
    assert call(q=view(sn=-8)) == STRIDE
    # two block-24 sequences need 101.7 MB of scratch, one fits (50.9 MB)
    big = view(sb=37810 * 3 * 56 * D, sn=3 * 56 * D)
    assert sage.sage_qkv_workspace_bytes(2, 37810, 56, D) > sage.sage_qkv_noalloc_max_bytes()
    assert sage.sage_qkv_workspace_bytes(1, 37810, 56, D) <= sage.sage_qkv_noalloc_max_bytes()
    assert call(q=big, Bv=2, Nv=37810, Hv=56) == WORKSPACE


def test_mx_quantize_validation():
    L = sage.lib()
    call = lambda x=None, c=A, s=A, fmt=0, Dv=D: L.sage_mx_quantize(ctypes.byref(x or view()), B, N, H, Dv, fmt, c, s,
                                                                   None)
    assert call(c=None) == NULL and call(s=None) == NULL
    assert call(x=view(data=None)) == NULL
    assert call(Dv=64) == SHAPE
    assert call(c=A + 8) == ALIGN
    assert call(x=view(data=A + 2)) == ALIGN
    assert call(x=view(sh=-D)) == STRIDE
    assert call(fmt=2) == VALUE and call(fmt=-1) == VALUE


def test_attn_fwd_mx_validation():
    L = sage.lib()
    call = lambda ptrs=(A,) * 6, c=A, s=A, sm=0.088, fmt=1, Nv=N: L.sage_attn_fwd_mx(*ptrs, B, Nv, H, D, sm, fmt, c, s,
                                                                                     None)
    assert call(ptrs=(A, A, A, A, None, A)) == NULL
    assert call(c=None) == NULL and call(s=None) == NULL
    assert call(Nv=0) == SHAPE
    assert call(c=A + 2) == ALIGN
    assert call(ptrs=(A, A, A + 4, A, A, A)) == ALIGN
    assert call(sm=float("inf")) == VALUE
    assert call(fmt=7) == VALUE


def test_qk_norm_rope_validation():
    L = sage.lib()
    io = lambda data=A, sn=3 * H * D, sh=D: sage.BF16Out(data, N * 3 * H * D, sn, sh)
    call = lambda q=None, g=(A, A, A), eps=1e-6, Dv=D: L.sage_qk_norm_rope(
        ctypes.byref(q or io()), ctypes.byref(io(A + 2 * H * D)), B, N, H, Dv, *g, eps, None)
    assert call(g=(A, None, A)) == NULL and call(g=(A, A, None)) == NULL
    assert call(q=io(data=None)) == NULL
    assert call(Dv=64) == SHAPE
    assert call(q=io(data=A + 8)) == ALIGN
    assert call(q=io(sn=3 * H * D + 4)) == ALIGN
    assert call(g=(A, A, A + 4)) == ALIGN and call(g=(A + 8, A, A)) == ALIGN
    assert call(q=io(sh=64)) == STRIDE                 # heads overlap
    assert call(eps=0.0) == VALUE and call(eps=float("nan")) == VALUE and call(eps=-1.0) == VALUE


def test_quantize_qkv_rope_validation():
    L = sage.lib()
    wsb = sage.sage_qkv_rope_workspace_bytes(B, N, H, D)
    # the qkv workspace plus one fp32 norm factor per (b, h, padded token)
    assert wsb == sage.sage_qkv_workspace_bytes(B, N, H, D) + B * H * sage.sage_npad(N) * 4
    call = lambda g=(A, A, A), eps=1e-6, ptrs=(A,) * 7, ws=A, w=wsb, Dv=D: L.sage_quantize_qkv_rope(
        ctypes.byref(view()), ctypes.byref(view(A + 2 * H * D)), ctypes.byref(view(A + 4 * H * D)), B, N, H, Dv,
        *g, eps, *ptrs, ws, w, None)
    assert call(g=(None, A, A)) == NULL
    assert call(ptrs=(A, A, None, A, A, A, A)) == NULL
    assert call(Dv=256) == SHAPE
    assert call(g=(A, A, A + 4)) == ALIGN
    assert call(ptrs=(A + 8, A, A, A, A, A, A)) == ALIGN
    assert call(eps=float("inf")) == VALUE
    assert call(w=wsb - 8) == WORKSPACE
    assert call(w=sage.sage_qkv_workspace_bytes(B, N, H, D)) == WORKSPACE   # the qkv size is not enough


@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++11")])
def test_header_is_plain_c_and_cxx(tmp_path, lang, std):
    # the public header needs nothing beyond the C standard headers it includes
    import subprocess
    src = tmp_path / ("use." + ("c" if lang == "c" else "cpp"))
    src.write_text('#include "sage_mi355x.h"\nint main(void) { return sage_npad(1) == 256 ? 0 : 1; }\n')
    cc = "gcc" if lang == "c" else "g++"
    r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-I", os.path.dirname(HEADER), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
