"""sage_quantize_qkv_noalloc on the GPU through the C ABI: the same codes, scales and
k_mean as sage_quantize_qkv with a caller workspace, bit for bit, on two calls in a
row (the second smaller, so it runs on the scratch the first left behind), and a
size beyond the library's scratch is refused before anything runs."""
import numpy as np
import pytest
import torch

from quantized_softmax_attention_amd import inputs, sage

pytestmark = pytest.mark.gpu


def _outputs(buf):
    return [t.cpu().numpy().view(np.uint8) for t in (buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.k_mean,
                                                     buf.v_codes, buf.v_scale)]


def _fill(buf, byte):
    for t in (buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.k_mean, buf.v_codes, buf.v_scale):
        t.view(torch.uint8).fill_(byte)


def _noalloc(g, buf):
    sage.sage_quantize_qkv_noalloc(g.q, g.k, g.v, buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.k_mean,
                                   buf.v_codes, buf.v_scale)


@pytest.mark.parametrize("first,second", [("block24", "tiny")])
def test_noalloc_equals_workspace_call_twice(first, second):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    for name in (first, second):
        print("no-alloc quantiser:", name, flush=True)
        case = inputs.config(name)
        assert sage.sage_qkv_workspace_bytes(case.B, case.N, case.H, case.D) <= sage.sage_qkv_noalloc_max_bytes()
        g = case.to("cuda")
        ref = sage.Buffers(case.B, case.N, case.H)
        _fill(ref, 0x5A)
        sage.quantize_qkv(g.q, g.k, g.v, ref)
        got = sage.Buffers(case.B, case.N, case.H)
        _fill(got, 0xA5)                     # different fill: a missed write cannot match
        _noalloc(g, got)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_outputs(got), _outputs(ref))):
            assert np.array_equal(a, b), (name, i)
        del g, ref, got


def test_noalloc_refuses_sizes_beyond_its_scratch():
    case = inputs.packed_case(2, 8, 1, seed=3)         # tiny tensors: only the declared sizes are too large
    g = case.to("cuda")
    B, N, H = 2, 37810, 56
    assert sage.sage_qkv_workspace_bytes(B, N, H, 128) > sage.sage_qkv_noalloc_max_bytes()
    L = sage.lib()
    sentinel = torch.full((64,), 7, dtype=torch.uint8, device="cuda")
    qi, ki, vi = (sage.BF16In(t.data_ptr(), N * 3 * H * 128, 3 * H * 128, 128) for t in (g.q, g.k, g.v))
    p = sentinel.data_ptr()
    st = L.sage_quantize_qkv_noalloc(*(ctypes_ref(x) for x in (qi, ki, vi)), B, N, H, 128, p, p, p, p, p, p, p, None)
    torch.cuda.synchronize()
    assert st == 5                                      # SAGE_ERR_WORKSPACE
    assert torch.all(sentinel == 7)


def ctypes_ref(x):
    import ctypes
    return ctypes.byref(x)
