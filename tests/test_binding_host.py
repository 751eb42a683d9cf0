"""The Python binding's argument checks, without a GPU: host tensors, undersized
or mistyped code buffers, mismatched views and MX buffers are refused with a
Python exception before the C ABI is called (the C ABI takes raw device
pointers and could not tell)."""
import os

import pytest
import torch

from quantized_softmax_attention_amd import sage

pytestmark = pytest.mark.skipif(not os.path.exists(sage.LIB_PATH), reason="library not built")

B, N, H, D = 1, 70, 2, 128


def views():
    x = torch.zeros(B, N, 3 * H * D, dtype=torch.bfloat16)
    return [x[:, :, i * H * D:(i + 1) * H * D].unflatten(2, (H, D)) for i in range(3)]


def buffers():
    npad = sage.sage_npad(N)
    return dict(q_codes=torch.zeros(B, H, npad, D, dtype=torch.int8), q_scale=torch.zeros(B, H, npad // 32),
                k_codes=torch.zeros(B, H, npad, D, dtype=torch.int8), k_scale=torch.zeros(B, H, npad // 64),
                k_mean=torch.zeros(B, H, D), v_codes=torch.zeros(B, H, npad // 64, D, 64, dtype=torch.uint8),
                v_scale=torch.zeros(B, H, D))


def test_host_tensors_are_refused():
    q, k, v = views()
    b = buffers()
    out = torch.zeros(B, N, H, D, dtype=torch.bfloat16)
    ws = torch.zeros(sage.sage_qkv_workspace_bytes(B, N, H, D) // 8, dtype=torch.float64)
    with pytest.raises(ValueError, match="device memory"):
        sage.sage_quantize_qkv(q, k, v, *b.values(), ws)
    with pytest.raises(ValueError, match="device memory"):
        sage.sage_attn_fwd(b["q_codes"], b["q_scale"], b["k_codes"], b["k_scale"], b["v_codes"], b["v_scale"], out)
    with pytest.raises(ValueError, match="device memory"):
        sage.sage_attn_fwd_bf16(q, k, v, out)
    with pytest.raises(ValueError, match="device memory"):
        sage.sage_mx_quantize(out, sage.MX_E4M3, torch.zeros(B, N, H * D, dtype=torch.uint8),
                              torch.zeros(B, N, H * D // 32, dtype=torch.uint8))


@pytest.fixture
def as_if_on_gpu(monkeypatch):
    # host tensors stand in for device ones so that the remaining checks run
    monkeypatch.setattr(sage, "_on_gpu", lambda name, t: None)


def test_code_buffers_sizes_types_layouts(as_if_on_gpu):
    b = buffers()
    sage._codes(B, N, H, D, **b)                               # the library's own sizes pass
    small = dict(b, q_codes=b["q_codes"][:, :, :N])             # padding rows missing
    with pytest.raises(ValueError, match="needed"):
        sage._codes(B, N, H, D, **dict(small, q_codes=small["q_codes"].contiguous()))
    with pytest.raises(TypeError, match="int8"):
        sage._codes(B, N, H, D, **dict(b, k_codes=b["k_codes"].view(torch.uint8)))
    with pytest.raises(TypeError, match="float32"):
        sage._codes(B, N, H, D, **dict(b, v_scale=b["v_scale"].double()))
    with pytest.raises(ValueError, match="contiguous"):
        sage._codes(B, N, H, D, **dict(b, k_mean=torch.zeros(B, H, 2 * D)[:, :, ::2]))
    with pytest.raises(ValueError, match="needed"):
        sage._codes(B, N + 300, H, D, **b)                     # buffers of a shorter sequence


def test_views_must_agree(as_if_on_gpu):
    q, k, v = views()
    with pytest.raises(ValueError, match="shape"):
        sage._views((B, N, H, D), q=q, k=k[:, :N - 1])
    with pytest.raises(ValueError, match="unit last stride"):
        sage._shape(q.transpose(2, 3))


def test_mx_buffers_must_match(as_if_on_gpu):
    codes = torch.zeros(B, N, H * D, dtype=torch.uint8)
    scales = torch.zeros(B, N, H * D // 32, dtype=torch.uint8)
    assert sage._mx_shape(codes, scales, sage.MX_E4M3) == (B, N, H)
    assert sage._mx_shape(codes[:, :, :H * D // 2].contiguous(), scales, sage.MX_E2M1) == (B, N, H)
    with pytest.raises(ValueError, match="does not match"):
        sage._mx_shape(codes, scales, sage.MX_E2M1)
    with pytest.raises(ValueError, match="does not match"):
        sage._mx_shape(codes, scales[:, 1:], sage.MX_E4M3)
    with pytest.raises(ValueError, match="unknown MX format"):
        sage._mx_shape(codes, scales, 7)
    with pytest.raises(ValueError, match="uint8"):
        sage._mx_shape(codes.to(torch.int8), scales, sage.MX_E4M3)
