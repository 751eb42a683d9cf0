"""Test-side glue: torch bf16 views -> oracle views, and small array helpers."""
import numpy as np
import torch

import oracle


def oracle_view(t: torch.Tensor) -> "oracle.View":
    """An oracle.View over the CPU storage of a [B, N, H, D] bf16 view (d-stride 1)."""
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu" and t.dim() == 4
    st = t.untyped_storage()
    flat = torch.empty(0, dtype=torch.bfloat16).set_(st, 0, (st.nbytes() // 2,), (1,))
    base = flat.view(torch.int16).numpy().view(np.uint16)
    B, N, H, D = t.shape
    sb, sn, sh, sd = t.stride()
    assert sd == 1
    return oracle.View(base, t.storage_offset(), sb, sn, sh, B, N, H, D)


def bf16_from_f32(x) -> torch.Tensor:
    """fp32 values (assumed exactly representable) as a bf16 tensor; asserts exactness."""
    x = torch.as_tensor(np.array(x, dtype=np.float32))
    y = x.to(torch.bfloat16)
    assert torch.equal(y.float(), x), "value not representable in bf16"
    return y


def bnhd(x_bnhd) -> torch.Tensor:
    """A contiguous [B, N, H, D] bf16 tensor from exactly representable values."""
    return bf16_from_f32(x_bnhd).contiguous()
