"""Launch errors are attributed to their own call: each entry point returns the
status of its own kernel launches (hipLaunchKernel's), so an error the caller's
earlier HIP work left in the thread's last-error state is not reported as the
library's SAGE_ERR_HIP (nor cleared by the library)."""
import ctypes
import math

import pytest
import torch

from quantized_softmax_attention_amd import inputs, sage

pytestmark = pytest.mark.gpu


def test_earlier_caller_error_is_not_the_librarys():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.init()
    hip = ctypes.CDLL("libamdhip64.so")            # the runtime torch and the library already use
    count = ctypes.c_int()
    assert hip.hipGetDeviceCount(ctypes.byref(count)) == 0
    case = inputs.config("tiny")
    g = case.to("cuda")
    buf = sage.Buffers(case.B, case.N, case.H)
    out = sage.token_major_out(case.B, case.N, case.H)
    torch.cuda.synchronize()
    assert hip.hipGetLastError() == 0                    # no error pending before the test's own
    # the caller's own failing HIP call: an invalid device ordinal (nothing is changed by it)
    err = hip.hipSetDevice(count.value + 7)
    assert err != 0
    # every entry point of the step still succeeds: it reports its own launches only (a launcher that
    # returned hipGetLastError() would report this error as SAGE_ERR_HIP and raise here) ...
    sage.quantize_qkv(g.q, g.k, g.v, buf)
    sage.sage_attn_fwd(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale, buf.v_codes, buf.v_scale, out,
                       1.0 / math.sqrt(128.0))
    sage.sage_attn_fwd_bf16(g.q, g.k, g.v, out, 1.0 / math.sqrt(128.0))
    # ... and leaves the caller's error for the caller (reading it here also clears it for torch)
    assert hip.hipGetLastError() == err
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
