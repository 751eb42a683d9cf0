"""The C ABI from plain C: tests/c_abi_client (built by build() from
tests/c_abi_client.c with gcc and the HIP runtime's C API; no torch, no Python)
quantises and attends a seeded case in a process of its own.  Its codes and scales
equal the oracle's bit for bit, and its two outputs pass the same gates as the
calls made through the Python binding."""
import os
import subprocess
import types

import numpy as np
import pytest
import torch

from quantized_softmax_attention_amd import inputs, sage
from tests import gpu_common as G
from tests.c_client_build import EXE

pytestmark = pytest.mark.gpu


def _read(f, dtype, shape):
    n = int(np.prod(shape))
    a = np.fromfile(f, dtype=dtype, count=n)
    assert a.size == n, "short output file"
    return torch.from_numpy(a.reshape(shape))


@pytest.mark.parametrize("B,N,H", [(1, 256, 2), (2, 333, 3)])
def test_c_client_matches_oracle(tmp_path, B, N, H):
    print("c client B=%d N=%d H=%d" % (B, N, H), flush=True)
    assert os.path.exists(EXE), "tests/c_abi_client is not built (run __graft_entry__.build())"
    case = inputs.packed_case(B, N, H, seed=90 + N, stress=(B == 2))
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([B, N, H], np.int32).tobytes())
        for t in (case.q, case.k, case.v):
            f.write(t.contiguous().view(torch.int16).numpy().tobytes())
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0
    D, npad = 128, sage.sage_npad(N)
    with open(dst, "rb") as f:
        assert int(np.fromfile(f, np.int32, 1)[0]) == 0
        buf = types.SimpleNamespace(
            q_codes=_read(f, np.int8, (B, H, npad, D)), k_codes=_read(f, np.int8, (B, H, npad, D)),
            v_codes=_read(f, np.uint8, (B, H, npad // 64, D, 64)), q_scale=_read(f, np.float32, (B, H, npad // 32)),
            k_scale=_read(f, np.float32, (B, H, npad // 64)), k_mean=_read(f, np.float32, (B, H, D)),
            v_scale=_read(f, np.float32, (B, H, D)))
        out8 = _read(f, np.int16, (B, N, H, D)).view(torch.bfloat16)
        out16 = _read(f, np.int16, (B, N, H, D)).view(torch.bfloat16)
        assert f.read() == b""
    ref = G.OracleRef(case)
    G.check_quant_bitexact(buf, ref)
    rows = inputs.sample_rows(B, H, N, count=N)
    G.gate(G.out_rows(out8, rows), G.bf16_round(ref.method(rows)), 1e-3, "C client quantised")
    G.gate(G.out_rows(out16, rows), ref.exact(rows), 5e-3, "C client bf16")
