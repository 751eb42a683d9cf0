"""The quantised step under HIP graph capture: sage_quantize_qkv and
sage_attn_fwd enqueue kernels only (no memsets, allocations or synchronisation),
so a captured step replays to the same bytes as the eager calls.  Replays are
interleaved with eager work and synchronisation, and each is checked."""
import pytest
import torch

from quantized_softmax_attention_amd import inputs, sage
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N", [300, 4096])
def test_captured_step_replays_match_eager(N):
    print("graph capture N =", N, flush=True)
    case = G.gpu_case(inputs.packed_case(1, N, 4, seed=60 + N))
    other = G.gpu_case(inputs.packed_case(1, N, 4, seed=61 + N))
    eager_buf = sage.Buffers(1, N, 4)
    eager_out = sage.token_major_out(1, N, 4)
    sage.forward(case.q, case.k, case.v, eager_out, eager_buf, G.SM)
    torch.cuda.synchronize()

    buf = sage.Buffers(1, N, 4)
    out = sage.token_major_out(1, N, 4)
    side = torch.cuda.Stream()                     # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                  # warm-up on the capture stream
        sage.forward(case.q, case.k, case.v, out, buf, G.SM)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        sage.forward(case.q, case.k, case.v, out, buf, G.SM)
    for r in range(3):
        out.fill_(0)
        buf.q_codes.fill_(0x5A)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16)), r
        for f in ("q_codes", "q_scale", "k_codes", "k_scale", "k_mean", "v_codes", "v_scale"):
            assert torch.equal(getattr(buf, f), getattr(eager_buf, f)), (r, f)
        # eager work on other inputs between replays
        tmp = sage.token_major_out(1, N, 4)
        sage.forward(other.q, other.k, other.v, tmp, sage.Buffers(1, N, 4), G.SM)
        torch.cuda.synchronize()
