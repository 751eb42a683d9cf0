"""Entry points under HIP graph capture: every call only enqueues kernels (no
memsets, allocations or synchronisation), so a captured quantised step, and a
captured sequence of all the other entry points, replay to the same bytes as the
eager calls.  Replays are interleaved with eager work and synchronisation, and
each is checked."""
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


def _other_calls(case, nr, bufs, outs, q_ip, k_ip):
    """Every other entry point once: the fused RMSNorm + RoPE quantiser, the MX
    epilogue and the standalone MX pass, the bf16 and INT8-QK / bf16-PV paths, and
    the in-place RMSNorm + RoPE."""
    rb, codes, scales, codes2, scales2, o16, o8 = bufs["rope"], *outs
    sage.quantize_qkv_rope(case.q, case.k, case.v, nr, rb)
    sage.sage_attn_fwd_mx(rb.q_codes, rb.q_scale, rb.k_codes, rb.k_scale, rb.v_codes, rb.v_scale, sage.MX_E4M3,
                          codes, scales, G.SM)
    sage.sage_attn_fwd_bf16(case.q, case.k, case.v, o16, G.SM)
    sage.sage_attn_fwd_int8qk(rb.q_codes, rb.q_scale, rb.k_codes, rb.k_scale, case.v, o8, G.SM)
    sage.sage_mx_quantize(o16, sage.MX_E2M1, codes2, scales2)
    sage.sage_qk_norm_rope(q_ip, k_ip, nr.gamma_q, nr.gamma_k, nr.rope, nr.eps)


def test_captured_other_entry_points_replay_match_eager():
    B, N, H = 1, 300, 4
    case = G.gpu_case(inputs.packed_case(B, N, H, seed=70))
    nr = inputs.norm_rope_params(N, seed=7).to("cuda")
    orig = case.packed.clone()                                   # the in-place transform works on a copy

    def state():
        ip = orig.clone()
        HD = H * 128
        q_ip, k_ip = (ip[:, :, i * HD:(i + 1) * HD].unflatten(2, (H, 128)) for i in range(2))
        bufs = {"rope": sage.Buffers(B, N, H)}
        outs = (*sage.mx_out(B, N, H, sage.MX_E4M3), *sage.mx_out(B, N, H, sage.MX_E2M1),
                sage.token_major_out(B, N, H), sage.token_major_out(B, N, H))
        return ip, q_ip, k_ip, bufs, outs

    e_ip, e_q, e_k, e_bufs, e_outs = state()
    _other_calls(case, nr, e_bufs, e_outs, e_q, e_k)
    torch.cuda.synchronize()

    ip, q_ip, k_ip, bufs, outs = state()
    side = torch.cuda.Stream()                                   # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _other_calls(case, nr, bufs, outs, q_ip, k_ip)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _other_calls(case, nr, bufs, outs, q_ip, k_ip)
    for r in range(3):
        ip.copy_(orig)                                           # eager: undo the in-place transform
        for t in outs:
            t.view(torch.uint8).fill_(0x5A)
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, e_outs)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (r, i)
        assert torch.equal(ip.view(torch.int16), e_ip.view(torch.int16)), r
        for f in ("q_codes", "q_scale", "k_codes", "k_scale", "k_mean", "v_codes", "v_scale"):
            assert torch.equal(getattr(bufs["rope"], f), getattr(e_bufs["rope"], f)), (r, f)
        tmp = sage.token_major_out(B, N, H)                      # eager work between replays
        sage.sage_attn_fwd_bf16(case.q, case.k, case.v, tmp, G.SM)
        torch.cuda.synchronize()
