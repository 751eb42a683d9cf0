"""One call of every entry point of libsage_mi355x.so, in a fixed order, after all
inputs and buffers are in place: run under `rocprofv3 --kernel-trace`, the
dispatches from the first library kernel on are exactly the kernels each call
launches (tests/test_gpu_launch_audit.py checks the list; no copy, transpose or
fill kernels appear between them)."""
import math
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import torch  # noqa: E402

from quantized_softmax_attention_amd import inputs, sage  # noqa: E402

# (entry point, the kernels it launches, in order)
EXPECTED = [
    ("sage_quantize_qk", ["kmean_partial_kernel", "chunk_final_kernel<true, false>", "quant_qk_kernel"]),
    ("sage_quantize_v", ["v_amax_partial_kernel", "chunk_final_kernel<false, true>", "quant_v_kernel"]),
    ("sage_quantize_qkv", ["qkv_pass1_kernel", "chunk_final_kernel<true, true>", "qkv_pass3_kernel<false>"]),
    ("sage_attn_fwd", ["attn_i8f8_kernel<-1>"]),
    ("sage_attn_fwd_bf16", ["attn_bf16_kernel"]),
    ("sage_attn_fwd_int8qk", ["attn_int8qk_kernel"]),
    ("sage_qk_norm_rope", ["norm_rope_kernel"]),
    ("sage_quantize_qkv_rope", ["qkv_rope_pass1_kernel", "chunk_final_kernel<true, true>",
                                "qkv_pass3_kernel<true>"]),
    ("sage_mx_quantize", ["mx_quantize_kernel<0>"]),
    ("sage_attn_fwd_mx", ["attn_i8f8_kernel<0>"]),
]


def main() -> None:
    B, N, H = 1, 1000, 4
    case = inputs.packed_case(B, N, H, seed=5).to("cuda")
    nr = inputs.norm_rope_params(N).to("cuda")
    pk = case.packed.clone()
    HD = H * 128
    pq, pkk = (pk[:, :, i * HD:(i + 1) * HD].unflatten(2, (H, 128)) for i in range(2))
    buf, rbuf = sage.Buffers(B, N, H), sage.Buffers(B, N, H)
    out, out2 = sage.token_major_out(B, N, H), sage.token_major_out(B, N, H)
    codes, scales = sage.mx_out(B, N, H, sage.MX_E4M3)
    sm = 1.0 / math.sqrt(128.0)
    torch.cuda.synchronize()
    calls = {
        "sage_quantize_qk": lambda: sage.sage_quantize_qk(case.q, case.k, buf.q_codes, buf.q_scale, buf.k_codes,
                                                          buf.k_scale, buf.k_mean, buf.ws_qk),
        "sage_quantize_v": lambda: sage.sage_quantize_v(case.v, buf.v_codes, buf.v_scale, buf.ws_v),
        "sage_quantize_qkv": lambda: sage.quantize_qkv(case.q, case.k, case.v, buf),
        "sage_attn_fwd": lambda: sage.sage_attn_fwd(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale,
                                                    buf.v_codes, buf.v_scale, out, sm),
        "sage_attn_fwd_bf16": lambda: sage.sage_attn_fwd_bf16(case.q, case.k, case.v, out2, sm),
        "sage_attn_fwd_int8qk": lambda: sage.sage_attn_fwd_int8qk(buf.q_codes, buf.q_scale, buf.k_codes,
                                                                  buf.k_scale, case.v, out2, sm),
        "sage_qk_norm_rope": lambda: sage.sage_qk_norm_rope(pq, pkk, nr.gamma_q, nr.gamma_k, nr.rope, nr.eps),
        "sage_quantize_qkv_rope": lambda: sage.quantize_qkv_rope(case.q, case.k, case.v, nr, rbuf),
        "sage_mx_quantize": lambda: sage.sage_mx_quantize(out, sage.MX_E4M3, codes, scales),
        "sage_attn_fwd_mx": lambda: sage.sage_attn_fwd_mx(buf.q_codes, buf.q_scale, buf.k_codes, buf.k_scale,
                                                          buf.v_codes, buf.v_scale, sage.MX_E4M3, codes, scales, sm),
    }
    for name, _ in EXPECTED:
        calls[name]()
        torch.cuda.synchronize()
    print("launch audit: %d calls done" % len(EXPECTED), flush=True)


if __name__ == "__main__":
    main()
