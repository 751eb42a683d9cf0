"""Write tests/golden/tiny_oracle.json: digests and a few values of the oracle's
results on the tiny workload (B=1, N=256, H=2, D=128, seed 0): quantisers, the
exact, method and INT8-QK/bf16-PV attention, MX blocks of the method's output
and the RMSNorm + RoPE transform of Q and K.  Calls only the
oracle (and the seeded input generators).  Re-run only when a change to the
oracle's arithmetic is justified by the method's definition.

    python tests/golden/make_golden.py
"""
import hashlib
import json
import math
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from quantized_softmax_attention_amd import inputs  # noqa: E402
from tests.helpers import oracle_view  # noqa: E402


def digest(a) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def compute():
    c = inputs.config("tiny")
    q, k, v = (oracle_view(t) for t in (c.q, c.k, c.v))
    sm = 1.0 / math.sqrt(128.0)
    km = oracle.kmean(k)
    qc, qs = oracle.quant_q(q, 32)
    kc, ks = oracle.quant_k(k, km, 64)
    vc, vs = oracle.quant_v(v)
    exact = oracle.attn_exact(q, k, v, sm)
    method = oracle.attn_method(qc, qs, kc, ks, vc, vs, sm)
    i8qk = oracle.attn_int8qk(qc, qs, kc, ks, v, sm)
    tok = np.ascontiguousarray(method.transpose(0, 2, 1, 3)).reshape(c.B, c.N, c.H * c.D)
    mx8c, mx8s = oracle.mx_quantize(tok, oracle.MX_E4M3)
    mx4c, mx4s = oracle.mx_quantize(tok, oracle.MX_E2M1)
    nr = inputs.norm_rope_params(c.N, seed=1)
    tq = oracle.norm_rope(q, nr.gamma_q.numpy(), nr.rope.numpy(), nr.eps)
    tk = oracle.norm_rope(k, nr.gamma_k.numpy(), nr.rope.numpy(), nr.eps)
    return {
        "inputs_sha256": {n: digest(t.contiguous().float().numpy())
                          for n, t in (("q", c.q), ("k", c.k), ("v", c.v))},
        "km_sha256": digest(km), "q_codes_sha256": digest(qc), "q_scales_sha256": digest(qs),
        "k_codes_sha256": digest(kc), "k_scales_sha256": digest(ks),
        "v_codes_sha256": digest(vc), "v_scales_sha256": digest(vs),
        "exact_row0_head0_first8": [float(x) for x in exact[0, 0, 0, :8]],
        "method_row0_head0_first8": [float(x) for x in method[0, 0, 0, :8]],
        "method_vs_exact_rel_l2": oracle.rel_l2(method, exact),
        "int8qk_row0_head0_first8": [float(x) for x in i8qk[0, 0, 0, :8]],
        "int8qk_vs_exact_rel_l2": oracle.rel_l2(i8qk, exact),
        "mx_e4m3_codes_sha256": digest(mx8c), "mx_e4m3_scales_sha256": digest(mx8s),
        "mx_e2m1_codes_sha256": digest(mx4c), "mx_e2m1_scales_sha256": digest(mx4s),
        "norm_rope_q_sha256": digest(tq), "norm_rope_k_sha256": digest(tk),
    }


if __name__ == "__main__":
    out = compute()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path, "rel_l2", out["method_vs_exact_rel_l2"])
