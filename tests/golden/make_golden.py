"""Write tests/golden/tiny_oracle.json: digests and a few values of the oracle's
results on the tiny workload (B=1, N=256, H=2, D=128, seed 0).  Calls only the
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
    return {
        "inputs_sha256": {n: digest(t.contiguous().float().numpy())
                          for n, t in (("q", c.q), ("k", c.k), ("v", c.v))},
        "km_sha256": digest(km), "q_codes_sha256": digest(qc), "q_scales_sha256": digest(qs),
        "k_codes_sha256": digest(kc), "k_scales_sha256": digest(ks),
        "v_codes_sha256": digest(vc), "v_scales_sha256": digest(vs),
        "exact_row0_head0_first8": [float(x) for x in exact[0, 0, 0, :8]],
        "method_row0_head0_first8": [float(x) for x in method[0, 0, 0, :8]],
        "method_vs_exact_rel_l2": oracle.rel_l2(method, exact),
    }


if __name__ == "__main__":
    out = compute()
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path, "rel_l2", out["method_vs_exact_rel_l2"])
