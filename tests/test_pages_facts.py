"""The shapes and tiling facts the pages print, checked against the workload
definitions used here (tests/golden/pages_facts.json holds them with citations)."""
import json
import math
import os

from quantized_softmax_attention_amd import inputs

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))


def test_block24_shape_matches_q_shape():
    B, N, H, D, layout, _ = inputs.CONFIGS["block24"]
    assert [B, N, H, D] == FACTS["q_shape"]["value"]
    assert N == FACTS["packed_tokens"]["value"]
    assert layout == "packed"


def test_token_major_output_rows_match_h_msa_shape():
    # q_shape fixes H = 56 heads of D = 128, so the attention output is the
    # token-major [N, H * D] = [37810, 7168]; h_msa_shape [37810, 5376] is the
    # block's hidden width after the output projection, which only shares N.
    B, N, H, D, _, _ = inputs.CONFIGS["block24"]
    assert N == FACTS["h_msa_shape"]["value"][0]
    assert H * D == 7168 != FACTS["h_msa_shape"]["value"][1]


def test_page_grid_is_query_tiles_times_heads():
    s = FACTS["scheduler"]["value"]
    B, N, H, D, _, _ = inputs.CONFIGS["block24"]
    assert math.ceil(N / s["cta_q"]) * H == s["grid_ctas"]
    # the page's smem fits one 128x128 int8 Q tile plus 64x128 int8 K and 64x128 fp8 V
    assert s["cta_q"] * D + 2 * s["cta_k"] * D == s["dynamic_shared_memory_bytes"]


def test_packed_view_geometry():
    c = inputs.packed_case(1, 7, 56, 128, seed=0)
    assert c.packed.shape == (1, 7, 3 * 7168)
    assert c.q.stride() == (7 * 21504, 21504, 128, 1)
    assert c.k.storage_offset() == 7168 and c.v.storage_offset() == 2 * 7168
