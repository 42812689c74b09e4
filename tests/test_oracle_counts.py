"""Pins of the oracle's cache accounting against figures printed on the pages
(tests/golden/page_figures.json carries each figure with its source)."""
import json
import os

import pytest

from oracle import cache_elements_per_token, kv_cache_bytes
from mla_synth import V2

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def test_v2_dims_match_symbol_table():
    s = GOLD["v2_symbols"]["value"]
    assert (V2.d_model, V2.n_heads, V2.d_nope, V2.d_rope, V2.d_cq, V2.d_latent) == (
        s["d"], s["n_h"], s["d_h_C"], s["d_h_R"], s["d_c_prime"], s["d_c"])
    assert V2.d_nope + V2.d_rope == s["d_h"]
    shp = GOLD["projection_shapes"]["value"]
    assert shp["W_UQ"] == [V2.n_heads * V2.d_nope, V2.d_cq]
    assert shp["W_QR"] == [V2.n_heads * V2.d_rope, V2.d_cq]
    assert shp["W_KR"] == [V2.d_rope, V2.d_model]


def test_mha_vs_mla_elements():
    mha = cache_elements_per_token("mha", n_heads=V2.n_heads, d_head=V2.d_nope)
    mla = cache_elements_per_token("mla", n_heads=V2.n_heads, d_latent=V2.d_latent, d_rope=V2.d_rope)
    assert mha == GOLD["mha_elements_per_token_layer"]["value"]
    assert mla == GOLD["mla_elements_per_token_layer"]["value"] == sum(GOLD["mla_elements_per_token_layer"]["parts"])
    assert round(mha / mla) == GOLD["mla_over_mha"]["value_inverse"]
    # and the row the cache layout stores is exactly that long
    assert V2.row == mla


def test_uncompressed_and_compression_factors():
    unc = cache_elements_per_token("mla_uncompressed", n_heads=V2.n_heads, d_head=V2.d_nope, d_rope=V2.d_rope)
    g = GOLD["mla_uncompressed_elements"]
    assert unc == g["value"]
    mha = cache_elements_per_token("mha", n_heads=V2.n_heads, d_head=V2.d_nope)
    assert abs(unc / mha - g["fraction_of_mha"]) < 0.01
    f = GOLD["compression_factors"]["value"]
    assert f["c_Q"][1] == V2.n_heads * V2.d_nope and round(f["c_Q"][1] / V2.d_cq) == f["c_Q"][2]
    assert f["c_KV"][1] / V2.d_latent == f["c_KV"][2]
    assert f["k_R"][1] == V2.n_heads * V2.d_rope and f["k_R"][1] / V2.d_rope == f["k_R"][2]


def test_gqa_equivalent_groups():
    g = GOLD["gqa_equivalent_groups"]["value"]
    mla = cache_elements_per_token("mla", n_heads=V2.n_heads, d_latent=V2.d_latent, d_rope=V2.d_rope)
    assert cache_elements_per_token("gqa", n_heads=V2.n_heads, d_head=V2.d_nope, groups=g) == mla


def test_128k_context_claims():
    """MHA 'hundreds of GB' and MLA 'under 10 GB' at 128K tokens in bf16 hold
    together for whole-model layer counts 12..66; per layer the latent cache of
    one 131072-token sequence is 150,994,944 bytes."""
    c = GOLD["context_128k"]["value"]
    mha = cache_elements_per_token("mha", n_heads=V2.n_heads, d_head=V2.d_nope)
    mla = cache_elements_per_token("mla", n_heads=V2.n_heads, d_latent=V2.d_latent, d_rope=V2.d_rope)
    assert kv_cache_bytes(mla, c["tokens"], 1, 2) == 150_994_944
    assert kv_cache_bytes(mha, c["tokens"], 1, 2) == 8_589_934_592
    ok = [L for L in range(1, 200)
          if kv_cache_bytes(mha, c["tokens"], L, 2) >= c["mha_at_least_bytes"]
          and kv_cache_bytes(mla, c["tokens"], L, 2) < c["mla_below_bytes"]]
    assert ok[0] == 12 and ok[-1] == 66 and len(ok) == 55


def test_absorbed_compute_factor():
    a = GOLD["absorbed_compute_factor"]
    assert a["parts"] == [V2.d_nope, V2.d_latent]
    assert V2.d_latent / V2.d_nope == a["value"]


def test_mha_fp16_byte_example():
    e = GOLD["mha_fp16_example"]["value"]
    per_tok = cache_elements_per_token("mha", n_heads=e["heads"], d_head=e["d_head"])
    assert kv_cache_bytes(per_tok, 1, 1, e["bytes_per_element"]) == e["per_token_layer_bytes"]
    assert kv_cache_bytes(per_tok, e["tokens"], 1, e["bytes_per_element"]) == e["per_layer_bytes"]
    assert kv_cache_bytes(per_tok, e["tokens"], e["layers"], e["bytes_per_element"]) == e["total_bytes"]


def test_unknown_kind_rejected():
    with pytest.raises(ValueError):
        cache_elements_per_token("mqa", n_heads=1)
