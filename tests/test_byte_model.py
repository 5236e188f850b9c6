"""The per-token byte accounting used by the roofline figures, pinned to the
capacity numbers printed on the Proxima README (tests/golden/byte_model.json)."""
import json
import os

from rank_compressed_paged_amd import metrics

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fx():
    with open(os.path.join(GOLDEN, "byte_model.json")) as f:
        return json.load(f)


def test_dense_kv_at_32768_is_16_gib():
    fx = _fx()
    per_tok = metrics.dense_bytes_per_token(fx["num_heads"], fx["head_size"])
    total = per_tok * fx["layers_assumed"] * fx["max_model_len_long"]
    assert total / 2**30 == fx["dense_kv_gib_at_32768"]


def test_capacity_ratio_consistent_with_rank_reading():
    """Same KV budget: plain blocks x dense bytes ~= STAR-KV blocks x latent
    bytes + fp16 bases, with r_k = 64 per head and a joint r_v = 512."""
    fx = _fx()
    H, d, bs, L = fx["num_heads"], fx["head_size"], fx["block_size"], fx["layers_assumed"]
    dense = fx["plain_vllm_blocks"] * bs * L * metrics.dense_bytes_per_token(H, d)
    lat = fx["star_kv_blocks"] * bs * L * metrics.latent_bytes_per_token(H, 64, 512)
    bases = L * metrics.basis_bytes(H, d, 64, 512)
    assert abs(lat + bases - dense) / dense < 0.01
    ratio = metrics.dense_bytes_per_token(H, d) / metrics.latent_bytes_per_token(H, 64, 512)
    assert abs(ratio - fx["capacity_ratio"]) / fx["capacity_ratio"] < 0.05
    assert round(fx["star_kv_blocks"] / fx["plain_vllm_blocks"], 2) == fx["capacity_ratio"]


def test_latent_bytes_per_token_main_shape():
    assert metrics.latent_bytes_per_token(32, 64, 512) == 5120
    assert metrics.latent_bytes_per_token(4, 16, 64) == 256
