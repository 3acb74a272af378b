"""Pins of the configurations against the numbers the pages print.

The fixture ``tests/golden/v3_key_dimensions.txt`` holds values printed by
the "DeepSeek-V3 Decoupled Implementation" README ("Key Dimensions (671B
variant)" table and "Architecture" list); every V3-shaped config the tests
and the bench use must carry exactly those sizes."""

import math
import os

import synth_inputs as si
from tests.helpers import oracle_cfg
import oracle as orc

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    out = {}
    for line in open(os.path.join(HERE, "golden", "v3_key_dimensions.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split()
        out[k] = int(v)
    return out


def test_v3_configs_carry_the_printed_dimensions():
    g = _golden()
    for name in ("v3_prefill", "v3_decode", "v3_yarn"):
        c = si.CONFIGS[name]
        for k in ("hidden_size", "num_attention_heads", "q_lora_rank", "kv_lora_rank",
                  "qk_nope_head_dim", "qk_rope_head_dim", "v_head_dim"):
            assert c[k] == g[k], (name, k)
        assert c["kv_lora_rank"] == g["latent_dim"]
        assert c["qk_rope_head_dim"] == g["decoupled_rope_dim"]


def test_latent_cache_row_is_latent_plus_rope():
    g = _golden()
    # V3 latent sizes; hidden size and head count shrunk to keep the draw small
    c = dict(si.CONFIGS["v3_decode"], hidden_size=8, num_attention_heads=1, q_lora_rank=8)
    _, _, _, cache = si.make_decode_inputs(c, batch=1, capacity=2, len_lo=1, len_hi=1)
    assert cache.shape[-1] == g["latent_dim"] + g["decoupled_rope_dim"]


def test_yarn_config_extends_to_the_printed_context():
    g = _golden()
    c = si.CONFIGS["v3_yarn"]
    assert c["rope_factor"] == g["yarn_factor"]
    assert c["rope_factor"] * c["original_max_position_embeddings"] == g["yarn_extended_context"]


def test_v3_softmax_scale_is_inverse_sqrt_dk():
    g = _golden()
    dk = g["qk_nope_head_dim"] + g["qk_rope_head_dim"]
    assert orc.softmax_scale(oracle_cfg(si.CONFIGS["v3_prefill"])) == 1.0 / math.sqrt(dk)
