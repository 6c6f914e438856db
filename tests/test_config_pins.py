"""Shapes of the path pinned by the parameter counts the pages print.

The pages give exact parameter totals (tests/golden/parameter_counts.json) and
the configuration (tests/golden/kimi_k2_config.json).  Rebuilding the totals
from the configuration pins the widths the oracle and the library assume:
64 heads of 128 (nope) + 64 (rope) query/key dims and 128 value dims, a single
64-wide rotary key shared by all heads (the key latent projects to 512 + 64),
and an 8,192 -> 7,168 output projection.
"""
import json
import os

import oracle
from transformer_attention_mla_amd import NOPE, ROPE, VDIM, inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def attention_params(c):
    H = c["num_attention_heads"]
    qk = c["qk_nope_head_dim"] + c["qk_rope_head_dim"]
    q_down = c["hidden_size"] * c["q_lora_rank"] + c["q_lora_rank"]          # + its RMSNorm gain
    q_up = c["q_lora_rank"] * H * qk
    kv_down = c["hidden_size"] * (c["kv_lora_rank"] + c["qk_rope_head_dim"]) + c["kv_lora_rank"]
    kv_up = c["kv_lora_rank"] * H * (c["qk_nope_head_dim"] + c["v_head_dim"])
    o_proj = H * c["v_head_dim"] * c["hidden_size"]
    return q_down + q_up + kv_down + kv_up + o_proj, o_proj


def test_o_proj_parameter_count():
    c, n = load("kimi_k2_config.json"), load("parameter_counts.json")
    _, o = attention_params(c)
    assert o == n["o_proj_per_block"] == 8192 * 7168
    assert o * 60 == n["o_proj_60_blocks"]


def test_block_parameter_counts_rebuild_exactly():
    c, n = load("kimi_k2_config.json"), load("parameter_counts.json")
    attn, _ = attention_params(c)
    d = c["hidden_size"]
    norms = 2 * d
    dense_mlp = 3 * d * c["intermediate_size"]
    assert attn + dense_mlp + norms == n["dense_block"]
    expert = 3 * d * c["moe_intermediate_size"]
    router = c["n_routed_experts"] * d + c["n_routed_experts"]  # gate weight + score correction bias
    moe = attn + norms + router + (c["n_routed_experts"] + c["n_shared_experts"]) * expert
    assert moe == n["moe_block"]
    n_moe = c["num_hidden_layers"] - c["first_k_dense_replace"]
    assert n_moe == 60 and moe * n_moe == n["moe_blocks_60"]
    assert n["dense_block"] + n["moe_blocks_60"] == n["stack_total"]
    assert c["vocab_size"] * d == n["embedding"]


def test_library_and_oracle_widths_follow_config():
    c = load("kimi_k2_config.json")
    want = (c["qk_nope_head_dim"], c["qk_rope_head_dim"], c["v_head_dim"])
    assert (NOPE, ROPE, VDIM) == want
    assert oracle.dims() == want
    assert c["num_attention_heads"] * c["v_head_dim"] == 8192
    assert c["attention_bias"] is False


def test_input_constants_follow_config():
    c = load("kimi_k2_config.json")
    assert inputs.ROPE_THETA == c["rope_theta"]
    assert inputs.ROT_DIM == c["qk_rope_head_dim"]
    assert inputs.D_MODEL == c["hidden_size"]
    assert abs(inputs.SOFTMAX_SCALE - (c["qk_nope_head_dim"] + c["qk_rope_head_dim"]) ** -0.5) < 1e-15
