"""Seeded input generators: reproducibility, angle tables, YaRN step."""
import math

import numpy as np
import torch

from transformer_attention_mla_amd import inputs


def test_plain_angles():
    R = inputs.rope_angles(100)
    assert R.shape == (100, 32) and R.dtype == np.float32
    assert np.all(R[0] == 0)
    assert R[1, 0] == 1.0
    assert R[37, 16] == np.float32(37 * 50000.0 ** -0.5)
    # frequencies fall monotonically with the pair index
    assert np.all(np.diff(R[1].astype(np.float64)) < 0)


def test_yarn_angles_step_at_one_turn():
    plain = inputs.rope_angles(16384)
    yarn = inputs.yarn_angles(16384)
    f = inputs.inv_freq()
    turns = 4096 * f / (2 * math.pi)
    keep = turns >= 1.0
    assert keep.sum() == 20 and np.all(keep[:20]) and not np.any(keep[20:])
    assert np.array_equal(yarn[:, :20], plain[:, :20])
    assert np.array_equal(yarn[:, 20:], plain[:, 20:] / np.float32(32))


def test_yarn_ramp_when_betas_differ():
    f = inputs.inv_freq()
    g = inputs.yarn_inv_freq(beta_fast=32.0, beta_slow=1.0)
    assert np.all(g <= f + 1e-300) and np.all(g >= f / 32 - 1e-300)


def test_generators_are_seeded():
    a = inputs.normal_bf16((3, 5), 123)
    b = inputs.normal_bf16((3, 5), 123)
    c = inputs.normal_bf16((3, 5), 124)
    assert a.dtype == torch.bfloat16
    assert torch.equal(a, b) and not torch.equal(a, c)
    w = inputs.normal_bf16((256, 256), 5, std=0.02).float()
    assert 0.015 < w.std().item() < 0.025


def test_prefill_inputs_shapes():
    d = inputs.prefill_inputs(2, 3, 17, workload=0)
    assert d["q_nope"].shape == (2, 3, 17, 128)
    assert d["q_pe"].shape == (2, 3, 17, 64)
    assert d["k_nope"].shape == (2, 3, 17, 128)
    assert d["k_pe"].shape == (2, 1, 17, 64)
    assert d["v"].shape == (2, 3, 17, 128)
    assert d["R"].shape == (17, 32) and d["R"].dtype == torch.float32
    d = inputs.decode_inputs(2, 3, 9, q_pos=9)
    assert d["k_cache"].shape == (2, 3, 9, 192) and d["R"].shape == (10, 32)
