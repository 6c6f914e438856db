"""GPU checks of mla_attend_prefill_fp8 (the attention output quantized for
the FP8 o_proj in the kernel's epilogue) and of mla_out_proj_fp8_q.

Gates (exact): the codes and scales equal the oracle's quantization
(oracle.act_quant) of the bf16 output of mla_attend_prefill, and equal the
GPU quantizer's (mla_act_quant) at the benchmark's size; lse equals the bf16
path's bit for bit; mla_out_proj_fp8_q on those codes equals
mla_out_proj_fp8_dyn on the bf16 output bit for bit (small-M split and
large-M tiles).  The bf16 attention output itself is gated against the fp64
oracle in test_prefill_gpu.py and the FP8 product in test_oproj_gpu.py.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_mla_amd as mla
from transformer_attention_mla_amd import inputs

from _gpu_helpers import SCALE, bits, say

pytestmark = pytest.mark.gpu


def both(B, H, T, dev, workload=0):
    d = inputs.prefill_inputs(B, H, T, workload=workload, device=dev)
    args = (d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], d["R"], SCALE)
    out16, lse16 = mla.mla_attend_prefill(*args, want_lse=True)
    x8, sT, lse8 = mla.mla_attend_prefill_fp8(*args, want_lse=True)
    torch.cuda.synchronize()
    return out16, lse16, x8, sT, lse8


@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 3, 17), (2, 2, 100), (1, 5, 300), (2, 4, 1000),
                                   (1, 64, 64)])
def test_prefill_fp8_matches_oracle_quantization(B, H, T, gpu_device):
    say(f"prefill fp8 B={B} H={H} T={T}")
    out16, lse16, x8, sT, lse8 = both(B, H, T, gpu_device)
    M, K = B * T, H * 128
    want_q, want_s = oracle.act_quant(bits(out16.view(M, K).cpu()))
    assert np.array_equal(x8.view(M, K).cpu().numpy(), want_q), "codes differ"
    got_s = sT.cpu().numpy()[:, :M].T
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), "scales differ"
    assert torch.equal(lse8, lse16), "lse differs from the bf16 path"


def test_prefill_fp8_benchmark_size(gpu_device):
    """B=4, T=4096, H=64 (the benchmark's launch): equal to mla_act_quant of
    the bf16 output, every code and scale."""
    B, H, T = 4, 64, 4096
    say("prefill fp8 B=4 H=64 T=4096")
    out16, _, x8, sT, _ = both(B, H, T, gpu_device, workload=3)
    M, K = B * T, H * 128
    q, s = mla.mla_act_quant(out16.view(M, K))
    torch.cuda.synchronize()
    assert torch.equal(x8.view(M, K), q), "codes differ"
    assert torch.equal(sT[:, :M], s[:, :M]), "scales differ"


@pytest.mark.parametrize("B,H,T", [(1, 64, 64), (1, 64, 33), (2, 64, 1000)])
def test_oproj_fp8_q_equals_dyn(B, H, T, gpu_device):
    """The attention's FP8 output through mla_out_proj_fp8_q equals the bf16
    output through mla_out_proj_fp8_dyn bit for bit (M = 64 and 33: split K;
    M = 2000: the 256 x 256 tiles)."""
    say(f"fp8 pipeline B={B} H={H} T={T}")
    out16, _, x8, sT, _ = both(B, H, T, gpu_device)
    M, K, N = B * T, H * 128, inputs.D_MODEL
    w8, ws = inputs.out_proj_weight_fp8(N, K, workload=3, device=gpu_device)
    y_q = mla.mla_out_proj_fp8_q(x8.view(M, K), sT, w8, ws, out_f32=True)
    y_d = mla.mla_out_proj_fp8_dyn(out16.view(M, K), w8, ws, out_f32=True)
    torch.cuda.synchronize()
    assert torch.equal(y_q, y_d), f"max diff {(y_q - y_d).abs().max().item()}"
