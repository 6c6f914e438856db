"""Shared helpers of the GPU parity tests (host-side conversions and gates)."""
import math
import sys

import numpy as np
import torch

from transformer_attention_mla_amd import inputs

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))
# Tolerance of the computation on floating-point outputs (max-abs).
TOL = 1e-2
# Relative tolerance of the weights-sum-to-one probe.
SUM_TOL = 1e-5


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print(*a, file=sys.stdout, flush=True)


def bits(t):
    return inputs.bits(t)


def bf16_half_spacing(x):
    """Half the bf16 spacing at |x| (the most a correct bf16 store can add)."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    e = np.floor(np.log2(ax))
    return 2.0 ** (e - 8)


def to_host64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check_bf16_is_rne_of_f32(out_bf16, out_f32):
    want = out_f32.to(torch.bfloat16)
    assert torch.equal(out_bf16.view(torch.int16), want.view(torch.int16)), \
        "bf16 output is not the round-to-nearest-even of the float32 output"


def check_close(got, want, tol, what):
    assert got.shape == want.shape, f"{what}: shape {got.shape} against {want.shape}"
    err = np.max(np.abs(got - want)) if got.size else 0.0
    say(f"  {what}: max-abs {err:.3e} (tol {tol:.1e})")
    assert err <= tol, f"{what}: {err} > {tol}"
    return err


def check_bf16_close(got_bf16, want64, what):
    got = to_host64(got_bf16)
    lim = TOL + bf16_half_spacing(want64)
    err = np.abs(got - want64)
    say(f"  {what}: max-abs {err.max():.3e} (tol {TOL:.0e} + half bf16 spacing)")
    assert np.all(err <= lim), f"{what}: max excess {(err - lim).max()}"
