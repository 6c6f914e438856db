"""GPU parity of the key-blocked value layout (flag MLA_V_BLOCKED).

The prefill with v key-blocked ([B, H, ceil(T/16), 128, 16]) performs the same
arithmetic in the same order as with v in [B, H, T, 128]: its outputs must be
bit-identical to the natural-layout call (which the other prefill tests hold
to the oracle), and within the tolerance of the oracle itself on small
shapes.  The slots of positions past T in the last block never reach a
result: NaN or infinity there gives the same bits as zeros.  The
up-projection writing v key-blocked must write the same values, element for
element, as its [B, H, T, 128] output.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_mla_amd as mla
from transformer_attention_mla_amd import inputs

from _gpu_helpers import SCALE, TOL, bits, check_close, say, to_host64

pytestmark = pytest.mark.gpu


def to_dev(d, dev):
    return {k: v.to(dev) for k, v in d.items()}


def prefill(g, v, **kw):
    out, lse = mla.mla_attend_prefill(g["q_nope"], g["q_pe"], g["k_nope"], g["k_pe"], v, g["R"],
                                      SCALE, want_lse=True, **kw)
    torch.cuda.synchronize()
    return out, lse


def assert_same(a, b, what):
    assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16)), what


# T % 16 in {1, 15, 0, 1, 8, 0, 1, 0}: a partial last block and whole ones; the
# B = 1, H = 64, T = 1024 case runs unpaired, (4, 64, 2048) the paired schedule.
@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (2, 3, 63), (1, 2, 64), (1, 3, 65), (2, 4, 1000),
                                   (1, 64, 1024), (1, 1, 513), (4, 64, 2048)])
def test_prefill_vblocked_matches_natural(B, H, T, gpu_device):
    say(f"prefill key-blocked v B={B} H={H} T={T}")
    d = inputs.prefill_inputs(B, H, T, workload=0)
    g = to_dev(d, gpu_device)
    vb = inputs.to_v_blocked(g["v"])
    for f32 in (True, False):
        want, want_lse = prefill(g, g["v"], out_f32=f32)
        got, got_lse = prefill(g, vb, out_f32=f32, v_blocked=True)
        assert_same(got, want, f"output (float32 store {f32}) differs from the natural layout")
        assert_same(got_lse, want_lse, "lse differs from the natural layout")
    if B * H * T <= 4 * 1000:
        o, ol = oracle.prefill(bits(d["q_nope"]), bits(d["q_pe"]), bits(d["k_nope"]),
                               bits(d["k_pe"]), bits(d["v"]), d["R"].numpy(), SCALE)
        out32, lse = prefill(g, vb, out_f32=True, v_blocked=True)
        check_close(to_host64(out32), o, TOL, "float32 output vs oracle")
        check_close(to_host64(lse), ol, TOL, "lse vs oracle")


@pytest.mark.parametrize("T", [1, 17, 63, 1000])
@pytest.mark.parametrize("fill", [float("nan"), float("inf"), float("-inf")])
def test_prefill_vblocked_padding_never_read(T, fill, gpu_device):
    say(f"prefill key-blocked v, padding {fill}, T={T}")
    d = inputs.prefill_inputs(1, 3, T, workload=0)
    g = to_dev(d, gpu_device)
    zero = inputs.to_v_blocked(g["v"], fill=0.0)
    junk = inputs.to_v_blocked(g["v"], fill=fill)
    want, want_lse = prefill(g, zero, out_f32=True, v_blocked=True)
    got, got_lse = prefill(g, junk, out_f32=True, v_blocked=True)
    assert torch.isfinite(got).all()
    assert_same(got, want, "padding slots reached the output")
    assert_same(got_lse, want_lse, "padding slots reached the lse")


@pytest.mark.parametrize("B,T,workload", [(4, 4096, 3), (1, 16384, 4)])
def test_prefill_vblocked_full_workload(B, T, workload, gpu_device):
    """The timed workloads with this layout (B = 4, T = 4096 and B = 1,
    T = 16384 with the YaRN table, 64 heads, paired launches): bit-identical
    to the natural layout."""
    H = 64
    say(f"prefill key-blocked v full B={B} H={H} T={T}")
    g = inputs.prefill_inputs(B, H, T, workload=workload, device=gpu_device)
    vb = inputs.to_v_blocked(g["v"])
    want, want_lse = prefill(g, g["v"])
    got, got_lse = prefill(g, vb, v_blocked=True)
    assert_same(got, want, "output differs from the natural layout")
    assert_same(got_lse, want_lse, "lse differs from the natural layout")


@pytest.mark.parametrize("B,H,T", [(1, 3, 65), (2, 64, 1024)])
def test_prefill_vblocked_fp8_and_noalloc(B, H, T, gpu_device):
    say(f"prefill key-blocked v, FP8 output and allocation-free forms B={B} H={H} T={T}")
    g = inputs.prefill_inputs(B, H, T, workload=0, device=gpu_device)
    vb = inputs.to_v_blocked(g["v"])
    args = (g["q_nope"], g["q_pe"], g["k_nope"], g["k_pe"])
    c8, s8, l8 = mla.mla_attend_prefill_fp8(*args, g["v"], g["R"], SCALE, want_lse=True)
    b8, bs8, bl8 = mla.mla_attend_prefill_fp8(*args, vb, g["R"], SCALE, want_lse=True,
                                             v_blocked=True)
    torch.cuda.synchronize()
    assert torch.equal(b8, c8)
    ms = B * T
    assert torch.equal(bs8[:, :ms], s8[:, :ms])
    assert_same(bl8, l8, "FP8-output lse differs")
    o, _ = mla.mla_attend_prefill(*args, g["v"], g["R"], SCALE)
    on, _ = mla.mla_attend_prefill_noalloc(*args, vb, g["R"], SCALE, v_blocked=True)
    torch.cuda.synchronize()
    assert_same(on, o, "allocation-free form differs")


# Small kernel (the first three), the wide kernel with whole 16-row blocks
# ((2, 800, 64), (4, 4096, 64)) and with blocks that span two sequences
# ((2, 1000, 64): T % 16 = 8).
@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (2, 17, 3), (1, 300, 4), (2, 800, 64), (2, 1000, 64),
                                   (4, 4096, 64)])
def test_up_project_vblocked(B, T, H, gpu_device):
    say(f"up-projection key-blocked v B={B} T={T} H={H}")
    g = inputs.up_project_inputs(B, T, H, workload=0, device=gpu_device)
    args = (g["q_lat"], g["ckv"], g["w_q_b"], g["w_kv_b"])
    f32_cases = (False, True) if B * T * H <= 2 * 1000 * 64 else (False,)
    for f32 in f32_cases:
        want = mla.mla_up_project(*args, out_f32=f32)
        odt = torch.float32 if f32 else torch.bfloat16
        nb = (T + 15) // 16
        vb = torch.full((B, H, nb, 128, 16), float("nan"), dtype=odt, device=gpu_device)
        outs = [torch.empty_like(want[0]), torch.empty_like(want[1]), torch.empty_like(want[2]), vb]
        got = mla.mla_up_project(*args, outs=outs, out_f32=f32, v_blocked=True)
        torch.cuda.synchronize()
        for i in range(3):
            assert_same(got[i], want[i], f"output {i} differs with the key-blocked v")
        assert_same(inputs.from_v_blocked(vb, T), want[3], "key-blocked v differs from v")
        # the padding slots stay as the caller left them
        if T % 16:
            pad = vb.transpose(3, 4).reshape(B, H, nb * 16, 128)[:, :, T:]
            assert torch.isnan(pad).all()


def test_up_project_vblocked_into_prefill(gpu_device):
    """Up-projection with the key-blocked v straight into the prefill, bit-identical
    to the natural-layout chain."""
    B, T, H = 2, 1000, 64
    say(f"up-projection then prefill, key-blocked v B={B} T={T} H={H}")
    g = inputs.up_project_inputs(B, T, H, workload=0, device=gpu_device)
    args = (g["q_lat"], g["ckv"], g["w_q_b"], g["w_kv_b"])
    qn, qp, kn, v = mla.mla_up_project(*args)
    *_, vb = mla.mla_up_project(*args, v_blocked=True)
    k_pe = inputs.normal_bf16((B, 1, T, 64), 77, device=gpu_device)
    R = torch.from_numpy(inputs.rope_angles(T)).to(gpu_device)
    want, wl = mla.mla_attend_prefill(qn, qp, kn, k_pe, v, R, SCALE, want_lse=True)
    got, gl = mla.mla_attend_prefill(qn, qp, kn, k_pe, vb, R, SCALE, want_lse=True, v_blocked=True)
    torch.cuda.synchronize()
    assert_same(got, want, "prefill output differs")
    assert_same(gl, wl, "prefill lse differs")
