"""The allocation-free prefill entry point (mla_attend_prefill_noalloc, for
callers that cannot allocate device memory): through the C ABI it must give
the same bytes as mla_attend_prefill with a caller workspace, on two calls in
a row, the second smaller than the first (so the static buffer still holds the
first call's contents), and agree with the oracle."""
import pytest
import torch

import oracle
import transformer_attention_mla_amd as mla
from transformer_attention_mla_amd import inputs

from _gpu_helpers import SCALE, TOL, bits, check_close, say, to_host64

pytestmark = pytest.mark.gpu


def _pair(d, out_f32):
    """Both entry points on the same inputs, outputs preallocated."""
    B, H, T = d["q_nope"].shape[:3]
    dev = d["q_nope"].device
    odt = torch.float32 if out_f32 else torch.bfloat16
    o_ref = torch.empty((B, T, H * 128), dtype=odt, device=dev)
    o_new = torch.full_like(o_ref, float("nan"))
    l_ref = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    l_new = torch.full_like(l_ref, float("nan"))
    args = (d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], d["R"], SCALE)
    mla.mla_attend_prefill(*args, out=o_ref, lse=l_ref, out_f32=out_f32)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    mla.mla_attend_prefill_noalloc(*args, out=o_new, lse=l_new, out_f32=out_f32)
    torch.cuda.synchronize()
    after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    assert after == before, "the allocation-free call allocated through torch"
    return o_ref, l_ref, o_new, l_new


def test_prefill_noalloc_matches_workspace_entry_point(gpu_device):
    # first call near the buffer's limit: T*256 + B*T*128 = 10.5 MiB of 16 MiB
    big = (8, 2, 8192)
    small = (1, 4, 300)
    for (B, H, T), out_f32 in ((big, True), (small, True), (small, False)):
        say(f"prefill noalloc B={B} H={H} T={T} out_f32={out_f32}")
        d = inputs.prefill_inputs(B, H, T, workload=0, device=gpu_device)
        o_ref, l_ref, o_new, l_new = _pair(d, out_f32)
        assert torch.equal(o_new, o_ref), "output differs from mla_attend_prefill"
        assert torch.equal(l_new, l_ref), "lse differs from mla_attend_prefill"
    want, wl = oracle.prefill(*[bits(d[k].cpu()) for k in ("q_nope", "q_pe", "k_nope", "k_pe", "v")],
                              d["R"].cpu().numpy(), SCALE)
    o32, l32, _, _ = _pair(d, True)
    check_close(to_host64(o32), want, TOL, "float32 output vs oracle")
    check_close(to_host64(l32), wl, TOL, "lse vs oracle")
