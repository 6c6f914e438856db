"""GPU parity of the KV-cache append and the chunked prefill (queries at
positions past .. past+T-1 over cache rows 0 .. past+t) against the fp64
oracle, and their agreement with the plain prefill."""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_mla_amd as mla
from transformer_attention_mla_amd import inputs

from _gpu_helpers import (SCALE, TOL, bits, check_bf16_close, check_bf16_is_rne_of_f32,
                          check_close, say, to_host64)

pytestmark = pytest.mark.gpu


def chunk_inputs(B, H, T, seed):
    g = lambda shape, k: inputs.normal_bf16(shape, seed + k)
    return dict(q_nope=g((B, H, T, 128), 0), q_pe=g((B, H, T, 64), 1), k_nope=g((B, H, T, 128), 2),
                k_pe=g((B, 1, T, 64), 3), v=g((B, H, T, 128), 4))


def junk_caches(B, H, L, seed):
    return (inputs.normal_bf16((B, H, L, 128), seed), inputs.normal_bf16((B, L, 64), seed + 1),
            inputs.normal_bf16((B, H, L, 128), seed + 2))


def test_append_matches_oracle(gpu_device):
    B, H, T, past, L = 2, 3, 45, 17, 80
    say(f"append B={B} H={H} T={T} past={past} L={L}")
    d = chunk_inputs(B, H, T, 3000)
    R = torch.from_numpy(inputs.rope_angles(L))
    kc, pc, vc = junk_caches(B, H, L, 3010)
    want = [bits(t).copy() for t in (kc, pc, vc)]
    oracle.append_kv(bits(d["k_nope"]), bits(d["k_pe"]), bits(d["v"]), R.numpy(), past, *want)
    g = [t.to(gpu_device) for t in (kc, pc, vc)]
    mla.mla_append_kv(d["k_nope"].to(gpu_device), d["k_pe"].to(gpu_device), d["v"].to(gpu_device),
                      R.to(gpu_device), past, *g)
    torch.cuda.synchronize()
    got = [bits(t) for t in g]
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[2], want[2])  # copies, untouched rows
    # rotated rope keys: float32 on the GPU, float64 in the oracle, each rounded once to bf16
    gk, wk = oracle.bf16_widen(got[1]), oracle.bf16_widen(want[1])
    same = np.mean(gk == wk)
    spacing = np.maximum(np.abs(wk), 2.0 ** -126)
    ulps = np.abs(gk - wk) / (2.0 ** (np.floor(np.log2(spacing)) - 7))
    say(f"  rotated keys equal: {same:.4f}; max difference {ulps.max():.1f} bf16 ulp")
    assert same > 0.99 and ulps.max() <= 1.0
    assert np.array_equal(got[1][:, :past], want[1][:, :past])
    assert np.array_equal(got[1][:, past + T:], want[1][:, past + T:])


def run_chunk(d, caches, R, past, dev, **kw):
    out, lse = mla.mla_attend_prefill_chunk(d["q_nope"].to(dev), d["q_pe"].to(dev), *caches,
                                            R.to(dev), past, SCALE, **kw)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("B,H,T,past,L", [(1, 1, 1, 0, 8), (2, 3, 17, 5, 40), (1, 2, 100, 300, 500),
                                          (2, 64, 200, 1000, 1300), (1, 4, 300, 33, 400),
                                          (3, 2, 64, 64, 128)])
def test_chunk_parity(B, H, T, past, L, gpu_device):
    """The chunk's keys appended on the GPU into caches whose earlier rows hold
    a seeded history; the oracle attends over the same cache contents."""
    say(f"prefill chunk parity B={B} H={H} T={T} past={past} L={L}")
    d = chunk_inputs(B, H, T, 3100 + T)
    R = torch.from_numpy(inputs.rope_angles(L))
    caches = [t.to(gpu_device) for t in junk_caches(B, H, L, 3200 + past)]
    mla.mla_append_kv(d["k_nope"].to(gpu_device), d["k_pe"].to(gpu_device), d["v"].to(gpu_device),
                      R.to(gpu_device), past, *caches)
    o32, lse = run_chunk(d, caches, R, past, gpu_device, out_f32=True, want_lse=True)
    o16, _ = run_chunk(d, caches, R, past, gpu_device)
    want, wl = oracle.prefill_chunk(bits(d["q_nope"]), bits(d["q_pe"]), *[bits(c) for c in caches],
                                    R.numpy(), past, SCALE)
    check_close(to_host64(o32), want, TOL, "float32 output vs oracle")
    check_close(to_host64(lse), wl, TOL, "lse vs oracle")
    check_bf16_is_rne_of_f32(o16, o32)
    check_bf16_close(o16, want, "bf16 output vs oracle")


@pytest.mark.parametrize("B,H,T,L", [(2, 3, 300, 300), (1, 64, 1024, 1500)])
def test_chunk_at_zero_is_the_prefill(B, H, T, L, gpu_device):
    """Append at 0 and the chunked prefill over the cache give the plain
    prefill's outputs bit for bit (same rotation code, same tiles)."""
    say(f"chunk at zero vs prefill B={B} H={H} T={T} L={L}")
    d = chunk_inputs(B, H, T, 3300)
    R = torch.from_numpy(inputs.rope_angles(L)).to(gpu_device)
    g = {k: v.to(gpu_device) for k, v in d.items()}
    caches = [t.to(gpu_device) for t in junk_caches(B, H, L, 3310)]
    mla.mla_append_kv(g["k_nope"], g["k_pe"], g["v"], R, 0, *caches)
    a, la = mla.mla_attend_prefill_chunk(g["q_nope"], g["q_pe"], *caches, R, 0, SCALE, out_f32=True,
                                         want_lse=True)
    b, lb = mla.mla_attend_prefill(g["q_nope"], g["q_pe"], g["k_nope"], g["k_pe"], g["v"], R, SCALE,
                                   out_f32=True, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_chunks_agree_with_one_prefill(gpu_device):
    """A 700-position prefill as chunks of 300 and 400 (append, then attend):
    the rows agree with the one-shot prefill to float32 rounding (the grouping
    of rows into waves differs, so the lazy rescale may round differently)."""
    B, H, T1, T2 = 2, 8, 300, 400
    T = T1 + T2
    say(f"chunks {T1}+{T2} vs one prefill B={B} H={H}")
    d = chunk_inputs(B, H, T, 3400)
    R = torch.from_numpy(inputs.rope_angles(T)).to(gpu_device)
    g = {k: v.to(gpu_device) for k, v in d.items()}
    full, fl = mla.mla_attend_prefill(g["q_nope"], g["q_pe"], g["k_nope"], g["k_pe"], g["v"], R, SCALE,
                                      out_f32=True, want_lse=True)
    caches = [t.to(gpu_device) for t in junk_caches(B, H, T, 3410)]
    outs, lses = [], []
    for past, n in ((0, T1), (T1, T2)):
        s = slice(past, past + n)
        part = {k: v[:, :, s].contiguous() for k, v in g.items()}
        mla.mla_append_kv(part["k_nope"], part["k_pe"], part["v"], R, past, *caches)
        o, l = mla.mla_attend_prefill_chunk(part["q_nope"], part["q_pe"], *caches, R, past, SCALE,
                                            out_f32=True, want_lse=True)
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    got, gl = torch.cat(outs, 1), torch.cat(lses, 2)
    err = (got - full).abs().max().item()
    lerr = (gl - fl).abs().max().item()
    say(f"  max |chunked - one-shot| {err:.2e}, lse {lerr:.2e}")
    assert err <= 1e-5 and lerr <= 1e-5


def test_chunk_long_history(gpu_device):
    """A 256-position chunk after 2048 cached positions, 8 heads."""
    B, H, T, past, L = 1, 8, 256, 2048, 2304
    say(f"prefill chunk long history B={B} H={H} T={T} past={past}")
    d = chunk_inputs(B, H, T, 3500)
    R = torch.from_numpy(inputs.rope_angles(L))
    caches = [t.to(gpu_device) for t in junk_caches(B, H, L, 3510)]
    mla.mla_append_kv(d["k_nope"].to(gpu_device), d["k_pe"].to(gpu_device), d["v"].to(gpu_device),
                      R.to(gpu_device), past, *caches)
    o32, lse = run_chunk(d, caches, R, past, gpu_device, out_f32=True, want_lse=True)
    want, wl = oracle.prefill_chunk(bits(d["q_nope"]), bits(d["q_pe"]), *[bits(c) for c in caches],
                                    R.numpy(), past, SCALE)
    check_close(to_host64(o32), want, TOL, "float32 output vs oracle")
    check_close(to_host64(lse), wl, TOL, "lse vs oracle")
