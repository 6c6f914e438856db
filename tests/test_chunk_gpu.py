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


def _chunk_sampled_check(c, past, heads, rows_per_head, dev, label):
    """Append the chunk, run the chunked prefill (float32 and bf16 stores) and
    compare sampled (head, row) outputs with the oracle, row by row."""
    B, H, T = c["q_nope"].shape[:3]
    caches = [c["k_nope_cache"], c["kpe_cache"], c["v_cache"]]
    mla.mla_append_kv(c["k_nope"], c["k_pe"], c["v"], c["R"], past, *caches)
    o32, lse = mla.mla_attend_prefill_chunk(c["q_nope"], c["q_pe"], *caches, c["R"], past, SCALE,
                                            out_f32=True, want_lse=True)
    o16, _ = mla.mla_attend_prefill_chunk(c["q_nope"], c["q_pe"], *caches, c["R"], past, SCALE)
    torch.cuda.synchronize()
    check_bf16_is_rne_of_f32(o16, o32)
    R = c["R"].cpu().numpy()
    for (b, h), rows in zip(heads, rows_per_head):
        one = lambda t: bits(t[b:b + 1, h:h + 1])
        sel = np.stack([np.zeros_like(rows), np.zeros_like(rows), rows], 1)
        want, wl = oracle.prefill_chunk_rows(one(c["q_nope"]), one(c["q_pe"]), one(caches[0]),
                                             bits(caches[1][b:b + 1]), one(caches[2]), R, past,
                                             SCALE, sel)
        idx = torch.from_numpy(rows).long().to(dev)
        check_close(to_host64(o32[b, idx, h * 128:(h + 1) * 128]), want, TOL,
                    f"{label} b={b} h={h} {len(rows)} rows")
        check_close(to_host64(lse[b, h, idx]), wl, TOL, f"{label} b={b} h={h} lse")
        check_bf16_close(o16[b, idx, h * 128:(h + 1) * 128], want, f"{label} b={b} h={h} bf16")


def test_chunk_paired_schedule_every_row(gpu_device):
    """B=4, H=64, T=1024 after 500 cached positions: enough work that every
    workgroup takes a pair of query tiles (the schedule of the long chunks);
    every row of four heads against the oracle."""
    B, H, T, past = 4, 64, 1024, 500
    say(f"prefill chunk paired schedule B={B} H={H} T={T} past={past}")
    c = inputs.chunk_inputs(B, H, T, past, seed=3600, device=gpu_device)
    rows = np.arange(T, dtype=np.int32)
    heads = [(0, 0), (1, 21), (2, 42), (3, 63)]
    _chunk_sampled_check(c, past, heads, [rows] * len(heads), gpu_device, "paired")


def test_chunk_benchmark_launch_sampled(gpu_device):
    """The chunk the benchmark times (B=1, H=64, a 4096-position chunk after
    12288 cached positions, same inputs and launch): first 128, last 128 and
    256 random rows of three heads against the oracle."""
    B, H, T, past = 1, 64, 4096, 12288
    say(f"prefill chunk benchmark launch B={B} H={H} T={T} past={past}")
    c = inputs.chunk_inputs(B, H, T, past, seed=7000, device=gpu_device)
    rng = np.random.default_rng(12288)
    heads = [(0, 0), (0, 31), (0, 63)]
    rows = []
    for _ in heads:
        r = set(range(128)) | set(range(T - 128, T)) | set(rng.integers(0, T, 256).tolist())
        rows.append(np.array(sorted(r), np.int32))
    _chunk_sampled_check(c, past, heads, rows, gpu_device, "benchmark chunk")


@pytest.mark.parametrize("B,H,T,past,L", [(2, 3, 45, 19, 100), (4, 64, 1000, 77, 1200)])
def test_chunk_unwritten_rows_never_reach_the_output(B, H, T, past, L, gpu_device):
    """Cache rows at and past past + T (never written by the append) holding
    bf16 NaN, +inf or -inf give outputs bit-identical to zero-filled rows
    (past + T is not a multiple of the 32-key tile, so the last key tile
    straddles it; the second case takes the paired schedule)."""
    say(f"prefill chunk unwritten rows B={B} H={H} T={T} past={past} L={L}")
    d = chunk_inputs(B, H, T, 3700 + T)
    R = torch.from_numpy(inputs.rope_angles(L)).to(gpu_device)
    hist = [t.to(gpu_device) for t in junk_caches(B, H, L, 3710)]
    outs = []
    for fill in (0x0000, 0x7FC0, 0x7F80, 0xFF80):  # zero, NaN, +inf, -inf
        caches = [t.clone() for t in hist]
        caches[0][:, :, past + T:].view(torch.int16).fill_(fill - (1 << 16 if fill >= 1 << 15 else 0))
        caches[1][:, past + T:].view(torch.int16).fill_(fill - (1 << 16 if fill >= 1 << 15 else 0))
        caches[2][:, :, past + T:].view(torch.int16).fill_(fill - (1 << 16 if fill >= 1 << 15 else 0))
        mla.mla_append_kv(d["k_nope"].to(gpu_device), d["k_pe"].to(gpu_device), d["v"].to(gpu_device),
                          R, past, *caches)
        o, l = run_chunk(d, caches, R, past, gpu_device, out_f32=True, want_lse=True)
        assert torch.isfinite(o).all() and torch.isfinite(l).all(), f"fill {fill:#06x}"
        outs.append((o, l))
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    want, _ = oracle.prefill_chunk(bits(d["q_nope"]), bits(d["q_pe"]),
                                   *[bits(t) for t in caches], R.cpu().numpy(), past, SCALE)
    check_close(to_host64(outs[0][0]), want, TOL, "float32 output vs oracle")
