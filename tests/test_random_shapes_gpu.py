"""Seeded random shapes through every entry point against the oracle, on top
of the chosen shapes of the other parity tests (all three decode cache
layouts included): ragged sizes nobody picked, split counts, K depths, past
offsets.  Gates as elsewhere: float32 outputs
and lse within 1e-2 of the fp64 oracle (the up-projection within 1e-4), the
key-blocked value layout bit-identical to the natural one with NaN in its
padding slots."""
import random

import pytest
import torch

import oracle
import transformer_attention_mla_amd as mla
from transformer_attention_mla_amd import inputs

from _gpu_helpers import SCALE, TOL, bits, check_close, say, to_host64

pytestmark = pytest.mark.gpu

_rng = random.Random(20261203)
PREFILL = [(_rng.choice([1, 2, 3]), h, _rng.randint(1, 300 if h == 64 else 700))
           for h in [_rng.choice([1, 2, 3, 5, 8, 64]) for _ in range(10)]]
DECODE = [(_rng.choice([1, 2, 4]), _rng.choice([1, 3, 8, 64]), _rng.randint(1, 3000),
           _rng.choice([0, 1, 2, 5, 17])) for _ in range(10)]
OPROJ = [(_rng.choice([1, 3, 17, 33, 64, 65, 130, 300, _rng.randint(1, 1200)]), 128 * _rng.randint(1, 24),
          _rng.randint(1, 900)) for _ in range(10)]
CHUNK = [(_rng.choice([1, 2]), _rng.choice([1, 3, 8]), _rng.randint(1, 300), _rng.randint(0, 500))
         for _ in range(6)]
UP = [(_rng.choice([1, 2, 3]), _rng.randint(1, 400), _rng.choice([1, 2, 4, 8])) for _ in range(6)]
SHARED = [(_rng.choice([1, 2, 5]), _rng.choice([1, 4, 16, 64]), _rng.randint(1, 2000),
           _rng.choice([0, 1, 3, 9])) for _ in range(6)]
LATENT = [(_rng.choice([1, 3, 17]), _rng.choice([1, 5, 16, 33, 64]), _rng.randint(1, 1500),
           _rng.choice([0, 1, 2, 7])) for _ in range(6)]


@pytest.mark.parametrize("B,H,T", PREFILL)
def test_random_prefill(B, H, T, gpu_device):
    say(f"random prefill B={B} H={H} T={T}")
    d = inputs.prefill_inputs(B, H, T, workload=0)
    want, want_lse = oracle.prefill(bits(d["q_nope"]), bits(d["q_pe"]), bits(d["k_nope"]), bits(d["k_pe"]),
                                    bits(d["v"]), d["R"].numpy(), SCALE)
    g = {k: v.to(gpu_device) for k, v in d.items()}
    args = (g["q_nope"], g["q_pe"], g["k_nope"], g["k_pe"])
    out, lse = mla.mla_attend_prefill(*args, g["v"], g["R"], SCALE, out_f32=True, want_lse=True)
    vb = inputs.to_v_blocked(g["v"], fill=float("nan"))
    outb, lseb = mla.mla_attend_prefill(*args, vb, g["R"], SCALE, out_f32=True, want_lse=True, v_blocked=True)
    torch.cuda.synchronize()
    check_close(to_host64(out), want, TOL, "output vs oracle")
    check_close(to_host64(lse), want_lse, TOL, "lse vs oracle")
    assert torch.equal(outb.view(torch.int32), out.view(torch.int32))
    assert torch.equal(lseb.view(torch.int32), lse.view(torch.int32))


@pytest.mark.parametrize("B,H,L,splits", DECODE)
def test_random_decode(B, H, L, splits, gpu_device):
    say(f"random decode B={B} H={H} L={L} splits={splits}")
    d = inputs.decode_inputs(B, H, L, q_pos=L + 3)
    want, want_lse = oracle.decode(bits(d["q_nope"]), bits(d["q_pe"]), bits(d["k_cache"]), bits(d["v_cache"]),
                                   d["R"].numpy(), d["q_pos"], SCALE)
    g = {k: (v.to(gpu_device) if torch.is_tensor(v) else v) for k, v in d.items()}
    out, lse = mla.mla_attend_decode(g["q_nope"], g["q_pe"], g["k_cache"], g["v_cache"], g["R"], g["q_pos"],
                                     SCALE, num_splits=splits, out_f32=True, want_lse=True)
    torch.cuda.synchronize()
    check_close(to_host64(out), want, TOL, "output vs oracle")
    check_close(to_host64(lse), want_lse, TOL, "lse vs oracle")


@pytest.mark.parametrize("M,K,N", OPROJ)
def test_random_oproj(M, K, N, gpu_device):
    say(f"random o_proj M={M} K={K} N={N}")
    x = inputs.normal_bf16((M, K), 1000 + M + K + N)
    w = inputs.normal_bf16((N, K), 2000 + M + K + N, std=0.02)
    w8, sc = inputs.out_proj_weight_fp8(N, K, workload=0)
    xd = x.to(gpu_device)
    y = mla.mla_out_proj(xd, w.to(gpu_device), out_f32=True)
    yd = mla.mla_out_proj_fp8_dyn(xd, w8.to(gpu_device), sc.to(gpu_device), out_f32=True)
    yw = mla.mla_out_proj_fp8(xd, w8.to(gpu_device), sc.to(gpu_device), out_f32=True)
    torch.cuda.synchronize()
    check_close(to_host64(y), oracle.out_proj(bits(x), bits(w)), TOL, "bf16 weight vs oracle")
    check_close(to_host64(yd), oracle.out_proj_fp8_dyn(bits(x), w8.numpy(), sc.numpy()), TOL,
                "FP8 activations vs oracle")
    check_close(to_host64(yw), oracle.out_proj_fp8(bits(x), w8.numpy(), sc.numpy()), TOL,
                "FP8 weight-only vs oracle")


@pytest.mark.parametrize("B,H,T,past", CHUNK)
def test_random_chunk(B, H, T, past, gpu_device):
    say(f"random chunk B={B} H={H} T={T} past={past}")
    c = inputs.chunk_inputs(B, H, T, past, seed=7000 + T + past)
    g = {k: v.to(gpu_device) for k, v in c.items()}
    mla.mla_append_kv(g["k_nope"], g["k_pe"], g["v"], g["R"], past, g["k_nope_cache"], g["kpe_cache"],
                      g["v_cache"])
    out, lse = mla.mla_attend_prefill_chunk(g["q_nope"], g["q_pe"], g["k_nope_cache"], g["kpe_cache"],
                                            g["v_cache"], g["R"], past, SCALE, out_f32=True, want_lse=True)
    torch.cuda.synchronize()
    kc, pc, vc = (g[k].cpu() for k in ("k_nope_cache", "kpe_cache", "v_cache"))
    want, want_lse = oracle.prefill_chunk(bits(c["q_nope"]), bits(c["q_pe"]), bits(kc), bits(pc), bits(vc),
                                          c["R"].numpy(), past, SCALE)
    check_close(to_host64(out), want, TOL, "output vs oracle")
    check_close(to_host64(lse), want_lse, TOL, "lse vs oracle")


@pytest.mark.parametrize("B,T,H", UP)
def test_random_up_project(B, T, H, gpu_device):
    say(f"random up-projection B={B} T={T} H={H}")
    d = inputs.up_project_inputs(B, T, H, workload=0)
    want = oracle.up_project(bits(d["q_lat"]), bits(d["ckv"]), bits(d["w_q_b"]), bits(d["w_kv_b"]))
    g = {k: v.to(gpu_device) for k, v in d.items()}
    args = (g["q_lat"], g["ckv"], g["w_q_b"], g["w_kv_b"])
    got = mla.mla_up_project(*args, out_f32=True)
    gotb = mla.mla_up_project(*args, out_f32=True, v_blocked=True)
    torch.cuda.synchronize()
    for a, w, name in zip(got, want, ("q_nope", "q_pe", "k_nope", "v")):
        check_close(to_host64(a), w, 1e-4, f"{name} vs oracle")
    assert torch.equal(inputs.from_v_blocked(gotb[3], T), got[3])


@pytest.mark.parametrize("B,H,L,splits", SHARED)
def test_random_decode_shared_kpe(B, H, L, splits, gpu_device):
    say(f"random decode, shared rotary key, B={B} H={H} L={L} splits={splits}")
    d = inputs.decode_shared_kpe_inputs(B, H, L, q_pos=L + 1)
    want, want_lse = oracle.decode_shared_kpe(bits(d["q_nope"]), bits(d["q_pe"]), bits(d["k_nope_cache"]),
                                              bits(d["kpe_cache"]), bits(d["v_cache"]), d["R"].numpy(),
                                              d["q_pos"], SCALE)
    g = {k: (v.to(gpu_device) if torch.is_tensor(v) else v) for k, v in d.items()}
    out, lse = mla.mla_attend_decode_shared_kpe(g["q_nope"], g["q_pe"], g["k_nope_cache"], g["kpe_cache"],
                                                g["v_cache"], g["R"], g["q_pos"], SCALE, num_splits=splits,
                                                out_f32=True, want_lse=True)
    torch.cuda.synchronize()
    check_close(to_host64(out), want, TOL, "output vs oracle")
    check_close(to_host64(lse), want_lse, TOL, "lse vs oracle")


@pytest.mark.parametrize("B,H,L,splits", LATENT)
def test_random_decode_latent(B, H, L, splits, gpu_device):
    say(f"random decode, latent cache, B={B} H={H} L={L} splits={splits}")
    d = inputs.decode_latent_inputs(B, H, L, q_pos=L + 2)
    want, want_lse = oracle.decode_latent(bits(d["q_nope"]), bits(d["q_pe"]), bits(d["ckv"]), bits(d["kpe"]),
                                          bits(d["w_kv_b"]), d["R"].numpy(), d["q_pos"], SCALE)
    g = {k: (v.to(gpu_device) if torch.is_tensor(v) else v) for k, v in d.items()}
    out, lse = mla.mla_attend_decode_latent(g["q_nope"], g["q_pe"], g["ckv"], g["kpe"], g["w_kv_b"], g["R"],
                                            g["q_pos"], SCALE, num_splits=splits, out_f32=True, want_lse=True)
    torch.cuda.synchronize()
    check_close(to_host64(out), want, TOL, "output vs oracle")
    check_close(to_host64(lse), want_lse, TOL, "lse vs oracle")
