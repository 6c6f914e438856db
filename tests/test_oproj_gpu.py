"""GPU parity of mla_out_proj (and of the attention + o_proj chain) against
the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_mla_amd as mla
from transformer_attention_mla_amd import inputs

from _gpu_helpers import (SCALE, TOL, bits, check_bf16_close, check_bf16_is_rne_of_f32,
                          check_close, say, to_host64)

pytestmark = pytest.mark.gpu


def xw(M, K, N, seed):
    x = inputs.normal_bf16((M, K), seed)
    w = inputs.normal_bf16((N, K), seed + 1, std=0.02)
    return x, w


# Small M at several K splits, N ragged against the tiles and against 4, M not
# a multiple of 16.  The last three shapes take the wide-tile kernel (>= 256
# tiles of 256 x 256): ragged last m-group and n-tile, a tile count that is
# not a multiple of the 8 XCDs, N not a multiple of 4 (element stores), and an
# exact 256-multiple.
@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (17, 256, 100), (130, 1024, 300), (64, 8192, 7168),
                                   (1, 512, 7168), (33, 1024, 500), (64, 2048, 225), (16, 4096, 447),
                                   (64, 16384, 300),
                                   (200, 512, 7168), (5, 8192, 33), (300, 128, 129),
                                   (4764, 128, 3803), (4100, 256, 4000), (8192, 512, 2048)])
def test_oproj_parity(M, K, N, gpu_device):
    say(f"o_proj parity M={M} K={K} N={N}")
    x, w = xw(M, K, N, 10 + M)
    want = oracle.out_proj(bits(x), bits(w))
    xg, wg = x.to(gpu_device), w.to(gpu_device)
    y32 = mla.mla_out_proj(xg, wg, out_f32=True)
    y16 = mla.mla_out_proj(xg, wg)
    torch.cuda.synchronize()
    check_close(to_host64(y32), want, TOL, "float32 output vs oracle")
    check_bf16_is_rne_of_f32(y16, y32)
    check_bf16_close(y16, want, "bf16 output vs oracle")


@pytest.mark.parametrize("M", [1024, 16384])
def test_oproj_large_sampled(M, gpu_device):
    K, N = 8192, 7168
    say(f"o_proj sampled M={M}")
    x = inputs.normal_bf16((M, K), 77, device=gpu_device)
    w = inputs.out_proj_weight(N, K, workload=3, device=gpu_device)
    y32 = mla.mla_out_proj(x, w, out_f32=True)
    y16 = mla.mla_out_proj(x, w)
    torch.cuda.synchronize()
    check_bf16_is_rne_of_f32(y16, y32)
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 30)])).astype(np.int32)
    want = oracle.out_proj_rows(bits(x), bits(w), rows)
    got = to_host64(y32[torch.from_numpy(rows).long().to(gpu_device)])
    check_close(got, want, TOL, f"{len(rows)} sampled rows")


@pytest.mark.parametrize("M", [70, 37])
def test_oproj_selection_weight_exact(M, gpu_device):
    K, N = 1024, 600
    x = inputs.normal_bf16((M, K), 5)
    w = torch.zeros((N, K), dtype=torch.bfloat16)
    w[torch.arange(N), torch.arange(N)] = 1
    y = mla.mla_out_proj(x.to(gpu_device), w.to(gpu_device))
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), x[:, :N])


def test_oproj_wide_selection_weight_exact(gpu_device):
    """Wide-tile kernel: with W = I every output is one input element times 1,
    so y must equal x bit for bit (every tile of the grouped order written)."""
    M, K, N = 4352, 4096, 4096
    say(f"o_proj wide selection M={M} K={K} N={N}")
    x = inputs.normal_bf16((M, K), 6, device=gpu_device)
    w = torch.eye(N, K, dtype=torch.bfloat16, device=gpu_device)
    y = mla.mla_out_proj(x, w)
    torch.cuda.synchronize()
    assert torch.equal(y, x[:, :N])


def test_attention_then_oproj_workload1(gpu_device):
    """The whole step at the 64-position workload: bf16 attention output into
    o_proj, against the oracle's projection of its own bf16-rounded output."""
    w_ = inputs.WORKLOADS[1]
    B, H, T = w_["B"], w_["H"], w_["T"]
    say("attention + o_proj, workload 1")
    d = inputs.prefill_inputs(B, H, T, workload=1)
    wo = inputs.out_proj_weight(workload=1)
    o, _ = oracle.prefill(bits(d["q_nope"]), bits(d["q_pe"]), bits(d["k_nope"]), bits(d["k_pe"]),
                          bits(d["v"]), d["R"].numpy(), SCALE, want_lse=False)
    o16 = oracle.bf16_round(o).reshape(B * T, H * 128)
    o16_bits = bits(torch.from_numpy(o16).to(torch.bfloat16))
    want = oracle.out_proj(o16_bits, bits(wo))
    g = {k: v.to(gpu_device) for k, v in d.items()}
    attn, _ = mla.mla_attend_prefill(g["q_nope"], g["q_pe"], g["k_nope"], g["k_pe"], g["v"], g["R"],
                                     SCALE)
    y32 = mla.mla_out_proj(attn.view(B * T, H * 128), wo.to(gpu_device), out_f32=True)
    torch.cuda.synchronize()
    check_close(to_host64(y32), want, TOL, "delta_attn (float32 store) vs oracle")
    # o_proj alone on the GPU's own bf16 attention output
    want_chain = oracle.out_proj(bits(attn.view(B * T, H * 128)), bits(wo))
    check_close(to_host64(y32), want_chain, 1e-3, "o_proj on the GPU's attention output")


def test_attention_then_oproj_workload2(gpu_device):
    """The whole step at the 1024-position workload, every output: the GPU's
    bf16 attention output into o_proj (float32 store) against the oracle's
    projection of its own bf16-rounded attention output (max-abs 1e-2)."""
    w_ = inputs.WORKLOADS[2]
    B, H, T = w_["B"], w_["H"], w_["T"]
    say("attention + o_proj, workload 2")
    d = inputs.prefill_inputs(B, H, T, workload=2)
    wo = inputs.out_proj_weight(workload=2)
    o, _ = oracle.prefill(bits(d["q_nope"]), bits(d["q_pe"]), bits(d["k_nope"]), bits(d["k_pe"]),
                          bits(d["v"]), d["R"].numpy(), SCALE, want_lse=False)
    o16_bits = bits(torch.from_numpy(oracle.bf16_round(o).reshape(B * T, H * 128)).to(torch.bfloat16))
    want = oracle.out_proj(o16_bits, bits(wo))
    g = {k: v.to(gpu_device) for k, v in d.items()}
    attn, _ = mla.mla_attend_prefill(g["q_nope"], g["q_pe"], g["k_nope"], g["k_pe"], g["v"], g["R"],
                                     SCALE)
    y32 = mla.mla_out_proj(attn.view(B * T, H * 128), wo.to(gpu_device), out_f32=True)
    torch.cuda.synchronize()
    check_close(to_host64(y32), want, TOL, "delta_attn (float32 store) vs oracle")


def test_attention_then_oproj_workload3_sampled(gpu_device):
    """The whole step at B=4, T=4096 in the benchmark's launch: for sampled
    (sequence, position) rows the oracle computes the attention of all 64
    heads, rounds it to bf16 and projects it; the GPU's projected rows
    (float32 store) must agree within 1e-2."""
    w_ = inputs.WORKLOADS[3]
    B, H, T = w_["B"], w_["H"], w_["T"]
    say("attention + o_proj, workload 3 sampled rows")
    d = inputs.prefill_inputs(B, H, T, workload=3, device=gpu_device)
    wo = inputs.out_proj_weight(workload=3, device=gpu_device)
    attn, _ = mla.mla_attend_prefill(d["q_nope"], d["q_pe"], d["k_nope"], d["k_pe"], d["v"], d["R"],
                                     SCALE)
    y32 = mla.mla_out_proj(attn.view(B * T, H * 128), wo, out_f32=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(33)
    picks = [(0, 0), (0, T - 1), (B - 1, T - 1), (1, 255), (2, 256), (3, 2047)]
    picks += [(int(rng.integers(0, B)), int(rng.integers(0, T))) for _ in range(10)]
    R = d["R"].cpu().numpy()
    wo_bits = bits(wo)
    worst = 0.0
    for b in sorted({p[0] for p in picks}):
        ts = np.array(sorted({t for bb, t in picks if bb == b}), np.int32)
        sel = np.array([[0, h, t] for t in ts for h in range(H)], np.int32)
        one = lambda x: bits(x[b:b + 1])
        o, _ = oracle.prefill_rows(one(d["q_nope"]), one(d["q_pe"]), one(d["k_nope"]),
                                   one(d["k_pe"]), one(d["v"]), R, SCALE, sel)
        x16 = oracle.bf16_round(o.reshape(len(ts), H * 128))
        x_bits = bits(torch.from_numpy(x16).to(torch.bfloat16))
        want = oracle.out_proj(x_bits, wo_bits)
        got = to_host64(y32[torch.from_numpy(b * T + ts).long().to(gpu_device)])
        worst = max(worst, check_close(got, want, TOL, f"b={b} {len(ts)} rows"))
    say(f"  worst {worst:.3e}")


# ------------------------------------------------------------- FP8 weights

@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (17, 256, 100), (64, 8192, 7168), (130, 1024, 300),
                                   (300, 384, 129), (1000, 512, 1000), (1, 512, 129), (40, 2048, 1000),
                                   (64, 1024, 7168), (33, 1024, 500), (64, 2048, 225), (16, 4096, 447),
                                   (64, 16384, 300), (40, 384, 200), (3, 640, 129)])
def test_oproj_fp8_parity(M, K, N, gpu_device):
    """The FP8 checkpoint weight, dequantized to bf16 in the kernel's load path:
    against the oracle's projection with the same dequantization.  M <= 64
    takes the 64-row tile with 128-deep slabs (one or several K splits, N
    ragged against the 128-feature tile and against 4, M not a multiple of
    16); larger M the 128-row tile with 64-deep slabs."""
    say(f"o_proj fp8 parity M={M} K={K} N={N}")
    x = inputs.normal_bf16((M, K), 30 + M)
    w8, sc = inputs.out_proj_weight_fp8(N, K, workload=1)
    want = oracle.out_proj_fp8(bits(x), w8.numpy(), sc.numpy())
    xg, wg, sg = x.to(gpu_device), w8.to(gpu_device), sc.to(gpu_device)
    y32 = mla.mla_out_proj_fp8(xg, wg, sg, out_f32=True)
    y16 = mla.mla_out_proj_fp8(xg, wg, sg)
    torch.cuda.synchronize()
    check_close(to_host64(y32), want, TOL, "float32 output vs oracle")
    check_bf16_is_rne_of_f32(y16, y32)
    check_bf16_close(y16, want, "bf16 output vs oracle")


@pytest.mark.parametrize("M", [70, 64])
def test_oproj_fp8_dequant_exact(M, gpu_device):
    """Scaled identity: w8 = 1.0 (0x38) on the diagonal, scale 2^-3 in every
    block, so y = x / 8 bit for bit -- the dequantized weight is exactly 0.125
    and zero elsewhere, each output one product; and a second block scale
    pattern (a power of two per block) moves each output by its block's scale.
    M = 64 takes the 64-row tile with 128-deep slabs, M = 70 the 128-row tile."""
    K, N = 1024, 600
    x = inputs.normal_bf16((M, K), 7)
    w8 = torch.zeros((N, K), dtype=torch.uint8)
    w8[torch.arange(N), torch.arange(N)] = 0x38
    NB, KB = (N + 127) // 128, K // 128
    sc = torch.full((NB, KB), 0.125, dtype=torch.float32)
    y = mla.mla_out_proj_fp8(x.to(gpu_device), w8.to(gpu_device), sc.to(gpu_device))
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), (x[:, :N].float() * 0.125).to(torch.bfloat16))
    sc2 = 2.0 ** -torch.arange(NB * KB, dtype=torch.float32).reshape(NB, KB)
    y2 = mla.mla_out_proj_fp8(x.to(gpu_device), w8.to(gpu_device), sc2.to(gpu_device), out_f32=True)
    torch.cuda.synchronize()
    n = torch.arange(N)
    want = x[:, :N].float() * sc2[n // 128, n // 128]
    assert torch.equal(y2.cpu(), want)


@pytest.mark.parametrize("M,K,N", [(4352, 1024, 4096), (4100, 512, 4000)])
def test_oproj_fp8_wide_equals_bf16_on_dequantized_weight(M, K, N, gpu_device):
    """Enough 256 x 256 tiles: the FP8 weight is dequantized once (value x
    block scale in float32, rounded to bf16) and the wide bf16 kernel runs, so
    the output must equal the bf16 projection with the oracle's dequantized
    weight bit for bit (ragged N against the tile and against 128 included)."""
    say(f"o_proj fp8 wide vs bf16 on the dequantized weight M={M} K={K} N={N}")
    x = inputs.normal_bf16((M, K), 31, device=gpu_device)
    w8, sc = inputs.out_proj_weight_fp8(N, K, workload=1)
    wd = torch.from_numpy(oracle.dequant_fp8(w8.numpy(), sc.numpy()).view(np.int16)).view(torch.bfloat16)
    y8 = mla.mla_out_proj_fp8(x, w8.to(gpu_device), sc.to(gpu_device), out_f32=True)
    yb = mla.mla_out_proj(x, wd.to(gpu_device), out_f32=True)
    torch.cuda.synchronize()
    assert torch.equal(y8, yb)


def test_oproj_fp8_large_sampled(gpu_device):
    """M = 16384, K = 8192, N = 7168 (the prefill projection) on sampled rows."""
    M, K, N = 16384, 8192, 7168
    say(f"o_proj fp8 sampled M={M}")
    x = inputs.normal_bf16((M, K), 78, device=gpu_device)
    w8, sc = inputs.out_proj_weight_fp8(N, K, workload=3, device=gpu_device)
    y32 = mla.mla_out_proj_fp8(x, w8, sc, out_f32=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 20)])).astype(np.int32)
    want = oracle.out_proj_fp8_rows(bits(x), w8.cpu().numpy(), sc.cpu().numpy(), rows)
    got = to_host64(y32[torch.from_numpy(rows).long().to(gpu_device)])
    check_close(got, want, TOL, f"{len(rows)} sampled rows")


# ------------------------------------------- FP8 activations (dynamic scheme)

@pytest.mark.parametrize("M,K", [(1, 128), (17, 384), (64, 8192), (300, 1024), (5, 256)])
def test_act_quant_bit_exact(M, K, gpu_device):
    """Codes and scales of the GPU quantizer equal the oracle's bit for bit
    (a zero block, a block below the 1e-4 clamp and a large-magnitude row
    included)."""
    say(f"act_quant M={M} K={K}")
    x = inputs.normal_bf16((M, K), 40 + M)
    x[0, :128] = 0
    if M > 1:
        x[1, -128:] = (x[1, -128:].float() * 1e-6).to(torch.bfloat16)
    if M > 2:
        x[2] = (x[2].float() * 300).to(torch.bfloat16)
    want_q, want_s = oracle.act_quant(bits(x))
    q, sT = mla.mla_act_quant(x.to(gpu_device))
    torch.cuda.synchronize()
    got_s = sT.cpu().numpy()[:, :M].T
    assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), "scales differ"
    assert np.array_equal(q.cpu().numpy(), want_q), "codes differ"


def test_act_quant_rounding_midpoints(gpu_device):
    """Blocks whose quotient x / scale lands exactly on e4m3 rounding midpoints
    (ties go to the even code) or one float32 step beside them, with scales
    whose reciprocal is inexact (block maxima 3*448, 5*448, 7*448 * 2^k): the
    codes must still equal those of the correctly rounded division."""
    import itertools
    say("act_quant midpoints")
    mids = []
    for e in range(-9, 9):  # normal and subnormal e4m3 midpoints below 448
        for m in range(16):
            val = (16 + m + 0.5) * 2.0 ** (e - 4) if e >= -6 else (m + 0.5) * 2.0 ** -9
            if val < 448:
                mids.append(val)
    rows = []
    for f, k in itertools.product((3.0, 5.0, 7.0), (-3, 0, 2)):
        sc = f * 2.0 ** k
        amax = 448.0 * sc
        for chunk in range(0, len(mids), 127):
            vals = [amax] + [sgn * mq * sc for mq, sgn in zip(mids[chunk:chunk + 127],
                                                               itertools.cycle((1.0, -1.0)))]
            vals += [0.0] * (128 - len(vals))
            rows.append(vals)
    x = torch.tensor(rows, dtype=torch.float32).to(torch.bfloat16)
    # keep only blocks whose maximum survived bf16 rounding exactly
    x = x[x.float().abs().amax(1) == torch.tensor([r[0] for r in rows])]
    want_q, want_s = oracle.act_quant(bits(x))
    q, sT = mla.mla_act_quant(x.to(gpu_device))
    torch.cuda.synchronize()
    assert np.array_equal(sT.cpu().numpy()[:, :x.shape[0]].T.view(np.uint32), want_s.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), want_q), "codes differ next to rounding midpoints"


@pytest.mark.parametrize("M,K,N", [(1, 128, 1), (17, 256, 100), (64, 8192, 7168), (130, 1024, 300),
                                   (300, 384, 129), (1000, 512, 1000), (1, 512, 129), (40, 2048, 1000),
                                   (64, 1024, 7168), (33, 1024, 500), (64, 2048, 225), (16, 4096, 447),
                                   (64, 16384, 300), (40, 384, 200), (3, 640, 129), (513, 768, 600)])
def test_oproj_fp8_dyn_parity(M, K, N, gpu_device):
    """FP8 activations and weights on the FP8 matrix cores against the
    oracle's product of the dequantized operands: M <= 64 takes the 128 x 64
    tile with K split over workgroups, larger M the 256 x 256 tile (ragged
    against both, N not a multiple of 4)."""
    say(f"o_proj fp8 dynamic parity M={M} K={K} N={N}")
    x = inputs.normal_bf16((M, K), 50 + M)
    w8, sc = inputs.out_proj_weight_fp8(N, K, workload=1)
    want = oracle.out_proj_fp8_dyn(bits(x), w8.numpy(), sc.numpy())
    xg, wg, sg = x.to(gpu_device), w8.to(gpu_device), sc.to(gpu_device)
    y32 = mla.mla_out_proj_fp8_dyn(xg, wg, sg, out_f32=True)
    y16 = mla.mla_out_proj_fp8_dyn(xg, wg, sg)
    torch.cuda.synchronize()
    check_close(to_host64(y32), want, TOL, "float32 output vs oracle")
    check_bf16_is_rne_of_f32(y16, y32)
    check_bf16_close(y16, want, "bf16 output vs oracle")


@pytest.mark.parametrize("M", [64, 300])
def test_oproj_fp8_dyn_scaled_identity_exact(M, gpu_device):
    """W = 1.0 on the diagonal with block scale 1/8: every output is one
    dequantized activation (code x scale, one float32 rounding) over 8,
    bit for bit."""
    K, N = 1024, 600
    x = inputs.normal_bf16((M, K), 8)
    w8 = torch.zeros((N, K), dtype=torch.uint8)
    w8[torch.arange(N), torch.arange(N)] = 0x38
    sc = torch.full(((N + 127) // 128, K // 128), 0.125, dtype=torch.float32)
    y = mla.mla_out_proj_fp8_dyn(x.to(gpu_device), w8.to(gpu_device), sc.to(gpu_device), out_f32=True)
    torch.cuda.synchronize()
    q, sx = oracle.act_quant(bits(x))
    qv = torch.from_numpy(q).view(torch.float8_e4m3fn).float().numpy()[:, :N]
    s_full = np.repeat(sx, 128, axis=1)[:, :N].astype(np.float32)
    want = (qv * s_full).astype(np.float32) * np.float32(0.125)
    assert np.array_equal(y.cpu().numpy(), want)


def test_oproj_fp8_dyn_large_sampled(gpu_device):
    """M = 16384, K = 8192, N = 7168 (the prefill projection) on sampled rows:
    quantization is per row, so the oracle's rows from the sampled x rows are
    exact."""
    M, K, N = 16384, 8192, 7168
    say(f"o_proj fp8 dynamic sampled M={M}")
    x = inputs.normal_bf16((M, K), 79, device=gpu_device)
    w8, sc = inputs.out_proj_weight_fp8(N, K, workload=3, device=gpu_device)
    y32 = mla.mla_out_proj_fp8_dyn(x, w8, sc, out_f32=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], rng.integers(0, M, 12)]))
    idx = torch.from_numpy(rows).long().to(gpu_device)
    want = oracle.out_proj_fp8_dyn(bits(x[idx]), w8.cpu().numpy(), sc.cpu().numpy())
    check_close(to_host64(y32[idx]), want, TOL, f"{len(rows)} sampled rows")
