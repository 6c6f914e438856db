"""Seeded synthetic inputs for the MLA attend-and-combine step.

This module generates data only: random activations and weights with the
shapes and distributions of the workloads, and the angle tables R that the
library takes as an input (page "Kimi K2 · Transformer blocks", I/O header:
R [T positions, 32 pairs]).  It holds none of the attention arithmetic; the
HIP library and the CPU oracle each consume what it produces.

Distributions: activations bf16 N(0, 1); the output-projection weight bf16
N(0, 0.02) (config.json ``initializer_range`` 0.02, page "Block input").
Values are drawn in float32 and rounded to bf16 (round to nearest even).
Seeds: ``1000 * workload + k`` with k = 0 q_nope, 1 q_pe, 2 k_nope, 3 k_pe,
4 v, 5 w_o, 6 k_cache, 7 v_cache.
"""
from __future__ import annotations

import math

import numpy as np

ROPE_THETA = 50000.0  # config.json rope_theta (page "Block input")
ROT_DIM = 64          # qk_rope_head_dim
PAIRS = ROT_DIM // 2

SEED_Q_NOPE, SEED_Q_PE, SEED_K_NOPE, SEED_K_PE, SEED_V, SEED_WO, SEED_KC, SEED_VC = range(8)
SEED_KNC, SEED_KPC = 8, 9  # shared-rotary cache layout: nope keys, rope keys
SEED_CKV, SEED_WKVB = 10, 11  # latent cache, up-projection weight
SEED_QLAT, SEED_WQB = 12, 13  # query latent, its up-projection weight

# The five workloads: (kind, B, T or L) with 64 heads.
WORKLOADS = {
    1: dict(kind="prefill", B=1, T=64, H=64, rope="plain"),
    2: dict(kind="prefill", B=1, T=1024, H=64, rope="plain"),
    3: dict(kind="prefill", B=4, T=4096, H=64, rope="plain"),
    4: dict(kind="prefill", B=1, T=16384, H=64, rope="yarn"),
    5: dict(kind="decode", B=64, L=8192, H=64, q_pos=8192, rope="plain"),
}
D_MODEL = 7168   # hidden_size
SOFTMAX_SCALE = 1.0 / math.sqrt(128 + 64)  # (qk_nope_head_dim + qk_rope_head_dim) ** -0.5


def inv_freq(theta: float = ROPE_THETA, rot_dim: int = ROT_DIM) -> np.ndarray:
    """theta ** (-2 i / rot_dim) for pair i, in float64."""
    i = np.arange(rot_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * i / rot_dim)


def rope_angles(n_pos: int, theta: float = ROPE_THETA, rot_dim: int = ROT_DIM) -> np.ndarray:
    """Plain rotary angle table R[t, i] = t * theta^(-2i/rot_dim), computed in
    float64 and stored as float32, shape [n_pos, rot_dim/2]."""
    t = np.arange(n_pos, dtype=np.float64)[:, None]
    return (t * inv_freq(theta, rot_dim)[None, :]).astype(np.float32)


def yarn_inv_freq(theta: float = ROPE_THETA, rot_dim: int = ROT_DIM, factor: float = 32.0,
                  original: int = 4096, beta_fast: float = 1.0,
                  beta_slow: float = 1.0) -> np.ndarray:
    """Per-pair frequencies of YaRN's "NTK-by-parts" interpolation (Peng et al.,
    2023), with config.json's rope_scaling (factor 32 over 4096 original
    positions, beta_fast = beta_slow = 1; page "Block input").

    For pair i with frequency f_i, r_i = original * f_i / (2 pi) is the number
    of turns it makes over the original context.  The ramp gamma(r) is 0 below
    beta_slow, 1 above beta_fast and linear in between; the new frequency is
    (1 - gamma) f_i / factor + gamma f_i.  With beta_fast = beta_slow the ramp
    is a step at r = beta: pairs turning at least once keep f_i, slower pairs
    are divided by the factor (for Kimi K2: pairs 0..19 keep, 20..31 scaled)."""
    f = inv_freq(theta, rot_dim)
    r = original * f / (2.0 * math.pi)
    if beta_fast == beta_slow:
        gamma = (r >= beta_fast).astype(np.float64)
    else:
        gamma = np.clip((r - beta_slow) / (beta_fast - beta_slow), 0.0, 1.0)
    return (1.0 - gamma) * f / factor + gamma * f


def yarn_angles(n_pos: int, **kw) -> np.ndarray:
    t = np.arange(n_pos, dtype=np.float64)[:, None]
    return (t * yarn_inv_freq(**kw)[None, :]).astype(np.float32)


def angles_for(workload: int, n_pos: int) -> np.ndarray:
    return yarn_angles(n_pos) if WORKLOADS[workload]["rope"] == "yarn" else rope_angles(n_pos)


def seed_of(workload: int, k: int) -> int:
    return 1000 * workload + k


def normal_bf16(shape, seed: int, std: float = 1.0, device="cpu"):
    """bf16 tensor of N(0, std^2) values drawn in float32 with a torch
    generator seeded by ``seed`` (on ``device``), in chunks of at most 2^27
    values so large tensors need little temporary memory."""
    import torch

    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    flat = out.view(-1)
    chunk = 1 << 27
    for s in range(0, flat.numel(), chunk):
        n = min(chunk, flat.numel() - s)
        x = torch.randn(n, generator=gen, dtype=torch.float32, device=dev)
        if std != 1.0:
            x.mul_(std)
        flat[s:s + n].copy_(x)
    return out


def prefill_inputs(B: int, H: int, T: int, workload: int = 0, device="cpu", r_rows=None):
    """q_nope, q_pe, k_nope, k_pe, v (bf16) and R (float32) for a causal prefill."""
    import torch

    g = lambda shape, k: normal_bf16(shape, seed_of(workload, k), device=device)
    q_nope = g((B, H, T, 128), SEED_Q_NOPE)
    q_pe = g((B, H, T, 64), SEED_Q_PE)
    k_nope = g((B, H, T, 128), SEED_K_NOPE)
    k_pe = g((B, 1, T, 64), SEED_K_PE)
    v = g((B, H, T, 128), SEED_V)
    rr = T if r_rows is None else r_rows
    R = torch.from_numpy(angles_for(workload, rr) if workload in WORKLOADS else rope_angles(rr))
    return dict(q_nope=q_nope, q_pe=q_pe, k_nope=k_nope, k_pe=k_pe, v=v, R=R.to(device))


def decode_inputs(B: int, H: int, L: int, q_pos: int, workload: int = 0, device="cpu"):
    """q_nope, q_pe (bf16), k_cache [B,H,L,192], v_cache [B,H,L,128] (bf16) and
    R with q_pos + 1 rows."""
    import torch

    g = lambda shape, k: normal_bf16(shape, seed_of(workload, k), device=device)
    q_nope = g((B, H, 128), SEED_Q_NOPE)
    q_pe = g((B, H, 64), SEED_Q_PE)
    k_cache = g((B, H, L, 192), SEED_KC)
    v_cache = g((B, H, L, 128), SEED_VC)
    R = torch.from_numpy(rope_angles(q_pos + 1)).to(device)
    return dict(q_nope=q_nope, q_pe=q_pe, k_cache=k_cache, v_cache=v_cache, R=R, q_pos=q_pos)


def decode_shared_kpe_inputs(B: int, H: int, L: int, q_pos: int, workload: int = 0, device="cpu"):
    """The shared-rotary cache layout: q_nope, q_pe (bf16), k_nope_cache
    [B,H,L,128], kpe_cache [B,L,64] (one rotated rope key per position for all
    heads), v_cache [B,H,L,128] (bf16) and R with q_pos + 1 rows."""
    import torch

    g = lambda shape, k: normal_bf16(shape, seed_of(workload, k), device=device)
    q_nope = g((B, H, 128), SEED_Q_NOPE)
    q_pe = g((B, H, 64), SEED_Q_PE)
    k_nope_cache = g((B, H, L, 128), SEED_KNC)
    kpe_cache = g((B, L, 64), SEED_KPC)
    v_cache = g((B, H, L, 128), SEED_VC)
    R = torch.from_numpy(rope_angles(q_pos + 1)).to(device)
    return dict(q_nope=q_nope, q_pe=q_pe, k_nope_cache=k_nope_cache, kpe_cache=kpe_cache,
                v_cache=v_cache, R=R, q_pos=q_pos)


def up_project_inputs(B: int, T: int, H: int, workload: int = 0, device="cpu"):
    """The up-projection's inputs: q_lat [B,T,1536] and ckv [B,T,512] (the two
    latents after their normalisations, unit scale: N(0,1)), w_q_b
    [H*192,1536] and w_kv_b [H*256,512] N(0, 0.02) (the configuration's
    initializer range), all bf16."""
    g = lambda shape, k, std=1.0: normal_bf16(shape, seed_of(workload, k), std=std, device=device)
    return dict(q_lat=g((B, T, 1536), SEED_QLAT), ckv=g((B, T, 512), SEED_CKV),
                w_q_b=g((H * 192, 1536), SEED_WQB, 0.02), w_kv_b=g((H * 256, 512), SEED_WKVB, 0.02))


def decode_latent_inputs(B: int, H: int, L: int, q_pos: int, workload: int = 0, device="cpu"):
    """The latent cache layout: q_nope [B,H,128], q_pe [B,H,64], ckv [B,L,512]
    (the cached latent after its normalisation, unit scale: N(0,1)), kpe
    [B,L,64] (rotated rope keys, N(0,1)), w_kv_b [H*256,512] N(0, 0.02) (the
    configuration's initializer range), all bf16, and R with q_pos + 1 rows."""
    import torch

    g = lambda shape, k, std=1.0: normal_bf16(shape, seed_of(workload, k), std=std, device=device)
    q_nope = g((B, H, 128), SEED_Q_NOPE)
    q_pe = g((B, H, 64), SEED_Q_PE)
    ckv = g((B, L, 512), SEED_CKV)
    kpe = g((B, L, 64), SEED_KPC)
    w_kv_b = g((H * 256, 512), SEED_WKVB, 0.02)
    R = torch.from_numpy(rope_angles(q_pos + 1)).to(device)
    return dict(q_nope=q_nope, q_pe=q_pe, ckv=ckv, kpe=kpe, w_kv_b=w_kv_b, R=R, q_pos=q_pos)


def chunk_inputs(B: int, H: int, T: int, past: int, seed: int = 7000, device="cpu"):
    """A prefill chunk of T positions after `past` cached ones: q_nope, q_pe,
    k_nope, k_pe, v of the chunk (bf16 N(0,1)), the shared-rotary caches
    k_nope_cache [B,H,L,128], kpe_cache [B,L,64], v_cache [B,H,L,128] with
    L = past + T (every row N(0,1): rows 0..past-1 stand for the history, rows
    past.. are overwritten by the append) and R with L rows.  Seeds
    seed + k, k = 0..7."""
    import torch

    L = past + T
    g = lambda shape, k: normal_bf16(shape, seed + k, device=device)
    return dict(q_nope=g((B, H, T, 128), 0), q_pe=g((B, H, T, 64), 1), k_nope=g((B, H, T, 128), 2),
                k_pe=g((B, 1, T, 64), 3), v=g((B, H, T, 128), 4), k_nope_cache=g((B, H, L, 128), 5),
                kpe_cache=g((B, L, 64), 6), v_cache=g((B, H, L, 128), 7),
                R=torch.from_numpy(rope_angles(L)).to(device))


def out_proj_weight(N: int = D_MODEL, K: int = 64 * 128, workload: int = 0, device="cpu"):
    """w_o [N, K] bf16 N(0, 0.02), stored as the linear layer stores it."""
    return normal_bf16((N, K), seed_of(workload, SEED_WO), std=0.02, device=device)


def out_proj_weight_fp8(N: int = D_MODEL, K: int = 64 * 128, workload: int = 0, device="cpu"):
    """The o_proj weight in the checkpoint's FP8 form: the bf16 N(0, 0.02)
    weight of out_proj_weight, one float32 scale per 128 x 128 block (block
    amax / 448, the largest e4m3 value), values divided by their scale and
    converted to e4m3 ("fn") by torch.  Returns (w8 uint8 [N,K], scale float32
    [ceil(N/128), ceil(K/128)])."""
    import torch

    w = out_proj_weight(N, K, workload, device).float()
    NB, KB = (N + 127) // 128, (K + 127) // 128
    pad = torch.zeros((NB * 128, KB * 128), dtype=torch.float32, device=w.device)
    pad[:N, :K] = w
    blocks = pad.view(NB, 128, KB, 128)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blocks / scale[:, None, :, None]).view(NB * 128, KB * 128)[:N, :K]
    w8 = q.contiguous().to(torch.float8_e4m3fn).view(torch.uint8)
    return w8, scale.contiguous()


def bits(t) -> np.ndarray:
    """uint16 bit patterns of a bf16 tensor (on the host)."""
    import torch

    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def to_v_blocked(v, fill: float = 0.0):
    """The key-blocked value layout (flag MLA_V_BLOCKED): v [B, H, T, 128] ->
    [B, H, ceil(T/16), 128, 16], the 16 positions of a block stored feature
    by feature; the slots past T hold ``fill``.  A copy in a new layout, no
    arithmetic."""
    import torch

    B, H, T, D = v.shape
    nb = (T + 15) // 16
    padded = torch.full((B, H, nb * 16, D), fill, dtype=v.dtype, device=v.device)
    padded[:, :, :T] = v
    return padded.view(B, H, nb, 16, D).transpose(3, 4).contiguous()


def from_v_blocked(vb, T: int):
    """Inverse of to_v_blocked: [B, H, NB, 128, 16] -> [B, H, T, 128]."""
    B, H, nb, D, _ = vb.shape
    return vb.transpose(3, 4).reshape(B, H, nb * 16, D)[:, :, :T].contiguous()
