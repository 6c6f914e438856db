"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

Every check here compares the oracle with something other than itself:
a library routine (torch's float32->bf16 conversion, torch's
scaled_dot_product_attention, numpy's float64 matmul), a closed form (prefix
means of V, integer row counts), an invariant of the definition (rows sum to
1, rotation preserves norm, relative-position invariance, future keys do not
matter, head permutation), or brute force through explicit [T, T] matrices
with the rotation written as complex multiplication.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from transformer_attention_mla_amd import inputs

SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


# ------------------------------------------------------------------ helpers

def rne_bf16(x):
    """Independent round-to-nearest-even to bf16 (8 significant bits) in numpy."""
    m, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def rand_bits(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    t = (torch.randn(shape, generator=g, dtype=torch.float32) * std).to(torch.bfloat16)
    return inputs.bits(t)


def widen(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def to_bits(x):
    return inputs.bits(torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def complex_rotate(x, ang):
    """Pair (x_i, x_{i+32}) as the complex number x_i + i*x_{i+32}, times e^{i*angle}."""
    z = x[..., :32] + 1j * x[..., 32:]
    y = z * np.exp(1j * ang)
    return np.concatenate([y.real, y.imag], axis=-1)


def brute_prefill(qn, qp, kn, kp, v, R, scale):
    """Explicit-matrix causal attention on widened float64 arrays."""
    B, H, T, _ = qn.shape
    ang = R[:T].astype(np.float64)
    qr = rne_bf16(complex_rotate(qp, ang))
    kr = rne_bf16(complex_rotate(kp, ang))
    Q = np.concatenate([qn, qr], axis=-1)
    K = np.concatenate([kn, np.broadcast_to(kr, (B, H, T, 64))], axis=-1)
    S = torch.from_numpy(Q) @ torch.from_numpy(np.ascontiguousarray(K)).transpose(-1, -2) * scale
    M = torch.full((T, T), float("-inf"), dtype=torch.float64).triu(1)
    P = torch.softmax(S + M, dim=-1)
    O = P @ torch.from_numpy(v)
    out = O.transpose(1, 2).reshape(B, T, H * 128).numpy()
    lse = torch.logsumexp(S + M, dim=-1).numpy()
    return out, lse, P.numpy()


def small_prefill(B, H, T, seed, r_rows=None):
    qn = rand_bits((B, H, T, 128), seed)
    qp = rand_bits((B, H, T, 64), seed + 1)
    kn = rand_bits((B, H, T, 128), seed + 2)
    kp = rand_bits((B, 1, T, 64), seed + 3)
    v = rand_bits((B, H, T, 128), seed + 4)
    R = inputs.rope_angles(r_rows or T)
    return qn, qp, kn, kp, v, R


# ------------------------------------------------------------ bf16 and dims

def test_dims_match_config():
    import json, os
    cfg = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "kimi_k2_config.json")))
    assert oracle.dims() == (cfg["qk_nope_head_dim"], cfg["qk_rope_head_dim"], cfg["v_head_dim"])


def test_bf16_round_matches_torch_on_float32_values():
    g = torch.Generator().manual_seed(7)
    x = torch.cat([torch.randn(200000, generator=g) * 3,
                   torch.randn(1000, generator=g) * 1e-30,
                   torch.randn(1000, generator=g) * 1e30])
    want = x.to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(x.to(torch.float64).numpy())
    assert np.array_equal(got, want)


def test_bf16_round_ties_to_even():
    ulp = 2.0 ** -7  # spacing of bf16 on [1, 2)
    x = np.array([1 + ulp / 2, 1 + 3 * ulp / 2, -(1 + ulp / 2), 2 + ulp, 1 + ulp / 2 + 2 ** -40])
    want = np.array([1.0, 1 + 2 * ulp, -1.0, 2.0, 1 + ulp])
    assert np.array_equal(oracle.bf16_round(x), want)
    assert np.array_equal(rne_bf16(x), want)


def test_widen_is_exact():
    b = rand_bits((4096,), 3)
    assert np.array_equal(oracle.bf16_widen(b), widen(b))


# ---------------------------------------------------------------- rotation

def test_rotation_position_zero_is_identity():
    x = rand_bits((5, 64), 11)
    R = inputs.rope_angles(8)
    assert np.all(R[0] == 0)
    f64, b16 = oracle.rope_rotate(x, R, np.zeros(5, np.int32))
    assert np.array_equal(b16, x)
    assert np.array_equal(f64, widen(x))


def test_rotation_is_complex_multiplication():
    x = rand_bits((64, 64), 12)
    R = inputs.rope_angles(5000)
    pos = np.random.default_rng(0).integers(0, 5000, 64).astype(np.int32)
    f64, b16 = oracle.rope_rotate(x, R, pos)
    want = complex_rotate(widen(x), R[pos].astype(np.float64))
    assert np.max(np.abs(f64 - want)) < 1e-12
    assert np.array_equal(widen(b16), rne_bf16(f64))


def test_rotation_preserves_pair_norm():
    x = rand_bits((32, 64), 13)
    R = inputs.rope_angles(16384)
    pos = np.arange(0, 16384, 512).astype(np.int32)
    f64, _ = oracle.rope_rotate(x, R, pos)
    xw = widen(x)
    n_in = xw[:, :32] ** 2 + xw[:, 32:] ** 2
    n_out = f64[:, :32] ** 2 + f64[:, 32:] ** 2
    assert np.max(np.abs(n_out - n_in) / np.maximum(n_in, 1e-30)) < 1e-12


def test_rotation_relative_position_invariance():
    """q at t+c against k at u+c scores the same as q at t against k at u
    (before rounding): pins that q and k use one pairing and one direction."""
    q = rand_bits((1, 64), 14)
    k = rand_bits((1, 64), 15)
    R = inputs.rope_angles(3000)
    for t, u, c in [(10, 3, 100), (500, 499, 1000), (7, 7, 2500), (2000, 0, 900)]:
        qa, _ = oracle.rope_rotate(q, R, np.array([t], np.int32))
        ka, _ = oracle.rope_rotate(k, R, np.array([u], np.int32))
        qb, _ = oracle.rope_rotate(q, R, np.array([t + c], np.int32))
        kb, _ = oracle.rope_rotate(k, R, np.array([u + c], np.int32))
        sa, sb = (qa @ ka.T).item(), (qb @ kb.T).item()
        # angles are float32, so t*f and (t+c)*f carry independent roundings
        assert abs(sa - sb) < 1e-3 * (1 + abs(sa)), (t, u, c, sa, sb)
    # exact version with an exactly representable angle table
    Rx = np.zeros((40, 32), np.float32)
    Rx[:, :] = np.arange(40, dtype=np.float32)[:, None] * np.float32(0.25)
    qa, _ = oracle.rope_rotate(q, Rx, np.array([5], np.int32))
    ka, _ = oracle.rope_rotate(k, Rx, np.array([2], np.int32))
    qb, _ = oracle.rope_rotate(q, Rx, np.array([35], np.int32))
    kb, _ = oracle.rope_rotate(k, Rx, np.array([32], np.int32))
    assert abs((qa @ ka.T).item() - (qb @ kb.T).item()) < 1e-12


def test_rotation_out_of_table_rejected():
    with pytest.raises(ValueError):
        oracle.rope_rotate(rand_bits((1, 64), 1), inputs.rope_angles(4), np.array([4], np.int32))


# ------------------------------------------------------------------ prefill

@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 3, 17), (2, 2, 9), (2, 3, 16)])
def test_prefill_matches_brute_force(B, H, T):
    qn, qp, kn, kp, v, R = small_prefill(B, H, T, 100 + T)
    out, lse = oracle.prefill(qn, qp, kn, kp, v, R, SCALE)
    bout, blse, P = brute_prefill(widen(qn), widen(qp), widen(kn), widen(kp), widen(v), R, SCALE)
    assert np.max(np.abs(out - bout)) < 1e-12
    assert np.max(np.abs(lse - blse)) < 1e-12
    assert np.max(np.abs(P.sum(-1) - 1)) < 1e-12


def test_prefill_rows_sum_to_one():
    """V = 1 makes every output the sum of the row's weights."""
    B, H, T = 1, 2, 50
    qn, qp, kn, kp, _, R = small_prefill(B, H, T, 200)
    ones = to_bits(np.ones((B, H, T, 128)))
    out, _ = oracle.prefill(qn, qp, kn, kp, ones, R, SCALE)
    assert np.max(np.abs(out - 1.0)) < 1e-13


def test_prefill_zero_query_gives_causal_prefix_means():
    B, H, T = 2, 2, 40
    _, _, kn, kp, v, R = small_prefill(B, H, T, 300)
    z128 = np.zeros((B, H, T, 128), np.uint16)
    z64 = np.zeros((B, H, T, 64), np.uint16)
    out, lse = oracle.prefill(z128, z64, kn, kp, v, R, SCALE)
    vw = widen(v)
    means = np.cumsum(vw, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    want = means.transpose(0, 2, 1, 3).reshape(B, T, H * 128)
    assert np.max(np.abs(out - want)) < 1e-13
    # count probe: every kept weight is exp(0) = 1, so exp(lse) = t + 1
    counts = np.rint(np.exp(lse)).astype(np.int64)
    assert np.array_equal(counts, np.broadcast_to(np.arange(1, T + 1), (B, H, T)))


def test_prefill_single_position_returns_v():
    qn, qp, kn, kp, v, R = small_prefill(2, 3, 1, 400)
    out, lse = oracle.prefill(qn, qp, kn, kp, v, R, SCALE)
    assert np.array_equal(out, widen(v)[:, :, 0, :].reshape(2, 3 * 128)[:, None, :])


def test_prefill_without_rotary_part_is_textbook_attention():
    """q_pe = k_pe = 0 reduces to causal attention over the 128-wide part with
    the 192-wide scale: torch's scaled_dot_product_attention in float64."""
    B, H, T = 2, 3, 33
    qn, _, kn, _, v, R = small_prefill(B, H, T, 500)
    out, _ = oracle.prefill(qn, np.zeros((B, H, T, 64), np.uint16), kn,
                            np.zeros((B, 1, T, 64), np.uint16), v, R, SCALE)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(widen(qn)), torch.from_numpy(widen(kn)), torch.from_numpy(widen(v)),
        is_causal=True, scale=SCALE)
    want = ref.transpose(1, 2).reshape(B, T, H * 128).numpy()
    assert np.max(np.abs(out - want)) < 1e-12


def test_prefill_future_keys_do_not_matter():
    B, H, T, t0 = 1, 2, 30, 12
    qn, qp, kn, kp, v, R = small_prefill(B, H, T, 600)
    out1, lse1 = oracle.prefill(qn, qp, kn, kp, v, R, SCALE)
    kn2, kp2, v2 = kn.copy(), kp.copy(), v.copy()
    kn2[:, :, t0 + 1:] = rand_bits(kn2[:, :, t0 + 1:].shape, 601)
    kp2[:, :, t0 + 1:] = rand_bits(kp2[:, :, t0 + 1:].shape, 602)
    v2[:, :, t0 + 1:] = rand_bits(v2[:, :, t0 + 1:].shape, 603)
    out2, lse2 = oracle.prefill(qn, qp, kn2, kp2, v2, R, SCALE)
    assert np.array_equal(out1[:, :t0 + 1], out2[:, :t0 + 1])
    assert np.array_equal(lse1[:, :, :t0 + 1], lse2[:, :, :t0 + 1])
    assert not np.array_equal(out1[:, t0 + 1:], out2[:, t0 + 1:])


def test_prefill_head_flatten_is_head_major():
    B, H, T, h = 1, 4, 10, 2
    qn, qp, kn, kp, v, R = small_prefill(B, H, T, 700)
    vh = np.zeros_like(v)
    vh[:, h] = v[:, h]
    out, _ = oracle.prefill(qn, qp, kn, kp, vh, R, SCALE)
    mask = np.zeros(H * 128, bool)
    mask[h * 128:(h + 1) * 128] = True
    assert np.all(out[:, :, ~mask] == 0)
    assert np.all(np.any(out[:, :, mask] != 0, axis=-1))


def test_prefill_head_permutation():
    B, H, T = 1, 4, 12
    qn, qp, kn, kp, v, R = small_prefill(B, H, T, 800)
    perm = np.array([2, 0, 3, 1])
    out, lse = oracle.prefill(qn, qp, kn, kp, v, R, SCALE)
    outp, lsep = oracle.prefill(qn[:, perm], qp[:, perm], kn[:, perm], kp, v[:, perm], R, SCALE)
    blocks = out.reshape(B, T, H, 128)
    assert np.array_equal(outp.reshape(B, T, H, 128), blocks[:, :, perm])
    assert np.array_equal(lsep, lse[:, perm])


def test_prefill_rows_equal_full():
    B, H, T = 2, 3, 21
    qn, qp, kn, kp, v, R = small_prefill(B, H, T, 900)
    out, lse = oracle.prefill(qn, qp, kn, kp, v, R, SCALE)
    sel = np.array([[0, 0, 0], [1, 2, 20], [0, 1, 7], [1, 0, 13]], np.int32)
    ro, rl = oracle.prefill_rows(qn, qp, kn, kp, v, R, SCALE, sel)
    for i, (b, h, t) in enumerate(sel):
        assert np.array_equal(ro[i], out[b, t, h * 128:(h + 1) * 128])
        assert rl[i] == lse[b, h, t]


def test_prefill_rejects_short_angle_table():
    qn, qp, kn, kp, v, R = small_prefill(1, 1, 8, 950)
    with pytest.raises(ValueError):
        oracle.prefill(qn, qp, kn, kp, v, R[:7], SCALE)


# ------------------------------------------------------------------- decode

def make_cache_from_prefill(kn, kp, R):
    """Decode cache rows [k_nope | rot(k_pe)] from a prefill's keys (rotated by the oracle)."""
    B, H, T, _ = kn.shape
    pos = np.broadcast_to(np.arange(T, dtype=np.int32), (B, T)).copy()
    _, kr = oracle.rope_rotate(kp.reshape(B, T, 64), R, pos)
    kr = np.broadcast_to(kr.reshape(B, 1, T, 64), (B, H, T, 64))
    return np.ascontiguousarray(np.concatenate([kn, kr], axis=-1))


def test_decode_equals_last_prefill_row():
    B, H, L = 2, 3, 24  # prefill over L + 1 positions; decode the last one
    qn, qp, kn, kp, v, R = small_prefill(B, H, L + 1, 1000)
    out, lse = oracle.prefill(qn, qp, kn, kp, v, R, SCALE)
    kc = make_cache_from_prefill(kn, kp, R)
    dout, dlse = oracle.decode(np.ascontiguousarray(qn[:, :, L]), np.ascontiguousarray(qp[:, :, L]),
                               kc, v, R, L, SCALE)
    assert np.array_equal(dout, out[:, L])
    assert np.array_equal(dlse, lse[:, :, L])


def test_decode_brute_force():
    B, H, L, qpos = 2, 3, 19, 40
    qn = rand_bits((B, H, 128), 1100)
    qp = rand_bits((B, H, 64), 1101)
    kc = rand_bits((B, H, L, 192), 1102)
    vc = rand_bits((B, H, L, 128), 1103)
    R = inputs.rope_angles(qpos + 1)
    out, lse = oracle.decode(qn, qp, kc, vc, R, qpos, SCALE)
    qr = rne_bf16(complex_rotate(widen(qp), R[qpos].astype(np.float64)))
    Q = np.concatenate([widen(qn), qr], -1)
    S = np.einsum("bhd,bhld->bhl", Q, widen(kc)) * SCALE
    P = np.exp(S - S.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    O = np.einsum("bhl,bhld->bhd", P, widen(vc)).reshape(B, H * 128)
    assert np.max(np.abs(out - O)) < 1e-12
    assert np.max(np.abs(lse - (S.max(-1) + np.log(np.exp(S - S.max(-1, keepdims=True)).sum(-1))))) < 1e-12


def test_decode_single_key_and_ones():
    B, H = 3, 2
    qn = rand_bits((B, H, 128), 1200)
    qp = rand_bits((B, H, 64), 1201)
    R = inputs.rope_angles(10)
    kc = rand_bits((B, H, 1, 192), 1202)
    vc = rand_bits((B, H, 1, 128), 1203)
    out, _ = oracle.decode(qn, qp, kc, vc, R, 9, SCALE)
    assert np.array_equal(out, widen(vc).reshape(B, H * 128))
    kc = rand_bits((B, H, 50, 192), 1204)
    out, _ = oracle.decode(qn, qp, kc, to_bits(np.ones((B, H, 50, 128))), R, 9, SCALE)
    assert np.max(np.abs(out - 1)) < 1e-13


def test_decode_zero_query_mean_and_count():
    B, H, L = 2, 2, 77
    kc = rand_bits((B, H, L, 192), 1300)
    vc = rand_bits((B, H, L, 128), 1301)
    out, lse = oracle.decode(np.zeros((B, H, 128), np.uint16), np.zeros((B, H, 64), np.uint16),
                             kc, vc, inputs.rope_angles(5), 4, SCALE)
    assert np.max(np.abs(out - widen(vc).mean(axis=2).reshape(B, H * 128))) < 1e-13
    assert np.array_equal(np.rint(np.exp(lse)), np.full((B, H), L))


def shared_kpe_case(B, H, L, seed):
    qn = rand_bits((B, H, 128), seed)
    qp = rand_bits((B, H, 64), seed + 1)
    kn = rand_bits((B, H, L, 128), seed + 2)
    kp = rand_bits((B, L, 64), seed + 3)
    vc = rand_bits((B, H, L, 128), seed + 4)
    return qn, qp, kn, kp, vc


def test_decode_shared_kpe_equals_joined_cache():
    """The shared-rotary layout is the joined layout with the one rope key per
    position copied into every head's rows: same outputs, bit for bit."""
    B, H, L, qpos = 3, 4, 45, 60
    qn, qp, kn, kp, vc = shared_kpe_case(B, H, L, 1500)
    R = inputs.rope_angles(qpos + 1)
    joined = np.concatenate([kn, np.broadcast_to(kp[:, None], (B, H, L, 64))], axis=-1)
    want, wl = oracle.decode(qn, qp, np.ascontiguousarray(joined), vc, R, qpos, SCALE)
    got, gl = oracle.decode_shared_kpe(qn, qp, kn, kp, vc, R, qpos, SCALE)
    assert np.array_equal(got, want) and np.array_equal(gl, wl)
    sel = np.array([[2, 3], [0, 1], [1, 0]], np.int32)
    ro, rl = oracle.decode_shared_kpe_rows(qn, qp, kn, kp, vc, R, qpos, SCALE, sel)
    for i, (b, h) in enumerate(sel):
        assert np.array_equal(ro[i], got[b, h * 128:(h + 1) * 128]) and rl[i] == gl[b, h]


def test_decode_shared_kpe_single_key_zero_query_and_sharing():
    B, H = 2, 3
    qn, qp, kn, kp, vc = shared_kpe_case(B, H, 1, 1600)
    R = inputs.rope_angles(4)
    out, _ = oracle.decode_shared_kpe(qn, qp, kn, kp, vc, R, 3, SCALE)
    assert np.array_equal(out, widen(vc).reshape(B, H * 128))  # one key: its value row
    L = 33
    qn, qp, kn, kp, vc = shared_kpe_case(B, H, L, 1700)
    z = np.zeros((B, H, 128), np.uint16), np.zeros((B, H, 64), np.uint16)
    out, lse = oracle.decode_shared_kpe(z[0], z[1], kn, kp, vc, R, 3, SCALE)
    assert np.max(np.abs(out - widen(vc).mean(axis=2).reshape(B, H * 128))) < 1e-13
    assert np.array_equal(np.rint(np.exp(lse)), np.full((B, H), L))
    # The rope table of sequence 1 feeds every head of sequence 1 and nothing else.
    base, _ = oracle.decode_shared_kpe(qn, qp, kn, kp, vc, R, 3, SCALE)
    kp2 = kp.copy()
    kp2[1] = rand_bits((L, 64), 1799)
    pert, _ = oracle.decode_shared_kpe(qn, qp, kn, kp2, vc, R, 3, SCALE)
    assert np.array_equal(pert[0], base[0])
    assert all(not np.array_equal(pert[1, h * 128:(h + 1) * 128], base[1, h * 128:(h + 1) * 128])
               for h in range(H))


def latent_case(B, H, L, seed):
    qn = rand_bits((B, H, 128), seed)
    qp = rand_bits((B, H, 64), seed + 1)
    ckv = rand_bits((B, L, 512), seed + 2)
    kpe = rand_bits((B, L, 64), seed + 3)
    w = rand_bits((H * 256, 512), seed + 4, std=0.02)
    return qn, qp, ckv, kpe, w


def test_decode_latent_selection_weights_equal_shared_kpe():
    """With a kv_b_proj whose rows are one-hot (a different permutation of the
    latent per head), every up-projected key and value is a latent element
    exactly, so the latent decode must equal the shared-rotary decode on the
    explicitly gathered caches, bit for bit: pins the head and row slicing."""
    B, H, L, qpos = 2, 3, 37, 50
    qn, qp, ckv, kpe, _ = latent_case(B, H, L, 2100)
    rng = np.random.default_rng(2105)
    perm = np.stack([rng.permutation(512) for _ in range(H)])
    w = np.zeros((H * 256, 512), np.uint16)
    for h in range(H):
        w[h * 256 + np.arange(256), perm[h, :256]] = 0x3F80  # bf16 1.0
    kn = np.stack([ckv[:, :, perm[h, :128]] for h in range(H)], axis=1)
    vc = np.stack([ckv[:, :, perm[h, 128:256]] for h in range(H)], axis=1)
    R = inputs.rope_angles(qpos + 1)
    want, wl = oracle.decode_shared_kpe(qn, qp, np.ascontiguousarray(kn), kpe,
                                        np.ascontiguousarray(vc), R, qpos, SCALE)
    got, gl = oracle.decode_latent(qn, qp, ckv, kpe, w, R, qpos, SCALE)
    assert np.array_equal(got, want) and np.array_equal(gl, wl)


def test_decode_latent_absorbed_form():
    """Without rounding the up-projected keys and values, the latent decode is
    (W_uk q)·c scores over the latent, the softmax-weighted latent mean, then
    W_uv: an independent evaluation (numpy, the query rotation as complex
    multiplication) of the same function in the absorbed order."""
    B, H, L, qpos = 2, 3, 29, 40
    qn, qp, ckv, kpe, w = latent_case(B, H, L, 2200)
    R = inputs.rope_angles(qpos + 1)
    got, gl = oracle.decode_latent(qn, qp, ckv, kpe, w, R, qpos, SCALE, round_kv=False)
    W = widen(w).reshape(H, 256, 512)
    Wk, Wv = W[:, :128], W[:, 128:]
    C, Kp = widen(ckv), widen(kpe)
    qr = rne_bf16(complex_rotate(widen(qp), R[qpos].astype(np.float64)))
    q_lat = np.einsum("bhd,hdc->bhc", widen(qn), Wk)
    s = SCALE * (np.einsum("bhc,blc->bhl", q_lat, C) + np.einsum("bhr,blr->bhl", qr, Kp))
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    o_lat = np.einsum("bhl,blc->bhc", e / e.sum(axis=-1, keepdims=True), C)
    want = np.einsum("hec,bhc->bhe", Wv, o_lat).reshape(B, H * 128)
    lse = (m[..., 0] + np.log(e.sum(axis=-1)))
    assert np.max(np.abs(got - want)) < 1e-12
    assert np.max(np.abs(gl - lse)) < 1e-12
    # with rounding (R3) the result moves, but only by the bf16 rounding of k and v
    r, _ = oracle.decode_latent(qn, qp, ckv, kpe, w, R, qpos, SCALE)
    assert 0 < np.max(np.abs(r - got)) < 5e-3


def test_decode_latent_equals_joined_decode_and_rows():
    """Up-project in numpy, round to bf16 (independent RNE), build the joined
    [nope | rope] cache per head: the joined-cache decode gives the same
    outputs; selected rows equal the full result."""
    B, H, L, qpos = 2, 2, 23, 30
    qn, qp, ckv, kpe, w = latent_case(B, H, L, 2300)
    R = inputs.rope_angles(qpos + 1)
    W = widen(w).reshape(H, 256, 512)
    up = np.einsum("hoc,blc->bhlo", W, widen(ckv))
    kn, vc = to_bits(rne_bf16(up[..., :128])), to_bits(rne_bf16(up[..., 128:]))
    joined = np.concatenate([kn, np.broadcast_to(kpe[:, None], (B, H, L, 64))], axis=-1)
    want, wl = oracle.decode(qn, qp, np.ascontiguousarray(joined), vc, R, qpos, SCALE)
    got, gl = oracle.decode_latent(qn, qp, ckv, kpe, w, R, qpos, SCALE)
    assert np.max(np.abs(got - want)) < 1e-14 and np.max(np.abs(gl - wl)) < 1e-13
    sel = np.array([[1, 1], [0, 0], [1, 0]], np.int32)
    ro, rl = oracle.decode_latent(qn, qp, ckv, kpe, w, R, qpos, SCALE, sel=sel)
    for i, (b, h) in enumerate(sel):
        assert np.array_equal(ro[i], got[b, h * 128:(h + 1) * 128]) and rl[i] == gl[b, h]


# --------------------------------------------------------- up-projection

def up_case(B, T, H, seed):
    return (rand_bits((B, T, 1536), seed), rand_bits((B, T, 512), seed + 1),
            rand_bits((H * 192, 1536), seed + 2, std=0.02), rand_bits((H * 256, 512), seed + 3, std=0.02))


def test_up_project_selection_weights():
    """One-hot weight rows (a different latent index per output feature):
    every output is one latent element exactly, at the place the head split
    puts it -- head h's q_nope from rows h*192.., its q_pe from h*192+128..,
    its nope key from rows h*256.., its value from h*256+128.. (pins the head
    and part slicing and the [B,H,T,d] layout)."""
    B, T, H = 2, 5, 3
    ql, ckv, _, _ = up_case(B, T, H, 2400)
    rng = np.random.default_rng(2405)
    iq = rng.integers(0, 1536, H * 192)
    ik = rng.integers(0, 512, H * 256)
    wq = np.zeros((H * 192, 1536), np.uint16)
    wq[np.arange(H * 192), iq] = 0x3F80
    wk = np.zeros((H * 256, 512), np.uint16)
    wk[np.arange(H * 256), ik] = 0x3F80
    qn, qp, kn, v = oracle.up_project(ql, ckv, wq, wk)
    Q, C = widen(ql), widen(ckv)
    for h in range(H):
        assert np.array_equal(qn[:, h], Q[:, :, iq[h * 192:h * 192 + 128]])
        assert np.array_equal(qp[:, h], Q[:, :, iq[h * 192 + 128:(h + 1) * 192]])
        assert np.array_equal(kn[:, h], C[:, :, ik[h * 256:h * 256 + 128]])
        assert np.array_equal(v[:, h], C[:, :, ik[h * 256 + 128:(h + 1) * 256]])


def test_up_project_one_hot_latent_reads_weight_columns():
    """A latent row that is one-hot at index k gives, for every head and
    feature, the weight's k-th column (the transposition of the linear layer:
    y = x · Wᵀ with W [out, in]); rows are independent of each other."""
    B, T, H = 1, 4, 2
    _, _, wq, wk = up_case(B, T, H, 2500)
    ql = np.zeros((B, T, 1536), np.uint16)
    ckv = np.zeros((B, T, 512), np.uint16)
    ks_q, ks_c = [7, 1535, 0, 800], [3, 511, 256, 0]
    for t in range(T):
        ql[0, t, ks_q[t]] = 0x3F80
        ckv[0, t, ks_c[t]] = 0x3F80
    qn, qp, kn, v = oracle.up_project(ql, ckv, wq, wk)
    Wq, Wk = widen(wq).reshape(H, 192, 1536), widen(wk).reshape(H, 256, 512)
    for t in range(T):
        assert np.array_equal(qn[0, :, t], Wq[:, :128, ks_q[t]])
        assert np.array_equal(qp[0, :, t], Wq[:, 128:, ks_q[t]])
        assert np.array_equal(kn[0, :, t], Wk[:, :128, ks_c[t]])
        assert np.array_equal(v[0, :, t], Wk[:, 128:, ks_c[t]])


def test_up_project_feeds_the_latent_decode():
    """Keys and values up-projected from a latent cache, rounded to bf16 and
    attended by the shared-rotary decode, give the latent decode's output
    (whose own up-projection is separate code): the kv half agrees with the
    latent reading.  Random weights are checked against numpy's float64
    matmul, and selected rows equal the full result."""
    B, T, H = 2, 19, 3
    ql, ckv, wq, wk = up_case(B, T, H, 2600)
    qn, qp, kn, v = oracle.up_project(ql, ckv, wq, wk)
    q = widen(ql) @ widen(wq).T
    kv = widen(ckv) @ widen(wk).T
    qh, kvh = q.reshape(B, T, H, 192).transpose(0, 2, 1, 3), kv.reshape(B, T, H, 256).transpose(0, 2, 1, 3)
    assert np.max(np.abs(qn - qh[..., :128])) < 1e-12 and np.max(np.abs(qp - qh[..., 128:])) < 1e-12
    assert np.max(np.abs(kn - kvh[..., :128])) < 1e-12 and np.max(np.abs(v - kvh[..., 128:])) < 1e-12
    qpos = T + 4
    R = inputs.rope_angles(qpos + 1)
    dq_n, dq_p = rand_bits((B, H, 128), 2610), rand_bits((B, H, 64), 2611)
    kpe = rand_bits((B, T, 64), 2612)
    want, wl = oracle.decode_latent(dq_n, dq_p, ckv, kpe, wk, R, qpos, SCALE)
    got, gl = oracle.decode_shared_kpe(dq_n, dq_p, to_bits(rne_bf16(kn)), kpe, to_bits(rne_bf16(v)), R,
                                       qpos, SCALE)
    assert np.max(np.abs(got - want)) < 1e-13 and np.max(np.abs(gl - wl)) < 1e-13
    rows = np.array([T + 3, 0, 2 * T - 1], np.int32)
    r = oracle.up_project(ql, ckv, wq, wk, rows=rows)
    for i, m in enumerate(rows):
        b, t = divmod(int(m), T)
        for full, part in zip((qn, qp, kn, v), r):
            assert np.array_equal(part[i], full[b, :, t])


def test_decode_rows_equal_full():
    B, H, L = 2, 3, 30
    qn = rand_bits((B, H, 128), 1400)
    qp = rand_bits((B, H, 64), 1401)
    kc = rand_bits((B, H, L, 192), 1402)
    vc = rand_bits((B, H, L, 128), 1403)
    R = inputs.rope_angles(8)
    out, lse = oracle.decode(qn, qp, kc, vc, R, 7, SCALE)
    sel = np.array([[1, 2], [0, 0], [1, 1]], np.int32)
    ro, rl = oracle.decode_rows(qn, qp, kc, vc, R, 7, SCALE, sel)
    for i, (b, h) in enumerate(sel):
        assert np.array_equal(ro[i], out[b, h * 128:(h + 1) * 128])
        assert rl[i] == lse[b, h]


# ------------------------------------------------- chunked prefill, append

def chunk_case(B, H, T, seed):
    return (rand_bits((B, H, T, 128), seed), rand_bits((B, H, T, 64), seed + 1),
            rand_bits((B, H, T, 128), seed + 2), rand_bits((B, 1, T, 64), seed + 3),
            rand_bits((B, H, T, 128), seed + 4))


def empty_caches(B, H, Lc, seed=None):
    if seed is None:
        z = lambda *s: np.zeros(s, np.uint16)
        return z(B, H, Lc, 128), z(B, Lc, 64), z(B, H, Lc, 128)
    return rand_bits((B, H, Lc, 128), seed), rand_bits((B, Lc, 64), seed + 1), rand_bits((B, H, Lc, 128), seed + 2)


def test_chunk_at_zero_equals_prefill():
    """Append at 0 then the chunked prefill over the cache is the prefill."""
    B, H, T, Lc = 2, 3, 37, 50
    qn, qp, kn, kp, v = chunk_case(B, H, T, 2400)
    R = inputs.rope_angles(Lc)
    want, wl = oracle.prefill(qn, qp, kn, kp, v, R, SCALE)
    kc, pc, vc = empty_caches(B, H, Lc, 2410)  # rows past T hold junk
    oracle.append_kv(kn, kp, v, R, 0, kc, pc, vc)
    got, gl = oracle.prefill_chunk(qn, qp, kc, pc, vc, R, 0, SCALE)
    assert np.array_equal(got, want) and np.array_equal(gl, wl)


def test_chunks_equal_one_prefill():
    """A 45-position prefill in chunks of 17 and 28 (append, then attend over
    the cache): every row equals the single prefill's, bit for bit."""
    B, H, T1, T2 = 2, 2, 17, 28
    T = T1 + T2
    qn, qp, kn, kp, v = chunk_case(B, H, T, 2500)
    R = inputs.rope_angles(64)
    want, wl = oracle.prefill(qn, qp, kn, kp, v, R, SCALE)
    kc, pc, vc = empty_caches(B, H, 64)
    c = lambda a, s: np.ascontiguousarray(a[:, :, s])
    oracle.append_kv(c(kn, slice(0, T1)), c(kp, slice(0, T1)), c(v, slice(0, T1)), R, 0, kc, pc, vc)
    o1, l1 = oracle.prefill_chunk(c(qn, slice(0, T1)), c(qp, slice(0, T1)), kc, pc, vc, R, 0, SCALE)
    oracle.append_kv(c(kn, slice(T1, T)), c(kp, slice(T1, T)), c(v, slice(T1, T)), R, T1, kc, pc, vc)
    o2, l2 = oracle.prefill_chunk(c(qn, slice(T1, T)), c(qp, slice(T1, T)), kc, pc, vc, R, T1, SCALE)
    assert np.array_equal(o1, want[:, :T1]) and np.array_equal(o2, want[:, T1:])
    assert np.array_equal(l1, wl[:, :, :T1]) and np.array_equal(l2, wl[:, :, T1:])


def test_chunk_of_one_equals_decode_and_ignores_later_rows():
    """A one-position chunk at past = L is the decode of that query over the
    L + 1 cached keys (shared-rotary layout); cache rows past it are unseen."""
    B, H, L, Lc = 2, 3, 30, 40
    kc, pc, vc = empty_caches(B, H, Lc, 2600)
    qn, qp = rand_bits((B, H, 1, 128), 2610), rand_bits((B, H, 1, 64), 2611)
    R = inputs.rope_angles(Lc)
    got, gl = oracle.prefill_chunk(qn, qp, kc, pc, vc, R, L, SCALE)
    c = lambda a: np.ascontiguousarray(a[:, :, :L + 1]) if a.ndim == 4 else np.ascontiguousarray(a[:, :L + 1])
    want, wl = oracle.decode_shared_kpe(qn[:, :, 0], qp[:, :, 0], c(kc), c(pc), c(vc), R, L, SCALE)
    assert np.array_equal(got[:, 0], want) and np.array_equal(gl[:, :, 0], wl)
    kc2, pc2, vc2 = kc.copy(), pc.copy(), vc.copy()
    kc2[:, :, L + 1:] = rand_bits(kc2[:, :, L + 1:].shape, 2620)
    pc2[:, L + 1:] = rand_bits(pc2[:, L + 1:].shape, 2621)
    g2, _ = oracle.prefill_chunk(qn, qp, kc2, pc2, vc2, R, L, SCALE)
    assert np.array_equal(g2, got)


def test_chunk_rows_equal_full_and_ignore_rows_past_the_chunk():
    """Sampled rows of the chunked prefill equal the full chunked prefill's
    rows bit for bit, and NaN / infinity in cache rows at or past past + T
    (never written by the append) change nothing."""
    B, H, T, past, Lc = 2, 3, 19, 23, 57
    qn, qp, kn, kp, v = chunk_case(B, H, T, 2700)
    R = inputs.rope_angles(Lc)
    kc, pc, vc = empty_caches(B, H, Lc)
    hist = empty_caches(B, H, past, 2710)
    kc[:, :, :past], pc[:, :past], vc[:, :, :past] = hist
    oracle.append_kv(kn, kp, v, R, past, kc, pc, vc)
    out, lse = oracle.prefill_chunk(qn, qp, kc, pc, vc, R, past, SCALE)
    sel = np.array([[0, 0, 0], [1, 2, T - 1], [0, 1, 7], [1, 0, 13], [1, 1, T - 1]], np.int32)
    ro, rl = oracle.prefill_chunk_rows(qn, qp, kc, pc, vc, R, past, SCALE, sel)
    for i, (b, h, t) in enumerate(sel):
        assert np.array_equal(ro[i], out[b, t, h * 128:(h + 1) * 128])
        assert rl[i] == lse[b, h, t]
    for bad in (0x7FC0, 0x7F80, 0xFF80):  # bf16 NaN, +inf, -inf
        kc2, pc2, vc2 = kc.copy(), pc.copy(), vc.copy()
        kc2[:, :, past + T:] = bad
        pc2[:, past + T:] = bad
        vc2[:, :, past + T:] = bad
        o2, l2 = oracle.prefill_chunk(qn, qp, kc2, pc2, vc2, R, past, SCALE)
        assert np.array_equal(o2, out) and np.array_equal(l2, lse)


# ------------------------------------------------------------ fp8 weights

def test_e4m3_decode_matches_torch():
    """Every byte value decodes to torch's float8_e4m3fn value (NaN codes too)."""
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_double(b)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_dequant_fp8_matches_torch_and_block_layout():
    """Dequantization equals torch's float32 product of the e4m3 value and its
    block's scale, rounded to bf16, bit for bit; ragged N and K; and a scale
    change in one block moves exactly that block."""
    N, K = 300, 384
    g = torch.Generator().manual_seed(1800)
    w8 = (torch.randn((N, K), generator=g) * 60).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    scale = (torch.rand((3, 3), generator=g) * 1e-3 + 1e-4).to(torch.float32)
    s_full = scale.repeat_interleave(128, 0).repeat_interleave(128, 1)[:N, :K]
    want = (torch.from_numpy(w8.copy()).view(torch.float8_e4m3fn).to(torch.float32) * s_full)
    want = inputs.bits(want.to(torch.bfloat16))
    got = oracle.dequant_fp8(w8, scale.numpy())
    assert np.array_equal(got, want)
    s2 = scale.clone()
    s2[1, 2] *= 2
    got2 = oracle.dequant_fp8(w8, s2.numpy())
    diff = got2 != got
    assert not diff[:128].any() and not diff[256:].any() and not diff[128:256, :256].any()
    assert diff[128:256, 256:].any()


def test_e4m3_encode_matches_torch():
    """Round to nearest even on the e4m3 grid, as torch converts float32 to
    float8_e4m3fn: random values over the whole range, exact ties between
    neighbours (normal and subnormal), the rounding edge above 448 and
    zeros."""
    g = torch.Generator().manual_seed(11)
    e = torch.randint(-12, 9, (20000,), generator=g).to(torch.float32)
    v = (torch.rand(20000, generator=g) * 2 - 1) * torch.pow(2.0, e)
    codes = torch.arange(0, 127, dtype=torch.uint8)
    grid = codes.view(torch.float8_e4m3fn).to(torch.float32)
    ties = (grid[:-1] + grid[1:]) / 2  # exact in float32
    extra = torch.tensor([448.0, 455.0, 464.0, 464.5, 480.0, 0.0, -0.0, 2.0 ** -10, 2.0 ** -12,
                          3 * 2.0 ** -11, 1e-30])
    vals = torch.cat([v, ties, -ties, grid, -grid, extra, -extra])
    want = vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_from_float(vals.numpy())
    # NaN results compare by being NaN codes (torch and the oracle both set 0x7F | sign)
    assert np.array_equal(got, want)


def test_act_quant_matches_the_published_per_token_cast():
    """Per row and 128-column block: amax (clamped at 1e-4) / 448 and e4m3 of
    x / scale, written here directly in torch float32 (the reference per-token
    cast of the FP8 recipe), including a zero block, a tiny block and a ragged
    last block."""
    M, K = 9, 300
    g = torch.Generator().manual_seed(12)
    x = (torch.randn((M, K), generator=g) * 3).to(torch.bfloat16)
    x[1, 128:256] = 0
    x[2, :128] = (torch.randn(128, generator=g) * 1e-6).to(torch.bfloat16)
    xf = x.float()
    pad = torch.zeros((M, 384))
    pad[:, :K] = xf
    amax = pad.view(M, 3, 128).abs().amax(-1).clamp(min=1e-4)
    scale = amax / 448.0
    q = (pad.view(M, 3, 128) / scale[:, :, None]).view(M, 384)[:, :K].to(torch.float8_e4m3fn)
    gq, gs = oracle.act_quant(inputs.bits(x))
    assert np.array_equal(gs, scale.numpy())
    assert np.array_equal(gq, q.view(torch.uint8).numpy())
    assert np.all(gq[1, 128:256] == 0)
    # every block's largest magnitude quantizes to the top code (448) unless the clamp applies
    big = np.abs(xf.numpy()[0, :128]).argmax()
    assert gq[0, big] & 0x7F == 0x7E


def test_out_proj_fp8_dyn_is_the_product_of_dequantized_operands():
    """The projection equals a numpy float64 matmul of the two dequantized
    operands (torch's e4m3 values times their block scales), and a scaled
    identity weight returns each row's dequantized activations."""
    M, K, N = 7, 384, 200
    g = torch.Generator().manual_seed(13)
    x = torch.randn((M, K), generator=g).to(torch.bfloat16)
    w8, ws = inputs.out_proj_weight_fp8(N, K, workload=2)
    y = oracle.out_proj_fp8_dyn(inputs.bits(x), w8.numpy(), ws.numpy())
    q, sx = oracle.act_quant(inputs.bits(x))
    xd = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy() * np.repeat(sx, 128, 1)[:, :K]
    wd = w8.view(torch.float8_e4m3fn).double().numpy() * np.repeat(np.repeat(ws.numpy(), 128, 0), 128, 1)[:N, :K]
    want = xd @ wd.T
    assert np.max(np.abs(y - want)) <= 1e-12 * np.max(np.abs(want))
    # W = 2^-3 I: y[m, n] = dequantized x[m, n] / 8, exactly
    w8i = np.zeros((K, K), np.uint8)
    w8i[np.arange(K), np.arange(K)] = 0x38  # 1.0
    wsi = np.full((3, 3), 0.125, np.float32)
    yi = oracle.out_proj_fp8_dyn(inputs.bits(x), w8i, wsi)
    assert np.array_equal(yi, xd / 8)


def test_out_proj_fp8_input_recipe():
    """The FP8 weight recipe reproduces the bf16 weight to e4m3 precision
    (relative error below 2^-4 of each block's largest element)."""
    N, K = 256, 256
    w = inputs.out_proj_weight(N, K, workload=3).float().numpy()
    w8, scale = inputs.out_proj_weight_fp8(N, K, workload=3)
    deq = widen(oracle.dequant_fp8(w8.numpy(), scale.numpy()))
    for nb in range(2):
        for kb in range(2):
            blk = np.s_[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            assert np.max(np.abs(deq[blk] - w[blk])) <= np.max(np.abs(w[blk])) * 2.0 ** -4


# ------------------------------------------------------------------- o_proj

def test_out_proj_matches_float64_matmul():
    M, K, N = 7, 256, 33
    x = rand_bits((M, K), 1500)
    w = rand_bits((N, K), 1501, std=0.02)
    y = oracle.out_proj(x, w)
    want = widen(x) @ widen(w).T
    assert np.max(np.abs(y - want)) < 1e-12


def test_out_proj_selection_weight_is_exact():
    M, K, N = 5, 384, 300
    x = rand_bits((M, K), 1600)
    w = np.zeros((N, K), np.float32)
    w[np.arange(N), np.arange(N)] = 1.0
    y = oracle.out_proj(x, to_bits(w))
    assert np.array_equal(y, widen(x)[:, :N])


def test_out_proj_rows_equal_full():
    M, K, N = 9, 128, 20
    x = rand_bits((M, K), 1700)
    w = rand_bits((N, K), 1701)
    y = oracle.out_proj(x, w)
    rows = np.array([8, 0, 3])
    assert np.array_equal(oracle.out_proj_rows(x, w, rows), y[rows])
