"""GPU check of the matrix-core rate probe (a measurement helper): its
outputs equal the products it is documented to chain, which pins the MFMA
lane layout it relies on, and it is deterministic.

Thread t = 64 w + l (wave w, lane l) supplies row l % 32 of A and column
l % 32 of B, k-elements 8 (l / 32) + e, with the values
A = 1 + ((5 t + 3 e) mod 128) / 128 and B = ((iters + e + 3 t) mod 4) / 2^20
(exact in bf16; every product and partial sum is exact in float32).  It then
holds column l % 32, rows (r / 4) * 8 + (l / 32) * 4 + r % 4 of D = iters * A B
in register r of each of its 4 chains, and writes the sum of those 64 values.
"""
import numpy as np
import pytest
import torch

import transformer_attention_mla_amd as mla

pytestmark = pytest.mark.gpu


def expected(iters):
    out = np.zeros(256)
    for w in range(4):
        A = np.zeros((32, 16))
        Bm = np.zeros((16, 32))
        for l in range(64):
            t = 64 * w + l
            for e in range(8):
                k = 8 * (l // 32) + e
                A[l % 32, k] = 1 + ((5 * t + 3 * e) % 128) / 128
                Bm[k, l % 32] = ((iters + e + 3 * t) % 4) * 2.0 ** -20
        D = iters * (A @ Bm)
        for l in range(64):
            rows = [(r // 4) * 8 + (l // 32) * 4 + r % 4 for r in range(16)]
            out[64 * w + l] = 4 * D[rows, l % 32].sum()
    return out


@pytest.mark.parametrize("iters", [1, 37, 1000])
def test_mfma_probe_values(iters, gpu_device):
    out = mla.mla_mfma_probe(iters, 0, device=gpu_device)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy().reshape(512, 256)
    want = expected(iters)
    for b in (0, 1, 255, 511):
        np.testing.assert_allclose(got[b], want, rtol=1e-6, atol=0)
    assert np.array_equal(got, np.broadcast_to(got[0], got.shape)), "workgroups differ"
    again = mla.mla_mfma_probe(iters, 0, out=torch.empty_like(out))
    torch.cuda.synchronize()
    assert torch.equal(out, again), "not deterministic"


@pytest.mark.parametrize("iters", [1, 2, 1001])
def test_mfma_probe_fp8_values(iters, gpu_device):
    """e4m3 kind: every 4-byte group of A is (a, a, a, 0), of B (0, b, b, b),
    a = 1 for even threads and 0.5 for odd ones, b = 1 (even iters) or 0.5:
    D[i][j] = 64 k-elements / 4 * 2 a_i b = 32 a_i b, rows i and i + 32 coming
    from lanes of the same parity.  A thread's 16 rows are 8 even and 8 odd,
    so it writes 4 chains * iters * 32 * (8 + 8 * 0.5) * b = 1536 iters b."""
    out = mla.mla_mfma_probe(iters, 1, device=gpu_device)
    torch.cuda.synchronize()
    b = 1.0 if iters % 2 == 0 else 0.5
    want = torch.full_like(out, 1536.0 * iters * b)
    assert torch.equal(out, want), (out[:4], want[:4])


def _xorshift32(h):
    h ^= (h << 13) & 0xFFFFFFFF
    h ^= h >> 17
    h ^= (h << 5) & 0xFFFFFFFF
    return h


def _rand_operands(t, iters, fp8):
    """Thread t's eight A and B operand sets as the probe documents them:
    bf16 -> float arrays [8, 8]; e4m3 -> byte arrays [8, 32]."""
    h = ((0x9E3779B9 * (t + 1)) & 0xFFFFFFFF) ^ iters
    if not fp8:
        a = np.zeros((8, 8), np.float32)
        b = np.zeros((8, 8), np.float32)
        for v in range(8):
            for e in range(8):
                h = _xorshift32(h)
                a[v, e] = (1.0 + (h & 0xFFFF) * 2.0 ** -16) * (-1.0 if (h >> 16) & 1 else 1.0)
                h = _xorshift32(h)
                b[v, e] = (0.5 + (h & 0xFFFF) * 2.0 ** -17) * (-1.0 if (h >> 16) & 1 else 1.0)
        rne = lambda x: torch.from_numpy(x).to(torch.bfloat16).double().numpy()
        return rne(a), rne(b)
    a = np.zeros((8, 32), np.uint8)
    b = np.zeros((8, 32), np.uint8)
    code = lambda h: ((h >> 7) & 0x80) | ((5 + (h >> 3) % 5) << 3) | (h & 7)
    for v in range(8):
        for e in range(8):
            for byte in range(4):
                h = _xorshift32(h)
                a[v, 4 * e + byte] = code(h)
                h = _xorshift32(h)
                b[v, 4 * e + byte] = code(h)
    return a, b


def _rand_expected(iters, fp8):
    """Per-thread outputs of kinds 2 (bf16) and 3 (e4m3) for one workgroup,
    in float64: lane l supplies row/column l % 32 with k-elements of half
    l // 32 (the order inside a half is the same for A and B); chain c over
    the 8-step cycle sums A set (v + c) % 8 times B set (v + 3c) % 8."""
    kw = 32 if fp8 else 8
    out = np.zeros(256)
    for w in range(4):
        ops = [_rand_operands(64 * w + l, iters, fp8) for l in range(64)]
        if fp8:
            dec = lambda x: torch.from_numpy(x).view(torch.float8_e4m3fn).double().numpy()
            ops = [(dec(a), dec(b)) for a, b in ops]
        # A_v [32, 2*kw], B_v [2*kw, 32]
        A = np.zeros((8, 32, 2 * kw))
        Bm = np.zeros((8, 2 * kw, 32))
        for l in range(64):
            a, b = ops[l]
            A[:, l % 32, (l // 32) * kw:(l // 32 + 1) * kw] = a
            Bm[:, (l // 32) * kw:(l // 32 + 1) * kw, l % 32] = b
        D = np.zeros((32, 32))
        for c in range(4):
            for v in range(8):
                D += A[(v + c) % 8] @ Bm[(v + 3 * c) % 8]
        D *= iters // 8
        for l in range(64):
            rows = [(r // 4) * 8 + (l // 32) * 4 + r % 4 for r in range(16)]
            out[64 * w + l] = D[rows, l % 32].sum()
    return out


@pytest.mark.parametrize("kind,iters", [(2, 8), (2, 64), (3, 8), (3, 40)])
def test_mfma_probe_random_operands(kind, iters, gpu_device):
    """Kinds 2 and 3 (operands that change with every instruction) compute the
    products the header documents: equal, up to float32 summation order, to a
    float64 model built from the documented generator -- which also pins the
    32x32x64 e4m3 lane layout (each lane's 32 bytes are one half of the k
    range of its row or column)."""
    out = mla.mla_mfma_probe(iters, kind, device=gpu_device)
    torch.cuda.synchronize()
    got = out.double().cpu().numpy().reshape(512, 256)
    want = _rand_expected(iters, fp8=(kind == 3))
    scale = np.abs(want).max()
    for b in (0, 1, 511):
        err = np.abs(got[b] - want).max()
        assert err <= 1e-5 * scale + 1e-6, (kind, iters, err, scale)
    again = mla.mla_mfma_probe(iters, kind, out=torch.empty_like(out))
    torch.cuda.synchronize()
    assert torch.equal(out, again), "not deterministic"
