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
