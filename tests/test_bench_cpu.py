"""bench.py's host-side figures (no GPU): the algorithmic units match the
workload table they are quoted against, and every measured-traffic entry
names a committed profile that records the same kernel-source hash."""
import os

import bench

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_units():
    # causal prefill: 2*(128+64+128)*T(T+1)/2*B*H flop
    assert bench.prefill_flops(4, 64, 4096) == 2 * 320 * 4096 * 4097 // 2 * 4 * 64
    assert abs(bench.prefill_flops(4, 64, 4096) - 1.3747e12) < 1e8
    assert abs(bench.prefill_flops(1, 64, 16384) - 5.4979e12) < 1e8
    # decode: every cached key (192 wide) and value (128 wide) once, plus q in and out
    kv = 64 * 64 * 8192 * (192 + 128) * 2
    assert kv == 21_474_836_480
    assert bench.decode_bytes(64, 64, 8192) == kv + 64 * 64 * (192 + 128) * 2
    # o_proj: 2*M*K*N flop; W, x and y bytes
    assert bench.oproj_flops(16384, 8192, 7168) == 2 * 16384 * 8192 * 7168
    assert bench.oproj_bytes(64, 8192, 7168) == (64 * 8192 + 7168 * 8192 + 64 * 7168) * 2


def test_measured_traffic_entries_match_their_profiles():
    for name, (digest, files, nbytes, profile) in bench.MEASURED_TRAFFIC.items():
        path = os.path.join(REPO, profile)
        assert os.path.exists(path), (name, profile)
        text = open(path).read()
        assert digest in text, f"{name}: {profile} does not record source hash {digest}"
        assert nbytes > 0
        for f in files:
            assert os.path.exists(os.path.join(bench.CSRC, f)), f
