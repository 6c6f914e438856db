"""The C-ABI library without a GPU: it loads, exports every symbol that
include/mla.h declares, and rejects bad arguments with the documented status
codes before touching the device.

Pointers passed here are fake, aligned addresses that are never dereferenced:
every call below fails validation (which happens before any HIP call), so no
work is ever enqueued.
"""
import ctypes
import os
import re

import pytest

import transformer_attention_mla_amd as mla

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mla.h")

OK, NULL, DIM, ALIGN, ALIAS, WORKSPACE, SCALE, DEVICE, LAUNCH, FLAGS = range(10)
GB = 1 << 30


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_header_symbols_exported():
    names = declared_functions()
    assert {"mla_attend_prefill", "mla_attend_decode", "mla_out_proj"} <= set(names)
    lib = mla.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_mfma_probe_rejects_and_counts():
    L = mla.lib()
    assert mla.mla_mfma_probe_flops(1, 0) == 512 * 4 * 4 * 2 * 32 * 32 * 16
    assert mla.mla_mfma_probe_flops(1, 1) == 512 * 4 * 4 * 2 * 32 * 32 * 64
    assert mla.mla_mfma_probe_flops(1000, 0) == 1000 * mla.mla_mfma_probe_flops(1, 0)
    assert mla.mla_mfma_probe_flops(0, 0) == 0.0
    assert mla.mla_mfma_probe_flops((1 << 24) + 1, 0) == 0.0
    assert mla.mla_mfma_probe_flops(8, 2) == 8 * mla.mla_mfma_probe_flops(1, 0)
    assert mla.mla_mfma_probe_flops(8, 3) == 8 * mla.mla_mfma_probe_flops(1, 1)
    assert mla.mla_mfma_probe_flops(10, 2) == 0.0  # random-operand kinds: multiples of 8
    assert mla.mla_mfma_probe_flops(8, 4) == 0.0
    assert L.mla_mfma_probe(None, 10, 0, None) == NULL
    assert L.mla_mfma_probe(A[0], 0, 0, None) == DIM
    assert L.mla_mfma_probe(A[0], (1 << 24) + 1, 0, None) == DIM
    assert L.mla_mfma_probe(A[0], 10, -1, None) == DIM
    assert L.mla_mfma_probe(A[0], 10, 2, None) == DIM
    assert L.mla_mfma_probe(A[0], 12, 3, None) == DIM
    assert L.mla_mfma_probe(A[0], 16, 4, None) == DIM
    assert L.mla_mfma_probe(ctypes.c_void_p(16 * GB + 4), 10, 0, None) == ALIGN


def test_version_and_strings():
    assert mla.mla_abi_version() == 1
    for code in range(10):
        s = mla.mla_status_string(code)
        assert s.startswith("MLA_")
    assert mla.mla_status_string(99) == "unknown status"


def test_workspace_sizes():
    assert mla.mla_prefill_workspace_bytes(4, 64, 4096) == 4096 * 32 * 8 + 4 * 4096 * 64 * 2
    assert mla.mla_prefill_workspace_bytes(0, 64, 10) == 0
    assert mla.mla_decode_splits(64, 64, 8192, 0) == 1
    assert mla.mla_decode_workspace_bytes(64, 64, 8192, 0) == 0
    assert mla.mla_decode_splits(1, 1, 100, 7) == 7
    assert mla.mla_decode_splits(1, 1, 5, 64) == 5
    assert mla.mla_decode_workspace_bytes(2, 3, 100, 4) == 2 * 3 * 4 * 136 * 4
    s = mla.mla_decode_splits(1, 64, 8192, 0)
    assert s > 1 and mla.mla_decode_workspace_bytes(1, 64, 8192, 0) == 64 * s * 136 * 4
    # latent decode: bf16 absorbed queries + float32 latent outputs (+ split partials)
    assert mla.mla_decode_latent_workspace_bytes(1, 64, 100, 1) == 64 * 512 * 2 + 64 * 512 * 4
    assert mla.mla_decode_latent_workspace_bytes(64, 64, 8192, 0) == (
        64 * 64 * 512 * 6 + 64 * 64 * 4 * 520 * 4)  # 4 splits: one workgroup per compute unit
    assert mla.mla_decode_latent_workspace_bytes(1, 65, 100, 1) == 0      # > 64 heads
    assert mla.mla_decode_latent_workspace_bytes(1, 64, 1 << 21, 1) == 0  # L too long
    assert mla.mla_out_proj_workspace_bytes(16384, 8192, 7168) == 0
    assert mla.mla_out_proj_workspace_bytes(64, 8192, 7168) > 0
    assert mla.mla_out_proj_workspace_bytes(64, 100, 7168) == 0  # K not a multiple of 128


# Fake device addresses: 16-byte aligned, disjoint, 1 GiB apart.
A = [ctypes.c_void_p((i + 1) * 16 * GB) for i in range(12)]


def prefill(**kw):
    a = dict(q_nope=A[0], q_pe=A[1], k_nope=A[2], k_pe=A[3], v=A[4], R=A[5], r_rows=64,
             scale=0.07, B=1, H=2, T=64, ws=A[6], ws_bytes=1 << 20, out=A[7], lse=None,
             flags=0)
    a.update(kw)
    return mla.lib().mla_attend_prefill(a["q_nope"], a["q_pe"], a["k_nope"], a["k_pe"], a["v"],
                                        a["R"], a["r_rows"], a["scale"], a["B"], a["H"], a["T"],
                                        a["ws"], a["ws_bytes"], a["out"], a["lse"], a["flags"],
                                        None)


def decode(**kw):
    a = dict(q_nope=A[0], q_pe=A[1], kc=A[2], vc=A[3], R=A[4], r_rows=10, q_pos=9, scale=0.07,
             B=1, H=2, L=100, splits=1, ws=None, ws_bytes=0, out=A[5], lse=None, flags=0)
    a.update(kw)
    return mla.lib().mla_attend_decode(a["q_nope"], a["q_pe"], a["kc"], a["vc"], a["R"],
                                       a["r_rows"], a["q_pos"], a["scale"], a["B"], a["H"],
                                       a["L"], a["splits"], a["ws"], a["ws_bytes"], a["out"],
                                       a["lse"], a["flags"], None)


def decode_shared(**kw):
    a = dict(q_nope=A[0], q_pe=A[1], kn=A[2], kp=A[8], vc=A[3], R=A[4], r_rows=10, q_pos=9,
             scale=0.07, B=1, H=2, L=100, splits=1, ws=None, ws_bytes=0, out=A[5], lse=None,
             flags=0)
    a.update(kw)
    return mla.lib().mla_attend_decode_shared_kpe(
        a["q_nope"], a["q_pe"], a["kn"], a["kp"], a["vc"], a["R"], a["r_rows"], a["q_pos"],
        a["scale"], a["B"], a["H"], a["L"], a["splits"], a["ws"], a["ws_bytes"], a["out"],
        a["lse"], a["flags"], None)


def latent(**kw):
    a = dict(q_nope=A[0], q_pe=A[1], ckv=A[2], kpe=A[3], w=A[4], R=A[5], r_rows=10, q_pos=9,
             scale=0.07, B=1, H=2, L=100, splits=1, ws=A[6], ws_bytes=1 << 20, out=A[7], lse=None,
             flags=0)
    a.update(kw)
    return mla.lib().mla_attend_decode_latent(
        a["q_nope"], a["q_pe"], a["ckv"], a["kpe"], a["w"], a["R"], a["r_rows"], a["q_pos"],
        a["scale"], a["B"], a["H"], a["L"], a["splits"], a["ws"], a["ws_bytes"], a["out"], a["lse"],
        a["flags"], None)


def oproj(**kw):
    a = dict(x=A[0], w=A[1], y=A[2], M=16384, K=8192, N=7168, ws=None, ws_bytes=0, flags=0)
    a.update(kw)
    return mla.lib().mla_out_proj(a["x"], a["w"], a["y"], a["M"], a["K"], a["N"], a["ws"],
                                  a["ws_bytes"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q_nope=None), NULL), (dict(k_pe=None), NULL), (dict(R=None), NULL), (dict(out=None), NULL),
    (dict(flags=4), FLAGS), (dict(flags=6), FLAGS),
    (dict(B=0), DIM), (dict(H=-1), DIM), (dict(T=0), DIM), (dict(T=65), DIM), (dict(r_rows=0), DIM),
    (dict(scale=0.0), SCALE), (dict(scale=-1.0), SCALE), (dict(scale=float("nan")), SCALE),
    (dict(scale=float("inf")), SCALE),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE),
    (dict(q_pe=ctypes.c_void_p(2 * 16 * GB + 8)), ALIGN), (dict(lse=ctypes.c_void_p(12 * GB + 4)), ALIGN),
    (dict(out=ctypes.c_void_p(1 * 16 * GB + 4096)), ALIAS),     # out inside q_nope
    (dict(ws=A[7]), ALIAS),                                   # workspace == out
    (dict(lse=ctypes.c_void_p(7 * 16 * GB + 1024)), ALIAS),    # lse inside workspace
    # key-blocked v spans whole 16-key blocks: at T = 63 it reaches 256 B past the
    # [B, H, T, 128] extent, into `out`
    (dict(T=63, flags=2, v=ctypes.c_void_p(8 * 16 * GB - 2 * 63 * 256 - 256)), ALIAS),
])
def test_prefill_rejects(kw, code):
    assert prefill(**kw) == code


def prefill_noalloc(**kw):
    a = dict(q_nope=A[0], q_pe=A[1], k_nope=A[2], k_pe=A[3], v=A[4], R=A[5], r_rows=1 << 20,
             scale=0.07, B=1, H=2, T=64, out=A[7], lse=None, flags=0)
    a.update(kw)
    return mla.lib().mla_attend_prefill_noalloc(a["q_nope"], a["q_pe"], a["k_nope"], a["k_pe"],
                                                a["v"], a["R"], a["r_rows"], a["scale"], a["B"],
                                                a["H"], a["T"], a["out"], a["lse"], a["flags"], None)


# Every case fails validation: B * T beyond the static buffer (16 MiB holds
# T*256 + B*T*128 bytes) is MLA_ERR_WORKSPACE, before any device call.
@pytest.mark.parametrize("kw,code", [
    (dict(q_nope=None), NULL), (dict(out=None), NULL), (dict(flags=4), FLAGS),
    (dict(T=0), DIM), (dict(scale=0.0), SCALE),
    (dict(B=7, T=16384), WORKSPACE), (dict(B=1, T=65536), WORKSPACE),
    (dict(B=127, T=1024), WORKSPACE),
    (dict(q_pe=ctypes.c_void_p(2 * 16 * GB + 8)), ALIGN),
    (dict(out=ctypes.c_void_p(1 * 16 * GB + 4096)), ALIAS),
])
def test_prefill_noalloc_rejects(kw, code):
    assert prefill_noalloc(**kw) == code


def test_prefill_noalloc_limit_matches_workspace_formula():
    limit = 16 << 20
    assert mla.mla_prefill_workspace_bytes(6, 1, 16384) <= limit < mla.mla_prefill_workspace_bytes(7, 1, 16384)
    assert mla.mla_prefill_workspace_bytes(126, 1, 1024) <= limit < mla.mla_prefill_workspace_bytes(127, 1, 1024)


def test_prefill_workspace_value_tail():
    # T % 16 != 0: one zero-padded key-blocked value tile (8 KiB) per (b, h)
    base = lambda B, T: -(-T * 32 * 8 // 256) * 256 + -(-B * T * 64 * 2 // 256) * 256
    assert mla.mla_prefill_workspace_bytes(2, 3, 1008) == base(2, 1008)
    assert mla.mla_prefill_workspace_bytes(2, 3, 1000) == base(2, 1000) + 2 * 3 * 8192
    assert mla.mla_prefill_workspace_bytes(2, 3, 1001) == base(2, 1001) + 2 * 3 * 8192
    assert mla.mla_prefill_workspace_bytes(4, 64, 4095) == base(4, 4095) + 4 * 64 * 8192


@pytest.mark.parametrize("kw,code", [
    (dict(kc=None), NULL), (dict(out=None), NULL),
    (dict(flags=4), FLAGS),
    (dict(L=0), DIM), (dict(q_pos=10), DIM), (dict(q_pos=-1), DIM), (dict(splits=-1), DIM),
    (dict(scale=0.0), SCALE),
    (dict(splits=4), WORKSPACE), (dict(splits=4, ws=A[6], ws_bytes=100), WORKSPACE),
    (dict(vc=ctypes.c_void_p(4 * 16 * GB + 2)), ALIGN),
    (dict(out=ctypes.c_void_p(3 * 16 * GB + 256)), ALIAS),
    (dict(splits=4, ws=A[5], ws_bytes=1 << 20), ALIAS),
])
def test_decode_rejects(kw, code):
    assert decode(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(kp=None), NULL), (dict(kn=None), NULL),
    (dict(flags=4), FLAGS), (dict(L=0), DIM), (dict(q_pos=10), DIM), (dict(scale=0.0), SCALE),
    (dict(splits=4), WORKSPACE),
    (dict(kp=ctypes.c_void_p(9 * 16 * GB + 8)), ALIGN),
    (dict(out=ctypes.c_void_p(9 * 16 * GB + 256)), ALIAS),     # out inside kpe_cache
    (dict(out=ctypes.c_void_p(3 * 16 * GB + 51200 - 16)), ALIAS),  # end of the 128-wide key cache
])
def test_decode_shared_kpe_rejects(kw, code):
    assert decode_shared(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(q_nope=None), NULL), (dict(ckv=None), NULL), (dict(kpe=None), NULL), (dict(w=None), NULL),
    (dict(R=None), NULL), (dict(out=None), NULL),
    (dict(flags=2), FLAGS),
    (dict(L=0), DIM), (dict(H=65), DIM), (dict(L=1 << 21), DIM), (dict(q_pos=10), DIM),
    (dict(splits=-1), DIM),
    (dict(scale=0.0), SCALE),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=1000), WORKSPACE),
    (dict(w=ctypes.c_void_p(5 * 16 * GB + 8)), ALIGN),
    (dict(out=ctypes.c_void_p(5 * 16 * GB + 256)), ALIAS),   # out inside w_kv_b
    (dict(ws=A[2]), ALIAS),                                  # workspace over the latent cache
    (dict(lse=ctypes.c_void_p(7 * 16 * GB + 4096)), ALIAS),  # lse inside the workspace
])
def test_decode_latent_rejects(kw, code):
    assert latent(**kw) == code


def append(**kw):
    a = dict(kn=A[0], kp=A[1], v=A[2], R=A[3], r_rows=100, past=10, B=1, H=2, T=20, L=64,
             kc=A[4], pc=A[5], vc=A[6], flags=0)
    a.update(kw)
    return mla.lib().mla_append_kv(a["kn"], a["kp"], a["v"], a["R"], a["r_rows"], a["past"], a["B"],
                                   a["H"], a["T"], a["L"], a["kc"], a["pc"], a["vc"], a["flags"], None)


def chunk(**kw):
    a = dict(qn=A[0], qp=A[1], kc=A[2], pc=A[3], vc=A[4], R=A[5], r_rows=100, past=10, scale=0.07,
             B=1, H=2, T=20, L=64, ws=A[6], ws_bytes=1 << 20, out=A[7], lse=None, flags=0)
    a.update(kw)
    return mla.lib().mla_attend_prefill_chunk(
        a["qn"], a["qp"], a["kc"], a["pc"], a["vc"], a["R"], a["r_rows"], a["past"], a["scale"],
        a["B"], a["H"], a["T"], a["L"], a["ws"], a["ws_bytes"], a["out"], a["lse"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(kn=None), NULL), (dict(pc=None), NULL), (dict(flags=1), FLAGS),
    (dict(past=-1), DIM), (dict(past=45), DIM), (dict(r_rows=29), DIM), (dict(T=0), DIM),
    (dict(kc=ctypes.c_void_p(5 * 16 * GB + 8)), ALIGN),
    (dict(kc=ctypes.c_void_p(1 * 16 * GB + 64)), ALIAS),  # cache over k_nope
])
def test_append_rejects(kw, code):
    assert append(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(qn=None), NULL), (dict(vc=None), NULL), (dict(flags=2), FLAGS),
    (dict(past=-1), DIM), (dict(past=45), DIM), (dict(r_rows=29), DIM), (dict(H=64, L=1 << 18), DIM),
    (dict(scale=0.0), SCALE), (dict(ws=None), WORKSPACE), (dict(ws_bytes=100), WORKSPACE),
    (dict(out=ctypes.c_void_p(3 * 16 * GB + 32)), ALIAS),  # out over the cache
])
def test_prefill_chunk_rejects(kw, code):
    assert chunk(**kw) == code


def test_prefill_chunk_workspace():
    assert mla.mla_prefill_chunk_workspace_bytes(300) == 300 * 32 * 8 + 256 - (300 * 32 * 8) % 256 \
        if (300 * 32 * 8) % 256 else 300 * 32 * 8
    assert mla.mla_prefill_chunk_workspace_bytes(0) == 0


def oproj8(**kw):
    a = dict(x=A[0], w8=A[1], s=A[2], y=A[3], M=16384, K=8192, N=7168, ws=None, ws_bytes=0, flags=0)
    a.update(kw)
    return mla.lib().mla_out_proj_fp8(a["x"], a["w8"], a["s"], a["y"], a["M"], a["K"], a["N"],
                                      a["ws"], a["ws_bytes"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(w8=None), NULL), (dict(s=None), NULL), (dict(y=None), NULL),
    (dict(flags=8), FLAGS),
    (dict(M=0), DIM), (dict(K=100), DIM),
    (dict(M=64), WORKSPACE),
    (dict(M=1000, s=ctypes.c_void_p(3 * 16 * GB + 4)), ALIGN),
    (dict(M=1000, y=ctypes.c_void_p(3 * 16 * GB + 16)), ALIAS),  # y over the scales
    (dict(ws=A[4], ws_bytes=7168 * 8192 * 2 - 1), WORKSPACE),  # wide: room for the bf16 weight
    (dict(ws=ctypes.c_void_p(1 * 16 * GB + 64), ws_bytes=1 << 30), ALIAS),  # workspace over w8
])
def test_oproj_fp8_rejects(kw, code):
    assert oproj8(**kw) == code


def test_oproj_fp8_workspace():
    assert mla.mla_out_proj_fp8_workspace_bytes(64, 8192, 7168) > 0      # split K
    # enough 256 x 256 tiles: the bf16 weight is formed once in the workspace
    assert mla.mla_out_proj_fp8_workspace_bytes(16384, 8192, 7168) == 7168 * 8192 * 2
    assert mla.mla_out_proj_fp8_workspace_bytes(1000, 8192, 7168) == 0  # small-tile kernel, no split
    assert mla.mla_out_proj_fp8_workspace_bytes(64, 100, 7168) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(w=None), NULL), (dict(y=None), NULL),
    (dict(flags=8), FLAGS),
    (dict(M=0), DIM), (dict(N=0), DIM), (dict(K=100), DIM), (dict(K=0), DIM),
    (dict(M=64), WORKSPACE),
    (dict(y=ctypes.c_void_p(1 * 16 * GB + 8)), ALIGN),
    (dict(y=ctypes.c_void_p(2 * 16 * GB + 64)), ALIAS),
])
def test_oproj_rejects(kw, code):
    assert oproj(**kw) == code


def up(**kw):
    a = dict(ql=A[0], c=A[1], wq=A[2], wk=A[3], B=4, T=4096, H=64, qn=A[4], qp=A[5], kn=A[6], v=A[7],
             flags=0)
    a.update(kw)
    return mla.lib().mla_up_project(a["ql"], a["c"], a["wq"], a["wk"], a["B"], a["T"], a["H"], a["qn"],
                                    a["qp"], a["kn"], a["v"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(ql=None), NULL), (dict(wk=None), NULL), (dict(v=None), NULL), (dict(flags=4), FLAGS),
    (dict(B=0), DIM), (dict(T=-1), DIM), (dict(H=0), DIM), (dict(B=1 << 20, T=1 << 12), DIM),
    (dict(qp=ctypes.c_void_p(5 * 16 * GB + 8)), ALIGN),
    (dict(kn=ctypes.c_void_p(1 * 16 * GB + 64)), ALIAS),   # k_nope over q_lat
    (dict(v=ctypes.c_void_p(4 * 16 * GB + 256)), ALIAS),   # v over w_kv_b
    (dict(v=ctypes.c_void_p(5 * 16 * GB + 256)), ALIAS),   # v over q_nope
    # key-blocked v (whole 16-position blocks) at T = 4095 reaches into q_nope,
    # which the [B, H, T, 128] extent ends 4 KiB short of
    (dict(T=4095, flags=2, v=ctypes.c_void_p(5 * 16 * GB - 4 * 64 * 4095 * 256 - 4096)), ALIAS),
    (dict(flags=6), FLAGS),
])
def test_up_project_rejects(kw, code):
    assert up(**kw) == code


def oproj_fp8_dyn(**kw):
    a = dict(x=A[0], w8=A[1], ws=A[2], y=A[3], M=64, K=8192, N=7168, work=A[4], wbytes=1 << 30,
             flags=0)
    a.update(kw)
    return mla.lib().mla_out_proj_fp8_dyn(a["x"], a["w8"], a["ws"], a["y"], a["M"], a["K"], a["N"],
                                          a["work"], a["wbytes"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), NULL), (dict(ws=None), NULL), (dict(y=None), NULL), (dict(flags=4), FLAGS),
    (dict(M=0), DIM), (dict(K=100), DIM), (dict(K=1 << 24), DIM),
    (dict(work=None), WORKSPACE), (dict(wbytes=1000), WORKSPACE),
    (dict(y=ctypes.c_void_p(16 * GB + 64)), ALIAS), (dict(w8=ctypes.c_void_p(2 * 16 * GB + 1)), ALIGN),
])
def test_oproj_fp8_dyn_rejects(kw, code):
    assert oproj_fp8_dyn(**kw) == code


def test_act_quant_rejects_and_sizes():
    lib = mla.lib()
    assert lib.mla_act_quant(None, 4, 128, A[1], A[2], None) == NULL
    assert lib.mla_act_quant(A[0], 4, 100, A[1], A[2], None) == DIM
    assert lib.mla_act_quant(A[0], 0, 128, A[1], A[2], None) == DIM
    assert mla.mla_act_scale_stride(17) == 20 and mla.mla_act_scale_stride(64) == 64
    # x8 + transposed scales (+ partials when K is split for M <= 64)
    ws = mla.mla_out_proj_fp8_dyn_workspace_bytes(16384, 8192, 7168)
    assert ws == 16384 * 8192 + 64 * 16384 * 4
    assert mla.mla_out_proj_fp8_dyn_workspace_bytes(64, 8192, 7168) > 64 * 8192 + 64 * 64 * 4
    assert mla.mla_out_proj_fp8_dyn_workspace_bytes(64, 100, 7168) == 0


def prefill_fp8(**kw):
    a = dict(q_nope=A[0], q_pe=A[1], k_nope=A[2], k_pe=A[3], v=A[4], R=A[5], r_rows=64,
             scale=0.07, B=1, H=2, T=64, ws=A[6], ws_bytes=1 << 20, out8=A[7], sT=A[8], lse=None,
             flags=0)
    a.update(kw)
    return mla.lib().mla_attend_prefill_fp8(a["q_nope"], a["q_pe"], a["k_nope"], a["k_pe"], a["v"],
                                            a["R"], a["r_rows"], a["scale"], a["B"], a["H"], a["T"],
                                            a["ws"], a["ws_bytes"], a["out8"], a["sT"], a["lse"],
                                            a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(out8=None), NULL), (dict(sT=None), NULL), (dict(q_pe=None), NULL),
    (dict(flags=1), FLAGS),  # no float32 variant of an FP8 output
    (dict(flags=3), FLAGS), (dict(flags=4), FLAGS),
    (dict(T=0), DIM), (dict(T=65), DIM),  # T beyond the angle table
    (dict(scale=-1.0), SCALE),
    (dict(ws_bytes=100), WORKSPACE),
    (dict(out8=ctypes.c_void_p(8 * 16 * GB + 4)), ALIGN),
    (dict(sT=ctypes.c_void_p(9 * 16 * GB + 8)), ALIGN),
    (dict(sT=ctypes.c_void_p(1 * 16 * GB + 64)), ALIAS),  # scales over q_nope
    (dict(sT=ctypes.c_void_p(8 * 16 * GB + 1024)), ALIAS),  # scales over the codes
    (dict(lse=ctypes.c_void_p(9 * 16 * GB)), ALIAS),  # lse over the scales
])
def test_prefill_fp8_rejects(kw, code):
    assert prefill_fp8(**kw) == code


def oproj8q(**kw):
    a = dict(x8=A[0], xs=A[1], w8=A[2], s=A[3], y=A[4], M=16384, K=8192, N=7168, ws=None, ws_bytes=0,
             flags=0)
    a.update(kw)
    return mla.lib().mla_out_proj_fp8_q(a["x8"], a["xs"], a["w8"], a["s"], a["y"], a["M"], a["K"],
                                        a["N"], a["ws"], a["ws_bytes"], a["flags"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x8=None), NULL), (dict(xs=None), NULL), (dict(w8=None), NULL), (dict(y=None), NULL),
    (dict(flags=2), FLAGS),
    (dict(M=0), DIM), (dict(K=100), DIM),
    (dict(M=64), WORKSPACE),  # K split: float32 partials
    (dict(x8=ctypes.c_void_p(1 * 16 * GB + 4)), ALIGN),
    (dict(y=ctypes.c_void_p(3 * 16 * GB + 16)), ALIAS),  # y over w8
    (dict(y=ctypes.c_void_p(2 * 16 * GB)), ALIAS),  # y over the activation scales
])
def test_oproj_fp8_q_rejects(kw, code):
    assert oproj8q(**kw) == code


def test_oproj_fp8_q_workspace():
    assert mla.mla_out_proj_fp8_q_workspace_bytes(16384, 8192, 7168) == 0
    # 4 K splits at M = 64: float32 partials only (no room for codes or scales)
    assert mla.mla_out_proj_fp8_q_workspace_bytes(64, 8192, 7168) == 4 * 64 * 7168 * 4
    assert mla.mla_out_proj_fp8_q_workspace_bytes(64, 100, 7168) == 0


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback: without the built library every entry point raises."""
    monkeypatch.setattr(mla, "_lib", None)
    monkeypatch.setattr(mla, "LIB_PATH", "/nonexistent/libmla.so")
    with pytest.raises(RuntimeError, match="missing"):
        mla.lib()
    with pytest.raises(RuntimeError, match="missing"):
        mla.mla_prefill_workspace_bytes(1, 1, 1)
