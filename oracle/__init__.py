"""Python front end of the fp64 CPU oracle (``oracle/mla_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, by the smoke check in
``__graft_entry__`` and by the CPU-baseline leg of ``bench.py``; never by the
product package, which must fail rather than fall back to it.  It shares no
code with the HIP library.

Arrays cross the boundary as numpy arrays: bf16 tensors as their ``uint16``
bit patterns (widened exactly inside the oracle), angle tables as float32,
results as float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: no fast-math and no contraction into FMA,
    so every double operation is the one written in the source."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wno-unused-function", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_bf16_round.argtypes = [D]
    lib.oracle_bf16_round.restype = D
    lib.oracle_bf16_round_array.argtypes = [P, P, ctypes.c_size_t]
    lib.oracle_bf16_widen_array.argtypes = [P, P, ctypes.c_size_t]
    lib.oracle_dims.argtypes = [P, P, P]
    lib.oracle_rope_rotate.argtypes = [P, P, I, P, I, P, P]
    lib.oracle_rope_rotate.restype = I
    lib.oracle_prefill.argtypes = [P, P, P, P, P, P, I, D, I, I, I, P, P, I]
    lib.oracle_prefill.restype = I
    lib.oracle_prefill_rows.argtypes = [P, P, P, P, P, P, I, D, I, I, I, I, P, P, P, I]
    lib.oracle_prefill_rows.restype = I
    lib.oracle_decode.argtypes = [P, P, P, P, P, I, I, D, I, I, I, P, P, I]
    lib.oracle_decode.restype = I
    lib.oracle_decode_rows.argtypes = [P, P, P, P, P, I, I, D, I, I, I, I, P, P, P, I]
    lib.oracle_decode_rows.restype = I
    lib.oracle_decode_shared_kpe.argtypes = [P, P, P, P, P, P, I, I, D, I, I, I, P, P, I]
    lib.oracle_decode_shared_kpe.restype = I
    lib.oracle_decode_shared_kpe_rows.argtypes = [P, P, P, P, P, P, I, I, D, I, I, I, I, P, P, P,
                                                  I]
    lib.oracle_decode_shared_kpe_rows.restype = I
    lib.oracle_decode_latent.argtypes = [P, P, P, P, P, P, I, I, D, I, I, I, I, P, I, P, P, I]
    lib.oracle_decode_latent.restype = I
    lib.oracle_e4m3_to_double_array.argtypes = [P, P, ctypes.c_size_t]
    lib.oracle_dequant_fp8.argtypes = [P, P, I, I, P]
    lib.oracle_dequant_fp8.restype = I
    lib.oracle_e4m3_from_float_array.argtypes = [P, P, ctypes.c_size_t]
    lib.oracle_act_quant.argtypes = [P, I, I, P, P]
    lib.oracle_act_quant.restype = I
    lib.oracle_out_proj_fp8_dyn.argtypes = [P, P, P, I, I, I, P, I]
    lib.oracle_out_proj_fp8_dyn.restype = I
    lib.oracle_append_kv.argtypes = [P, P, P, P, I, I, I, I, I, I, P, P, P]
    lib.oracle_append_kv.restype = I
    lib.oracle_prefill_chunk.argtypes = [P, P, P, P, P, P, I, I, D, I, I, I, I, P, P, I]
    lib.oracle_prefill_chunk.restype = I
    lib.oracle_prefill_chunk_rows.argtypes = [P, P, P, P, P, P, I, I, D, I, I, I, I, I, P, P, P, I]
    lib.oracle_prefill_chunk_rows.restype = I
    lib.oracle_up_project.argtypes = [P, P, P, P, I, I, I, I, P, P, P, P, P, I]
    lib.oracle_up_project.restype = I
    lib.oracle_out_proj.argtypes = [P, P, I, I, I, P, I]
    lib.oracle_out_proj.restype = I
    lib.oracle_out_proj_rows.argtypes = [P, P, I, I, I, I, P, P, I]
    lib.oracle_out_proj_rows.restype = I
    _lib = lib
    return lib


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns as uint16, got {a.dtype}")
    return a


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def dims():
    lib = _load()
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    lib.oracle_dims(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return a.value, b.value, c.value


def bf16_round(x) -> np.ndarray:
    """Round doubles to the nearest bf16 value (ties to even), returned as doubles."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    lib.oracle_bf16_round_array(_p(x), _p(y), x.size)
    return y


def bf16_widen(bits) -> np.ndarray:
    lib = _load()
    bits = _u16(bits)
    y = np.empty(bits.shape, dtype=np.float64)
    lib.oracle_bf16_widen_array(_p(bits), _p(y), bits.size)
    return y


def rope_rotate(x_bits, R, pos):
    """Rotate rows of 64 bf16 values (shape [..., 64]) at positions ``pos``
    (shape [...]).  Returns (double result before rounding, bf16 bits after)."""
    lib = _load()
    x_bits = _u16(x_bits)
    R = _f32(R)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    n = pos.size
    if x_bits.size != n * 64:
        raise ValueError("x must hold 64 values per position")
    f64 = np.empty(x_bits.shape, dtype=np.float64)
    b16 = np.empty(x_bits.shape, dtype=np.uint16)
    rc = lib.oracle_rope_rotate(_p(x_bits), _p(R), R.shape[0], _p(pos), n, _p(f64), _p(b16))
    if rc:
        raise ValueError("position outside the angle table")
    return f64, b16


def prefill(q_nope, q_pe, k_nope, k_pe, v, R, scale, nthreads=None, want_lse=True):
    """Full causal prefill.  Shapes: q_nope/k_nope/v [B,H,T,128], q_pe
    [B,H,T,64], k_pe [B,1,T,64], R [>=T,32].  Returns out [B,T,H*128] (double)
    and lse [B,H,T] (or None)."""
    lib = _load()
    q_nope, q_pe, k_nope, k_pe, v = map(_u16, (q_nope, q_pe, k_nope, k_pe, v))
    R = _f32(R)
    B, H, T, _ = q_nope.shape
    _check_prefill_shapes(q_nope, q_pe, k_nope, k_pe, v, B, H, T)
    out = np.empty((B, T, H * 128), dtype=np.float64)
    lse = np.empty((B, H, T), dtype=np.float64) if want_lse else None
    rc = lib.oracle_prefill(_p(q_nope), _p(q_pe), _p(k_nope), _p(k_pe), _p(v), _p(R), R.shape[0],
                            float(scale), B, H, T, _p(out), _p(lse) if want_lse else None,
                            nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_prefill failed ({rc})")
    return out, lse


def prefill_rows(q_nope, q_pe, k_nope, k_pe, v, R, scale, sel, nthreads=None):
    """Selected rows: ``sel`` is an int array [n,3] of (b, h, t).  Returns
    out [n,128] and lse [n]."""
    lib = _load()
    q_nope, q_pe, k_nope, k_pe, v = map(_u16, (q_nope, q_pe, k_nope, k_pe, v))
    R = _f32(R)
    B, H, T, _ = q_nope.shape
    _check_prefill_shapes(q_nope, q_pe, k_nope, k_pe, v, B, H, T)
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 3)
    n = sel.shape[0]
    out = np.empty((n, 128), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_prefill_rows(_p(q_nope), _p(q_pe), _p(k_nope), _p(k_pe), _p(v), _p(R),
                                 R.shape[0], float(scale), B, H, T, n, _p(sel), _p(out), _p(lse),
                                 nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_prefill_rows failed ({rc})")
    return out, lse


def decode(q_nope, q_pe, k_cache, v_cache, R, q_pos, scale, nthreads=None):
    """Decode one query per (b, h) over L cached, already rotated keys.
    Shapes: q_nope [B,H,128], q_pe [B,H,64], k_cache [B,H,L,192], v_cache
    [B,H,L,128].  Returns out [B,H*128] and lse [B,H]."""
    lib = _load()
    q_nope, q_pe, k_cache, v_cache = map(_u16, (q_nope, q_pe, k_cache, v_cache))
    R = _f32(R)
    B, H, L, _ = k_cache.shape
    _check_decode_shapes(q_nope, q_pe, k_cache, v_cache, B, H, L)
    out = np.empty((B, H * 128), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    rc = lib.oracle_decode(_p(q_nope), _p(q_pe), _p(k_cache), _p(v_cache), _p(R), R.shape[0],
                           int(q_pos), float(scale), B, H, L, _p(out), _p(lse),
                           nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_decode failed ({rc})")
    return out, lse


def decode_rows(q_nope, q_pe, k_cache, v_cache, R, q_pos, scale, sel, nthreads=None):
    lib = _load()
    q_nope, q_pe, k_cache, v_cache = map(_u16, (q_nope, q_pe, k_cache, v_cache))
    R = _f32(R)
    B, H, L, _ = k_cache.shape
    _check_decode_shapes(q_nope, q_pe, k_cache, v_cache, B, H, L)
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 2)
    n = sel.shape[0]
    out = np.empty((n, 128), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_decode_rows(_p(q_nope), _p(q_pe), _p(k_cache), _p(v_cache), _p(R),
                                R.shape[0], int(q_pos), float(scale), B, H, L, n, _p(sel),
                                _p(out), _p(lse), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_decode_rows failed ({rc})")
    return out, lse


def _check_shared_kpe_shapes(q_nope, q_pe, k_nope_cache, kpe_cache, v_cache):
    B, H, L, dn = k_nope_cache.shape
    if dn != 128 or q_nope.shape != (B, H, 128) or q_pe.shape != (B, H, 64):
        raise ValueError("k_nope_cache must be [B,H,L,128], q_nope [B,H,128], q_pe [B,H,64]")
    if kpe_cache.shape != (B, L, 64) or v_cache.shape != (B, H, L, 128):
        raise ValueError("kpe_cache must be [B,L,64] and v_cache [B,H,L,128]")
    return B, H, L


def decode_shared_kpe(q_nope, q_pe, k_nope_cache, kpe_cache, v_cache, R, q_pos, scale,
                      nthreads=None):
    """Decode against the shared-rotary cache layout: k_nope_cache [B,H,L,128],
    kpe_cache [B,L,64] (rotated keys, one per position for every head), v_cache
    [B,H,L,128].  Returns out [B,H*128] and lse [B,H]."""
    lib = _load()
    q_nope, q_pe, k_nope_cache, kpe_cache, v_cache = map(
        _u16, (q_nope, q_pe, k_nope_cache, kpe_cache, v_cache))
    R = _f32(R)
    B, H, L = _check_shared_kpe_shapes(q_nope, q_pe, k_nope_cache, kpe_cache, v_cache)
    out = np.empty((B, H * 128), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    rc = lib.oracle_decode_shared_kpe(_p(q_nope), _p(q_pe), _p(k_nope_cache), _p(kpe_cache),
                                      _p(v_cache), _p(R), R.shape[0], int(q_pos), float(scale),
                                      B, H, L, _p(out), _p(lse), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_decode_shared_kpe failed ({rc})")
    return out, lse


def decode_shared_kpe_rows(q_nope, q_pe, k_nope_cache, kpe_cache, v_cache, R, q_pos, scale, sel,
                           nthreads=None):
    """As decode_shared_kpe for selected (b, h) pairs ``sel`` [n,2]: out [n,128], lse [n]."""
    lib = _load()
    q_nope, q_pe, k_nope_cache, kpe_cache, v_cache = map(
        _u16, (q_nope, q_pe, k_nope_cache, kpe_cache, v_cache))
    R = _f32(R)
    B, H, L = _check_shared_kpe_shapes(q_nope, q_pe, k_nope_cache, kpe_cache, v_cache)
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 2)
    n = sel.shape[0]
    out = np.empty((n, 128), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_decode_shared_kpe_rows(_p(q_nope), _p(q_pe), _p(k_nope_cache), _p(kpe_cache),
                                           _p(v_cache), _p(R), R.shape[0], int(q_pos),
                                           float(scale), B, H, L, n, _p(sel), _p(out), _p(lse),
                                           nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_decode_shared_kpe_rows failed ({rc})")
    return out, lse


def _check_latent_shapes(q_nope, q_pe, ckv, kpe, w_kv_b):
    B, L, r = ckv.shape
    if r != 512 or q_nope.ndim != 3 or q_nope.shape[0] != B or q_nope.shape[2] != 128:
        raise ValueError("ckv must be [B,L,512] and q_nope [B,H,128]")
    H = q_nope.shape[1]
    if q_pe.shape != (B, H, 64) or kpe.shape != (B, L, 64) or w_kv_b.shape != (H * 256, 512):
        raise ValueError("q_pe must be [B,H,64], kpe [B,L,64], w_kv_b [H*256,512]")
    return B, H, L


def decode_latent(q_nope, q_pe, ckv, kpe, w_kv_b, R, q_pos, scale, sel=None, round_kv=True,
                  nthreads=None):
    """Decode against a latent cache: ckv [B,L,512] (the cached latent), kpe
    [B,L,64] (rotated rope keys, one per position for every head), w_kv_b
    [H*256,512] (the up-projection, rows h*256.. nope key, h*256+128.. value).
    Every (b, h): out [B,H*128], lse [B,H]; with ``sel`` [n,2] (b, h) pairs:
    out [n,128], lse [n].  ``round_kv=False`` keeps the up-projected keys and
    values unrounded."""
    lib = _load()
    q_nope, q_pe, ckv, kpe, w_kv_b = map(_u16, (q_nope, q_pe, ckv, kpe, w_kv_b))
    R = _f32(R)
    B, H, L = _check_latent_shapes(q_nope, q_pe, ckv, kpe, w_kv_b)
    if sel is None:
        n, psel = 0, None
        out = np.empty((B, H * 128), dtype=np.float64)
        lse = np.empty((B, H), dtype=np.float64)
    else:
        sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 2)
        n, psel = sel.shape[0], _p(sel)
        out = np.empty((n, 128), dtype=np.float64)
        lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_decode_latent(_p(q_nope), _p(q_pe), _p(ckv), _p(kpe), _p(w_kv_b), _p(R),
                                  R.shape[0], int(q_pos), float(scale), B, H, L, n, psel,
                                  1 if round_kv else 0, _p(out), _p(lse),
                                  nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_decode_latent failed ({rc})")
    return out, lse


def up_project(q_lat, ckv, w_q_b, w_kv_b, rows=None, nthreads=None):
    """The MLA up-projection: q_lat [B,T,1536] and ckv [B,T,512] (bf16 bits),
    w_q_b [H*192,1536] (rows h*192.. q_nope, h*192+128.. q_pe of head h) and
    w_kv_b [H*256,512] (rows h*256.. nope key, h*256+128.. value).  Returns
    (q_nope, q_pe, k_nope, v) in double, unrounded: [B,H,T,d] each, or with
    ``rows`` (flat indices b*T + t) [n,H,d]."""
    lib = _load()
    q_lat, ckv, w_q_b, w_kv_b = map(_u16, (q_lat, ckv, w_q_b, w_kv_b))
    if q_lat.ndim != 3 or q_lat.shape[2] != 1536 or ckv.shape != q_lat.shape[:2] + (512,):
        raise ValueError("q_lat must be [B,T,1536] and ckv [B,T,512]")
    B, T, _ = q_lat.shape
    H = w_q_b.shape[0] // 192
    if w_q_b.shape != (H * 192, 1536) or w_kv_b.shape != (H * 256, 512) or H < 1:
        raise ValueError("w_q_b must be [H*192,1536] and w_kv_b [H*256,512]")
    if rows is None:
        n, prow = 0, None
        lead = (B, H, T)
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int32).ravel()
        n, prow = rows.size, _p(rows)
        lead = (n, H)
    outs = [np.empty(lead + (d,), dtype=np.float64) for d in (128, 64, 128, 128)]
    rc = lib.oracle_up_project(_p(q_lat), _p(ckv), _p(w_q_b), _p(w_kv_b), B, T, H, n, prow,
                               *[_p(o) for o in outs], nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_up_project failed ({rc})")
    return tuple(outs)


def e4m3_to_double(b):
    """Exact values of e4m3 ("fn") bytes; NaN for the NaN codes."""
    lib = _load()
    b = np.ascontiguousarray(b, dtype=np.uint8)
    out = np.empty(b.shape, dtype=np.float64)
    lib.oracle_e4m3_to_double_array(_p(b), _p(out), b.size)
    return out


def dequant_fp8(w8, scale):
    """bf16 bits [N,K] of the dequantized weight: float32(e4m3 value x block
    scale), rounded to bf16; w8 [N,K] uint8, scale [ceil(N/128), ceil(K/128)]."""
    lib = _load()
    w8 = np.ascontiguousarray(w8, dtype=np.uint8)
    scale = _f32(scale)
    N, K = w8.shape
    if scale.shape != ((N + 127) // 128, (K + 127) // 128):
        raise ValueError("scale must be [ceil(N/128), ceil(K/128)]")
    out = np.empty((N, K), dtype=np.uint16)
    if lib.oracle_dequant_fp8(_p(w8), _p(scale), N, K, _p(out)):
        raise ValueError("oracle_dequant_fp8 failed")
    return out


def e4m3_from_float(v):
    """e4m3 ("fn") codes of float32 values, round to nearest even; values that
    round above 448 (and NaN) give NaN codes."""
    lib = _load()
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib.oracle_e4m3_from_float_array(_p(v), _p(out), v.size)
    return out


def act_quant(x):
    """Dynamic activation quantization of x [M,K] (bf16 bits): per row and
    128-column block, scale = max(amax, 1e-4) / 448 in float32 and codes
    e4m3(x / scale).  Returns (q uint8 [M,K], scale float32 [M,ceil(K/128)])."""
    lib = _load()
    x = _u16(x)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, (K + 127) // 128), dtype=np.float32)
    if lib.oracle_act_quant(_p(x), M, K, _p(q), _p(s)):
        raise ValueError("oracle_act_quant failed")
    return q, s


def out_proj_fp8_dyn(x, w8, scale, nthreads=None):
    """y = dequant(act_quant(x)) · dequant(w8, scale)ᵀ in double: the
    projection with FP8 activations (dynamic 1 x 128 scales) and the FP8
    checkpoint weight (128 x 128 block scales).  x [M,K] bf16 bits, w8 [N,K]
    uint8, scale [ceil(N/128), ceil(K/128)] float32; returns y [M,N] double."""
    lib = _load()
    x = _u16(x)
    w8 = np.ascontiguousarray(w8, dtype=np.uint8)
    scale = _f32(scale)
    M, K = x.shape
    N = w8.shape[0]
    if w8.shape != (N, K) or scale.shape != ((N + 127) // 128, (K + 127) // 128):
        raise ValueError("out_proj_fp8_dyn shapes")
    y = np.empty((M, N), dtype=np.float64)
    if lib.oracle_out_proj_fp8_dyn(_p(x), _p(w8), _p(scale), M, K, N, _p(y),
                                   nthreads or default_threads()):
        raise ValueError("oracle_out_proj_fp8_dyn failed")
    return y


def out_proj_fp8(x, w8, scale, nthreads=None):
    """y = x · dequant(w8, scale)ᵀ: the projection with the FP8 checkpoint
    weight, dequantized to bf16 first; returns y [M,N] double."""
    return out_proj(x, dequant_fp8(w8, scale), nthreads)


def out_proj_fp8_rows(x, w8, scale, rows, nthreads=None):
    return out_proj_rows(x, dequant_fp8(w8, scale), rows, nthreads)


def append_kv(k_nope, k_pe, v, R, past, k_nope_cache, kpe_cache, v_cache):
    """Write a chunk's keys and values into the shared-rotary cache layout at
    rows past .. past+T-1 (rope key rotated at its position, bf16).  k_nope
    [B,H,T,128], k_pe [B,1,T,64] or [B,T,64], v [B,H,T,128]; the caches
    (k_nope_cache [B,H,Lc,128], kpe_cache [B,Lc,64], v_cache [B,H,Lc,128]) are
    uint16 arrays updated in place."""
    lib = _load()
    k_nope, v = _u16(k_nope), _u16(v)
    k_pe = _u16(k_pe).reshape(k_nope.shape[0], -1, 64)
    R = _f32(R)
    B, H, T, _ = k_nope.shape
    Lc = k_nope_cache.shape[2]
    for a in (k_nope_cache, kpe_cache, v_cache):
        if a.dtype != np.uint16 or not a.flags["C_CONTIGUOUS"]:
            raise ValueError("caches must be contiguous uint16 arrays")
    if k_nope_cache.shape != (B, H, Lc, 128) or kpe_cache.shape != (B, Lc, 64) or \
            v_cache.shape != (B, H, Lc, 128) or k_pe.shape != (B, T, 64) or v.shape != (B, H, T, 128):
        raise ValueError("append_kv shapes")
    if lib.oracle_append_kv(_p(k_nope), _p(k_pe), _p(v), _p(R), R.shape[0], int(past), B, H, T, Lc,
                            _p(k_nope_cache), _p(kpe_cache), _p(v_cache)):
        raise ValueError("oracle_append_kv failed")


def prefill_chunk(q_nope, q_pe, k_nope_cache, kpe_cache, v_cache, R, past, scale, nthreads=None):
    """Chunked prefill: queries [B,H,T,·] at positions past .. past+T-1 against
    cache rows 0 .. past+t.  Returns out [B,T,H*128] and lse [B,H,T]."""
    lib = _load()
    q_nope, q_pe, k_nope_cache, kpe_cache, v_cache = map(
        _u16, (q_nope, q_pe, k_nope_cache, kpe_cache, v_cache))
    R = _f32(R)
    B, H, T, _ = q_nope.shape
    Lc = k_nope_cache.shape[2]
    if q_pe.shape != (B, H, T, 64) or k_nope_cache.shape != (B, H, Lc, 128) or \
            kpe_cache.shape != (B, Lc, 64) or v_cache.shape != (B, H, Lc, 128):
        raise ValueError("prefill_chunk shapes")
    out = np.empty((B, T, H * 128), dtype=np.float64)
    lse = np.empty((B, H, T), dtype=np.float64)
    rc = lib.oracle_prefill_chunk(_p(q_nope), _p(q_pe), _p(k_nope_cache), _p(kpe_cache),
                                  _p(v_cache), _p(R), R.shape[0], int(past), float(scale), B, H, T,
                                  Lc, _p(out), _p(lse), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_prefill_chunk failed ({rc})")
    return out, lse


def prefill_chunk_rows(q_nope, q_pe, k_nope_cache, kpe_cache, v_cache, R, past, scale, sel,
                       nthreads=None):
    """Selected rows of the chunked prefill: ``sel`` is an int array [n,3] of
    (b, h, t); query t sits at position past + t and sees cache rows
    0 .. past + t.  Returns out [n,128] and lse [n]."""
    lib = _load()
    q_nope, q_pe, k_nope_cache, kpe_cache, v_cache = map(
        _u16, (q_nope, q_pe, k_nope_cache, kpe_cache, v_cache))
    R = _f32(R)
    B, H, T, _ = q_nope.shape
    Lc = k_nope_cache.shape[2]
    if q_pe.shape != (B, H, T, 64) or k_nope_cache.shape != (B, H, Lc, 128) or \
            kpe_cache.shape != (B, Lc, 64) or v_cache.shape != (B, H, Lc, 128):
        raise ValueError("prefill_chunk_rows shapes")
    sel = np.ascontiguousarray(sel, dtype=np.int32).reshape(-1, 3)
    n = sel.shape[0]
    out = np.empty((n, 128), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib.oracle_prefill_chunk_rows(_p(q_nope), _p(q_pe), _p(k_nope_cache), _p(kpe_cache),
                                       _p(v_cache), _p(R), R.shape[0], int(past), float(scale), B,
                                       H, T, Lc, n, _p(sel), _p(out), _p(lse),
                                       nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_prefill_chunk_rows failed ({rc})")
    return out, lse


def out_proj(x, w, nthreads=None):
    """y = x · wᵀ with x [M,K] and w [N,K] (bf16 bits); returns y [M,N] double."""
    lib = _load()
    x, w = _u16(x), _u16(w)
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("inner sizes differ")
    y = np.empty((M, N), dtype=np.float64)
    rc = lib.oracle_out_proj(_p(x), _p(w), M, K, N, _p(y), nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_out_proj failed ({rc})")
    return y


def out_proj_rows(x, w, rows, nthreads=None):
    lib = _load()
    x, w = _u16(x), _u16(w)
    M, K = x.shape
    N, K2 = w.shape
    if K != K2:
        raise ValueError("inner sizes differ")
    rows = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1)
    y = np.empty((rows.size, N), dtype=np.float64)
    rc = lib.oracle_out_proj_rows(_p(x), _p(w), M, K, N, rows.size, _p(rows), _p(y),
                                  nthreads or default_threads())
    if rc:
        raise ValueError(f"oracle_out_proj_rows failed ({rc})")
    return y


def _check_prefill_shapes(q_nope, q_pe, k_nope, k_pe, v, B, H, T):
    want = {"q_nope": (B, H, T, 128), "q_pe": (B, H, T, 64), "k_nope": (B, H, T, 128),
            "k_pe": (B, 1, T, 64), "v": (B, H, T, 128)}
    for name, arr in zip(want, (q_nope, q_pe, k_nope, k_pe, v)):
        if tuple(arr.shape) != want[name]:
            raise ValueError(f"{name} has shape {arr.shape}, expected {want[name]}")


def _check_decode_shapes(q_nope, q_pe, k_cache, v_cache, B, H, L):
    want = {"q_nope": (B, H, 128), "q_pe": (B, H, 64), "k_cache": (B, H, L, 192),
            "v_cache": (B, H, L, 128)}
    for name, arr in zip(want, (q_nope, q_pe, k_cache, v_cache)):
        if tuple(arr.shape) != want[name]:
            raise ValueError(f"{name} has shape {arr.shape}, expected {want[name]}")
