"""Python binding of ``libmla.so``: Kimi K2 latent-attention (MLA)
attend-and-combine on MI355X (gfx950).

The functions carry the C-ABI names (see ``include/mla.h``) and only marshal
arguments: they check torch tensors (device, dtype, layout, shapes), allocate
outputs and workspaces through torch when the caller passes none, hand raw
device pointers and the current HIP stream to the library, and raise
``MlaError`` (a ``ValueError``) on a nonzero status.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "MLA_OUT_F32", "MlaError", "lib", "mla_abi_version", "mla_status_string",
    "mla_prefill_workspace_bytes", "mla_attend_prefill", "mla_decode_splits",
    "mla_decode_workspace_bytes", "mla_attend_decode", "mla_attend_decode_shared_kpe",
    "mla_decode_latent_workspace_bytes", "mla_attend_decode_latent",
    "mla_append_kv", "mla_prefill_chunk_workspace_bytes", "mla_attend_prefill_chunk",
    "mla_out_proj_workspace_bytes", "mla_out_proj_fp8_workspace_bytes", "mla_out_proj_fp8",
    "mla_out_proj", "mla_up_project", "NOPE", "ROPE", "VDIM", "PAIRS", "LATENT", "Q_RANK",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")

MLA_OUT_F32 = 0x1
MLA_V_BLOCKED = 0x2  # v key-blocked: [B, H, ceil(T/16), 128, 16]
NOPE, ROPE, VDIM, PAIRS = 128, 64, 128, 32
LATENT = 512  # kv_lora_rank
Q_RANK = 1536  # q_lora_rank

_lib = None


class MlaError(ValueError):
    """A nonzero status from the library (mirrors the pages' ValueError on bad shapes)."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mla_status_string(status)}")


def lib():
    """The loaded ``libmla.so`` with ctypes signatures.  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m transformer_attention_mla_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, U, Z, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32, ctypes.c_size_t, ctypes.c_float
    L.mla_abi_version.argtypes = []
    L.mla_abi_version.restype = I
    L.mla_status_string.argtypes = [I]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_prefill_workspace_bytes.argtypes = [I, I, I]
    L.mla_prefill_workspace_bytes.restype = Z
    L.mla_attend_prefill.argtypes = [P, P, P, P, P, P, I, F, I, I, I, P, Z, P, P, U, P]
    L.mla_attend_prefill_noalloc.argtypes = [P, P, P, P, P, P, I, F, I, I, I, P, P, U, P]
    L.mla_attend_prefill_noalloc.restype = I
    L.mla_attend_prefill.restype = I
    L.mla_append_kv.argtypes = [P, P, P, P, I, I, I, I, I, I, P, P, P, U, P]
    L.mla_append_kv.restype = I
    L.mla_prefill_chunk_workspace_bytes.argtypes = [I]
    L.mla_prefill_chunk_workspace_bytes.restype = Z
    L.mla_attend_prefill_chunk.argtypes = [P, P, P, P, P, P, I, I, F, I, I, I, I, P, Z, P, P, U, P]
    L.mla_attend_prefill_chunk.restype = I
    L.mla_decode_splits.argtypes = [I, I, I, I]
    L.mla_decode_splits.restype = I
    L.mla_decode_workspace_bytes.argtypes = [I, I, I, I]
    L.mla_decode_workspace_bytes.restype = Z
    L.mla_attend_decode.argtypes = [P, P, P, P, P, I, I, F, I, I, I, I, P, Z, P, P, U, P]
    L.mla_attend_decode.restype = I
    L.mla_attend_decode_shared_kpe.argtypes = [P, P, P, P, P, P, I, I, F, I, I, I, I, P, Z, P, P,
                                               U, P]
    L.mla_attend_decode_shared_kpe.restype = I
    L.mla_decode_latent_workspace_bytes.argtypes = [I, I, I, I]
    L.mla_decode_latent_workspace_bytes.restype = Z
    L.mla_attend_decode_latent.argtypes = [P, P, P, P, P, P, I, I, F, I, I, I, I, P, Z, P, P, U, P]
    L.mla_attend_decode_latent.restype = I
    L.mla_out_proj_workspace_bytes.argtypes = [I, I, I]
    L.mla_out_proj_workspace_bytes.restype = Z
    L.mla_out_proj.argtypes = [P, P, P, I, I, I, P, Z, U, P]
    L.mla_out_proj_fp8_workspace_bytes.argtypes = [I, I, I]
    L.mla_out_proj_fp8_workspace_bytes.restype = Z
    L.mla_out_proj_fp8.argtypes = [P, P, P, P, I, I, I, P, Z, U, P]
    L.mla_out_proj_fp8.restype = I
    L.mla_out_proj.restype = I
    L.mla_act_scale_stride.argtypes = [I]
    L.mla_act_scale_stride.restype = I
    L.mla_act_quant.argtypes = [P, I, I, P, P, P]
    L.mla_act_quant.restype = I
    L.mla_out_proj_fp8_dyn_workspace_bytes.argtypes = [I, I, I]
    L.mla_out_proj_fp8_dyn_workspace_bytes.restype = Z
    L.mla_out_proj_fp8_dyn.argtypes = [P, P, P, P, I, I, I, P, Z, U, P]
    L.mla_out_proj_fp8_dyn.restype = I
    L.mla_up_project.argtypes = [P, P, P, P, I, I, I, P, P, P, P, U, P]
    L.mla_up_project.restype = I
    L.mla_attend_prefill_fp8.argtypes = [P, P, P, P, P, P, I, F, I, I, I, P, Z, P, P, P, U, P]
    L.mla_attend_prefill_fp8.restype = I
    L.mla_out_proj_fp8_q_workspace_bytes.argtypes = [I, I, I]
    L.mla_out_proj_fp8_q_workspace_bytes.restype = Z
    L.mla_out_proj_fp8_q.argtypes = [P, P, P, P, P, I, I, I, P, Z, U, P]
    L.mla_out_proj_fp8_q.restype = I
    L.mla_mfma_probe_flops.argtypes = [I, I]
    L.mla_mfma_probe_flops.restype = ctypes.c_double
    L.mla_mfma_probe.argtypes = [P, I, I, P]
    L.mla_mfma_probe.restype = I
    _lib = L
    return L


def mla_abi_version() -> int:
    return lib().mla_abi_version()


def mla_status_string(status: int) -> str:
    return lib().mla_status_string(int(status)).decode()


def mla_prefill_workspace_bytes(B: int, H: int, T: int) -> int:
    return lib().mla_prefill_workspace_bytes(B, H, T)


def mla_decode_splits(B: int, H: int, L: int, num_splits: int = 0) -> int:
    return lib().mla_decode_splits(B, H, L, num_splits)


def mla_decode_workspace_bytes(B: int, H: int, L: int, num_splits: int = 0) -> int:
    return lib().mla_decode_workspace_bytes(B, H, L, num_splits)


def mla_out_proj_fp8_workspace_bytes(M: int, K: int, N: int) -> int:
    return lib().mla_out_proj_fp8_workspace_bytes(M, K, N)


def mla_decode_latent_workspace_bytes(B: int, H: int, L: int, num_splits: int = 0) -> int:
    return lib().mla_decode_latent_workspace_bytes(B, H, L, num_splits)


def mla_out_proj_workspace_bytes(M: int, K: int, N: int) -> int:
    return lib().mla_out_proj_workspace_bytes(M, K, N)


# ------------------------------------------------------------------ helpers

def _torch():
    import torch
    return torch


def _check(t, name, dtype, shape, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _workspace(workspace, nbytes, device):
    torch = _torch()
    if nbytes == 0:
        return workspace, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    return workspace, workspace.numel() * workspace.element_size()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------------ calls

def _v_shape(B, H, T, v_blocked):
    return (B, H, (T + 15) // 16, VDIM, 16) if v_blocked else (B, H, T, VDIM)


def mla_attend_prefill(q_nope, q_pe, k_nope, k_pe, v, R, softmax_scale, *, out=None, lse=None,
                       want_lse=False, out_f32=False, v_blocked=False, workspace=None,
                       stream=None):
    """Causal prefill attention.  Shapes: q_nope/k_nope/v [B,H,T,128] bf16,
    q_pe [B,H,T,64] bf16 (unrotated), k_pe [B,1,T,64] bf16 (unrotated, shared
    by heads), R [r_rows,32] float32 (angles, r_rows >= T); with v_blocked, v
    is key-blocked [B,H,ceil(T/16),128,16] (MLA_V_BLOCKED).  Returns
    (out [B,T,H*128] bf16 or float32, lse [B,H,T] float32 or None)."""
    torch = _torch()
    if q_nope.dim() != 4:
        raise ValueError("q_nope must be [B, H, T, 128]")
    B, H, T, _ = q_nope.shape
    dev = q_nope.device
    bf = torch.bfloat16
    _check(q_nope, "q_nope", bf, (B, H, T, NOPE), dev)
    _check(q_pe, "q_pe", bf, (B, H, T, ROPE), dev)
    _check(k_nope, "k_nope", bf, (B, H, T, NOPE), dev)
    _check(k_pe, "k_pe", bf, (B, 1, T, ROPE), dev)
    _check(v, "v", bf, _v_shape(B, H, T, v_blocked), dev)
    if R.dim() != 2:
        raise ValueError("R must be [r_rows, 32]")
    _check(R, "R", torch.float32, (R.shape[0], PAIRS), dev)
    odt = torch.float32 if out_f32 else bf
    if out is None:
        out = torch.empty((B, T, H * VDIM), dtype=odt, device=dev)
    _check(out, "out", odt, (B, T, H * VDIM), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, T), dev)
    workspace, ws_bytes = _workspace(workspace, mla_prefill_workspace_bytes(B, H, T), dev)
    flags = (MLA_OUT_F32 if out_f32 else 0) | (MLA_V_BLOCKED if v_blocked else 0)
    rc = lib().mla_attend_prefill(_ptr(q_nope), _ptr(q_pe), _ptr(k_nope), _ptr(k_pe), _ptr(v),
                                  _ptr(R), R.shape[0], float(softmax_scale), B, H, T,
                                  _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                                  flags, _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_attend_prefill")
    return out, lse


def mla_attend_prefill_fp8(q_nope, q_pe, k_nope, k_pe, v, R, softmax_scale, *, out8=None,
                           out_scaleT=None, lse=None, want_lse=False, v_blocked=False,
                           workspace=None, stream=None):
    """Causal prefill attention with its output quantized for the FP8 o_proj
    in the epilogue (the codes and scales mla_act_quant gives for the bf16
    output).  Shapes as for mla_attend_prefill.  Returns (out8 [B,T,H*128]
    uint8 e4m3, out_scaleT [H, mla_act_scale_stride(B*T)] float32, lse or
    None)."""
    torch = _torch()
    if q_nope.dim() != 4:
        raise ValueError("q_nope must be [B, H, T, 128]")
    B, H, T, _ = q_nope.shape
    dev = q_nope.device
    bf = torch.bfloat16
    _check(q_nope, "q_nope", bf, (B, H, T, NOPE), dev)
    _check(q_pe, "q_pe", bf, (B, H, T, ROPE), dev)
    _check(k_nope, "k_nope", bf, (B, H, T, NOPE), dev)
    _check(k_pe, "k_pe", bf, (B, 1, T, ROPE), dev)
    _check(v, "v", bf, _v_shape(B, H, T, v_blocked), dev)
    if R.dim() != 2:
        raise ValueError("R must be [r_rows, 32]")
    _check(R, "R", torch.float32, (R.shape[0], PAIRS), dev)
    ms = mla_act_scale_stride(B * T)
    if out8 is None:
        out8 = torch.empty((B, T, H * VDIM), dtype=torch.uint8, device=dev)
    if out_scaleT is None:
        out_scaleT = torch.empty((H, ms), dtype=torch.float32, device=dev)
    _check(out8, "out8", torch.uint8, (B, T, H * VDIM), dev)
    _check(out_scaleT, "out_scaleT", torch.float32, (H, ms), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, T), dev)
    workspace, ws_bytes = _workspace(workspace, mla_prefill_workspace_bytes(B, H, T), dev)
    rc = lib().mla_attend_prefill_fp8(_ptr(q_nope), _ptr(q_pe), _ptr(k_nope), _ptr(k_pe), _ptr(v),
                                      _ptr(R), R.shape[0], float(softmax_scale), B, H, T,
                                      _ptr(workspace), ws_bytes, _ptr(out8), _ptr(out_scaleT),
                                      _ptr(lse), MLA_V_BLOCKED if v_blocked else 0,
                                      _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_attend_prefill_fp8")
    return out8, out_scaleT, lse


def mla_attend_prefill_noalloc(q_nope, q_pe, k_nope, k_pe, v, R, softmax_scale, *, out=None,
                               lse=None, want_lse=False, out_f32=False, v_blocked=False,
                               stream=None):
    """mla_attend_prefill without a workspace argument: the library's static
    per-device buffer (MLA_PREFILL_NOALLOC_SCRATCH_BYTES) holds the cos/sin
    table and the rotated shared key.  Same shapes and results; calls that
    overlap on one GPU race.  Allocates `out` / `lse` here only when they are
    not given (pass them to allocate nothing at all)."""
    torch = _torch()
    if q_nope.dim() != 4:
        raise ValueError("q_nope must be [B, H, T, 128]")
    B, H, T, _ = q_nope.shape
    dev = q_nope.device
    bf = torch.bfloat16
    _check(q_nope, "q_nope", bf, (B, H, T, NOPE), dev)
    _check(q_pe, "q_pe", bf, (B, H, T, ROPE), dev)
    _check(k_nope, "k_nope", bf, (B, H, T, NOPE), dev)
    _check(k_pe, "k_pe", bf, (B, 1, T, ROPE), dev)
    _check(v, "v", bf, _v_shape(B, H, T, v_blocked), dev)
    if R.dim() != 2:
        raise ValueError("R must be [r_rows, 32]")
    _check(R, "R", torch.float32, (R.shape[0], PAIRS), dev)
    odt = torch.float32 if out_f32 else bf
    if out is None:
        out = torch.empty((B, T, H * VDIM), dtype=odt, device=dev)
    _check(out, "out", odt, (B, T, H * VDIM), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, T), dev)
    flags = (MLA_OUT_F32 if out_f32 else 0) | (MLA_V_BLOCKED if v_blocked else 0)
    rc = lib().mla_attend_prefill_noalloc(_ptr(q_nope), _ptr(q_pe), _ptr(k_nope), _ptr(k_pe),
                                          _ptr(v), _ptr(R), R.shape[0], float(softmax_scale), B, H,
                                          T, _ptr(out), _ptr(lse), flags,
                                          _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_attend_prefill_noalloc")
    return out, lse


def mla_attend_decode(q_nope, q_pe, k_cache, v_cache, R, q_pos, softmax_scale, *, num_splits=0,
                      out=None, lse=None, want_lse=False, out_f32=False, workspace=None,
                      stream=None):
    """Decode attention for one new query per (b, h).  Shapes: q_nope [B,H,128],
    q_pe [B,H,64] (unrotated; rotated at q_pos), k_cache [B,H,L,192] (rotated
    keys), v_cache [B,H,L,128], R [r_rows,32].  Returns (out [B,H*128], lse [B,H] or None)."""
    torch = _torch()
    if k_cache.dim() != 4:
        raise ValueError("k_cache must be [B, H, L, 192]")
    B, H, L, _ = k_cache.shape
    dev = k_cache.device
    bf = torch.bfloat16
    _check(q_nope, "q_nope", bf, (B, H, NOPE), dev)
    _check(q_pe, "q_pe", bf, (B, H, ROPE), dev)
    _check(k_cache, "k_cache", bf, (B, H, L, NOPE + ROPE), dev)
    _check(v_cache, "v_cache", bf, (B, H, L, VDIM), dev)
    if R.dim() != 2:
        raise ValueError("R must be [r_rows, 32]")
    _check(R, "R", torch.float32, (R.shape[0], PAIRS), dev)
    odt = torch.float32 if out_f32 else bf
    if out is None:
        out = torch.empty((B, H * VDIM), dtype=odt, device=dev)
    _check(out, "out", odt, (B, H * VDIM), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H), dev)
    need = mla_decode_workspace_bytes(B, H, L, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    rc = lib().mla_attend_decode(_ptr(q_nope), _ptr(q_pe), _ptr(k_cache), _ptr(v_cache), _ptr(R),
                                 R.shape[0], int(q_pos), float(softmax_scale), B, H, L,
                                 int(num_splits), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                                 MLA_OUT_F32 if out_f32 else 0, _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_attend_decode")
    return out, lse


def mla_attend_decode_shared_kpe(q_nope, q_pe, k_nope_cache, kpe_cache, v_cache, R, q_pos,
                                 softmax_scale, *, num_splits=0, out=None, lse=None,
                                 want_lse=False, out_f32=False, workspace=None, stream=None):
    """Decode against the shared-rotary cache layout.  Shapes: q_nope [B,H,128],
    q_pe [B,H,64] (unrotated; rotated at q_pos), k_nope_cache [B,H,L,128],
    kpe_cache [B,L,64] (rotated keys, one per position for every head),
    v_cache [B,H,L,128], R [r_rows,32].  Returns (out [B,H*128], lse [B,H] or None)."""
    torch = _torch()
    if k_nope_cache.dim() != 4:
        raise ValueError("k_nope_cache must be [B, H, L, 128]")
    B, H, L, _ = k_nope_cache.shape
    dev = k_nope_cache.device
    bf = torch.bfloat16
    _check(q_nope, "q_nope", bf, (B, H, NOPE), dev)
    _check(q_pe, "q_pe", bf, (B, H, ROPE), dev)
    _check(k_nope_cache, "k_nope_cache", bf, (B, H, L, NOPE), dev)
    _check(kpe_cache, "kpe_cache", bf, (B, L, ROPE), dev)
    _check(v_cache, "v_cache", bf, (B, H, L, VDIM), dev)
    if R.dim() != 2:
        raise ValueError("R must be [r_rows, 32]")
    _check(R, "R", torch.float32, (R.shape[0], PAIRS), dev)
    odt = torch.float32 if out_f32 else bf
    if out is None:
        out = torch.empty((B, H * VDIM), dtype=odt, device=dev)
    _check(out, "out", odt, (B, H * VDIM), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H), dev)
    need = mla_decode_workspace_bytes(B, H, L, num_splits)
    workspace, ws_bytes = _workspace(workspace, need, dev)
    rc = lib().mla_attend_decode_shared_kpe(
        _ptr(q_nope), _ptr(q_pe), _ptr(k_nope_cache), _ptr(kpe_cache), _ptr(v_cache), _ptr(R),
        R.shape[0], int(q_pos), float(softmax_scale), B, H, L, int(num_splits), _ptr(workspace),
        ws_bytes, _ptr(out), _ptr(lse), MLA_OUT_F32 if out_f32 else 0, _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_attend_decode_shared_kpe")
    return out, lse


def mla_attend_decode_latent(q_nope, q_pe, ckv_cache, kpe_cache, w_kv_b, R, q_pos, softmax_scale,
                             *, num_splits=0, out=None, lse=None, want_lse=False, out_f32=False,
                             workspace=None, stream=None):
    """Decode against a latent cache.  Shapes: q_nope [B,H,128], q_pe [B,H,64]
    (unrotated; rotated at q_pos), ckv_cache [B,L,512], kpe_cache [B,L,64]
    (rotated keys, one per position for every head), w_kv_b [H*256,512] (the
    up-projection, per head 128 key rows then 128 value rows), R [r_rows,32].
    Returns (out [B,H*128], lse [B,H] or None)."""
    torch = _torch()
    if ckv_cache.dim() != 3 or q_nope.dim() != 3:
        raise ValueError("ckv_cache must be [B, L, 512] and q_nope [B, H, 128]")
    B, L, _ = ckv_cache.shape
    H = q_nope.shape[1]
    dev = ckv_cache.device
    bf = torch.bfloat16
    _check(q_nope, "q_nope", bf, (B, H, NOPE), dev)
    _check(q_pe, "q_pe", bf, (B, H, ROPE), dev)
    _check(ckv_cache, "ckv_cache", bf, (B, L, LATENT), dev)
    _check(kpe_cache, "kpe_cache", bf, (B, L, ROPE), dev)
    _check(w_kv_b, "w_kv_b", bf, (H * (NOPE + VDIM), LATENT), dev)
    if R.dim() != 2:
        raise ValueError("R must be [r_rows, 32]")
    _check(R, "R", torch.float32, (R.shape[0], PAIRS), dev)
    odt = torch.float32 if out_f32 else bf
    if out is None:
        out = torch.empty((B, H * VDIM), dtype=odt, device=dev)
    _check(out, "out", odt, (B, H * VDIM), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H), dev)
    workspace, ws_bytes = _workspace(workspace, mla_decode_latent_workspace_bytes(B, H, L, num_splits),
                                     dev)
    rc = lib().mla_attend_decode_latent(
        _ptr(q_nope), _ptr(q_pe), _ptr(ckv_cache), _ptr(kpe_cache), _ptr(w_kv_b), _ptr(R),
        R.shape[0], int(q_pos), float(softmax_scale), B, H, L, int(num_splits), _ptr(workspace),
        ws_bytes, _ptr(out), _ptr(lse), MLA_OUT_F32 if out_f32 else 0, _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_attend_decode_latent")
    return out, lse


def mla_out_proj(x, w_o, *, y=None, out_f32=False, workspace=None, stream=None):
    """y = x · w_oᵀ with x [M,K] bf16 and w_o [N,K] bf16 (a linear layer's
    weight, one row per output feature).  Returns y [M,N] bf16 or float32."""
    torch = _torch()
    if x.dim() != 2 or w_o.dim() != 2:
        raise ValueError("x must be [M, K] and w_o [N, K]")
    M, K = x.shape
    N = w_o.shape[0]
    dev = x.device
    bf = torch.bfloat16
    _check(x, "x", bf, (M, K), dev)
    _check(w_o, "w_o", bf, (N, K), dev)
    odt = torch.float32 if out_f32 else bf
    if y is None:
        y = torch.empty((M, N), dtype=odt, device=dev)
    _check(y, "y", odt, (M, N), dev)
    workspace, ws_bytes = _workspace(workspace, mla_out_proj_workspace_bytes(M, K, N), dev)
    rc = lib().mla_out_proj(_ptr(x), _ptr(w_o), _ptr(y), M, K, N, _ptr(workspace), ws_bytes,
                            MLA_OUT_F32 if out_f32 else 0, _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_out_proj")
    return y


def mla_up_project(q_lat, ckv, w_q_b, w_kv_b, *, outs=None, out_f32=False, v_blocked=False,
                   stream=None):
    """The MLA up-projection: q_lat [B,T,1536] and ckv [B,T,512] bf16, w_q_b
    [H*192,1536] and w_kv_b [H*256,512] bf16.  Returns (q_nope [B,H,T,128],
    q_pe [B,H,T,64] unrotated, k_nope [B,H,T,128], v [B,H,T,128]), bf16 or
    float32; with v_blocked, v is key-blocked [B,H,ceil(T/16),128,16] (the
    slots past T unwritten).  ``outs`` may hold the four output tensors."""
    torch = _torch()
    if q_lat.dim() != 3 or w_q_b.dim() != 2:
        raise ValueError("q_lat must be [B, T, 1536] and w_q_b [H*192, 1536]")
    B, T = q_lat.shape[:2]
    H = w_q_b.shape[0] // (NOPE + ROPE)
    dev = q_lat.device
    _check(q_lat, "q_lat", torch.bfloat16, (B, T, Q_RANK), dev)
    _check(ckv, "ckv", torch.bfloat16, (B, T, LATENT), dev)
    _check(w_q_b, "w_q_b", torch.bfloat16, (H * (NOPE + ROPE), Q_RANK), dev)
    _check(w_kv_b, "w_kv_b", torch.bfloat16, (H * (NOPE + VDIM), LATENT), dev)
    odt = torch.float32 if out_f32 else torch.bfloat16
    shapes = [(B, H, T, NOPE), (B, H, T, ROPE), (B, H, T, NOPE), _v_shape(B, H, T, v_blocked)]
    if outs is None:
        outs = [torch.empty(sh, dtype=odt, device=dev) for sh in shapes]
    for t, sh, name in zip(outs, shapes, ("q_nope", "q_pe", "k_nope", "v")):
        _check(t, name, odt, sh, dev)
    rc = lib().mla_up_project(_ptr(q_lat), _ptr(ckv), _ptr(w_q_b), _ptr(w_kv_b), B, T, H,
                              *[_ptr(t) for t in outs],
                              (MLA_OUT_F32 if out_f32 else 0) | (MLA_V_BLOCKED if v_blocked else 0),
                              _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_up_project")
    return tuple(outs)


def mla_out_proj_fp8(x, w8, w_scale, *, y=None, out_f32=False, workspace=None, stream=None):
    """y = x · dequant(w8, w_scale)ᵀ with x [M,K] bf16, w8 [N,K] uint8 (e4m3)
    and w_scale [ceil(N/128), K/128] float32 block scales.  Returns y [M,N]."""
    torch = _torch()
    if x.dim() != 2 or w8.dim() != 2:
        raise ValueError("x must be [M, K] and w8 [N, K]")
    M, K = x.shape
    N = w8.shape[0]
    dev = x.device
    _check(x, "x", torch.bfloat16, (M, K), dev)
    _check(w8, "w8", torch.uint8, (N, K), dev)
    _check(w_scale, "w_scale", torch.float32, ((N + 127) // 128, (K + 127) // 128), dev)
    odt = torch.float32 if out_f32 else torch.bfloat16
    if y is None:
        y = torch.empty((M, N), dtype=odt, device=dev)
    _check(y, "y", odt, (M, N), dev)
    workspace, ws_bytes = _workspace(workspace, mla_out_proj_fp8_workspace_bytes(M, K, N), dev)
    rc = lib().mla_out_proj_fp8(_ptr(x), _ptr(w8), _ptr(w_scale), _ptr(y), M, K, N, _ptr(workspace),
                                ws_bytes, MLA_OUT_F32 if out_f32 else 0, _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_out_proj_fp8")
    return y


def mla_act_scale_stride(M):
    return lib().mla_act_scale_stride(int(M))


def mla_out_proj_fp8_dyn_workspace_bytes(M, K, N):
    return lib().mla_out_proj_fp8_dyn_workspace_bytes(int(M), int(K), int(N))


def mla_act_quant(x, *, x8=None, x_scaleT=None, stream=None):
    """FP8 activations of x [M,K] bf16 (1 x 128 blocks, dynamic scales):
    returns (x8 [M,K] uint8 e4m3 codes, x_scaleT [K/128, stride] float32, the
    scales transposed; columns past M unspecified)."""
    torch = _torch()
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    dev = x.device
    _check(x, "x", torch.bfloat16, (M, K), dev)
    ms = mla_act_scale_stride(M)
    if x8 is None:
        x8 = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if x_scaleT is None:
        x_scaleT = torch.empty((K // 128, ms), dtype=torch.float32, device=dev)
    _check(x8, "x8", torch.uint8, (M, K), dev)
    _check(x_scaleT, "x_scaleT", torch.float32, (K // 128, ms), dev)
    rc = lib().mla_act_quant(_ptr(x), M, K, _ptr(x8), _ptr(x_scaleT), _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_act_quant")
    return x8, x_scaleT


def mla_out_proj_fp8_dyn(x, w8, w_scale, *, y=None, out_f32=False, workspace=None, stream=None):
    """y = dequant(act_quant(x)) · dequant(w8, w_scale)ᵀ on the FP8 matrix
    cores: x [M,K] bf16 (quantized to e4m3 per row and 128 columns inside the
    call), w8 [N,K] uint8 e4m3, w_scale [ceil(N/128), K/128] float32.
    Returns y [M,N]."""
    torch = _torch()
    if x.dim() != 2 or w8.dim() != 2:
        raise ValueError("x must be [M, K] and w8 [N, K]")
    M, K = x.shape
    N = w8.shape[0]
    dev = x.device
    _check(x, "x", torch.bfloat16, (M, K), dev)
    _check(w8, "w8", torch.uint8, (N, K), dev)
    _check(w_scale, "w_scale", torch.float32, ((N + 127) // 128, (K + 127) // 128), dev)
    odt = torch.float32 if out_f32 else torch.bfloat16
    if y is None:
        y = torch.empty((M, N), dtype=odt, device=dev)
    _check(y, "y", odt, (M, N), dev)
    workspace, ws_bytes = _workspace(workspace, mla_out_proj_fp8_dyn_workspace_bytes(M, K, N), dev)
    rc = lib().mla_out_proj_fp8_dyn(_ptr(x), _ptr(w8), _ptr(w_scale), _ptr(y), M, K, N,
                                    _ptr(workspace), ws_bytes, MLA_OUT_F32 if out_f32 else 0,
                                    _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_out_proj_fp8_dyn")
    return y


def mla_out_proj_fp8_q_workspace_bytes(M: int, K: int, N: int) -> int:
    return lib().mla_out_proj_fp8_q_workspace_bytes(M, K, N)


def mla_out_proj_fp8_q(x8, x_scaleT, w8, w_scale, *, y=None, out_f32=False, workspace=None,
                       stream=None):
    """The FP8 product on activations already quantized: x8 [M,K] uint8
    e4m3, x_scaleT [K/128, mla_act_scale_stride(M)] float32 (from
    mla_act_quant or mla_attend_prefill_fp8), w8 [N,K] uint8 e4m3, w_scale
    [ceil(N/128), K/128] float32.  Returns y [M,N]."""
    torch = _torch()
    if x8.dim() != 2 or w8.dim() != 2:
        raise ValueError("x8 must be [M, K] and w8 [N, K]")
    M, K = x8.shape
    N = w8.shape[0]
    dev = x8.device
    _check(x8, "x8", torch.uint8, (M, K), dev)
    _check(x_scaleT, "x_scaleT", torch.float32, (K // 128, mla_act_scale_stride(M)), dev)
    _check(w8, "w8", torch.uint8, (N, K), dev)
    _check(w_scale, "w_scale", torch.float32, ((N + 127) // 128, (K + 127) // 128), dev)
    odt = torch.float32 if out_f32 else torch.bfloat16
    if y is None:
        y = torch.empty((M, N), dtype=odt, device=dev)
    _check(y, "y", odt, (M, N), dev)
    workspace, ws_bytes = _workspace(workspace, mla_out_proj_fp8_q_workspace_bytes(M, K, N), dev)
    rc = lib().mla_out_proj_fp8_q(_ptr(x8), _ptr(x_scaleT), _ptr(w8), _ptr(w_scale), _ptr(y), M, K,
                                  N, _ptr(workspace), ws_bytes, MLA_OUT_F32 if out_f32 else 0,
                                  _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_out_proj_fp8_q")
    return y


def mla_append_kv(k_nope, k_pe, v, R, past, k_nope_cache, kpe_cache, v_cache, *, stream=None):
    """Write a chunk (k_nope [B,H,T,128], k_pe [B,1,T,64] unrotated, v
    [B,H,T,128]) into the shared-rotary cache at rows past .. past+T-1
    (k_nope_cache [B,H,L,128], kpe_cache [B,L,64], v_cache [B,H,L,128])."""
    torch = _torch()
    if k_nope.dim() != 4 or k_nope_cache.dim() != 4:
        raise ValueError("k_nope must be [B, H, T, 128] and k_nope_cache [B, H, L, 128]")
    B, H, T, _ = k_nope.shape
    L = k_nope_cache.shape[2]
    dev = k_nope.device
    bf = torch.bfloat16
    _check(k_nope, "k_nope", bf, (B, H, T, NOPE), dev)
    _check(k_pe, "k_pe", bf, (B, 1, T, ROPE), dev)
    _check(v, "v", bf, (B, H, T, VDIM), dev)
    _check(k_nope_cache, "k_nope_cache", bf, (B, H, L, NOPE), dev)
    _check(kpe_cache, "kpe_cache", bf, (B, L, ROPE), dev)
    _check(v_cache, "v_cache", bf, (B, H, L, VDIM), dev)
    if R.dim() != 2:
        raise ValueError("R must be [r_rows, 32]")
    _check(R, "R", torch.float32, (R.shape[0], PAIRS), dev)
    rc = lib().mla_append_kv(_ptr(k_nope), _ptr(k_pe), _ptr(v), _ptr(R), R.shape[0], int(past), B, H,
                             T, L, _ptr(k_nope_cache), _ptr(kpe_cache), _ptr(v_cache), 0,
                             _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_append_kv")


def mla_prefill_chunk_workspace_bytes(T: int) -> int:
    return lib().mla_prefill_chunk_workspace_bytes(T)


def mla_attend_prefill_chunk(q_nope, q_pe, k_nope_cache, kpe_cache, v_cache, R, past,
                             softmax_scale, *, out=None, lse=None, want_lse=False, out_f32=False,
                             workspace=None, stream=None):
    """Chunked prefill: q_nope [B,H,T,128], q_pe [B,H,T,64] at positions past ..
    past+T-1 against cache rows 0 .. past+t.  Returns (out [B,T,H*128], lse
    [B,H,T] or None)."""
    torch = _torch()
    if q_nope.dim() != 4 or k_nope_cache.dim() != 4:
        raise ValueError("q_nope must be [B, H, T, 128] and k_nope_cache [B, H, L, 128]")
    B, H, T, _ = q_nope.shape
    L = k_nope_cache.shape[2]
    dev = q_nope.device
    bf = torch.bfloat16
    _check(q_nope, "q_nope", bf, (B, H, T, NOPE), dev)
    _check(q_pe, "q_pe", bf, (B, H, T, ROPE), dev)
    _check(k_nope_cache, "k_nope_cache", bf, (B, H, L, NOPE), dev)
    _check(kpe_cache, "kpe_cache", bf, (B, L, ROPE), dev)
    _check(v_cache, "v_cache", bf, (B, H, L, VDIM), dev)
    if R.dim() != 2:
        raise ValueError("R must be [r_rows, 32]")
    _check(R, "R", torch.float32, (R.shape[0], PAIRS), dev)
    odt = torch.float32 if out_f32 else bf
    if out is None:
        out = torch.empty((B, T, H * VDIM), dtype=odt, device=dev)
    _check(out, "out", odt, (B, T, H * VDIM), dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    if lse is not None:
        _check(lse, "lse", torch.float32, (B, H, T), dev)
    workspace, ws_bytes = _workspace(workspace, mla_prefill_chunk_workspace_bytes(T), dev)
    rc = lib().mla_attend_prefill_chunk(
        _ptr(q_nope), _ptr(q_pe), _ptr(k_nope_cache), _ptr(kpe_cache), _ptr(v_cache), _ptr(R),
        R.shape[0], int(past), float(softmax_scale), B, H, T, L, _ptr(workspace), ws_bytes, _ptr(out),
        _ptr(lse), MLA_OUT_F32 if out_f32 else 0, _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_attend_prefill_chunk")
    return out, lse


MLA_MFMA_PROBE_OUT = 512 * 256


def mla_mfma_probe_flops(iters: int, kind: int = 0) -> float:
    return lib().mla_mfma_probe_flops(int(iters), int(kind))


def mla_mfma_probe(iters, kind=0, *, out=None, device=None, stream=None):
    """One launch of the matrix-core rate probe (a measurement helper, not a
    step of the path): mla_mfma_probe_flops(iters, kind) flops of MFMA chains
    on every compute unit, kind 0 bf16 32x32x16, kind 1 e4m3 32x32x64 on fixed
    operands; kinds 2 (bf16) and 3 (e4m3) on random operands that change with
    every instruction (iters a multiple of 8).  Returns the out buffer
    (float32 per-thread sums of the products)."""
    torch = _torch()
    dev = out.device if out is not None else torch.device(device or "cuda:0")
    if out is None:
        out = torch.empty(MLA_MFMA_PROBE_OUT, dtype=torch.float32, device=dev)
    _check(out, "out", torch.float32, (MLA_MFMA_PROBE_OUT,), dev)
    rc = lib().mla_mfma_probe(_ptr(out), int(iters), int(kind), _stream_handle(stream, dev))
    if rc:
        raise MlaError(rc, "mla_mfma_probe")
    return out
