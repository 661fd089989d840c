"""ctypes binding of libflashattn.so (argument marshalling only).

Each function checks the torch tensors it is given (device, dtype, shape,
contiguity), allocates the outputs the caller did not pass, and calls the C
entry point of the same name on torch's current HIP stream. Every step of
the computation runs in the library's kernels; if the library is missing
the call fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashattn.so")
_lib = None

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_SCRATCH_LIMIT = 0, 1, 2, 3, 4
NOALLOC_MAX_ROWS = 4 << 20  # B*H*N limit of flash_attn_bwd_noalloc
FA_BWD_PRECISE = 1
FA_BWD_DQ_ATOMIC = 2

EXPORTED = ("flash_attn_fwd", "flash_attn_bwd", "flash_attn_bwd_noalloc", "flash_attn_bwd_workspace_bytes",
            "flash_attn_fwd_f32", "flash_attn_bwd_f32", "flash_attn_decode_fwd",
            "flash_attn_decode_workspace_bytes", "flash_attn_fwd_dropout", "flash_attn_bwd_dropout",
            "flash_attn_dropout_mask", "flash_attn_fwd_block_sparse", "flash_attn_fwd_fp8",
            "flash_attn_status_string")


class FlashAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {flash_attn_status_string(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libflashattn.so (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m io_aware_exact_11_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i, f, u, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint, ctypes.c_size_t
    fwd_args = [p, p, p, p, p, i, i, i, i, f, i, p, p]
    bwd_args = [p, p, p, p, p, p, p, p, p, p, sz, i, i, i, i, f, i, p, u, p]
    for name, args in (("flash_attn_fwd", fwd_args), ("flash_attn_fwd_f32", fwd_args),
                       ("flash_attn_bwd", bwd_args), ("flash_attn_bwd_f32", bwd_args)):
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.flash_attn_bwd_noalloc.argtypes = bwd_args[:9] + bwd_args[11:]
    lib.flash_attn_bwd_noalloc.restype = ctypes.c_int
    lib.flash_attn_bwd_workspace_bytes.argtypes = [i, i, i, i, u]
    lib.flash_attn_bwd_workspace_bytes.restype = sz
    lib.flash_attn_decode_fwd.argtypes = [p, p, p, p, p, p, sz, i, i, i, i, i, f, i, p, p]
    lib.flash_attn_decode_fwd.restype = ctypes.c_int
    lib.flash_attn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.flash_attn_decode_workspace_bytes.restype = sz
    u64 = ctypes.c_uint64
    lib.flash_attn_fwd_dropout.argtypes = fwd_args[:-1] + [f, u64, u, p]
    lib.flash_attn_fwd_dropout.restype = ctypes.c_int
    lib.flash_attn_bwd_dropout.argtypes = bwd_args[:-2] + [f, u64, u, u, p]
    lib.flash_attn_bwd_dropout.restype = ctypes.c_int
    lib.flash_attn_dropout_mask.argtypes = [p, i, i, i, i, f, u64, u, p]
    lib.flash_attn_dropout_mask.restype = ctypes.c_int
    lib.flash_attn_fwd_block_sparse.argtypes = fwd_args[:-1] + [p, ctypes.c_int64, p]
    lib.flash_attn_fwd_block_sparse.restype = ctypes.c_int
    lib.flash_attn_fwd_fp8.argtypes = fwd_args[:-1] + [f, f, f, p]
    lib.flash_attn_fwd_fp8.restype = ctypes.c_int
    lib.flash_attn_status_string.argtypes = [i]
    lib.flash_attn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def flash_attn_status_string(status: int) -> str:
    return load_library().flash_attn_status_string(int(status)).decode()


def flash_attn_bwd_workspace_bytes(B: int, H: int, N: int, d: int, flags: int = 0) -> int:
    return int(load_library().flash_attn_bwd_workspace_bytes(B, H, N, d, flags))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(name, t, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.device.index != torch.cuda.current_device():
        # the library launches on the current device and its current stream
        raise ValueError(f"{name} is on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _kv(kv_len, B, device):
    if kv_len is None:
        return None
    _check("kv_len", kv_len, torch.int32, (B,))
    return kv_len


def _scale(scale, d):
    return float(d) ** -0.5 if scale is None else float(scale)


def _fwd(name, dtype, q, k, v, causal, scale, kv_len, out, lse, extra=()):
    lib = load_library()
    _check("q", q, dtype, q.shape)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _check("k", k, dtype, q.shape)
    _check("v", v, dtype, q.shape)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    _check("out", out, dtype, q.shape)
    _check("lse", lse, torch.float32, (B, H, N))
    kv_len = _kv(kv_len, B, q.device)
    st = getattr(lib, name)(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d,
                            _scale(scale, d), int(bool(causal)), _ptr(kv_len), *extra, _stream())
    if st != FA_OK:
        raise FlashAttnError(st, name)
    return out, lse


def _bwd(name, dtype, q, k, v, o, do, lse, causal, scale, kv_len, flags, dq, dk, dv, workspace, extra=None):
    lib = load_library()
    _check("q", q, dtype, q.shape)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for nm, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _check(nm, t, dtype, q.shape)
    _check("lse", lse, torch.float32, (B, H, N))
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32) if dq is None else dq
    dk = torch.empty(q.shape, **f32) if dk is None else dk
    dv = torch.empty(q.shape, **f32) if dv is None else dv
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(nm, t, torch.float32, q.shape)
    need = flash_attn_bwd_workspace_bytes(B, H, N, d, flags)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    kv_len = _kv(kv_len, B, q.device)
    tail = (int(flags),) if extra is None else tuple(extra)
    st = getattr(lib, name)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                            _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(),
                            B, H, N, d, _scale(scale, d), int(bool(causal)), _ptr(kv_len), *tail,
                            _stream())
    if st != FA_OK:
        raise FlashAttnError(st, name)
    return dq, dk, dv


def flash_attn_fwd(q, k, v, causal=False, scale=None, kv_len=None, out=None, lse=None):
    """bf16 forward: returns (O bf16 [B,H,N,d], LSE fp32 [B,H,N])."""
    return _fwd("flash_attn_fwd", torch.bfloat16, q, k, v, causal, scale, kv_len, out, lse)


def flash_attn_fwd_f32(q, k, v, causal=False, scale=None, kv_len=None, out=None, lse=None):
    """fp32 forward: returns (O fp32, LSE fp32)."""
    return _fwd("flash_attn_fwd_f32", torch.float32, q, k, v, causal, scale, kv_len, out, lse)


def flash_attn_bwd(q, k, v, o, do, lse, causal=False, scale=None, kv_len=None, precise=False,
                   dq_atomic=False, dq=None, dk=None, dv=None, workspace=None):
    """bf16 backward: returns fp32 (dQ, dK, dV)."""
    flags = (FA_BWD_PRECISE if precise else 0) | (FA_BWD_DQ_ATOMIC if dq_atomic else 0)
    return _bwd("flash_attn_bwd", torch.bfloat16, q, k, v, o, do, lse, causal, scale, kv_len, flags,
                dq, dk, dv, workspace)


def flash_attn_bwd_noalloc(q, k, v, o, do, lse, causal=False, scale=None, kv_len=None, precise=False,
                           dq_atomic=False, dq=None, dk=None, dv=None):
    """bf16 backward without a workspace (the library's fixed scratch holds D_i): returns fp32 (dQ, dK, dV).
    Outputs the caller does not pass are allocated here; pass dq, dk, dv to allocate nothing."""
    lib = load_library()
    _check("q", q, torch.bfloat16, q.shape)
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for nm, t in (("k", k), ("v", v), ("o", o), ("do", do)):
        _check(nm, t, torch.bfloat16, q.shape)
    _check("lse", lse, torch.float32, (B, H, N))
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty(q.shape, **f32) if dq is None else dq
    dk = torch.empty(q.shape, **f32) if dk is None else dk
    dv = torch.empty(q.shape, **f32) if dv is None else dv
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(nm, t, torch.float32, q.shape)
    kv_len = _kv(kv_len, B, q.device)
    flags = (FA_BWD_PRECISE if precise else 0) | (FA_BWD_DQ_ATOMIC if dq_atomic else 0)
    st = lib.flash_attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
                                    _ptr(dv), B, H, N, d, _scale(scale, d), int(bool(causal)), _ptr(kv_len),
                                    int(flags), _stream())
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_bwd_noalloc")
    return dq, dk, dv


def flash_attn_bwd_f32(q, k, v, o, do, lse, causal=False, scale=None, kv_len=None,
                       dq=None, dk=None, dv=None, workspace=None):
    """fp32 backward: returns fp32 (dQ, dK, dV)."""
    return _bwd("flash_attn_bwd_f32", torch.float32, q, k, v, o, do, lse, causal, scale, kv_len, 0,
                dq, dk, dv, workspace)


def flash_attn_decode_workspace_bytes(B: int, H: int, Nq: int, Nk: int, d: int) -> int:
    return int(load_library().flash_attn_decode_workspace_bytes(B, H, Nq, Nk, d))


def flash_attn_decode_fwd(q, k, v, causal=False, scale=None, kv_len=None, out=None, lse=None,
                          workspace=None):
    """bf16 decoding forward: q [B,H,Nq,d] against the cache k, v [B,H,Nk,d].

    Returns (O bf16 [B,H,Nq,d], LSE fp32 [B,H,Nq])."""
    lib = load_library()
    _check("q", q, torch.bfloat16, q.shape)
    _check("k", k, torch.bfloat16, k.shape)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be [B, H, N, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    _check("k", k, torch.bfloat16, (B, H, Nk, d))
    _check("v", v, torch.bfloat16, (B, H, Nk, d))
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check("out", out, torch.bfloat16, q.shape)
    _check("lse", lse, torch.float32, (B, H, Nq))
    need = flash_attn_decode_workspace_bytes(B, H, Nq, Nk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    kv_len = _kv(kv_len, B, q.device)
    st = lib.flash_attn_decode_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), B, H, Nq, Nk, d,
                                   _scale(scale, d), int(bool(causal)), _ptr(kv_len), _stream())
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_decode_fwd")
    return out, lse


def _drop_args(p_drop, seed, offset):
    return (float(p_drop), int(seed) & 0xFFFFFFFFFFFFFFFF, int(offset) & 0xFFFFFFFF)


def flash_attn_fwd_dropout(q, k, v, p_drop, seed, offset=0, causal=False, scale=None, kv_len=None, out=None,
                           lse=None):
    """bf16 forward with fused dropout: returns (O bf16, LSE fp32 of the undropped scores)."""
    return _fwd("flash_attn_fwd_dropout", torch.bfloat16, q, k, v, causal, scale, kv_len, out, lse,
                _drop_args(p_drop, seed, offset))


def flash_attn_bwd_dropout(q, k, v, o, do, lse, p_drop, seed, offset=0, causal=False, scale=None, kv_len=None,
                           precise=False, dq=None, dk=None, dv=None, workspace=None):
    """bf16 backward with the dropout mask regenerated: returns fp32 (dQ, dK, dV)."""
    flags = FA_BWD_PRECISE if precise else 0
    return _bwd("flash_attn_bwd_dropout", torch.bfloat16, q, k, v, o, do, lse, causal, scale, kv_len, flags,
                dq, dk, dv, workspace, _drop_args(p_drop, seed, offset) + (flags,))


def flash_attn_dropout_mask(B, H, N_q, N_k, p_drop, seed, offset=0, out=None, device="cuda"):
    """The keep mask of the dropout calls as uint8 [B, H, N_q, N_k] (1 = kept)."""
    lib = load_library()
    out = torch.empty((B, H, N_q, N_k), dtype=torch.uint8, device=device) if out is None else out
    _check("out", out, torch.uint8, (B, H, N_q, N_k))
    st = lib.flash_attn_dropout_mask(_ptr(out), B, H, N_q, N_k, *_drop_args(p_drop, seed, offset), _stream())
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_dropout_mask")
    return out


def flash_attn_fwd_block_sparse(q, k, v, block_mask, causal=False, scale=None, kv_len=None, out=None, lse=None):
    """bf16 block-sparse forward. block_mask: uint8 (or bool) device tensor [nb, nb] shared by every head, or
    [B, H, nb, nb], nb = ceil(N / 128). Returns (O bf16, LSE fp32)."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    nb = (N + 127) // 128
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.to(torch.uint8)
    if tuple(block_mask.shape) == (nb, nb):
        stride = 0
    else:
        _check("block_mask", block_mask, torch.uint8, (B, H, nb, nb))
        stride = nb * nb
    _check("block_mask", block_mask, torch.uint8, block_mask.shape)
    return _fwd("flash_attn_fwd_block_sparse", torch.bfloat16, q, k, v, causal, scale, kv_len, out, lse,
                (_ptr(block_mask), stride))


def flash_attn_fwd_fp8(q8, k8, vt8, descale_q, descale_k, descale_v, causal=False, scale=None, kv_len=None,
                       out=None, lse=None):
    """8-bit forward: q8, k8 uint8 E4M3 codes [B, H, N, d]; vt8 [B, H, d, N] (V transposed); fp32
    dequantisation factors. Returns (O bf16 [B, H, N, d], LSE fp32 [B, H, N])."""
    lib = load_library()
    _check("q8", q8, torch.uint8, q8.shape)
    if q8.dim() != 4:
        raise ValueError("q8 must be [B, H, N, d]")
    B, H, N, d = q8.shape
    _check("k8", k8, torch.uint8, (B, H, N, d))
    _check("vt8", vt8, torch.uint8, (B, H, d, N))
    out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device) if out is None else out
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device) if lse is None else lse
    _check("out", out, torch.bfloat16, (B, H, N, d))
    _check("lse", lse, torch.float32, (B, H, N))
    kv_len = _kv(kv_len, B, q8.device)
    st = lib.flash_attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), _ptr(out), _ptr(lse), B, H, N, d, _scale(scale, d),
                                int(bool(causal)), _ptr(kv_len), float(descale_q), float(descale_k),
                                float(descale_v), _stream())
    if st != FA_OK:
        raise FlashAttnError(st, "flash_attn_fwd_fp8")
    return out, lse
