"""Online-softmax kernels for MI355X (gfx950) behind the C ABI of libtea.so.

This module only marshals arguments: torch tensors in, device pointers,
sizes, dtype codes and the current HIP stream out; every step of the
computation runs in the HIP kernels of ``csrc/``.  There is no CPU fallback:
if libtea.so is missing, or a call's status is not TEA_OK, an exception is
raised.  The C contract of each call is documented in ``include/tea.h``.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

import torch

__all__ = [
    "row_softmax", "attn_fwd", "attn_fwd_splitk", "attn_fwd_splitk_workspace_bytes", "attn_decode_splitkv",
    "attn_decode_workspace_bytes", "attn_decode_splitkv_noalloc", "attn_decode_fused", "merge_partials",
    "TeaError", "library_path", "load_library",
    "TEA_OK", "TEA_EINVAL", "TEA_EUNSUPPORTED", "TEA_EHIP", "TEA_ENOSPACE", "TEA_F32", "TEA_BF16",
]

TEA_OK, TEA_EINVAL, TEA_EUNSUPPORTED, TEA_EHIP, TEA_ENOSPACE = 0, 1, 2, 3, 4
DECODE_NOALLOC_MAX_BYTES = 32 << 20  # TEA_DECODE_NOALLOC_MAX_BYTES
TEA_F32, TEA_BF16 = 0, 1
TEA_RESCALE_ALWAYS, TEA_RESCALE_IF_RISE, TEA_RESCALE_L0_ONE = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtea.so")
_lib = None
_lock = threading.Lock()

EXPORTS = ("row_softmax", "row_softmax_variant", "attn_fwd", "attn_fwd_splitk_workspace_bytes", "attn_fwd_splitk",
           "attn_decode_workspace_bytes", "attn_decode_splitkv", "attn_decode_splitkv_noalloc", "attn_decode_fused",
           "merge_partials",
           "tea_status_string", "tea_abi_version")


class TeaError(RuntimeError):
    def __init__(self, name: str, status: int, msg: str):
        super().__init__(f"{name}: status {status} ({msg})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libtea.so (built by ``tiled_exact_attention_amd.build``) and
    declare its signatures.  Raises if the library is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                                   "`python -m tiled_exact_attention_amd.build` (or __graft_entry__.build())")
            lib = ctypes.CDLL(_LIB_PATH)
            P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
            lib.row_softmax.argtypes = [P, P, I64, I64, I, I, P, P, P]
            lib.row_softmax.restype = I
            lib.row_softmax_variant.argtypes = [P, P, I64, I64, I, I, I, P, P, P]
            lib.row_softmax_variant.restype = I
            lib.attn_fwd.argtypes = [P, P, P, P, I, I, I, I, I, F, I, I, P, P]
            lib.attn_fwd.restype = I
            lib.attn_decode_workspace_bytes.argtypes = [I, I, I, I]
            lib.attn_decode_workspace_bytes.restype = SZ
            lib.attn_decode_splitkv.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P, SZ, P]
            lib.attn_decode_splitkv.restype = I
            lib.attn_decode_splitkv_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
            lib.attn_decode_splitkv_noalloc.restype = I
            lib.attn_decode_fused.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, P]
            lib.attn_decode_fused.restype = I
            lib.attn_fwd_splitk_workspace_bytes.argtypes = [I, I, I, I, I]
            lib.attn_fwd_splitk_workspace_bytes.restype = SZ
            lib.attn_fwd_splitk.argtypes = [P, P, P, P, I, I, I, I, I, F, I, I, I, P, P, SZ, P]
            lib.attn_fwd_splitk.restype = I
            lib.merge_partials.argtypes = [P, P, P, I64, I, I, P, P, P, I, I, P]
            lib.merge_partials.restype = I
            lib.tea_status_string.argtypes = [I]
            lib.tea_status_string.restype = ctypes.c_char_p
            lib.tea_abi_version.restype = I
            _lib = lib
    return _lib


def _check(name: str, status: int):
    if status != TEA_OK:
        raise TeaError(name, status, load_library().tea_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _shape(name: str, t, shape, dtype=None):
    """The C ABI takes bare pointers and sizes, so a tensor whose shape or
    dtype disagrees with the sizes passed would be read or written out of
    bounds: check it here."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or (dtype is not None and t.dtype != dtype):
        want = f"{tuple(shape)}" + (f" {dtype}" if dtype is not None else "")
        raise ValueError(f"{name} must be {want}, got {tuple(t.shape)} {t.dtype}")


def _dcode(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return TEA_F32
    if dt == torch.bfloat16:
        return TEA_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on a GPU")


def row_softmax(x: torch.Tensor, out: torch.Tensor | None = None, block: int = 8, stats: bool = False):
    """Softmax of every row of a 2-D fp32/bf16 tensor; y has x's dtype.
    ``stats=True`` also returns the row maxima and normalisers (fp32)."""
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    _shape("out", out, x.shape, x.dtype)
    y = torch.empty_like(x) if out is None else out
    _dev(x, y)
    rows, cols = x.shape
    m = torch.empty(rows, dtype=torch.float32, device=x.device) if stats else None
    l = torch.empty(rows, dtype=torch.float32, device=x.device) if stats else None
    _check("row_softmax", load_library().row_softmax(_ptr(x), _ptr(y), rows, cols, _dcode(x.dtype), int(block),
                                                     _ptr(m), _ptr(l), _stream(x)))
    return (y, m, l) if stats else y


def row_softmax_variant(x: torch.Tensor, rescale: int, out: torch.Tensor | None = None, block: int = 8,
                        stats: bool = False):
    """row_softmax with the rescale policy of the online fold chosen:
    TEA_RESCALE_ALWAYS, TEA_RESCALE_IF_RISE or TEA_RESCALE_L0_ONE (same bits
    as row_softmax for every policy)."""
    if x.dim() != 2:
        raise ValueError("x must be [rows, cols]")
    _shape("out", out, x.shape, x.dtype)
    y = torch.empty_like(x) if out is None else out
    _dev(x, y)
    rows, cols = x.shape
    m = torch.empty(rows, dtype=torch.float32, device=x.device) if stats else None
    l = torch.empty(rows, dtype=torch.float32, device=x.device) if stats else None
    _check("row_softmax_variant", load_library().row_softmax_variant(_ptr(x), _ptr(y), rows, cols, _dcode(x.dtype),
                                                                     int(block), int(rescale), _ptr(m), _ptr(l),
                                                                     _stream(x)))
    return (y, m, l) if stats else y


def attn_fwd(q, k, v, scale: float | None = None, causal: bool = False, out_dtype=torch.bfloat16,
             return_lse: bool = False, out: torch.Tensor | None = None):
    """O = softmax(q k^T * scale) v for bf16 q [B,H,Sq,D], k, v [B,H,Sk,D]."""
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    _shape("k", k, (B, H, Sk, D))
    _shape("v", v, (B, H, Sk, D))
    _shape("out", out, (B, H, Sq, D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty((B, H, Sq, D), dtype=out_dtype, device=q.device) if out is None else out
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    _dev(q, k, v, o, lse)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    _check("attn_fwd", load_library().attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, Sq, Sk, D, float(scale),
                                               int(bool(causal)), _dcode(o.dtype), _ptr(lse), _stream(q)))
    return (o, lse) if return_lse else o


def attn_fwd_splitk_workspace_bytes(B: int, H: int, Sq: int, D: int, num_splits: int) -> int:
    return int(load_library().attn_fwd_splitk_workspace_bytes(B, H, Sq, D, num_splits))


def attn_fwd_splitk(q, k, v, num_splits: int, scale: float | None = None, causal: bool = False,
                    out_dtype=torch.bfloat16, return_lse: bool = False, workspace: torch.Tensor | None = None,
                    out: torch.Tensor | None = None):
    """attn_fwd with each query block's KV range split num_splits ways and the
    partial states merged; same arguments as attn_fwd."""
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    _shape("k", k, (B, H, Sk, D))
    _shape("v", v, (B, H, Sk, D))
    _shape("out", out, (B, H, Sq, D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = attn_fwd_splitk_workspace_bytes(B, H, Sq, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty((B, H, Sq, D), dtype=out_dtype, device=q.device) if out is None else out
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    _dev(q, k, v, o, lse, workspace)
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    _check("attn_fwd_splitk", load_library().attn_fwd_splitk(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), B, H, Sq, Sk, D, float(scale), int(bool(causal)), int(num_splits),
        _dcode(o.dtype), _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q)))
    return (o, lse) if return_lse else o


def attn_decode_workspace_bytes(B: int, H: int, D: int, num_splits: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, H, D, num_splits))


def attn_decode_splitkv(q, k, v, kv_len, num_splits: int = 64, scale: float | None = None,
                        out_dtype=torch.bfloat16, workspace: torch.Tensor | None = None,
                        out: torch.Tensor | None = None):
    """Split-KV decode: q [B,H,1,D], k/v [B,H,Lmax,D] bf16, kv_len [B] int32
    (device).  Returns O [B,H,D]."""
    B, H, _, D = q.shape
    Lmax = k.shape[2]
    _shape("q", q, (B, H, 1, D))
    _shape("k", k, (B, H, Lmax, D))
    _shape("v", v, (B, H, Lmax, D))
    _shape("kv_len", kv_len, (B,))
    _shape("out", out, (B, H, D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = attn_decode_workspace_bytes(B, H, D, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    o = torch.empty((B, H, D), dtype=out_dtype, device=q.device) if out is None else out
    _dev(q, k, v, kv_len, o, workspace)
    if kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be int32")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    _check("attn_decode_splitkv", load_library().attn_decode_splitkv(
        _ptr(q), _ptr(k), _ptr(v), _ptr(kv_len), _ptr(o), B, H, Lmax, D, int(num_splits), float(scale),
        _dcode(o.dtype), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q)))
    return o


def attn_decode_splitkv_noalloc(q, k, v, kv_len, out: torch.Tensor, num_splits: int = 64,
                                scale: float | None = None):
    """attn_decode_splitkv with the partials in the library's device scratch
    instead of a workspace: nothing is allocated on this path, so the output
    ``out`` [B,H,D] (bf16 or fp32) must be passed.  Returns ``out``."""
    B, H, _, D = q.shape
    Lmax = k.shape[2]
    _shape("q", q, (B, H, 1, D))
    _shape("k", k, (B, H, Lmax, D))
    _shape("v", v, (B, H, Lmax, D))
    _shape("kv_len", kv_len, (B,))
    _shape("out", out, (B, H, D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _dev(q, k, v, kv_len, out)
    if kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be int32")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    _check("attn_decode_splitkv_noalloc", load_library().attn_decode_splitkv_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(kv_len), _ptr(out), B, H, Lmax, D, int(num_splits), float(scale),
        _dcode(out.dtype), _stream(q)))
    return out


def attn_decode_fused(q, k, v, kv_len, num_splits: int = 64, scale: float | None = None,
                      out_dtype=torch.bfloat16, out: torch.Tensor | None = None):
    """Split-KV decode in one launch, no workspace (num_splits <= 64): q
    [B,H,1,D], k/v [B,H,Lmax,D] bf16, kv_len [B] int32 (device).  Returns
    O [B,H,D]."""
    B, H, _, D = q.shape
    Lmax = k.shape[2]
    _shape("q", q, (B, H, 1, D))
    _shape("k", k, (B, H, Lmax, D))
    _shape("v", v, (B, H, Lmax, D))
    _shape("kv_len", kv_len, (B,))
    _shape("out", out, (B, H, D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = torch.empty((B, H, D), dtype=out_dtype, device=q.device) if out is None else out
    _dev(q, k, v, kv_len, o)
    if kv_len.dtype != torch.int32:
        raise TypeError("kv_len must be int32")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError("q, k, v must be bfloat16")
    _check("attn_decode_fused", load_library().attn_decode_fused(
        _ptr(q), _ptr(k), _ptr(v), _ptr(kv_len), _ptr(o), B, H, Lmax, D, int(num_splits), float(scale),
        _dcode(o.dtype), _stream(q)))
    return o


def merge_partials(m, l, O, out_dtype=torch.float32, normalize: bool = True, stats: bool = False,
                   out: torch.Tensor | None = None):
    """Merge partial states m, l [N,S], O [N,S,D] (fp32) into O [N,D]."""
    N, S, D = O.shape
    _shape("O", O, (N, S, D), torch.float32)
    _shape("m", m, (N, S), torch.float32)
    _shape("l", l, (N, S), torch.float32)
    _shape("out", out, (N, D))
    o = torch.empty((N, D), dtype=out_dtype, device=O.device) if out is None else out
    mo = torch.empty(N, dtype=torch.float32, device=O.device) if stats else None
    lo = torch.empty(N, dtype=torch.float32, device=O.device) if stats else None
    _dev(m, l, O, o, mo, lo)
    _check("merge_partials", load_library().merge_partials(_ptr(m), _ptr(l), _ptr(O), N, S, D, _ptr(mo), _ptr(lo),
                                                           _ptr(o), _dcode(o.dtype), int(bool(normalize)),
                                                           _stream(O)))
    return (o, mo, lo) if stats else o
