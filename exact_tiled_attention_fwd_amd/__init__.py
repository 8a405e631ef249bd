"""Exact attention forward (FlashAttention-2 style) on MI355X / gfx950.

A thin ctypes binding over the C ABI of ``include/fa.h`` (``libfa.so``, built
by ``exact_tiled_attention_fwd_amd.build``). Every step of the computation
runs in the HIP kernels of that library; this module only marshals arguments.
PyTorch supplies device memory and the current stream.

Raw entry points, same names and argument order as the C header:
    fa_fwd, fa_fwd_strided, fa_fwd_varlen, fa_fwd_varlen_strided, fa_fwd_fp8, fa_bwd,
    fa_bwd_workspace_bytes, fa_decode, fa_decode_noalloc, fa_decode_paged,
    fa_decode_workspace_bytes, fa_set_prefill_schedule, fa_status_string, fa_last_error,
    fa_abi_version
Tensor-level helpers:
    attention(q, k, v, causal=False, scale=None) -> (o, lse)
        q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d], any strides with a unit last one
    attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                     causal=False, scale=None) -> (o, lse)
        q [Hq,total_q,d], k/v [Hkv,total_k,d], any strides likewise
    flash_attn_func(q, k, v, dropout_p=0.0, softmax_scale=None, causal=False)
        -> o, for q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d]; differentiable (fa_bwd)
        when an input requires grad
    flash_attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                           max_seqlen_k, dropout_p=0.0, softmax_scale=None,
                           causal=False) -> o, for q [total_q,Hq,d]
    attention_fp8(q, k, v, q_descale, k_descale, v_descale, causal=False,
                  scale=None) -> (o bf16, lse), E4M3 inputs [B,H,N,128]
    attention_bwd(q, k, v, o, lse, dout, causal=False, scale=None)
        -> (dq, dk, dv), for the contiguous layouts of attention()
    decode(q, k_cache, v_cache, seqlens, scale=None, num_splits=0) -> (o, lse)
    decode_paged(q, k_pages, v_pages, block_table, seqlens, scale=None,
                 num_splits=0) -> (o, lse)

There is no fallback: if the library is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch  # loads the HIP runtime that libfa.so then binds to

__all__ = [
    "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP",
    "FA_DTYPE_BF16", "FA_DTYPE_FP16", "FA_SCHEDULE_AUTO", "FA_SCHEDULE_TILES", "FA_SCHEDULE_SPLIT",
    "FAError", "lib_path", "load_library", "fa_set_prefill_schedule",
    "fa_fwd", "fa_fwd_strided", "fa_fwd_varlen", "fa_fwd_varlen_strided", "fa_fwd_fp8", "attention_fp8", "fa_bwd",
    "fa_bwd_workspace_bytes",
    "attention_bwd", "fa_decode", "fa_decode_noalloc", "fa_decode_paged",
    "fa_decode_workspace_bytes", "fa_status_string", "fa_last_error", "fa_abi_version", "attention",
    "attention_varlen", "flash_attn_func", "flash_attn_varlen_func", "decode", "decode_paged", "dtype_code",
]

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP = 0, 1, 2, 3
FA_DTYPE_BF16, FA_DTYPE_FP16 = 0, 1
FA_SCHEDULE_AUTO, FA_SCHEDULE_TILES, FA_SCHEDULE_SPLIT = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def lib_path() -> str:
    """The library to load: ``libfa.so`` beside this file, or the build named
    by the environment variable FA_LIBRARY (the host-sanitizer test points it
    at ``libfa_hostsan.so``)."""
    return os.environ.get("FA_LIBRARY") or os.path.join(_HERE, "libfa.so")


class FAError(RuntimeError):
    """A non-OK status from the library (status code in ``.status``)."""

    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class FAInvalidArgument(FAError, ValueError):
    pass


class FAUnsupported(FAError, NotImplementedError):
    pass


def load_library():
    """Load libfa.so once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"HIP library not found at {path}; build it with "
            "`python -m exact_tiled_attention_fwd_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_varlen.restype = i
    lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_strided.restype = i
    lib.fa_fwd_varlen_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_varlen_strided.restype = i
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i]
    lib.fa_bwd_workspace_bytes.restype = sz
    lib.fa_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, f, i, i, vp]
    lib.fa_decode.restype = i
    lib.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_decode_noalloc.restype = i
    lib.fa_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, sz, i, i, i, i, i, i, i, f, i, i, vp]
    lib.fa_decode_paged.restype = i
    lib.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.fa_decode_workspace_bytes.restype = sz
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i
    lib.fa_set_prefill_schedule.argtypes = [i]
    lib.fa_set_prefill_schedule.restype = i
    _LIB = lib
    return lib


def _raise_for(status: int):
    if status == FA_OK:
        return
    lib = load_library()
    msg = f"{lib.fa_status_string(status).decode()}: {lib.fa_last_error().decode()}"
    if status == FA_ERR_INVALID_ARG:
        raise FAInvalidArgument(status, msg)
    if status == FA_ERR_UNSUPPORTED:
        raise FAUnsupported(status, msg)
    raise FAError(status, msg)


# ------------------------------------------------------------------ raw C ABI
def fa_set_prefill_schedule(mode: int) -> int:
    """Call the C ``fa_set_prefill_schedule`` (FA_SCHEDULE_*); returns the
    previous mode, or -1 for an unknown one."""
    return load_library().fa_set_prefill_schedule(mode)


def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, stream) -> int:
    """Call the C ``fa_fwd`` with integer device addresses; returns the status."""
    return load_library().fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, stream)


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q, total_k, max_seqlen_q,
                  d, scale, causal, dtype, stream) -> int:
    """Call the C ``fa_fwd_varlen`` with integer device addresses; returns the status."""
    return load_library().fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q, total_k,
                                        max_seqlen_q, d, scale, causal, dtype, stream)


def _i64_array(strides):
    arr = (ctypes.c_int64 * len(strides))(*[int(x) for x in strides])
    return arr


def fa_fwd_strided(q, k, v, o, lse, strides, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, stream) -> int:
    """Call the C ``fa_fwd_strided``; `strides` is a sequence of 12 ints
    (batch, head, row strides of q, k, v, o in elements)."""
    if len(strides) != 12:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "fa_fwd_strided needs 12 strides")
    arr = _i64_array(strides)
    return load_library().fa_fwd_strided(q, k, v, o, lse, ctypes.cast(arr, ctypes.c_void_p), B, Hq, Hkv, Nq, Nk, d,
                                         scale, causal, dtype, stream)


def fa_fwd_varlen_strided(q, k, v, o, lse, strides, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, total_q, total_k,
                          max_seqlen_q, d, scale, causal, dtype, stream) -> int:
    """Call the C ``fa_fwd_varlen_strided``; `strides` is a sequence of 8 ints
    (head, token strides of q, k, v, o in elements)."""
    if len(strides) != 8:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "fa_fwd_varlen_strided needs 8 strides")
    arr = _i64_array(strides)
    return load_library().fa_fwd_varlen_strided(q, k, v, o, lse, ctypes.cast(arr, ctypes.c_void_p), cu_seqlens_q,
                                                cu_seqlens_k, B, Hq, Hkv, total_q, total_k, max_seqlen_q, d, scale,
                                                causal, dtype, stream)


def fa_fwd_fp8(q, k, v, o, lse, q_descale, k_descale, v_descale, B, Hq, Hkv, Nq, Nk, d, scale, causal,
               stream) -> int:
    """Call the C ``fa_fwd_fp8`` with integer device addresses; returns the status."""
    return load_library().fa_fwd_fp8(q, k, v, o, lse, q_descale, k_descale, v_descale, B, Hq, Hkv, Nq, Nk, d, scale,
                                     causal, stream)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale, causal,
           dtype, stream) -> int:
    """Call the C ``fa_bwd`` with integer device addresses; returns the status."""
    return load_library().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk,
                                 d, scale, causal, dtype, stream)


def fa_bwd_workspace_bytes(B, Hq, Nq) -> int:
    return load_library().fa_bwd_workspace_bytes(B, Hq, Nq)


def fa_decode(q, k_cache, v_cache, seqlens, o, lse, workspace, workspace_bytes,
              B, Hq, Hkv, Lcap, d, scale, num_splits, dtype, stream) -> int:
    """Call the C ``fa_decode`` with integer device addresses; returns the status."""
    return load_library().fa_decode(q, k_cache, v_cache, seqlens, o, lse, workspace, workspace_bytes,
                                    B, Hq, Hkv, Lcap, d, scale, num_splits, dtype, stream)


def fa_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Lcap, d, scale, num_splits, dtype,
                      stream) -> int:
    """Call the C ``fa_decode_noalloc`` (decode on the library's static
    workspace) with integer device addresses; returns the status."""
    return load_library().fa_decode_noalloc(q, k_cache, v_cache, seqlens, o, lse, B, Hq, Hkv, Lcap, d, scale,
                                            num_splits, dtype, stream)


def fa_decode_paged(q, k_pages, v_pages, block_table, seqlens, o, lse, workspace, workspace_bytes,
                    B, Hq, Hkv, num_pages, page_size, max_pages, d, scale, num_splits, dtype, stream) -> int:
    """Call the C ``fa_decode_paged`` with integer device addresses; returns the status."""
    return load_library().fa_decode_paged(q, k_pages, v_pages, block_table, seqlens, o, lse, workspace,
                                          workspace_bytes, B, Hq, Hkv, num_pages, page_size, max_pages, d, scale,
                                          num_splits, dtype, stream)


def fa_decode_workspace_bytes(B, Hq, Hkv, Lcap, d, num_splits) -> int:
    return load_library().fa_decode_workspace_bytes(B, Hq, Hkv, Lcap, d, num_splits)


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(status).decode()


def fa_last_error() -> str:
    return load_library().fa_last_error().decode()


def fa_abi_version() -> int:
    return load_library().fa_abi_version()


# ------------------------------------------------------------------ torch helpers
def dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return FA_DTYPE_BF16
    if dt == torch.float16:
        return FA_DTYPE_FP16
    raise FAUnsupported(FA_ERR_UNSUPPORTED, f"unsupported dtype {dt}; use bfloat16 or float16")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_tensor(name, t, ndim, device=None, strided=False):
    if not isinstance(t, torch.Tensor):
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must be on the GPU")
    if strided:
        if t.stride(-1) != 1 and t.shape[-1] > 1:
            raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must have a unit stride in its last dim")
    elif not t.is_contiguous():
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} is on {t.device}, expected {device}")


def _check_out(name, t, shape, dtype, device, strided=False):
    """A caller-supplied output or workspace: a torch.Tensor on ``device``
    with exactly ``shape`` and ``dtype`` (contiguous unless ``strided``, then
    with a unit last stride). The C layer only sees a pointer, so a tensor
    that is too small, of the wrong type or on the host must be refused
    here, before anything is launched."""
    if not isinstance(t, torch.Tensor):
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must be a torch.Tensor")
    if t.device != device:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must be {dtype}, got {t.dtype}")
    if strided:
        if t.dim() and t.stride(-1) != 1 and t.shape[-1] > 1:
            raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must have a unit stride in its last dim")
    elif not t.is_contiguous():
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must be contiguous")


def _check_workspace(t, need, device):
    """A caller-supplied workspace: contiguous bytes on ``device``, at least ``need`` of them."""
    if not isinstance(t, torch.Tensor):
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "workspace must be a torch.Tensor")
    if t.device != device:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"workspace is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "workspace must be contiguous")
    if t.numel() * t.element_size() < need:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG,
                                f"workspace holds {t.numel() * t.element_size()} bytes, {need} needed")


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def attention(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """O, LSE for q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] (bf16/fp16, same GPU). Any
    strides with a unit last one are accepted (e.g. transposed views of
    (batch, seq, heads, dim) tensors); contiguous tensors go through fa_fwd,
    others through fa_fwd_strided."""
    _check_tensor("q", q, 4, strided=True)
    dev = q.device
    _check_tensor("k", k, 4, dev, strided=True)
    _check_tensor("v", v, 4, dev, strided=True)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "q, k and v must share a dtype")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if (Bk, dk) != (B, d) or tuple(v.shape) != tuple(k.shape):
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_out("out", out, q.shape, q.dtype, dev, strided=True)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    _check_out("lse", lse, (B, Hq, Nq), torch.float32, dev)
    with torch.cuda.device(dev):
        if all(t.is_contiguous() for t in (q, k, v, out)):
            st = fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
                        float(scale), int(bool(causal)), dtype_code(q.dtype), _stream(dev))
        else:
            strides = [*q.stride()[:3], *k.stride()[:3], *v.stride()[:3], *out.stride()[:3]]
            st = fa_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), strides, B, Hq, Hkv, Nq, Nk, d,
                                float(scale), int(bool(causal)), dtype_code(q.dtype), _stream(dev))
    _raise_for(st)
    return out, lse


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False,
                     scale: float | None = None, out=None, lse=None):
    """Packed variable-length batch: q [Hq,total_q,d], k/v [Hkv,total_k,d],
    cu_seqlens_* int32 [B+1] on the device, max_seqlen_q a host int. Any
    strides with a unit last one are accepted (e.g. transposed views of
    (total, heads, dim) tensors)."""
    _check_tensor("q", q, 3, strided=True)
    dev = q.device
    _check_tensor("k", k, 3, dev, strided=True)
    _check_tensor("v", v, 3, dev, strided=True)
    _check_tensor("cu_seqlens_q", cu_seqlens_q, 1, dev)
    _check_tensor("cu_seqlens_k", cu_seqlens_k, 1, dev)
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "cu_seqlens must be int32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "q, k and v must share a dtype")
    Hq, total_q, d = q.shape
    Hkv, total_k, dk = k.shape
    B = cu_seqlens_q.shape[0] - 1
    if dk != d or tuple(v.shape) != tuple(k.shape) or cu_seqlens_k.shape[0] != B + 1 or B < 1:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "shape mismatch between q, k, v and cu_seqlens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    _check_out("out", out, q.shape, q.dtype, dev, strided=True)
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=dev)
    _check_out("lse", lse, (Hq, total_q), torch.float32, dev)
    with torch.cuda.device(dev):
        if all(t.is_contiguous() for t in (q, k, v, out)):
            st = fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                               _ptr(cu_seqlens_k), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), d, float(scale),
                               int(bool(causal)), dtype_code(q.dtype), _stream(dev))
        else:
            strides = [*q.stride()[:2], *k.stride()[:2], *v.stride()[:2], *out.stride()[:2]]
            st = fa_fwd_varlen_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), strides,
                                       _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Hq, Hkv, total_q, total_k,
                                       int(max_seqlen_q), d, float(scale), int(bool(causal)), dtype_code(q.dtype),
                                       _stream(dev))
    _raise_for(st)
    return out, lse


def _no_dropout(dropout_p):
    if dropout_p:
        raise FAUnsupported(FA_ERR_UNSUPPORTED, "dropout is not supported (forward inference path only)")


class _AttentionFn(torch.autograd.Function):
    """Autograd node over fa_fwd / fa_bwd for [B,H,N,d] tensors (any strides
    in the forward; the backward reads contiguous copies)."""

    @staticmethod
    def forward(ctx, q, k, v, causal, scale):
        o, lse = attention(q, k, v, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.causal, ctx.scale = causal, scale
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse = ctx.saved_tensors
        qc, kc, vc, oc, doc = (t.contiguous() for t in (q, k, v, o, do))
        dq, dk, dv = attention_bwd(qc, kc, vc, oc, lse, doc, causal=ctx.causal, scale=ctx.scale)
        return dq, dk, dv, None, None


def _needs_grad(*ts):
    return torch.is_grad_enabled() and any(t.requires_grad for t in ts)


def flash_attn_func(q, k, v, dropout_p: float = 0.0, softmax_scale: float | None = None, causal: bool = False,
                    return_lse: bool = False):
    """The flash_attn_func calling convention: q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d]
    (batch, seq, heads, dim); returns o [B,Nq,Hq,d] in the same layout (and
    the LSE [B,Hq,Nq] fp32 with return_lse). No copies: the kernels read and
    write the (batch, seq, heads, dim) tensors through their strides. When
    an input requires grad, the result is differentiable: the backward pass
    runs fa_bwd (on contiguous copies)."""
    _no_dropout(dropout_p)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, 4, strided=True)
    if _needs_grad(q, k, v):
        scale = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(q.shape[-1])
        o, lse = _AttentionFn.apply(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), bool(causal), scale)
        out = o.transpose(1, 2)
        return (out, lse) if return_lse else out
    out = torch.empty_like(q)
    o, lse = attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2), causal=causal,
                       scale=softmax_scale, out=out.transpose(1, 2))
    return (out, lse) if return_lse else out


def flash_attn_varlen_func(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                           dropout_p: float = 0.0, softmax_scale: float | None = None, causal: bool = False,
                           return_lse: bool = False):
    """The flash_attn_varlen_func calling convention: q [total_q,Hq,d],
    k/v [total_k,Hkv,d] (packed tokens, heads, dim), cu_seqlens_* int32 [B+1];
    returns o [total_q,Hq,d] (and the LSE [Hq,total_q] fp32 with return_lse).
    max_seqlen_k is accepted for the signature and not needed."""
    _no_dropout(dropout_p)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, 3, strided=True)
    out = torch.empty_like(q)
    o, lse = attention_varlen(q.transpose(0, 1), k.transpose(0, 1), v.transpose(0, 1), cu_seqlens_q, cu_seqlens_k,
                              max_seqlen_q, causal=causal, scale=softmax_scale, out=out.transpose(0, 1))
    return (out, lse) if return_lse else out


def attention_fp8(q, k, v, q_descale, k_descale, v_descale, causal: bool = False, scale: float | None = None,
                  out=None, lse=None):
    """O (bf16), LSE for E4M3 inputs: q [B,Hq,Nq,128], k/v [B,Hkv,Nk,128] as
    torch.uint8 or torch.float8_e4m3fn (contiguous), descales float32
    [B,Hq] / [B,Hkv]: element x of a slab stands for x * descale."""
    def u8(name, t):
        _check_tensor(name, t, 4, q.device if name != "q" else None)
        if t.dtype == getattr(torch, "float8_e4m3fn", None):
            return t.view(torch.uint8)
        if t.dtype != torch.uint8:
            raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must be uint8 or float8_e4m3fn")
        return t
    q8, k8, v8 = u8("q", q), u8("k", k), u8("v", v)
    dev = q.device
    B, Hq, Nq, d = q8.shape
    Bk, Hkv, Nk, dk = k8.shape
    if (Bk, dk) != (B, d) or tuple(v8.shape) != tuple(k8.shape):
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "shape mismatch between q, k and v")
    for name, t, shape in (("q_descale", q_descale, (B, Hq)), ("k_descale", k_descale, (B, Hkv)),
                           ("v_descale", v_descale, (B, Hkv))):
        _check_tensor(name, t, 2, dev)
        if t.dtype != torch.float32 or tuple(t.shape) != shape:
            raise FAInvalidArgument(FA_ERR_INVALID_ARG, f"{name} must be float32 of shape {shape}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=dev)
    _check_out("out", out, (B, Hq, Nq, d), torch.bfloat16, dev)
    _check_out("lse", lse, (B, Hq, Nq), torch.float32, dev)
    with torch.cuda.device(dev):
        st = fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(out), _ptr(lse), _ptr(q_descale), _ptr(k_descale),
                        _ptr(v_descale), B, Hq, Hkv, Nq, Nk, d, float(scale), int(bool(causal)), _stream(dev))
    _raise_for(st)
    return out, lse


def attention_bwd(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None, dq=None, dk=None,
                  dv=None, workspace=None):
    """dQ, dK, dV for the forward attention(q, k, v) whose output o and LSE
    lse are given, and an upstream gradient dout of o. q, o, dout
    [B,Hq,Nq,d], k/v [B,Hkv,Nk,d], lse [B,Hq,Nq] fp32, all contiguous."""
    _check_tensor("q", q, 4)
    dev = q.device
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, 4, dev)
    _check_tensor("lse", lse, 3, dev)
    if any(t.dtype != q.dtype for t in (k, v, o, dout)) or lse.dtype != torch.float32:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "q, k, v, o, dout must share a dtype and lse be float32")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk_ = k.shape
    if ((Bk, dk_) != (B, d) or tuple(v.shape) != tuple(k.shape) or tuple(o.shape) != tuple(q.shape)
            or tuple(dout.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Nq)):
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "shape mismatch between q, k, v, o, lse and dout")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_out(name, t, ref.shape, ref.dtype, dev)
    need = fa_bwd_workspace_bytes(B, Hq, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check_workspace(workspace, need, dev)
    with torch.cuda.device(dev):
        st = fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                    _ptr(workspace), workspace.numel() * workspace.element_size(), B, Hq, Hkv, Nq, Nk, d,
                    float(scale), int(bool(causal)), dtype_code(q.dtype), _stream(dev))
    _raise_for(st)
    return dq, dk, dv


def decode(q, k_cache, v_cache, seqlens, scale: float | None = None, num_splits: int = 0,
           workspace=None, out=None, lse=None):
    """One new token per sequence: q [B,Hq,d], caches [B,Hkv,Lcap,d], seqlens int32 [B]."""
    _check_tensor("q", q, 3)
    dev = q.device
    _check_tensor("k_cache", k_cache, 4, dev)
    _check_tensor("v_cache", v_cache, 4, dev)
    _check_tensor("seqlens", seqlens, 1, dev)
    if seqlens.dtype != torch.int32:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "seqlens must be int32")
    if k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "q and the caches must share a dtype")
    B, Hq, d = q.shape
    Bk, Hkv, Lcap, dk = k_cache.shape
    if (Bk, dk) != (B, d) or tuple(v_cache.shape) != tuple(k_cache.shape) or seqlens.shape[0] != B:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "shape mismatch between q, caches and seqlens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_decode_workspace_bytes(B, Hq, Hkv, Lcap, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _check_workspace(workspace, need, dev)
    _check_out("out", out, q.shape, q.dtype, dev)
    _check_out("lse", lse, (B, Hq), torch.float32, dev)
    with torch.cuda.device(dev):
        st = fa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seqlens), _ptr(out), _ptr(lse),
                       _ptr(workspace), workspace.numel() * workspace.element_size(),
                       B, Hq, Hkv, Lcap, d, float(scale), int(num_splits), dtype_code(q.dtype), _stream(dev))
    _raise_for(st)
    return out, lse


def decode_paged(q, k_pages, v_pages, block_table, seqlens, scale: float | None = None, num_splits: int = 0,
                 workspace=None, out=None, lse=None):
    """Decode against a paged cache: q [B,Hq,d], pages [num_pages,Hkv,page_size,d],
    block_table int32 [B,max_pages], seqlens int32 [B]."""
    _check_tensor("q", q, 3)
    dev = q.device
    _check_tensor("k_pages", k_pages, 4, dev)
    _check_tensor("v_pages", v_pages, 4, dev)
    _check_tensor("block_table", block_table, 2, dev)
    _check_tensor("seqlens", seqlens, 1, dev)
    if seqlens.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "seqlens and block_table must be int32")
    if k_pages.dtype != q.dtype or v_pages.dtype != q.dtype:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "q and the pages must share a dtype")
    B, Hq, d = q.shape
    num_pages, Hkv, page_size, dk = k_pages.shape
    Bt, max_pages = block_table.shape
    if dk != d or tuple(v_pages.shape) != tuple(k_pages.shape) or Bt != B or seqlens.shape[0] != B:
        raise FAInvalidArgument(FA_ERR_INVALID_ARG, "shape mismatch between q, pages, block_table and seqlens")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_decode_workspace_bytes(B, Hq, Hkv, max_pages * page_size, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _check_workspace(workspace, need, dev)
    _check_out("out", out, q.shape, q.dtype, dev)
    _check_out("lse", lse, (B, Hq), torch.float32, dev)
    with torch.cuda.device(dev):
        st = fa_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(seqlens), _ptr(out),
                             _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(), B, Hq, Hkv,
                             num_pages, page_size, max_pages, d, float(scale), int(num_splits), dtype_code(q.dtype),
                             _stream(dev))
    _raise_for(st)
    return out, lse
