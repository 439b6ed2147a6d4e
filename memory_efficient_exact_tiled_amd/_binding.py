"""ctypes binding of libmea.so: the same entry points as include/mea.h.

Argument marshalling only: shapes and dtypes of torch tensors are turned into
the pointers and sizes of the C ABI, and the current HIP stream is passed
along. Every step of the computation runs in the library's kernels; there is
no fallback. Importing this module fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import math
import os

# torch owns the device memory and streams handed to the library, so its HIP
# runtime must be the one the library binds to: import it before loading
# libmea.so, whose libamdhip64 dependency then resolves to torch's copy.
import torch  # noqa: F401

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmea.so")

MEA_OK, MEA_EINVAL, MEA_EUNSUPPORTED, MEA_EWORKSPACE, MEA_EHIP, MEA_ESCRATCH = 0, 1, 2, 3, 4, 5
MEA_DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20   # include/mea.h
MEA_FP16, MEA_BF16 = 0, 1
MEA_MASK_CAUSAL, MEA_MASK_BLOCKDIAG, MEA_BIAS_ALIBI = 1, 2, 4

EXPORTS = ("mea_fwd", "mea_fwd_blocksparse", "mea_block_sparse_block", "mea_bwd", "mea_bwd_blocksparse", "mea_bwd_workspace_bytes", "mea_fwd_kvcache", "mea_kv_append", "mea_decode",
           "mea_decode_noalloc", "mea_decode_workspace_bytes", "mea_strerror", "mea_supported", "mea_decode_chunk")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python memory_efficient_exact_tiled_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i, _f, _u, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint, ctypes.c_size_t
_lib.mea_fwd.restype = _i
_lib.mea_fwd.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _u, _vp, _vp, _vp, _i, _vp, _vp]
_lib.mea_fwd_blocksparse.restype = _i
_lib.mea_fwd_blocksparse.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _u, _vp, _vp, _i, _vp, _vp]
_lib.mea_block_sparse_block.restype = _i
_lib.mea_block_sparse_block.argtypes = []
_lib.mea_bwd.restype = _i
_lib.mea_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _u, _vp, _vp, _vp,
                         _i, _vp, _sz, _vp]
_lib.mea_bwd_blocksparse.restype = _i
_lib.mea_bwd_blocksparse.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _u,
                                     _vp, _vp, _i, _vp, _sz, _vp]
_lib.mea_bwd_workspace_bytes.restype = _sz
_lib.mea_bwd_workspace_bytes.argtypes = [_i, _i, _i, _u]
_lib.mea_fwd_kvcache.restype = _i
_lib.mea_fwd_kvcache.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _u, _vp, _i, _vp, _vp]
_lib.mea_kv_append.restype = _i
_lib.mea_kv_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]
_lib.mea_decode.restype = _i
_lib.mea_decode.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _i, _vp, _sz, _vp]
_lib.mea_decode_noalloc.restype = _i
_lib.mea_decode_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _i, _vp]
_lib.mea_decode_workspace_bytes.restype = _sz
_lib.mea_decode_workspace_bytes.argtypes = [_i, _i, _i, _i]
_lib.mea_strerror.restype = ctypes.c_char_p
_lib.mea_strerror.argtypes = [_i]
_lib.mea_supported.restype = _i
_lib.mea_supported.argtypes = [_i, _i]
_lib.mea_decode_chunk.restype = _i
_lib.mea_decode_chunk.argtypes = []


class MeaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"mea status {status}: {_lib.mea_strerror(status).decode()}")


def lib():
    """The loaded ctypes library (for callers that pass raw pointers)."""
    return _lib


def strerror(status: int) -> str:
    return _lib.mea_strerror(status).decode()


def supported(dtype_code: int, D: int) -> bool:
    return bool(_lib.mea_supported(dtype_code, D))


def decode_chunk() -> int:
    return int(_lib.mea_decode_chunk())


def decode_workspace_bytes(B: int, Hq: int, D: int, S_max: int) -> int:
    return int(_lib.mea_decode_workspace_bytes(B, Hq, D, S_max))


def bwd_workspace_bytes(B: int, M: int, Hq: int, bias_kind: int) -> int:
    return int(_lib.mea_bwd_workspace_bytes(B, M, Hq, bias_kind))


def _check(status: int) -> None:
    if status != MEA_OK:
        raise MeaError(status)


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return MEA_FP16
    if t.dtype == torch.bfloat16:
        return MEA_BF16
    raise TypeError(f"q/k/v must be float16 or bfloat16, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


# Shape checks of the arrays the kernels index by the problem's sizes: the C
# ABI takes plain pointers, so an output or side array smaller than the sizes
# given would be written or read past its end. They run before any device call.
def _need_like(t, shape, dtype, what):
    if t is not None and (tuple(t.shape) != tuple(shape) or t.dtype != dtype):
        raise ValueError(f"{what} must be {dtype} shaped {tuple(shape)}")


def _need_numel(t, n, dtype, what):
    if t is not None and (t.numel() != n or t.dtype != dtype):
        raise ValueError(f"{what} must hold {n} values of {dtype}")


def _need_seqstart(seqstart_q, seqstart_k):
    torch = _torch()
    for s in (seqstart_q, seqstart_k):
        if s is not None and (s.dtype != torch.int32 or s.dim() != 1):
            raise TypeError("seqstart arrays must be 1-D int32 device tensors")
    if seqstart_k is not None and seqstart_k.numel() != seqstart_q.numel():
        raise ValueError("seqstart_k must have as many entries as seqstart_q")
    if seqstart_q.numel() < 2:
        raise ValueError("seqstart_q needs at least two entries (one segment)")


def fwd(q, k, v, *, causal: bool = False, seqstart_q=None, seqstart_k=None, alibi_slopes=None,
        scale: float | None = None, out=None, lse=None, stream=None):
    """Exact attention forward (``mea_fwd``).

    Dense: q ``[B,M,Hq,D]``, k/v ``[B,N,Hkv,D]``. Packed (``seqstart_q`` given):
    q ``[1,M,Hq,D]`` (or ``[M,Hq,D]``), k/v ``[1,N,Hkv,D]``, int32 prefix sums
    ``seqstart_q`` (``seqstart_k`` defaults to it) on the device. ``lse`` (fp32,
    ``[B,Hq,M]`` / ``[Hq,M]``) is filled if given. Returns ``out``.
    """
    torch = _torch()
    varlen = seqstart_q is not None
    B, M, N, Hq, Hkv, D = _shapes(q, k, seqstart_q, seqstart_k)
    if v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must match in shape and dtype, and q, k, v in dtype")
    _need_like(out, q.shape, q.dtype, "out")
    _need_numel(lse, (1 if varlen else B) * Hq * M, torch.float32, "lse")
    _need_numel(alibi_slopes, Hq, torch.float32, "alibi_slopes")
    _need_cuda(q, k, v, out, lse, alibi_slopes, seqstart_q, seqstart_k)
    if out is None:
        out = torch.empty_like(q)
    if alibi_slopes is not None and alibi_slopes.dtype != torch.float32:
        raise TypeError("alibi_slopes must be float32")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kind = ((MEA_MASK_CAUSAL if causal else 0) | (MEA_MASK_BLOCKDIAG if varlen else 0)
            | (MEA_BIAS_ALIBI if alibi_slopes is not None else 0))
    _check(_lib.mea_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, M, N, Hq, Hkv, D, float(scale), kind,
                        _ptr(seqstart_q), _ptr(seqstart_k), _ptr(alibi_slopes), _dtype_code(q), _ptr(lse),
                        _stream(stream)))
    return out


def block_sparse_block() -> int:
    return int(_lib.mea_block_sparse_block())


def fwd_blocksparse(q, k, v, block_mask, *, causal: bool = False, alibi_slopes=None, scale: float | None = None,
                    out=None, lse=None, stream=None):
    """Block-sparse exact attention forward (``mea_fwd_blocksparse``): dense
    q ``[B,M,Hq,D]``, k/v ``[B,N,Hkv,D]``; ``block_mask`` uint8 (or bool)
    device tensor ``[ceil(M/64), ceil(N/64)]``, nonzero = block on."""
    torch = _torch()
    B, M, N, Hq, Hkv, D = _shapes(q, k, None, None)
    if v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must match in shape and dtype, and q, k, v in dtype")
    blk = block_sparse_block()
    if block_mask.dtype not in (torch.uint8, torch.bool) or tuple(block_mask.shape) != (-(-M // blk), -(-N // blk)):
        raise ValueError(f"block_mask must be uint8/bool [{-(-M // blk)}, {-(-N // blk)}]")
    if alibi_slopes is not None and alibi_slopes.dtype != torch.float32:
        raise TypeError("alibi_slopes must be float32")
    _need_like(out, q.shape, q.dtype, "out")
    _need_numel(lse, B * Hq * M, torch.float32, "lse")
    _need_numel(alibi_slopes, Hq, torch.float32, "alibi_slopes")
    _need_cuda(q, k, v, out, lse, alibi_slopes, block_mask)
    out = torch.empty_like(q) if out is None else out
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kind = (MEA_MASK_CAUSAL if causal else 0) | (MEA_BIAS_ALIBI if alibi_slopes is not None else 0)
    _check(_lib.mea_fwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, M, N, Hq, Hkv, D, float(scale), kind,
                                    _ptr(block_mask), _ptr(alibi_slopes), _dtype_code(q), _ptr(lse),
                                    _stream(stream)))
    return out


def _shapes(q, k, seqstart_q, seqstart_k):
    torch = _torch()
    if seqstart_q is not None:
        if q.dim() not in (3, 4) or k.dim() not in (3, 4):
            raise ValueError("packed q/k must be [1,T,H,D] or [T,H,D]")
        M, Hq, D = q.shape[-3:]
        N, Hkv, Dk = k.shape[-3:]
        if q.numel() != M * Hq * D or k.numel() != N * Hkv * Dk or Dk != D:
            raise ValueError("packed q/k must be [1,T,H,D] or [T,H,D]")
        _need_seqstart(seqstart_q, seqstart_k)
        return seqstart_q.numel() - 1, M, N, Hq, Hkv, D
    if seqstart_k is not None:
        raise ValueError("seqstart_k needs seqstart_q")
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("dense q/k must be [B,M,Hq,D] / [B,N,Hkv,D]")
    B, M, Hq, D = q.shape
    Bk, N, Hkv, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("q and k shapes disagree")
    return B, M, N, Hq, Hkv, D


def bwd(q, k, v, out, dout, lse, *, causal: bool = False, seqstart_q=None, seqstart_k=None, alibi_slopes=None,
        scale: float | None = None, dq=None, dk=None, dv=None, workspace=None, block_mask=None, stream=None):
    """Backward of :func:`fwd` (``mea_bwd``), or of :func:`fwd_blocksparse`
    when ``block_mask`` is given (``mea_bwd_blocksparse``): gradients of
    ``sum(dout * out)``.

    ``out`` and ``lse`` are what the forward returned/filled for the same
    arguments; ``dout`` is shaped like q. The workspace is allocated with torch
    when not given. Returns ``(dq, dk, dv)``.
    """
    torch = _torch()
    B, M, N, Hq, Hkv, D = _shapes(q, k, seqstart_q, seqstart_k)
    if v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("v must match k, out and dout must match q")
    if len({q.dtype, k.dtype, v.dtype, out.dtype, dout.dtype}) != 1:
        raise ValueError("q, k, v, out, dout must share a dtype")
    if lse.dtype != torch.float32 or lse.numel() != (1 if seqstart_q is not None else B) * Hq * M:
        raise ValueError("lse must be the float32 [B,Hq,M] (packed [Hq,M]) array the forward filled")
    if alibi_slopes is not None and alibi_slopes.dtype != torch.float32:
        raise TypeError("alibi_slopes must be float32")
    _need_numel(alibi_slopes, Hq, torch.float32, "alibi_slopes")
    _need_like(dq, q.shape, q.dtype, "dq")
    _need_like(dk, k.shape, q.dtype, "dk")
    _need_like(dv, v.shape, q.dtype, "dv")
    _need_cuda(q, k, v, out, dout, lse, dq, dk, dv, alibi_slopes, workspace, seqstart_q, seqstart_k)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    kind = ((MEA_MASK_CAUSAL if causal else 0) | (MEA_MASK_BLOCKDIAG if seqstart_q is not None else 0)
            | (MEA_BIAS_ALIBI if alibi_slopes is not None else 0))
    if workspace is None:
        workspace = torch.empty(bwd_workspace_bytes(B, M, Hq, kind), dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nbytes = workspace.numel() * workspace.element_size()
    if block_mask is not None:
        blk = block_sparse_block()
        if seqstart_q is not None or tuple(block_mask.shape) != (-(-M // blk), -(-N // blk)):
            raise ValueError("block_mask needs dense inputs and shape [ceil(M/64), ceil(N/64)]")
        _need_cuda(block_mask)
        _check(_lib.mea_bwd_blocksparse(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
                                        _ptr(dk), _ptr(dv), B, M, N, Hq, Hkv, D, float(scale), kind,
                                        _ptr(block_mask), _ptr(alibi_slopes), _dtype_code(q), _ptr(workspace),
                                        nbytes, _stream(stream)))
        return dq, dk, dv
    _check(_lib.mea_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        B, M, N, Hq, Hkv, D, float(scale), kind, _ptr(seqstart_q), _ptr(seqstart_k),
                        _ptr(alibi_slopes), _dtype_code(q), _ptr(workspace), nbytes, _stream(stream)))
    return dq, dk, dv


def decode(q, kcache, vcache, ctx_lens, *, scale: float | None = None, alibi_slopes=None, out=None,
           workspace=None, stream=None):
    """One KV-cache decode step (``mea_decode``): q ``[B,Hq,D]``, caches
    ``[B,S_max,Hkv,D]``, int32 ``ctx_lens`` ``[B]`` on the device. The workspace
    is allocated with torch when not given. Returns ``out`` ``[B,Hq,D]``."""
    torch = _torch()
    B, Hq, D = q.shape
    Bc, S_max, Hkv, Dc = kcache.shape
    if Bc != B or Dc != D or vcache.shape != kcache.shape:
        raise ValueError("q and cache shapes disagree")
    if kcache.dtype != q.dtype or vcache.dtype != q.dtype:
        raise ValueError("q and caches must share a dtype")
    if ctx_lens.dtype != torch.int32 or ctx_lens.numel() != B:
        raise TypeError("ctx_lens must be an int32 device tensor of B entries")
    _need_like(out, q.shape, q.dtype, "out")
    _need_numel(alibi_slopes, Hq, torch.float32, "alibi_slopes")
    _need_cuda(q, kcache, vcache, ctx_lens, out, alibi_slopes, workspace)
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_bytes(B, Hq, D, S_max)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(_lib.mea_decode(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(ctx_lens), _ptr(out), B, Hq, Hkv, D, S_max,
                           float(scale), _ptr(alibi_slopes), _dtype_code(q), _ptr(workspace),
                           workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def decode_noalloc(q, kcache, vcache, ctx_lens, out, *, scale: float | None = None, alibi_slopes=None,
                   stream=None):
    """``mea_decode_noalloc``: the decode step of :func:`decode` with the
    library's static per-device scratch instead of a workspace. ``out``
    ``[B,Hq,D]`` is required (this call allocates nothing). Calls that may
    overlap on one device race on the scratch."""
    torch = _torch()
    B, Hq, D = q.shape
    Bc, S_max, Hkv, Dc = kcache.shape
    if Bc != B or Dc != D or vcache.shape != kcache.shape:
        raise ValueError("q and cache shapes disagree")
    if kcache.dtype != q.dtype or vcache.dtype != q.dtype or out.dtype != q.dtype or out.shape != q.shape:
        raise ValueError("q, caches and out must share a dtype; out is shaped like q")
    if ctx_lens.dtype != torch.int32 or ctx_lens.numel() != B:
        raise TypeError("ctx_lens must be an int32 device tensor of B entries")
    _need_numel(alibi_slopes, Hq, torch.float32, "alibi_slopes")
    _need_cuda(q, kcache, vcache, ctx_lens, out, alibi_slopes)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(_lib.mea_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(ctx_lens), _ptr(out), B, Hq, Hkv, D,
                                   S_max, float(scale), _ptr(alibi_slopes), _dtype_code(q), _stream(stream)))
    return out


def fwd_kvcache(q, kcache, vcache, ctx_lens, *, causal: bool = True, alibi_slopes=None,
                scale: float | None = None, out=None, lse=None, stream=None):
    """Chunked prefill / multi-token decode (``mea_fwd_kvcache``): q ``[B,M,Hq,D]``
    are the M newest tokens of each sequence, already appended to the caches
    ``[B,S_max,Hkv,D]``; int32 ``ctx_lens`` ``[B]`` on the device."""
    torch = _torch()
    B, M, Hq, D = q.shape
    Bc, S_max, Hkv, Dc = kcache.shape
    if Bc != B or Dc != D or vcache.shape != kcache.shape:
        raise ValueError("q and cache shapes disagree")
    if kcache.dtype != q.dtype or vcache.dtype != q.dtype:
        raise ValueError("q and caches must share a dtype")
    if ctx_lens.dtype != torch.int32 or ctx_lens.numel() != B:
        raise TypeError("ctx_lens must be an int32 device tensor of B entries")
    _need_like(out, q.shape, q.dtype, "out")
    _need_numel(lse, B * Hq * M, torch.float32, "lse")
    _need_numel(alibi_slopes, Hq, torch.float32, "alibi_slopes")
    _need_cuda(q, kcache, vcache, ctx_lens, out, lse, alibi_slopes)
    if out is None:
        out = torch.empty_like(q)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kind = (MEA_MASK_CAUSAL if causal else 0) | (MEA_BIAS_ALIBI if alibi_slopes is not None else 0)
    _check(_lib.mea_fwd_kvcache(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(ctx_lens), _ptr(out), B, M, Hq, Hkv, D,
                                S_max, float(scale), kind, _ptr(alibi_slopes), _dtype_code(q), _ptr(lse),
                                _stream(stream)))
    return out


def kv_append(kcache, vcache, k_new, v_new, ctx_lens, *, stream=None):
    """Append ``k_new``/``v_new`` ``[B,T,Hkv,D]`` to the caches at rows
    ``ctx_lens[b] ..`` (``mea_kv_append``). ``ctx_lens`` is not updated."""
    torch = _torch()
    B, S_max, Hkv, D = kcache.shape
    Bn, T, Hn, Dn = k_new.shape
    if (Bn, Hn, Dn) != (B, Hkv, D) or v_new.shape != k_new.shape or vcache.shape != kcache.shape:
        raise ValueError("cache and new-row shapes disagree")
    if len({kcache.dtype, vcache.dtype, k_new.dtype, v_new.dtype}) != 1:
        raise ValueError("caches and new rows must share a dtype")
    if ctx_lens.dtype != torch.int32 or ctx_lens.numel() != B:
        raise TypeError("ctx_lens must be an int32 device tensor of B entries")
    _need_cuda(kcache, vcache, k_new, v_new, ctx_lens)
    _check(_lib.mea_kv_append(_ptr(kcache), _ptr(vcache), _ptr(k_new), _ptr(v_new), _ptr(ctx_lens), B, S_max, Hkv,
                              D, T, _dtype_code(kcache), _stream(stream)))
    return kcache, vcache
