"""Python binding of libfa355 (exact tiled attention on MI355X / gfx950).

Two layers, both argument marshalling only — every step of the computation
runs in the HIP kernels of ``libfa355.so``:

* ``fa_fwd``, ``fa_fwd_varlen``, ``fa_decode_splitkv``, ... mirror the C ABI
  of ``include/fa355.h`` one to one (integers for device pointers and the
  stream) and return the status code.
* ``fwd``, ``fwd_varlen``, ``decode_splitkv`` take torch tensors (torch
  provides device memory and streams), allocate outputs when none are
  given, call the C ABI on the current stream and raise ``FaError`` on a
  non-zero status.

There is no fallback: if the shared library is missing or cannot be loaded,
every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

__all__ = [
    "FA_F32", "FA_F16", "FA_BF16",
    "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_WORKSPACE", "FA_ERR_HIP",
    "FA_ERR_TOO_LARGE", "FA_NOALLOC_SCRATCH_BYTES", "fa_fwd_varlen_noalloc", "fwd_varlen_noalloc",
    "FaError", "library_path", "load",
    "fa_fwd", "fa_fwd_masked", "fa_fwd_dropout", "fa_bwd", "fa_bwd_masked", "fa_bwd_dropout",
    "fa_bwd_varlen", "fa_fwd_varlen_masked", "fa_fwd_varlen_dropout", "fa_bwd_varlen_masked",
    "fa_bwd_varlen_dropout", "fa_fwd_ex", "fa_bwd_ex", "fa_fwd_varlen_ex", "fa_bwd_varlen_ex",
    "fa_bwd_workspace_bytes", "fa_fwd_varlen", "fa_fwd_varlen_workspace_bytes", "fa_decode_splitkv",
    "fa_decode_splitkv_paged", "fa_decode_workspace_bytes", "fa_status_string", "fa_version",
    "fwd", "fwd_masked", "fwd_dropout", "fwd_ex", "bwd", "fwd_varlen", "bwd_varlen", "decode_splitkv",
    "decode_splitkv_paged",
]

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = 0, 1, 2, 3, 4
FA_ERR_TOO_LARGE = 5
FA_NOALLOC_SCRATCH_BYTES = 1 << 20

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_u64 = ctypes.c_uint64
_SIGS = {
    "fa_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _i, _vp]),
    "fa_fwd_masked": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _i, _vp, _i,
                           _vp]),
    "fa_fwd_dropout": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _f, _u64,
                            _i, _vp]),
    "fa_bwd_dropout": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                            _i, _vp, _f, _u64, _vp, _sz, _i, _vp]),
    "fa_bwd_masked": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                           _i, _vp, _i, _vp, _vp, _sz, _i, _vp]),
    "fa_bwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i,
                           _i, _i, _i, _f, _i, _vp, _sz, _i, _vp]),
    "fa_fwd_varlen_masked": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                                  _i, _vp, _vp, _sz, _i, _vp]),
    "fa_fwd_varlen_dropout": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                                   _f, _u64, _vp, _sz, _i, _vp]),
    "fa_bwd_varlen_masked": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i,
                                  _i, _i, _i, _i, _i, _f, _i, _i, _vp, _vp, _sz, _i, _vp]),
    "fa_bwd_varlen_dropout": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i,
                                   _i, _i, _i, _i, _i, _f, _i, _f, _u64, _vp, _sz, _i, _vp]),
    "fa_fwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp, _i, _vp, _f,
                       _u64, _i, _vp]),
    "fa_bwd_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                       _vp, _i, _vp, _f, _u64, _vp, _sz, _i, _vp]),
    "fa_fwd_varlen_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i,
                              _vp, _f, _u64, _vp, _sz, _i, _vp]),
    "fa_bwd_varlen_ex": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i,
                              _i, _i, _i, _i, _f, _i, _i, _vp, _f, _u64, _vp, _sz, _i, _vp]),
    "fa_bwd_workspace_bytes": (_sz, [_i, _i, _i]),
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp,
                    _vp, _sz, _i, _vp]),
    "fa_fwd_varlen_workspace_bytes": (_sz, [_i, _i]),
    "fa_fwd_varlen_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                                   _i, _vp]),
    "fa_fwd_varlen": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp,
                           _sz, _i, _vp]),
    "fa_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "fa_decode_splitkv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _f, _i, _vp, _sz,
                               _i, _vp]),
    "fa_decode_splitkv_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i,
                                     _f, _i, _vp, _sz, _i, _vp]),
    "fa_status_string": (ctypes.c_char_p, [_i]),
    "fa_version": (ctypes.c_char_p, []),
}


class FaError(RuntimeError):
    """A libfa355 call returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: status %d (%s)" % (fn, status, fa_status_string(status)))


def library_path() -> str:
    return os.environ.get("FA355_LIB", os.path.join(_HERE, "libfa355.so"))


def load() -> ctypes.CDLL:
    """Load libfa355.so (built by ``python -m exact_tiled_attention_11_amd.build``)."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError("libfa355.so not found at %s; build it with "
                              "`python -m exact_tiled_attention_11_amd.build`" % path)
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


# ---------------------------------------------------------------------------
# C ABI, one to one
# ---------------------------------------------------------------------------

def fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, dtype, stream) -> int:
    return load().fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, dtype, stream)


def fa_fwd_masked(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, prefix, alibi_slopes,
                  dtype, stream) -> int:
    return load().fa_fwd_masked(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, prefix,
                                alibi_slopes, dtype, stream)


def fa_fwd_dropout(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, dropout_p, seed,
                   dtype, stream) -> int:
    return load().fa_fwd_dropout(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k,
                                 dropout_p, seed, dtype, stream)


def fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, seqlens_k,
                   dropout_p, seed, workspace, workspace_bytes, dtype, stream) -> int:
    return load().fa_bwd_dropout(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal,
                                 seqlens_k, dropout_p, seed, workspace, workspace_bytes, dtype,
                                 stream)


def fa_bwd_masked(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, seqlens_k,
                  prefix, alibi_slopes, workspace, workspace_bytes, dtype, stream) -> int:
    return load().fa_bwd_masked(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal,
                                seqlens_k, prefix, alibi_slopes, workspace, workspace_bytes, dtype,
                                stream)


def fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, nseq, total_q,
                  total_k, max_seqlen_q, max_seqlen_k, H, D, scale, causal, workspace,
                  workspace_bytes, dtype, stream) -> int:
    return load().fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k,
                                nseq, total_q, total_k, max_seqlen_q, max_seqlen_k, H, D, scale,
                                causal, workspace, workspace_bytes, dtype, stream)


def fa_fwd_varlen_masked(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k, H,
                         D, scale, causal, prefix, alibi_slopes, workspace, workspace_bytes, dtype,
                         stream) -> int:
    return load().fa_fwd_varlen_masked(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q,
                                       total_k, H, D, scale, causal, prefix, alibi_slopes,
                                       workspace, workspace_bytes, dtype, stream)


def fa_fwd_varlen_dropout(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k, H,
                          D, scale, causal, dropout_p, seed, workspace, workspace_bytes, dtype,
                          stream) -> int:
    return load().fa_fwd_varlen_dropout(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq,
                                        total_q, total_k, H, D, scale, causal, dropout_p, seed,
                                        workspace, workspace_bytes, dtype, stream)


def fa_bwd_varlen_masked(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, nseq,
                         total_q, total_k, max_seqlen_q, max_seqlen_k, H, D, scale, causal, prefix,
                         alibi_slopes, workspace, workspace_bytes, dtype, stream) -> int:
    return load().fa_bwd_varlen_masked(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q,
                                       cu_seqlens_k, nseq, total_q, total_k, max_seqlen_q,
                                       max_seqlen_k, H, D, scale, causal, prefix, alibi_slopes,
                                       workspace, workspace_bytes, dtype, stream)


def fa_bwd_varlen_dropout(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, nseq,
                          total_q, total_k, max_seqlen_q, max_seqlen_k, H, D, scale, causal,
                          dropout_p, seed, workspace, workspace_bytes, dtype, stream) -> int:
    return load().fa_bwd_varlen_dropout(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q,
                                        cu_seqlens_k, nseq, total_q, total_k, max_seqlen_q,
                                        max_seqlen_k, H, D, scale, causal, dropout_p, seed,
                                        workspace, workspace_bytes, dtype, stream)


def fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, prefix, alibi_slopes,
              dropout_p, seed, dtype, stream) -> int:
    return load().fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, D, scale, causal, seqlens_k, prefix,
                            alibi_slopes, dropout_p, seed, dtype, stream)


def fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, seqlens_k, prefix,
              alibi_slopes, dropout_p, seed, workspace, workspace_bytes, dtype, stream) -> int:
    return load().fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal,
                            seqlens_k, prefix, alibi_slopes, dropout_p, seed, workspace,
                            workspace_bytes, dtype, stream)


def fa_fwd_varlen_ex(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k, H, D,
                     scale, causal, prefix, alibi_slopes, dropout_p, seed, workspace,
                     workspace_bytes, dtype, stream) -> int:
    return load().fa_fwd_varlen_ex(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q,
                                   total_k, H, D, scale, causal, prefix, alibi_slopes, dropout_p,
                                   seed, workspace, workspace_bytes, dtype, stream)


def fa_bwd_varlen_ex(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k, nseq, total_q,
                     total_k, max_seqlen_q, max_seqlen_k, H, D, scale, causal, prefix,
                     alibi_slopes, dropout_p, seed, workspace, workspace_bytes, dtype,
                     stream) -> int:
    return load().fa_bwd_varlen_ex(q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens_q, cu_seqlens_k,
                                   nseq, total_q, total_k, max_seqlen_q, max_seqlen_k, H, D,
                                   scale, causal, prefix, alibi_slopes, dropout_p, seed,
                                   workspace, workspace_bytes, dtype, stream)


def fa_bwd_workspace_bytes(B, H, Nq) -> int:
    return load().fa_bwd_workspace_bytes(B, H, Nq)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal, seqlens_k, workspace,
           workspace_bytes, dtype, stream) -> int:
    return load().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, D, scale, causal,
                         seqlens_k, workspace, workspace_bytes, dtype, stream)


def fa_fwd_varlen_workspace_bytes(nseq, total_q) -> int:
    return load().fa_fwd_varlen_workspace_bytes(nseq, total_q)


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k, H, D,
                  scale, causal, workspace, workspace_bytes, dtype, stream) -> int:
    return load().fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q,
                                total_k, H, D, scale, causal, workspace, workspace_bytes, dtype,
                                stream)


def fa_fwd_varlen_noalloc(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq, total_q, total_k,
                          H, D, scale, causal, dtype, stream) -> int:
    return load().fa_fwd_varlen_noalloc(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, nseq,
                                        total_q, total_k, H, D, scale, causal, dtype, stream)


def fa_decode_workspace_bytes(B, H, Nk_max, D, chunk) -> int:
    return load().fa_decode_workspace_bytes(B, H, Nk_max, D, chunk)


def fa_decode_splitkv(q, k_cache, v_cache, o, lse, seqlens_k, B, H, Nk_max, D, scale, chunk,
                      workspace, workspace_bytes, dtype, stream) -> int:
    return load().fa_decode_splitkv(q, k_cache, v_cache, o, lse, seqlens_k, B, H, Nk_max, D,
                                    scale, chunk, workspace, workspace_bytes, dtype, stream)


def fa_decode_splitkv_paged(q, k_pages, v_pages, o, lse, seqlens_k, block_table, B, H, num_pages,
                            page_size, max_pages, D, scale, chunk, workspace, workspace_bytes,
                            dtype, stream) -> int:
    return load().fa_decode_splitkv_paged(q, k_pages, v_pages, o, lse, seqlens_k, block_table, B,
                                          H, num_pages, page_size, max_pages, D, scale, chunk,
                                          workspace, workspace_bytes, dtype, stream)


def fa_status_string(status: int) -> str:
    return load().fa_status_string(status).decode()


def fa_version() -> str:
    return load().fa_version().decode()


# ---------------------------------------------------------------------------
# torch convenience layer
# ---------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}
    if t.dtype not in codes:
        raise FaError("dtype", FA_ERR_UNSUPPORTED)
    return codes[t.dtype]


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, status: int) -> None:
    if status != FA_OK:
        raise FaError(fn, status)


def _expect(t, name: str, shape, dtype, device=None) -> None:
    """Raise ValueError unless tensor t (if given) has this shape, dtype and device.  The
    kernels address every buffer from the sizes of q (and k), so a mismatch would make them
    read or write past an allocation."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError("%s must be %s of shape %s, got %s of shape %s"
                         % (name, dtype, list(shape), t.dtype, list(t.shape)))
    if device is not None and t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))


def _index(t, name: str, n: int, device) -> None:
    """int32 index vector of n entries (cu_seqlens, seqlens_k)."""
    import torch
    if t is None:
        return
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() != n:
        raise ValueError("%s must be int32 of shape [%d], got %s of shape %s"
                         % (name, n, t.dtype, list(t.shape)))
    if t.device != device:
        raise ValueError("%s must be on %s, got %s" % (name, device, t.device))


def _check_fixed(q, k, v, seqlens_k, alibi_slopes, out, lse):
    """Shapes of a fixed-length call: q [B,Nq,H,D], k and v [B,Nk,H,D] of q's dtype."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B,Nq,H,D], [B,Nk,H,D], [B,Nk,H,D] of one dtype")
    B, Nq, H, D = q.shape
    Nk = k.shape[1]
    if k.shape != (B, Nk, H, D) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must be [B,Nq,H,D], [B,Nk,H,D], [B,Nk,H,D] of one dtype")
    _expect(k, "k", k.shape, q.dtype, q.device)
    _expect(v, "v", k.shape, q.dtype, q.device)
    _expect(out, "out", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, H, Nq), torch.float32, q.device)
    _index(seqlens_k, "seqlens_k", B, q.device)
    _expect(alibi_slopes, "alibi_slopes", (H,), torch.float32, q.device)
    return B, Nq, H, D, Nk


def _check_packed(q, k, v, cu_seqlens_q, cu_seqlens_k, alibi_slopes, out, lse):
    """Shapes of a packed call: q [total_q,H,D], k and v [total_k,H,D] of q's dtype, int32
    cu_seqlens of equal length."""
    import torch
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("q, k, v must be [total_q,H,D], [total_k,H,D], [total_k,H,D] of one dtype")
    total_q, H, D = q.shape
    total_k = k.shape[0]
    if k.shape != (total_k, H, D) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must be [total_q,H,D], [total_k,H,D], [total_k,H,D] of one dtype")
    _expect(k, "k", k.shape, q.dtype, q.device)
    _expect(v, "v", k.shape, q.dtype, q.device)
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q must be int32 of shape [nseq + 1]")
    nseq = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != nseq + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    _index(cu_seqlens_q, "cu_seqlens_q", nseq + 1, q.device)
    _index(cu_seqlens_k, "cu_seqlens_k", nseq + 1, q.device)
    _expect(out, "out", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (H, total_q), torch.float32, q.device)
    _expect(alibi_slopes, "alibi_slopes", (H,), torch.float32, q.device)
    return total_q, H, D, total_k, nseq


def fwd(q, k, v, *, causal: bool = False, scale: Optional[float] = None, seqlens_k=None,
        out=None, lse=None, return_lse: bool = True, stream=None) -> Tuple:
    """Fixed-length attention. q [B, Nq, H, D]; k, v [B, Nk, H, D] -> (o, lse [B, H, Nq])."""
    import torch
    B, Nq, H, D, Nk = _check_fixed(q, k, v, seqlens_k, None, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, D, float(scale),
                int(bool(causal)), _ptr(seqlens_k), _dtype_code(q), _stream(stream))
    _check("fa_fwd", st)
    return out, lse


def fwd_masked(q, k, v, *, causal: bool = False, scale: Optional[float] = None, seqlens_k=None,
               prefix: int = 0, alibi_slopes=None, out=None, lse=None, return_lse: bool = True,
               stream=None) -> Tuple:
    """fwd with the prefix mask (causal only) and/or ALiBi slopes (float32 [H] on the device)."""
    import torch
    B, Nq, H, D, Nk = _check_fixed(q, k, v, seqlens_k, alibi_slopes, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = fa_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, D,
                       float(scale), int(bool(causal)), _ptr(seqlens_k), int(prefix),
                       _ptr(alibi_slopes), _dtype_code(q), _stream(stream))
    _check("fa_fwd_masked", st)
    return out, lse


def fwd_dropout(q, k, v, *, dropout_p: float, seed: int, causal: bool = False,
                scale: Optional[float] = None, seqlens_k=None, out=None, lse=None,
                return_lse: bool = True, stream=None) -> Tuple:
    """fwd with attention dropout (training): keep decisions from Philox4x32-10 keyed by seed."""
    import torch
    B, Nq, H, D, Nk = _check_fixed(q, k, v, seqlens_k, None, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, D,
                        float(scale), int(bool(causal)), _ptr(seqlens_k), float(dropout_p),
                        int(seed) & 0xFFFFFFFFFFFFFFFF, _dtype_code(q), _stream(stream))
    _check("fa_fwd_dropout", st)
    return out, lse


def fwd_ex(q, k, v, *, causal: bool = False, scale: Optional[float] = None, seqlens_k=None,
           prefix: int = 0, alibi_slopes=None, dropout_p: float = 0.0, seed: int = 0, out=None,
           lse=None, return_lse: bool = True, stream=None) -> Tuple:
    """fwd with every option at once: the prefix mask (causal only), ALiBi slopes (float32 [H]
    on the device) and attention dropout (fp16/bf16 for any option)."""
    import torch
    B, Nq, H, D, Nk = _check_fixed(q, k, v, seqlens_k, alibi_slopes, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    st = fa_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, D, float(scale),
                   int(bool(causal)), _ptr(seqlens_k), int(prefix), _ptr(alibi_slopes),
                   float(dropout_p), int(seed) & 0xFFFFFFFFFFFFFFFF, _dtype_code(q),
                   _stream(stream))
    _check("fa_fwd_ex", st)
    return out, lse


def bwd(q, k, v, o, lse, dout, *, causal: bool = False, scale: Optional[float] = None,
        seqlens_k=None, dropout_p: float = 0.0, seed: int = 0, prefix: int = 0,
        alibi_slopes=None, dq=None, dk=None, dv=None, workspace=None, stream=None) -> Tuple:
    """Gradients (dq, dk, dv) for the forward fwd(q, k, v) that produced o and lse, given dout
    (with dropout_p > 0: for fwd_dropout with the same dropout_p and seed; with prefix or
    alibi_slopes: for fwd_masked with the same ones; with both: for fwd_ex)."""
    import torch
    B, Nq, H, D, Nk = _check_fixed(q, k, v, seqlens_k, alibi_slopes, None, lse)
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(dout, "dout", q.shape, q.dtype, q.device)
    _expect(dq, "dq", q.shape, q.dtype, q.device)
    _expect(dk, "dk", k.shape, q.dtype, q.device)
    _expect(dv, "dv", k.shape, q.dtype, q.device)
    if lse is None or o is None or dout is None:
        raise ValueError("o, lse and dout of the forward call are required")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(max(fa_bwd_workspace_bytes(B, H, Nq), 16), dtype=torch.uint8,
                                device=q.device)
    if dropout_p and (prefix or alibi_slopes is not None):
        st = fa_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                       _ptr(dk), _ptr(dv), B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                       _ptr(seqlens_k), int(prefix), _ptr(alibi_slopes), float(dropout_p),
                       int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(workspace), workspace.numel(),
                       _dtype_code(q), _stream(stream))
        _check("fa_bwd_ex", st)
        return dq, dk, dv
    if prefix or alibi_slopes is not None:
        st = fa_bwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                           _ptr(dk), _ptr(dv), B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                           _ptr(seqlens_k), int(prefix), _ptr(alibi_slopes), _ptr(workspace),
                           workspace.numel(), _dtype_code(q), _stream(stream))
        _check("fa_bwd_masked", st)
        return dq, dk, dv
    if dropout_p:
        st = fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                            _ptr(dk), _ptr(dv), B, H, Nq, Nk, D, float(scale), int(bool(causal)),
                            _ptr(seqlens_k), float(dropout_p), int(seed) & 0xFFFFFFFFFFFFFFFF,
                            _ptr(workspace), workspace.numel(), _dtype_code(q), _stream(stream))
        _check("fa_bwd_dropout", st)
        return dq, dk, dv
    st = fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                _ptr(dv), B, H, Nq, Nk, D, float(scale), int(bool(causal)), _ptr(seqlens_k),
                _ptr(workspace), workspace.numel(), _dtype_code(q), _stream(stream))
    _check("fa_bwd", st)
    return dq, dk, dv


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, causal: bool = False,
               scale: Optional[float] = None, prefix: int = 0, alibi_slopes=None,
               dropout_p: float = 0.0, seed: int = 0, out=None, lse=None, return_lse: bool = True,
               workspace=None, stream=None) -> Tuple:
    """Packed varlen attention. q [total_q, H, D], k, v [total_k, H, D] -> (o, lse [H, total_q]).
    prefix / alibi_slopes (float32 [H] on the device) select fa_fwd_varlen_masked, dropout_p > 0
    fa_fwd_varlen_dropout (positions and dropout counters per sequence)."""
    import torch
    total_q, H, D, total_k, nseq = _check_packed(q, k, v, cu_seqlens_q, cu_seqlens_k,
                                                 alibi_slopes, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    need = fa_fwd_varlen_workspace_bytes(max(nseq, 1), total_q)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    common = (_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
              _ptr(cu_seqlens_k), nseq, total_q, total_k, H, D, float(scale), int(bool(causal)))
    tail = (_ptr(workspace), workspace.numel(), _dtype_code(q), _stream(stream))
    if dropout_p and (prefix or alibi_slopes is not None):
        st = fa_fwd_varlen_ex(*common, int(prefix), _ptr(alibi_slopes), float(dropout_p),
                              int(seed) & 0xFFFFFFFFFFFFFFFF, *tail)
        _check("fa_fwd_varlen_ex", st)
    elif dropout_p:
        st = fa_fwd_varlen_dropout(*common, float(dropout_p), int(seed) & 0xFFFFFFFFFFFFFFFF, *tail)
        _check("fa_fwd_varlen_dropout", st)
    elif prefix or alibi_slopes is not None:
        st = fa_fwd_varlen_masked(*common, int(prefix), _ptr(alibi_slopes), *tail)
        _check("fa_fwd_varlen_masked", st)
    else:
        st = fa_fwd_varlen(*common, *tail)
        _check("fa_fwd_varlen", st)
    return out, lse


def fwd_varlen_noalloc(q, k, v, cu_seqlens_q, cu_seqlens_k, *, causal: bool = False,
                       scale: Optional[float] = None, out=None, lse=None, return_lse: bool = True,
                       stream=None) -> Tuple:
    """fwd_varlen through fa_fwd_varlen_noalloc: the library allocates nothing (the tile
    schedule lives in its static per-GPU scratch; calls that overlap on one GPU race).  Pass
    out (and lse) to allocate nothing here either."""
    import torch
    total_q, H, D, total_k, nseq = _check_packed(q, k, v, cu_seqlens_q, cu_seqlens_k, None, out,
                                                 lse)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    st = fa_fwd_varlen_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                               _ptr(cu_seqlens_k), nseq, total_q, total_k, H, D, float(scale),
                               int(bool(causal)), _dtype_code(q), _stream(stream))
    _check("fa_fwd_varlen_noalloc", st)
    return out, lse


def bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, *, causal: bool = False,
               scale: Optional[float] = None, max_seqlen_q: Optional[int] = None,
               max_seqlen_k: Optional[int] = None, prefix: int = 0, alibi_slopes=None,
               dropout_p: float = 0.0, seed: int = 0, dq=None, dk=None, dv=None, workspace=None,
               stream=None) -> Tuple:
    """Gradients for fwd_varlen (packed q [total_q, H, D], k, v [total_k, H, D], lse [H, total_q]),
    with the forward call's prefix / alibi_slopes / dropout_p and seed.
    max_seqlen_q / max_seqlen_k default to the longest ranges of cu_seqlens (read on the host:
    pass them to avoid that synchronisation)."""
    import torch
    total_q, H, D, total_k, nseq = _check_packed(q, k, v, cu_seqlens_q, cu_seqlens_k,
                                                 alibi_slopes, None, lse)
    _expect(o, "o", q.shape, q.dtype, q.device)
    _expect(dout, "dout", q.shape, q.dtype, q.device)
    _expect(dq, "dq", q.shape, q.dtype, q.device)
    _expect(dk, "dk", k.shape, q.dtype, q.device)
    _expect(dv, "dv", k.shape, q.dtype, q.device)
    if lse is None or o is None or dout is None:
        raise ValueError("o, lse and dout of the forward call are required")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seqlen_q is None:
        max_seqlen_q = int(torch.diff(cu_seqlens_q).max().item()) if nseq > 0 else 0
    if max_seqlen_k is None:
        max_seqlen_k = int(torch.diff(cu_seqlens_k).max().item()) if nseq > 0 else 0
    dq = torch.zeros_like(q) if dq is None else dq
    dk = torch.zeros_like(k) if dk is None else dk
    dv = torch.zeros_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(max(fa_bwd_workspace_bytes(1, H, total_q), 16), dtype=torch.uint8,
                                device=q.device)
    common = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
              _ptr(dv), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), nseq, total_q, total_k,
              int(max_seqlen_q), int(max_seqlen_k), H, D, float(scale), int(bool(causal)))
    tail = (_ptr(workspace), workspace.numel(), _dtype_code(q), _stream(stream))
    if dropout_p and (prefix or alibi_slopes is not None):
        st = fa_bwd_varlen_ex(*common, int(prefix), _ptr(alibi_slopes), float(dropout_p),
                              int(seed) & 0xFFFFFFFFFFFFFFFF, *tail)
        _check("fa_bwd_varlen_ex", st)
    elif dropout_p:
        st = fa_bwd_varlen_dropout(*common, float(dropout_p), int(seed) & 0xFFFFFFFFFFFFFFFF, *tail)
        _check("fa_bwd_varlen_dropout", st)
    elif prefix or alibi_slopes is not None:
        st = fa_bwd_varlen_masked(*common, int(prefix), _ptr(alibi_slopes), *tail)
        _check("fa_bwd_varlen_masked", st)
    else:
        st = fa_bwd_varlen(*common, *tail)
        _check("fa_bwd_varlen", st)
    return dq, dk, dv


def decode_splitkv(q, k_cache, v_cache, seqlens_k, *, scale: Optional[float] = None,
                   chunk: int = 256, out=None, lse=None, return_lse: bool = True,
                   workspace=None, stream=None) -> Tuple:
    """Split-KV decode. q [B, H, D]; caches [B, Nk_max, H, D] -> (o [B, H, D], lse [B, H])."""
    import torch
    if q.dim() != 3 or k_cache.dim() != 4:
        raise ValueError("q must be [B,H,D] and the caches [B,Nk_max,H,D]")
    B, H, D = q.shape
    Nk_max = k_cache.shape[1]
    _expect(k_cache, "k_cache", (B, Nk_max, H, D), q.dtype, q.device)
    _expect(v_cache, "v_cache", (B, Nk_max, H, D), q.dtype, q.device)
    if seqlens_k is None:
        raise ValueError("seqlens_k is required")
    _index(seqlens_k, "seqlens_k", B, q.device)
    _expect(out, "out", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, H), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    need = fa_decode_workspace_bytes(B, H, Nk_max, D, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = fa_decode_splitkv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse),
                           _ptr(seqlens_k), B, H, Nk_max, D, float(scale), chunk,
                           _ptr(workspace), workspace.numel(), _dtype_code(q), _stream(stream))
    _check("fa_decode_splitkv", st)
    return out, lse


def decode_splitkv_paged(q, k_pages, v_pages, seqlens_k, block_table, *,
                         scale: Optional[float] = None, chunk: int = 256, out=None, lse=None,
                         return_lse: bool = True, workspace=None, stream=None) -> Tuple:
    """Split-KV decode over a paged cache. q [B, H, D]; pages [num_pages, page_size, H, D];
    block_table int32 [B, max_pages] -> (o [B, H, D], lse [B, H])."""
    import torch
    if q.dim() != 3 or k_pages.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q must be [B,H,D], the pages [num_pages,page_size,H,D] and "
                         "block_table [B,max_pages]")
    B, H, D = q.shape
    num_pages, page_size = k_pages.shape[0], k_pages.shape[1]
    max_pages = block_table.shape[1]
    _expect(k_pages, "k_pages", (num_pages, page_size, H, D), q.dtype, q.device)
    _expect(v_pages, "v_pages", (num_pages, page_size, H, D), q.dtype, q.device)
    _expect(block_table, "block_table", (B, max_pages), torch.int32, q.device)
    if seqlens_k is None:
        raise ValueError("seqlens_k is required")
    _index(seqlens_k, "seqlens_k", B, q.device)
    _expect(out, "out", q.shape, q.dtype, q.device)
    _expect(lse, "lse", (B, H), torch.float32, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    need = fa_decode_workspace_bytes(B, H, max_pages * page_size, D, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = fa_decode_splitkv_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(out), _ptr(lse),
                                 _ptr(seqlens_k), _ptr(block_table), B, H, num_pages, page_size,
                                 max_pages, D, float(scale), chunk, _ptr(workspace),
                                 workspace.numel(), _dtype_code(q), _stream(stream))
    _check("fa_decode_splitkv_paged", st)
    return out, lse
