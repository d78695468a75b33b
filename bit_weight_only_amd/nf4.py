"""ctypes binding of libnf4.so with the same entry-point names as include/nf4.h.

Argument marshalling only: every step of the layer runs in the HIP kernels.
Tensors supply device pointers; the stream defaults to torch's current
stream.  A missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4.so")

NF4_OK, NF4_ERR_NULL, NF4_ERR_SHAPE, NF4_ERR_ALIGN, NF4_ERR_CODEBOOK, NF4_ERR_WORKSPACE, \
    NF4_ERR_HIP, NF4_ERR_SCRATCH = range(8)

EXPORTS = ("nf4_status_string", "nf4_codebook", "nf4_qweight_bytes", "nf4_absmax_bytes", "nf4_workspace_bytes",
           "nf4_pack", "nf4_dequant", "nf4_repack", "nf4_unpack", "nf4_gemv", "nf4_gemm",
           "nf4_gemv_argmax_workspace_bytes", "nf4_gemv_argmax", "nf4_gemv_argmax_noalloc",
           "nf4_gemv_prefetch",
           "nf4_awq_params_bytes", "nf4_awq_workspace_bytes", "nf4_awq_pack", "nf4_awq_repack",
           "nf4_awq_unpack", "nf4_awq_dequant", "nf4_gather_columns", "nf4_awq_gemv_prefetch", "nf4_awq_gemv", "nf4_awq_gemm")

_lib = None


class NF4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {nf4_status_string(status)}")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_weight_only_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, sz, st = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        fp = ctypes.POINTER(ctypes.c_float)
        L.nf4_status_string.restype = ctypes.c_char_p
        L.nf4_status_string.argtypes = [st]
        L.nf4_codebook.restype = st
        L.nf4_codebook.argtypes = [ctypes.c_double, fp]
        for f in (L.nf4_qweight_bytes, L.nf4_absmax_bytes):
            f.restype = sz
            f.argtypes = [i64, i64]
        L.nf4_workspace_bytes.restype = sz
        L.nf4_workspace_bytes.argtypes = [i64, i64, i64]
        L.nf4_pack.restype = st
        L.nf4_pack.argtypes = [vp, i64, i64, fp, vp, vp, vp]
        L.nf4_dequant.restype = st
        L.nf4_dequant.argtypes = [vp, vp, fp, i64, i64, vp, vp]
        L.nf4_repack.restype = st
        L.nf4_repack.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        L.nf4_unpack.restype = st
        L.nf4_unpack.argtypes = [vp, vp, i64, i64, vp, vp, vp]
        for f in (L.nf4_gemv, L.nf4_gemm):
            f.restype = st
            f.argtypes = [vp, i64, vp, vp, fp, i64, i64, vp, vp, sz, vp]
        L.nf4_gemv_argmax_workspace_bytes.restype = sz
        L.nf4_gemv_argmax_workspace_bytes.argtypes = [i64, i64, i64]
        L.nf4_gemv_argmax.restype = st
        L.nf4_gemv_argmax.argtypes = [vp, i64, vp, vp, fp, i64, i64, vp, vp, vp, sz, vp]
        L.nf4_gemv_argmax_noalloc.restype = st
        L.nf4_gemv_argmax_noalloc.argtypes = [vp, i64, vp, vp, fp, i64, i64, vp, vp, vp]
        L.nf4_gemv_prefetch.restype = st
        L.nf4_gemv_prefetch.argtypes = [vp, i64, vp, vp, fp, i64, i64, vp, vp, sz, vp, vp, i64,
                                        i64, vp]
        L.nf4_awq_params_bytes.restype = sz
        L.nf4_awq_params_bytes.argtypes = [i64, i64]
        L.nf4_awq_workspace_bytes.restype = sz
        L.nf4_awq_workspace_bytes.argtypes = [i64, i64, i64]
        L.nf4_awq_pack.restype = st
        L.nf4_awq_pack.argtypes = [vp, i64, i64, vp, vp, vp]
        L.nf4_awq_repack.restype = st
        L.nf4_awq_repack.argtypes = [vp, vp, vp, i64, i64, vp, vp, vp]
        L.nf4_awq_unpack.restype = st
        L.nf4_awq_unpack.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp]
        L.nf4_awq_dequant.restype = st
        L.nf4_awq_dequant.argtypes = [vp, vp, i64, i64, vp, vp]
        L.nf4_awq_gemv_prefetch.restype = st
        L.nf4_awq_gemv_prefetch.argtypes = [vp, i64, vp, vp, i64, i64, vp, vp, sz, vp, vp, i64,
                                            i64, vp]
        L.nf4_gather_columns.restype = st
        L.nf4_gather_columns.argtypes = [vp, i64, i64, vp, vp, vp]
        for f in (L.nf4_awq_gemv, L.nf4_awq_gemm):
            f.restype = st
            f.argtypes = [vp, i64, vp, vp, i64, i64, vp, vp, sz, vp]
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _codebook(cb) -> ctypes.Array:
    a = np.ascontiguousarray(np.asarray(cb, dtype=np.float32).reshape(16))
    return (ctypes.c_float * 16)(*a.tolist())


def _check(status: int, where: str) -> None:
    if status != NF4_OK:
        raise NF4Error(status, where)


def nf4_status_string(status: int) -> str:
    return lib().nf4_status_string(int(status)).decode()


DEFAULT_DELTA = 0.9677083  # tail probability of the default codebook


def nf4_codebook(delta: float = DEFAULT_DELTA) -> np.ndarray:
    """The library's default 16-entry codebook (host computation): normal
    quantiles normalised to [-1, 1] with an exact zero, each a bfloat16 value."""
    out = (ctypes.c_float * 16)()
    _check(lib().nf4_codebook(float(delta), out), "nf4_codebook")
    return np.array(out[:], dtype=np.float32)


def nf4_qweight_bytes(N: int, K: int) -> int:
    return lib().nf4_qweight_bytes(N, K)


def nf4_absmax_bytes(N: int, K: int) -> int:
    return lib().nf4_absmax_bytes(N, K)


def nf4_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib().nf4_workspace_bytes(M, N, K)


def nf4_pack(W, N: int, K: int, codebook, qweight, absmax, stream=None) -> None:
    _check(lib().nf4_pack(_ptr(W), N, K, _codebook(codebook), _ptr(qweight), _ptr(absmax),
                          _stream(stream)), "nf4_pack")


def nf4_dequant(qweight, absmax, codebook, N: int, K: int, W_out, stream=None) -> None:
    _check(lib().nf4_dequant(_ptr(qweight), _ptr(absmax), _codebook(codebook), N, K,
                             _ptr(W_out), _stream(stream)), "nf4_dequant")


def nf4_repack(codes, scales, N: int, K: int, qweight, absmax, stream=None) -> None:
    _check(lib().nf4_repack(_ptr(codes), _ptr(scales), N, K, _ptr(qweight), _ptr(absmax),
                            _stream(stream)), "nf4_repack")


def nf4_unpack(qweight, absmax, N: int, K: int, codes, scales, stream=None) -> None:
    _check(lib().nf4_unpack(_ptr(qweight), _ptr(absmax), N, K, _ptr(codes), _ptr(scales),
                            _stream(stream)), "nf4_unpack")


def nf4_gemv(x, M: int, qweight, absmax, codebook, N: int, K: int, y, workspace=None,
             ws_bytes: int = 0, stream=None) -> None:
    _check(lib().nf4_gemv(_ptr(x), M, _ptr(qweight), _ptr(absmax), _codebook(codebook), N, K,
                          _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)), "nf4_gemv")


def nf4_gemv_prefetch(x, M: int, qweight, absmax, codebook, N: int, K: int, y, workspace=None,
                      ws_bytes: int = 0, next_qweight=None, next_absmax=None, next_N: int = 0,
                      next_K: int = 0, stream=None) -> None:
    _check(lib().nf4_gemv_prefetch(_ptr(x), M, _ptr(qweight), _ptr(absmax), _codebook(codebook),
                                   N, K, _ptr(y), _ptr(workspace), ws_bytes, _ptr(next_qweight),
                                   _ptr(next_absmax), next_N, next_K, _stream(stream)),
           "nf4_gemv_prefetch")


def nf4_gemm(x, M: int, qweight, absmax, codebook, N: int, K: int, y, workspace=None,
             ws_bytes: int = 0, stream=None) -> None:
    _check(lib().nf4_gemm(_ptr(x), M, _ptr(qweight), _ptr(absmax), _codebook(codebook), N, K,
                          _ptr(y), _ptr(workspace), ws_bytes, _stream(stream)), "nf4_gemm")


def nf4_gemv_argmax_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib().nf4_gemv_argmax_workspace_bytes(M, N, K)


def nf4_gemv_argmax(x, M: int, qweight, absmax, codebook, N: int, K: int, y, index, workspace,
                    ws_bytes: int, stream=None) -> None:
    _check(lib().nf4_gemv_argmax(_ptr(x), M, _ptr(qweight), _ptr(absmax), _codebook(codebook),
                                 N, K, _ptr(y), _ptr(index), _ptr(workspace), ws_bytes,
                                 _stream(stream)), "nf4_gemv_argmax")


def nf4_gemv_argmax_noalloc(x, M: int, qweight, absmax, codebook, N: int, K: int, y, index,
                            stream=None) -> None:
    _check(lib().nf4_gemv_argmax_noalloc(_ptr(x), M, _ptr(qweight), _ptr(absmax),
                                         _codebook(codebook), N, K, _ptr(y), _ptr(index),
                                         _stream(stream)), "nf4_gemv_argmax_noalloc")


def nf4_awq_params_bytes(N: int, K: int) -> int:
    return lib().nf4_awq_params_bytes(N, K)


def nf4_awq_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib().nf4_awq_workspace_bytes(M, N, K)


def nf4_awq_pack(W, N: int, K: int, qweight, params, stream=None) -> None:
    _check(lib().nf4_awq_pack(_ptr(W), N, K, _ptr(qweight), _ptr(params), _stream(stream)),
           "nf4_awq_pack")


def nf4_awq_repack(codes, scales, zeros, N: int, K: int, qweight, params, stream=None) -> None:
    _check(lib().nf4_awq_repack(_ptr(codes), _ptr(scales), _ptr(zeros), N, K, _ptr(qweight),
                                _ptr(params), _stream(stream)), "nf4_awq_repack")


def nf4_awq_unpack(qweight, params, N: int, K: int, codes, scales, zeros, stream=None) -> None:
    _check(lib().nf4_awq_unpack(_ptr(qweight), _ptr(params), N, K, _ptr(codes), _ptr(scales),
                                _ptr(zeros), _stream(stream)), "nf4_awq_unpack")


def nf4_awq_dequant(qweight, params, N: int, K: int, W_out, stream=None) -> None:
    _check(lib().nf4_awq_dequant(_ptr(qweight), _ptr(params), N, K, _ptr(W_out),
                                 _stream(stream)), "nf4_awq_dequant")


def nf4_gather_columns(x, M: int, K: int, perm, x_out, stream=None) -> None:
    _check(lib().nf4_gather_columns(_ptr(x), M, K, _ptr(perm), _ptr(x_out), _stream(stream)),
           "nf4_gather_columns")


def nf4_awq_gemv(x, M: int, qweight, params, N: int, K: int, y, workspace=None,
                 ws_bytes: int = 0, stream=None) -> None:
    _check(lib().nf4_awq_gemv(_ptr(x), M, _ptr(qweight), _ptr(params), N, K, _ptr(y),
                              _ptr(workspace), ws_bytes, _stream(stream)), "nf4_awq_gemv")


def nf4_awq_gemv_prefetch(x, M: int, qweight, params, N: int, K: int, y, workspace=None,
                          ws_bytes: int = 0, next_qweight=None, next_params=None,
                          next_N: int = 0, next_K: int = 0, stream=None) -> None:
    _check(lib().nf4_awq_gemv_prefetch(_ptr(x), M, _ptr(qweight), _ptr(params), N, K, _ptr(y),
                                       _ptr(workspace), ws_bytes, _ptr(next_qweight),
                                       _ptr(next_params), next_N, next_K, _stream(stream)),
           "nf4_awq_gemv_prefetch")


def nf4_awq_gemm(x, M: int, qweight, params, N: int, K: int, y, workspace=None,
                 ws_bytes: int = 0, stream=None) -> None:
    _check(lib().nf4_awq_gemm(_ptr(x), M, _ptr(qweight), _ptr(params), N, K, _ptr(y),
                              _ptr(workspace), ws_bytes, _stream(stream)), "nf4_awq_gemm")


# ------------------------------------------------------------ conveniences
class PackedWeight:
    """Device-layout codes and scales of one N x K weight (torch uint8/fp32)."""

    def __init__(self, N: int, K: int, device="cuda"):
        import torch
        qb, ab = nf4_qweight_bytes(N, K), nf4_absmax_bytes(N, K)
        if qb == 0:
            raise NF4Error(NF4_ERR_SHAPE, "PackedWeight")
        self.N, self.K = N, K
        self.qweight = torch.empty(qb, dtype=torch.uint8, device=device)
        self.absmax = torch.empty(ab // 4, dtype=torch.float32, device=device)

    @property
    def nbytes(self) -> int:
        """Algorithmic bytes a full read moves: 4-bit codes plus fp32 scales."""
        return self.N * self.K // 2 + 4 * self.N * (self.K // 64)

    def rows(self, n0: int, n1: int) -> "PackedWeight":
        """Rows [n0, n1) as a view of this weight's buffers (one part of a
        matrix fused along N; n0, n1 multiples of 16).  The device layout keeps
        each group of 16 rows contiguous, so the part is itself a weight in
        the device layout."""
        if n0 % 16 or n1 % 16 or not 0 <= n0 < n1 <= self.N:
            raise NF4Error(NF4_ERR_SHAPE, "PackedWeight.rows")
        v = PackedWeight.__new__(PackedWeight)
        v.N, v.K = n1 - n0, self.K
        per_q = self.qweight.numel() // (self.N // 16)
        per_a = self.absmax.numel() // (self.N // 16)
        v.qweight = self.qweight[n0 // 16 * per_q:n1 // 16 * per_q]
        v.absmax = self.absmax[n0 // 16 * per_a:n1 // 16 * per_a]
        return v


def pack_weight(W, codebook, stream=None) -> PackedWeight:
    """Quantize a device fp32 [N, K] tensor into a new PackedWeight."""
    N, K = W.shape
    pw = PackedWeight(N, K, device=W.device)
    nf4_pack(W, N, K, codebook, pw.qweight, pw.absmax, stream)
    return pw


class AwqWeight:
    """Device-layout codes and (s, z) params (int32 dwords) of one N x K int4 weight."""

    def __init__(self, N: int, K: int, device="cuda"):
        import torch
        qb, pb = nf4_qweight_bytes(N, K), nf4_awq_params_bytes(N, K)
        if qb == 0 or pb == 0:
            raise NF4Error(NF4_ERR_SHAPE, "AwqWeight")
        self.N, self.K = N, K
        self.qweight = torch.empty(qb, dtype=torch.uint8, device=device)
        self.params = torch.empty(pb // 4, dtype=torch.int32, device=device)

    @property
    def nbytes(self) -> int:
        """Algorithmic bytes a full read moves: 4-bit codes plus one 4-byte (s, z) per group."""
        return self.N * self.K // 2 + 4 * self.N * (self.K // 128)


def awq_pack_weight(W, stream=None) -> AwqWeight:
    """Quantize a device fp32 [N, K] tensor into a new AwqWeight."""
    N, K = W.shape
    aw = AwqWeight(N, K, device=W.device)
    nf4_awq_pack(W, N, K, aw.qweight, aw.params, stream)
    return aw
