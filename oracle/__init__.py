"""CPU oracle for the NF4-style 4-bit weight-only linear layer.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use it.  The product library never imports,
links or runs anything here, and nothing here imports the product package.

The arithmetic lives in ``nf4_oracle.c`` (plain scalar C, fp64 reductions,
built without fast-math or contraction); this module only marshals numpy
arrays through ctypes and states the acceptance test.

Page cited throughout: the vibevoice.c README (section "Quantization" >
"Weights"), which fixes blocks of 64 weights along the input dimension with
one absmax scale each, codes that index a non-uniform table, and a
deterministic quantizer run once at load.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nf4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BLOCK = 64
# Tail probability of the normal-quantile construction.  The pages never
# print the table; this value is the reading taken for it (a common choice
# for NF4 tables) and nothing downstream depends on it: every kernel takes
# the codebook as an argument.
DELTA = 0.9677083

_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle into ``oracle/liboracle.so`` with gcc."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm", "-lpthread"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        d, i64, vp = ctypes.c_double, ctypes.c_int64, ctypes.c_void_p
        L.oracle_norm_cdf.restype = d
        L.oracle_norm_cdf.argtypes = [d]
        L.oracle_norm_ppf.restype = d
        L.oracle_norm_ppf.argtypes = [d]
        L.oracle_round_bf16.restype = d
        L.oracle_round_bf16.argtypes = [d]
        L.oracle_nf4_codebook.restype = None
        L.oracle_nf4_codebook.argtypes = [d, vp, vp]
        L.oracle_quantize.restype = ctypes.c_int
        L.oracle_quantize.argtypes = [vp, i64, i64, vp, vp, vp, ctypes.c_int]
        L.oracle_pack_canonical.restype = None
        L.oracle_pack_canonical.argtypes = [vp, i64, i64, vp]
        L.oracle_unpack_canonical.restype = None
        L.oracle_unpack_canonical.argtypes = [vp, i64, i64, vp]
        L.oracle_dequant.restype = None
        L.oracle_dequant.argtypes = [vp, vp, vp, i64, i64, vp]
        L.oracle_linear.restype = ctypes.c_int
        L.oracle_linear.argtypes = [vp, i64, vp, vp, vp, i64, i64, vp, i64, vp, vp, ctypes.c_int]
        L.oracle_round_fp16.restype = d
        L.oracle_round_fp16.argtypes = [d]
        L.oracle_awq_quantize.restype = ctypes.c_int
        L.oracle_awq_quantize.argtypes = [vp, i64, i64, vp, vp, vp, ctypes.c_int]
        L.oracle_awq_dequant.restype = None
        L.oracle_awq_dequant.argtypes = [vp, vp, vp, i64, i64, vp]
        L.oracle_awq_linear.restype = ctypes.c_int
        L.oracle_awq_linear.argtypes = [vp, i64, vp, vp, vp, i64, i64, vp, i64, vp, vp,
                                        ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---------------------------------------------------------------- codebook
def norm_cdf(z: float) -> float:
    return lib().oracle_norm_cdf(float(z))


def norm_ppf(p: float) -> float:
    return lib().oracle_norm_ppf(float(p))


def round_bf16(v: float) -> float:
    return lib().oracle_round_bf16(float(v))


def codebook(delta: float = DELTA):
    """16 sorted codes (bf16-exact fp32) and their unrounded double values.

    Normal quantiles normalised to [-1, 1] with an exact zero: 8 positive
    levels at probabilities 1/2 + (delta - 1/2) j/8 and 7 negative levels at
    1/2 + (delta - 1/2) j/7, each divided by Phi^-1(delta)."""
    out = np.zeros(16, np.float32)
    unr = np.zeros(16, np.float64)
    lib().oracle_nf4_codebook(float(delta), _ptr(out), _ptr(unr))
    return out, unr


# ---------------------------------------------------------------- quantizer
def quantize(W: np.ndarray, cb: np.ndarray, threads: int | None = None):
    """Per 64-block absmax and nearest code (ties to the lower index).

    Returns (codes uint8 [N, K], absmax float32 [N, K/64])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    cb = np.ascontiguousarray(cb, dtype=np.float32)
    N, K = W.shape
    codes = np.empty((N, K), np.uint8)
    absmax = np.empty((N, K // BLOCK), np.float32)
    rc = lib().oracle_quantize(_ptr(W), N, K, _ptr(cb), _ptr(codes), _ptr(absmax),
                               threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_quantize: bad shape or codebook without +0.0")
    return codes, absmax


def pack(codes: np.ndarray) -> np.ndarray:
    """Canonical packing: byte j of a row = code[2j] | code[2j+1] << 4."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    N, K = codes.shape
    out = np.empty((N, K // 2), np.uint8)
    lib().oracle_pack_canonical(_ptr(codes), N, K, _ptr(out))
    return out


def unpack(packed: np.ndarray) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    N, K2 = packed.shape
    out = np.empty((N, 2 * K2), np.uint8)
    lib().oracle_unpack_canonical(_ptr(packed), N, 2 * K2, _ptr(out))
    return out


def dequant(packed: np.ndarray, absmax: np.ndarray, cb: np.ndarray) -> np.ndarray:
    """W'[n, k] = fl32(c[idx] * s): one binary32 multiply per weight."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    absmax = np.ascontiguousarray(absmax, dtype=np.float32)
    cb = np.ascontiguousarray(cb, dtype=np.float32)
    N, K2 = packed.shape
    K = 2 * K2
    assert absmax.shape == (N, K // BLOCK)
    out = np.empty((N, K), np.float32)
    lib().oracle_dequant(_ptr(packed), _ptr(absmax), _ptr(cb), N, K, _ptr(out))
    return out


def linear(x_bf16: np.ndarray, packed: np.ndarray, absmax: np.ndarray, cb: np.ndarray,
           rows=None, threads: int | None = None):
    """y[m, n] = sum_k x[m, k] * W'[n, k] in double, natural k order.

    x_bf16: uint16 bit patterns [M, K].  rows: optional output rows to compute.
    Returns (y float64 [M, nrows], bound float64 [M, nrows]) where
    bound = sum_k |x * W'|."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    absmax = np.ascontiguousarray(absmax, dtype=np.float32)
    cb = np.ascontiguousarray(cb, dtype=np.float32)
    M, K = x_bf16.shape
    N = packed.shape[0]
    assert packed.shape == (N, K // 2)
    if rows is None:
        rows_arr, nrows, rp = None, N, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rp = rows_arr.size, _ptr(rows_arr)
    y = np.empty((M, nrows), np.float64)
    bound = np.empty((M, nrows), np.float64)
    rc = lib().oracle_linear(_ptr(x_bf16), M, _ptr(packed), _ptr(absmax), _ptr(cb), N, K, rp,
                             nrows, _ptr(y), _ptr(bound), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_linear: bad arguments")
    return y, bound


# ---------------------------------------------------------------- second format
# Asymmetric int4 in groups of 128 along K (vibevoice.c README, "Quantization"
# > "Weights", the AWQ/GPTQ paragraph): w = (q - z) * s with an exact integer
# zero point z per group and an FP16 scale s per group.  The pages give the
# dequantization; the quantizer is the plain min-max round-to-nearest of that
# form (a reading: the pages load quantized checkpoints).
GROUP = 128


def round_fp16(v: float) -> float:
    """Nearest binary16 value (ties to even), as a float."""
    return lib().oracle_round_fp16(float(v))


def awq_quantize(W: np.ndarray, threads: int | None = None):
    """Per row and group of 128: s = fp16(max(wmax - wmin, 1e-5) / 15),
    z = clamp(rint(-wmin / s), 0, 15), q = clamp(rint(w / s) + z, 0, 15).

    Returns (codes uint8 [N, K], scales float32 [N, K/128], zeros uint8
    [N, K/128])."""
    W = np.ascontiguousarray(W, dtype=np.float32)
    N, K = W.shape
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, K // GROUP), np.float32)
    zeros = np.empty((N, K // GROUP), np.uint8)
    rc = lib().oracle_awq_quantize(_ptr(W), N, K, _ptr(codes), _ptr(scales), _ptr(zeros),
                                   threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_awq_quantize: K must be a positive multiple of 128")
    return codes, scales, zeros


def awq_dequant(packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray) -> np.ndarray:
    """W'[n, k] = fl32((q - z) * s): one binary32 multiply per weight."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    N, K2 = packed.shape
    K = 2 * K2
    assert scales.shape == (N, K // GROUP) and zeros.shape == (N, K // GROUP)
    out = np.empty((N, K), np.float32)
    lib().oracle_awq_dequant(_ptr(packed), _ptr(scales), _ptr(zeros), N, K, _ptr(out))
    return out


def awq_linear(x_bf16: np.ndarray, packed: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
               rows=None, threads: int | None = None):
    """y[m, n] = sum_k x[m, k] * W'[n, k] in double, natural k order, with the
    second format's W'; returns (y, bound) as linear()."""
    x_bf16 = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    M, K = x_bf16.shape
    N = packed.shape[0]
    assert packed.shape == (N, K // 2)
    if rows is None:
        rows_arr, nrows, rp = None, N, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, rp = rows_arr.size, _ptr(rows_arr)
    y = np.empty((M, nrows), np.float64)
    bound = np.empty((M, nrows), np.float64)
    rc = lib().oracle_awq_linear(_ptr(x_bf16), M, _ptr(packed), _ptr(scales), _ptr(zeros), N, K,
                                 rp, nrows, _ptr(y), _ptr(bound), threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_awq_linear: bad arguments")
    return y, bound


# Act-order checkpoints (vibevoice.c README, "Quantization" > "Weights", the
# GPTQ act-order bullet): the input channels were quantized in order of
# importance, so a group's channels are scattered over K.  The loader sorts
# the channels by group, which makes every group a contiguous run of 128, and
# keeps that order; the decoder gathers the activations through it before the
# product: y = sum_j x[perm[j]] * W[n][perm[j]].
def act_order_perm(g_idx: np.ndarray) -> np.ndarray:
    """Channel order sorted by group, channels of one group in ascending
    order (a stable sort of the group index): perm[j] = the j-th channel."""
    g_idx = np.asarray(g_idx)
    return np.argsort(g_idx, kind="stable").astype(np.int32)


def gather_columns(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """x_out[m][j] = x[m][perm[j]]."""
    return np.ascontiguousarray(np.asarray(x)[:, np.asarray(perm)])


# ---------------------------------------------------------------- acceptance
REL_L2 = 1e-5
ELEM = 1e-4


def check_linear(y_test: np.ndarray, y_ref: np.ndarray, bound: np.ndarray):
    """Acceptance of an fp32 output against the double oracle.

    rel-L2 <= 1e-5 over the call, every element within 1e-4 * sum|x*w|, and
    exact zeros where the reference is identically zero.  Returns
    (ok, rel_l2, worst_elem_ratio)."""
    yt = np.asarray(y_test, np.float64)
    yr = np.asarray(y_ref, np.float64)
    b = np.asarray(bound, np.float64)
    assert yt.shape == yr.shape == b.shape
    if not np.all(np.isfinite(yt)):
        return False, float("inf"), float("inf")
    diff = yt - yr
    nref = float(np.linalg.norm(yr))
    if nref == 0.0:
        ok = bool(np.all(yt == 0.0))
        return ok, 0.0 if ok else float("inf"), 0.0 if ok else float("inf")
    rel = float(np.linalg.norm(diff)) / nref
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(b > 0, np.abs(diff) / (ELEM * b), np.where(diff == 0, 0.0, np.inf))
    worst = float(ratio.max()) if ratio.size else 0.0
    return (rel <= REL_L2 and worst <= 1.0), rel, worst
