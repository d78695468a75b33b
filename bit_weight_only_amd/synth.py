"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no part of the layer's arithmetic: it only draws numbers.
Weights are N(0, 0.02^2) rounded to fp32 and activations are N(0, 1) rounded
to fp32 and then to bfloat16 (ties to even), matching the workloads' stated
distributions.  Draws come from SplitMix64 (Steele, Lea and Flood, 2014: add
the golden-ratio increment to a 64-bit state and pass it through the
published two-multiply finaliser), which is counter based, so any row of any
matrix can be regenerated on its own.  Normals use the Box-Muller transform
in double.  The bulk generation runs in ``synth.c`` (threaded, gcc-built
``libsynth.so``); ``splitmix64`` and ``normal_numpy`` here restate the same
definitions in numpy for the generator's own tests.

Every stream's seed is  MASTER ^ cfg << 32 ^ layer << 16 ^ matrix_id.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_clib = None

MASTER = 0x4E4634  # "NF4"
_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22

# matrix ids inside a decoder layer
Q, K_, V, O, GATE, UP, DOWN, LM_HEAD = range(8)
X_LAYER = 0xFFFF  # layer field used for activation streams


def stream_seed(cfg: int, layer: int, matrix_id: int) -> int:
    return (MASTER ^ (cfg << 32) ^ (layer << 16) ^ matrix_id) & 0xFFFFFFFFFFFFFFFF


def splitmix64(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Outputs offset .. offset+n-1 of the SplitMix64 stream started at `seed`."""
    i = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + i * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def build() -> str:
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-o", _LIB + ".tmp", _SRC, "-lm", "-lpthread"]
    subprocess.check_call(cmd)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _c():
    global _clib
    if _clib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        L.synth_fill.restype = None
        L.synth_fill.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                 ctypes.c_double, ctypes.c_void_p, ctypes.c_int]
        _clib = L
    return _clib


def _threads() -> int:
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS")
    return min(n, int(env)) if env and env.isdigit() and int(env) > 0 else n


def _fill(kind: int, seed: int, n: int, offset: int, dtype, scale: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype)
    _c().synth_fill(kind, seed & 0xFFFFFFFFFFFFFFFF, offset, n, scale, out.ctypes.data,
                    _threads())
    return out


def normal(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Standard normals offset .. offset+n-1 (float64)."""
    return _fill(0, seed, n, offset, np.float64)


def normal_numpy(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """The same normals restated in numpy (slow; for the generator's tests).
    Normal 2i and 2i+1 come from draws 2i and 2i+1 by Box-Muller."""
    out = np.empty(n, np.float64)
    done = 0
    while done < n:
        lo = offset + done
        take = min(_CHUNK, n - done)
        p0 = lo // 2
        p1 = (lo + take + 1) // 2
        r = splitmix64(seed, 2 * (p1 - p0), 2 * p0)
        u1 = ((r[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0**-53
        u2 = (r[1::2] >> np.uint64(11)).astype(np.float64) * 2.0**-53
        rad = np.sqrt(-2.0 * np.log(u1))
        z = np.empty(2 * (p1 - p0), np.float64)
        z[0::2] = rad * np.cos(2.0 * np.pi * u2)
        z[1::2] = rad * np.sin(2.0 * np.pi * u2)
        s = lo - 2 * p0
        out[done:done + take] = z[s:s + take]
        done += take
    return out


def fp32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_fp32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def weights(cfg: int, layer: int, matrix_id: int, N: int, K: int, rows=None,
            std: float = 0.02) -> np.ndarray:
    """fp32 W[N][K] ~ N(0, std^2); element (n, k) is draw n*K + k.
    `rows` selects a subset of rows (returned in that order)."""
    seed = stream_seed(cfg, layer, matrix_id)
    if rows is None:
        return _fill(1, seed, N * K, 0, np.float32, std).reshape(N, K)
    rows = np.asarray(rows, np.int64)
    out = np.empty((rows.size, K), np.float32)
    for i, n in enumerate(rows):
        out[i] = _fill(1, seed, K, int(n) * K, np.float32, std)
    return out


def activations(cfg: int, M: int, K: int, stream: int = 0, rows=None) -> np.ndarray:
    """bf16 bit patterns x[M][K] ~ N(0, 1), one stream per (cfg, K, stream)."""
    seed = stream_seed(cfg, X_LAYER, (K << 4 | stream) & 0xFFFF_FFFF)
    if rows is None:
        return _fill(2, seed, M * K, 0, np.uint16).reshape(M, K)
    rows = np.asarray(rows, np.int64)
    out = np.empty((rows.size, K), np.uint16)
    for i, m in enumerate(rows):
        out[i] = _fill(2, seed, K, int(m) * K, np.uint16)
    return out
