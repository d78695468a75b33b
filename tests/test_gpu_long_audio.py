"""Long-audio prefill parity: the 32-minute recording's prompt of M = 14449
rows (vibevoice.c README, "Benchmarks": 14449 prompt tokens) through every
fused Qwen2-7B layer linear (q|k|v, o, gate|up, down), in the NF4 format and
in the int4 group-128 format, run as a prefill runs it: 14 chunks of 1024
rows and a ragged tail of 113 ("Quantization" > "Weights", M > 1 bullet:
the prefill chunk on the matrix-core GEMM).

Against the oracle on sampled output columns (every row of W the oracle
quantizes is regenerated from the same counter-based stream): every row of
the 113-row tail and rows {first, last} of each 1024-row chunk.  The tail
also equals the same rows computed inside a full 1024-row chunk, bit for
bit (a row of y does not depend on the other rows of the batch).
"""
import numpy as np
import pytest

import oracle
from bit_weight_only_amd import synth

from gpu_helpers import QWEN_FUSED, Side, assert_linear_ok, say

pytestmark = pytest.mark.gpu

M = 14449
CHUNK = 1024
TAIL0 = 14 * CHUNK  # first row of the 113-row tail


@pytest.fixture(scope="module")
def side():
    return Side()


@pytest.fixture(scope="module")
def cb():
    return oracle.codebook()[0]


@pytest.fixture(scope="module")
def xs():
    """One seeded 14449-row activation matrix per K, shared by the linears."""
    return {K: synth.activations(4, M, K, stream=7) for K in sorted({K for _, K in
                                                                     QWEN_FUSED.values()})}


def columns(N, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 15, 16, N // 2, N - 16, N - 1],
                                     rng.integers(0, N, 120)]))


def picked_rows():
    firsts_lasts = np.concatenate([[c, c + CHUNK - 1] for c in range(0, TAIL0, CHUNK)])
    return np.concatenate([firsts_lasts, np.arange(TAIL0, M)])


def run_chunks(side, fmt, x, w, cb):
    """y rows picked_rows() of the chunked 14449-row prefill, and the last
    1024 rows computed as one full chunk (its last 113 rows are the tail)."""
    t = side.torch
    N = w.N
    xd = side.x_dev(x)
    y = t.empty((CHUNK, N), dtype=t.float32, device="cuda")
    picks = picked_rows()
    out = np.empty((len(picks), N), np.float32)
    for c0 in range(0, M, CHUNK):
        rows = min(CHUNK, M - c0)
        say(f"[{fmt} gemm] long audio N={N} K={w.K} rows {c0}..{c0 + rows}")
        if fmt == "nf4":
            side.linear("gemm", xd[c0:c0 + rows], rows, w, cb, y=y[:rows])
        else:
            side.awq_linear("gemm", xd[c0:c0 + rows], rows, w, y=y[:rows])
        sel = (picks >= c0) & (picks < c0 + rows)
        out[sel] = y[:rows].cpu().numpy()[picks[sel] - c0]
    c0 = M - CHUNK
    if fmt == "nf4":
        yin = side.linear("gemm", xd[c0:], CHUNK, w, cb, y=y)
    else:
        yin = side.awq_linear("gemm", xd[c0:], CHUNK, w, y=y)
    return out, yin.cpu().numpy()[CHUNK - (M - TAIL0):]


@pytest.mark.parametrize("fmt", ["nf4", "int4"])
@pytest.mark.parametrize("name", list(QWEN_FUSED))
def test_long_audio_prefill_every_linear(side, cb, xs, name, fmt):
    N, K = QWEN_FUSED[name]
    mid = 80 + list(QWEN_FUSED).index(name)
    cols = columns(N, mid)
    W = synth.weights(4, 0, mid, N, K)
    if fmt == "nf4":
        w = side.pack(W, cb)
    else:
        w = side.awq_pack(W)
    del W
    Wr = synth.weights(4, 0, mid, N, K, rows=cols)
    x = xs[K]
    out, tail_in_chunk = run_chunks(side, fmt, x, w, cb)
    picks = picked_rows()
    if fmt == "nf4":
        codes, absmax = oracle.quantize(Wr, cb)
        yr, b = oracle.linear(x[picks], oracle.pack(codes), absmax, cb)
    else:
        codes, scales, zeros = oracle.awq_quantize(Wr)
        yr, b = oracle.awq_linear(x[picks], oracle.pack(codes), scales, zeros)
    ntail = M - TAIL0
    assert_linear_ok(out[:-ntail][:, cols], yr[:-ntail], b[:-ntail],
                     f"{fmt} {name} chunk rows")
    assert_linear_ok(out[-ntail:][:, cols], yr[-ntail:], b[-ntail:], f"{fmt} {name} tail")
    assert np.all(np.isfinite(out))
    np.testing.assert_array_equal(tail_in_chunk, out[-ntail:])
    del w
    side.torch.cuda.empty_cache()
