"""GPU parity of nf4_gemv_argmax, the lm_head step that turns the decode
GEMV's logits into one index per row on the device (vibevoice.c README, "The
kernels that matter").

The index is an integer decided by floating point, so the two sides are
compared on what is unique and the rest is checked for validity:
  - y equals nf4_gemv's y bit for bit and passes the oracle's bar;
  - index[m] is the first n holding the maximum of the kernel's own fp32 y
    (exact: that is the definition the entry point promises);
  - the oracle's value at index[m] is within the error bar of the oracle's
    maximum, i.e. the choice is a maximum of the exact result up to the
    rounding the bar allows.
"""
import numpy as np
import pytest

import oracle
from bit_weight_only_amd import synth

from gpu_helpers import QWEN, Side, assert_linear_ok, oracle_layer, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def side():
    return Side()


@pytest.fixture(scope="module")
def cb():
    return oracle.codebook()[0]


def run_argmax(side, x_bits, pw, cb, ws=None):
    t = side.torch
    M = x_bits.shape[0]
    xd = side.x_dev(x_bits)
    y = t.empty((M, pw.N), dtype=t.float32, device="cuda")
    idx = t.full((8,), -7, dtype=t.int32, device="cuda")
    need = side.nf4.nf4_gemv_argmax_workspace_bytes(M, pw.N, pw.K)
    if ws is None:
        ws = t.zeros(need, dtype=t.uint8, device="cuda")
    assert ws.numel() >= need
    side.stream.wait_stream(t.cuda.current_stream())
    side.nf4.nf4_gemv_argmax(xd, M, pw.qweight, pw.absmax, cb, pw.N, pw.K, y, idx, ws,
                             ws.numel(), stream=side.stream)
    side.sync()
    out = idx.cpu().numpy()
    assert np.all(out[M:] == -7), "index written past row M"
    return y.cpu().numpy(), out[:M]


def check_index(y, idx, yr=None, b=None, what=""):
    M = y.shape[0]
    for m in range(M):
        assert idx[m] == int(np.argmax(y[m])), f"{what}: row {m} index {idx[m]}"
        if yr is not None:
            j = int(np.argmax(yr[m]))
            bar = 1e-4 * (b[m, idx[m]] + b[m, j])
            assert yr[m, idx[m]] >= yr[m, j] - bar, f"{what}: row {m} not a maximum"


@pytest.mark.parametrize("M", [1, 3, 8])
def test_argmax_tiny(side, cb, M):
    N, K = 256, 256
    _, packed, absmax = oracle_layer(0, 0, 30, N, K, cb)
    pw = side.repack(packed, absmax)
    x = synth.activations(0, M, K, stream=M)
    y, idx = run_argmax(side, x, pw, cb)
    yr, b = oracle.linear(x, packed, absmax, cb)
    assert_linear_ok(y, yr, b, f"argmax tiny M={M}")
    check_index(y, idx, yr, b, f"tiny M={M}")


def test_argmax_logits_equal_gemv(side, cb):
    N, K, M = 4608, 3584, 2
    _, packed, absmax = oracle_layer(2, 0, 31, N, K, cb)
    pw = side.repack(packed, absmax)
    x = synth.activations(2, M, K)
    y, idx = run_argmax(side, x, pw, cb)
    np.testing.assert_array_equal(y, side.run("gemv", x, pw, cb))
    check_index(y, idx, what="qkv-shaped")


def test_argmax_planted_tie_takes_lower_index(side, cb):
    """Rows 35 and 42 (one 16-row group, so the same operations) hold the
    same weights, aligned with x: an exact tie for the maximum."""
    N, K = 512, 256
    x = synth.activations(0, 1, K, stream=7)
    xf = synth.bf16_bits_to_fp32(x)[0].astype(np.float64)
    W = synth.weights(0, 0, 32, N, K)
    W[35] = W[42] = (0.05 * xf).astype(np.float32)
    codes, absmax = oracle.quantize(W, cb)
    packed = oracle.pack(codes)
    pw = side.repack(packed, absmax)
    y, idx = run_argmax(side, x, pw, cb)
    assert y[0, 35] == y[0, 42] and y[0, 35] == y[0].max()
    assert idx[0] == 35
    yr, b = oracle.linear(x, packed, absmax, cb)
    check_index(y, idx, yr, b, "planted tie")


def test_argmax_all_equal_and_workspace_reuse(side, cb):
    """Zero codes give y = 0 everywhere: the first column wins.  One
    workspace serves calls with M = 2 then M = 1 (its counter is left at
    zero after each call)."""
    N, K = 1024, 512
    packed = np.full((N, K // 2), 0x77, dtype=np.uint8)  # code 7 is +0.0 in both nibbles
    absmax = np.ones((N, K // 64), dtype=np.float32)
    assert cb[7] == 0.0
    pw = side.repack(packed, absmax)
    t = side.torch
    ws = t.zeros(side.nf4.nf4_gemv_argmax_workspace_bytes(2, N, K), dtype=t.uint8, device="cuda")
    for M in (2, 1, 2):
        x = synth.activations(0, M, K, stream=11)
        y, idx = run_argmax(side, x, pw, cb, ws=ws)
        assert np.all(y == 0.0)
        assert np.all(idx == 0)
    assert int(ws[:4].cpu().view(t.int32)[0]) == 0


def test_argmax_three_term_codebook_path(side):
    """A codebook that is not bf16-exact runs the generic GEMV and a separate
    argmax over y; the result definition is the same."""
    cb32 = np.sort(np.random.default_rng(5).uniform(-1, 1, 16)).astype(np.float32)
    cb32[7] = 0.0
    cb32 = np.sort(cb32)
    N, K, M = 2048, 512, 2
    W = synth.weights(0, 0, 33, N, K)
    codes, absmax = oracle.quantize(W, cb32)
    packed = oracle.pack(codes)
    pw = side.repack(packed, absmax)
    x = synth.activations(0, M, K, stream=9)
    y, idx = run_argmax(side, x, pw, cb32)
    yr, b = oracle.linear(x, packed, absmax, cb32)
    assert_linear_ok(y, yr, b, "argmax 3-term")
    check_index(y, idx, yr, b, "3-term codebook")


@pytest.mark.parametrize("M", [1, 2])
def test_argmax_lm_head_full_size(side, cb, M):
    """Qwen2-7B lm_head (152064 x 3584): the oracle computes every logit."""
    N, K = QWEN["lm_head"]
    say(f"[argmax] lm_head M={M} N={N} K={K}: oracle quantizes and multiplies all rows")
    W = synth.weights(2, 0, 54, N, K)
    codes, absmax = oracle.quantize(W, cb)
    del W
    packed = oracle.pack(codes)
    del codes
    pw = side.repack(packed, absmax)
    x = synth.activations(2, M, K, stream=5)
    y, idx = run_argmax(side, x, pw, cb)
    yr, b = oracle.linear(x, packed, absmax, cb)
    assert_linear_ok(y, yr, b, f"lm_head M={M}")
    check_index(y, idx, yr, b, f"lm_head M={M}")
