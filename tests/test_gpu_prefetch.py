"""GPU parity of nf4_gemv_prefetch: the read-ahead hint names the next
launch's matrix and must not change any output (vibevoice.c README,
"Quantization" > "Weights", the decode-GEMV bullet of the int4 GPU path, on
the fixed cost per kernel that the hint addresses).

y from the hinted call equals nf4_gemv's y bit for bit, on tiny shapes that
the oracle also checks, on the full-size decode linears with their neighbours
in a decode step as hints, with a next matrix larger or smaller than the
current one, with the current matrix as its own next one, and on the paths
that ignore the hint (x too long for the fast GEMV's LDS)."""
import numpy as np
import pytest

import oracle
from bit_weight_only_amd import synth

from gpu_helpers import QWEN_FUSED, Side, assert_linear_ok, oracle_layer, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def side():
    return Side()


@pytest.fixture(scope="module")
def cb():
    return oracle.codebook()[0]


def hinted(side, x_bits, pw, cb, nxt):
    t = side.torch
    M = x_bits.shape[0]
    xd = side.x_dev(x_bits)
    y = t.empty((M, pw.N), dtype=t.float32, device="cuda")
    side.stream.wait_stream(t.cuda.current_stream())
    if nxt is None:
        side.nf4.nf4_gemv_prefetch(xd, M, pw.qweight, pw.absmax, cb, pw.N, pw.K, y,
                                   stream=side.stream)
    else:
        side.nf4.nf4_gemv_prefetch(xd, M, pw.qweight, pw.absmax, cb, pw.N, pw.K, y,
                                   next_qweight=nxt.qweight, next_absmax=nxt.absmax,
                                   next_N=nxt.N, next_K=nxt.K, stream=side.stream)
    side.sync()
    return y.cpu().numpy()


def device_weight(side, cb, N, K, seed):
    t = side.torch
    gen = t.Generator(device="cuda")
    gen.manual_seed(seed)
    W = t.randn((N, K), generator=gen, device="cuda", dtype=t.float32) * 0.02
    side.stream.wait_stream(t.cuda.current_stream())  # W was made on torch's stream
    pw = side.nf4.pack_weight(W, cb, stream=side.stream)
    side.sync()
    del W
    return pw


@pytest.mark.parametrize("M", [1, 4])
def test_prefetch_tiny_matches_gemv_and_oracle(side, cb, M):
    _, packed, absmax = oracle_layer(0, 0, 40, 256, 256, cb)
    pw = side.repack(packed, absmax)
    _, packed2, absmax2 = oracle_layer(0, 0, 41, 512, 512, cb)
    nxt = side.repack(packed2, absmax2)
    x = synth.activations(0, M, 256, stream=21)
    y0 = side.run("gemv", x, pw, cb)
    for n in (None, nxt, pw):
        np.testing.assert_array_equal(hinted(side, x, pw, cb, n), y0)
    yr, b = oracle.linear(x, packed, absmax, cb)
    assert_linear_ok(y0, yr, b, f"prefetch tiny M={M}")


@pytest.mark.parametrize("M", [1, 2, 8])
def test_prefetch_decode_chain_bitwise(side, cb, M):
    """Each fused Qwen2-7B linear with the next one of a decode step as the
    hint (down hints the next layer's q|k|v), plus a larger-than-current
    next matrix for q|k|v."""
    names = list(QWEN_FUSED)
    pws = {n: device_weight(side, cb, *QWEN_FUSED[n], seed=100 + i) for i, n in enumerate(names)}
    for i, name in enumerate(names):
        pw = pws[name]
        nxt = pws[names[(i + 1) % len(names)]]
        x = synth.activations(2, M, pw.K, stream=30 + i)
        say(f"[prefetch] M={M} {name} -> {names[(i + 1) % len(names)]}")
        y0 = side.run("gemv", x, pw, cb)
        np.testing.assert_array_equal(hinted(side, x, pw, cb, nxt), y0, err_msg=name)
        np.testing.assert_array_equal(hinted(side, x, pw, cb, None), y0, err_msg=name)
    x = synth.activations(2, M, pws["qkv"].K, stream=39)
    y0 = side.run("gemv", x, pws["qkv"], cb)
    np.testing.assert_array_equal(hinted(side, x, pws["qkv"], cb, pws["gate_up"]), y0)
