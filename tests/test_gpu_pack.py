"""GPU parity of the load-time path: nf4_pack, nf4_repack/nf4_unpack and the
debug nf4_dequant, bit-exact against the oracle on the same seeded weights.

The quantizer runs once per projection at load (vibevoice.c README,
"Quantization" > "Weights"); the device layout is a permutation of the
canonical bytes.  Integer outputs (codes) and the dequantized binary32 values
must match bit for bit."""
import numpy as np
import pytest

import oracle
from bit_weight_only_amd import synth

from gpu_helpers import QWEN_FUSED, Side, oracle_layer, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def side():
    return Side()


@pytest.fixture(scope="module")
def cb():
    return oracle.codebook()[0]


SHAPES = [(16, 64), (16, 128), (48, 192), (256, 256), (512, 3584), (64, 18944), (4608, 320)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_pack_bit_exact(side, cb, N, K):
    say(f"[pack] N={N} K={K}")
    W, packed, absmax = oracle_layer(0, 1, 10, N, K, cb)
    W[3, 64:128] = 0.0  # an all-zero block
    codes, absmax = oracle.quantize(W, cb)
    packed = oracle.pack(codes)
    pw = side.pack(W, cb)
    gc, gs = side.unpack(pw)
    np.testing.assert_array_equal(gc, packed)
    np.testing.assert_array_equal(gs.view(np.uint32), absmax.view(np.uint32))
    deq = side.dequant(pw, cb)
    np.testing.assert_array_equal(deq.view(np.uint32),
                                  oracle.dequant(packed, absmax, cb).view(np.uint32))


def test_pack_exact_midpoint_ties(side, cb):
    """w/s exactly on a midpoint goes to the lower code on the GPU too."""
    mids = np.array([(float(cb[i]) + float(cb[i + 1])) / 2 for i in range(15)], np.float32)
    W = np.zeros((16, 128), np.float32)
    W[:, 0] = 1.0
    W[:, 1:16] = mids
    W[:, 16:31] = np.nextafter(mids, np.float32(2))
    W[:, 31:46] = -mids
    W[:, 64] = -3.0
    W[:, 65:80] = 3 * mids
    codes, absmax = oracle.quantize(W, cb)
    gc, gs = side.unpack(side.pack(W, cb))
    np.testing.assert_array_equal(gc, oracle.pack(codes))
    np.testing.assert_array_equal(gs, absmax)


def test_repack_unpack_roundtrip(side, cb):
    rng = np.random.default_rng(11)
    for N, K in [(16, 64), (48, 192), (256, 512)]:
        codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
        scales = rng.random((N, K // 64)).astype(np.float32)
        pw = side.repack(codes, scales)
        gc, gs = side.unpack(pw)
        np.testing.assert_array_equal(gc, codes)
        np.testing.assert_array_equal(gs, scales)
        np.testing.assert_array_equal(side.dequant(pw, cb).view(np.uint32),
                                      oracle.dequant(codes, scales, cb).view(np.uint32))


def test_dequant_one_hot_layout(side, cb):
    """A single nonzero code at every position in turn lands at (n, k)."""
    N, K = 32, 256
    for n, k in [(0, 0), (0, 1), (1, 7), (15, 8), (16, 31), (17, 32), (5, 127), (30, 128),
                 (31, 255), (9, 200)]:
        codes = np.full((N, K), 7, np.uint8)
        codes[n, k] = 15
        scales = np.ones((N, K // 64), np.float32)
        deq = side.dequant(side.repack(oracle.pack(codes), scales), cb)
        want = np.zeros((N, K), np.float32)
        want[n, k] = 1.0
        np.testing.assert_array_equal(deq, want)


def test_pack_full_size_gate_up(side, cb):
    """The largest decoder weight at its real shape (gate|up, 37888 x 3584);
    the oracle quantizes a sample of rows from the same stream."""
    N, K = QWEN_FUSED["gate_up"]
    say(f"[pack] full gate_up N={N} K={K}")
    W = synth.weights(2, 0, synth.GATE, N, K)
    pw = side.pack(W, cb)
    rows = np.array([0, 1, 15, 16, 4095, 18943, 18944, 30000, N - 1])
    codes, absmax = oracle.quantize(W[rows], cb)
    gc, gs = side.unpack(pw)
    np.testing.assert_array_equal(gc[rows], oracle.pack(codes))
    np.testing.assert_array_equal(gs[rows], absmax)
