"""Pins of the oracle's linear layer y = x . dequant(W)^T (CPU only).

The method computes every output as a plain dot product of a bf16 activation
row with a dequantized weight row (vibevoice.c README, "The kernels that
matter": dequantization is fused into the multiply-accumulate).  The oracle
sums exact double products in natural k order.  It is pinned against exact
rational arithmetic, numpy's float64 matmul, an exactly representable dyadic
case, one-hot activations and row selection, and its acceptance test is shown
to reject planted mistakes.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from bit_weight_only_amd import synth


@pytest.fixture(scope="module")
def cb():
    return oracle.codebook()[0]


def make_layer(cb, N, K, cfg=0, layer=0, mid=50):
    W = synth.weights(cfg, layer, mid, N, K)
    codes, absmax = oracle.quantize(W, cb)
    return oracle.pack(codes), absmax


def test_linear_exact_rationals(cb):
    M, K, N = 4, 64, 16
    packed, absmax = make_layer(cb, N, K)
    x = synth.activations(0, M, K)
    y, bound = oracle.linear(x, packed, absmax, cb)
    Wd = oracle.dequant(packed, absmax, cb)
    xf = synth.bf16_bits_to_fp32(x)
    for m in range(M):
        for n in range(N):
            prods = [Fraction(float(xf[m, k])) * Fraction(float(Wd[n, k])) for k in range(K)]
            exact = sum(prods)
            babs = sum(abs(p) for p in prods)
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(K) * Fraction(2) ** -52 * babs
            assert abs(Fraction(bound[m, n]) - babs) <= Fraction(K) * Fraction(2) ** -52 * babs


def test_linear_matches_numpy_float64(cb):
    M, K, N = 4, 256, 256
    packed, absmax = make_layer(cb, N, K, mid=51)
    x = synth.activations(0, M, K)
    y, bound = oracle.linear(x, packed, absmax, cb)
    ref = synth.bf16_bits_to_fp32(x).astype(np.float64) @ oracle.dequant(packed, absmax, cb).astype(np.float64).T
    assert np.all(np.abs(y - ref) <= 1e-13 * bound)
    babs = np.abs(synth.bf16_bits_to_fp32(x).astype(np.float64)) @ np.abs(oracle.dequant(packed, absmax, cb).astype(np.float64)).T
    np.testing.assert_allclose(bound, babs, rtol=1e-13)


def test_linear_dyadic_exact(cb):
    """Codebook (i-7)/8, scales 2^[-4,0], integer x with |x| <= 2: every
    partial sum is a multiple of 2^-7 below 2^13, so y is an exact integer
    combination that any summation order must reproduce."""
    rng = np.random.default_rng(4)
    M, K, N = 3, 1024, 32
    dy = ((np.arange(16) - 7) / 8).astype(np.float32)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    absmax = np.ldexp(np.float32(1), rng.integers(-4, 1, size=(N, K // 64))).astype(np.float32)
    xi = rng.integers(-2, 3, size=(M, K))
    x = synth.fp32_to_bf16_bits(xi.astype(np.float32))
    y, _ = oracle.linear(x, oracle.pack(codes), absmax, dy)
    W = ((codes.astype(np.int64) - 7) * np.repeat((absmax * 128).astype(np.int64), 64, axis=1))  # units of 2^-10
    exact = (xi @ W.T).astype(np.float64) / 1024.0
    np.testing.assert_array_equal(y, exact)


def test_linear_one_hot(cb):
    K, N = 192, 48
    packed, absmax = make_layer(cb, N, K, mid=52)
    Wd = oracle.dequant(packed, absmax, cb)
    x = np.zeros((K, K), np.uint16)
    x[np.arange(K), np.arange(K)] = 0x3F80  # bf16 1.0
    y, _ = oracle.linear(x, packed, absmax, cb)
    np.testing.assert_array_equal(y, Wd.T.astype(np.float64))


def test_linear_row_selection_and_threads(cb):
    M, K, N = 2, 320, 80
    packed, absmax = make_layer(cb, N, K, mid=53)
    x = synth.activations(0, M, K)
    full, bfull = oracle.linear(x, packed, absmax, cb, threads=1)
    rows = [79, 0, 13, 13, 40]
    sub, bsub = oracle.linear(x, packed, absmax, cb, rows=rows, threads=3)
    np.testing.assert_array_equal(sub, full[:, rows])
    np.testing.assert_array_equal(bsub, bfull[:, rows])


def test_acceptance_check_rejects_planted_mistakes(cb):
    M, K, N = 2, 256, 64
    packed, absmax = make_layer(cb, N, K, mid=54)
    x = synth.activations(0, M, K)
    y, b = oracle.linear(x, packed, absmax, cb)
    ok, rel, worst = oracle.check_linear(y.astype(np.float32), y, b)
    assert ok and rel < 1e-6
    # dropped term: the last k of every dot product
    Wd = oracle.dequant(packed, absmax, cb)
    xf = synth.bf16_bits_to_fp32(x).astype(np.float64)
    dropped = y - np.outer(xf[:, -1], Wd[:, -1])
    assert not oracle.check_linear(dropped, y, b)[0]
    # transposed nibble order inside a byte
    swapped = oracle.pack(oracle.unpack(packed).reshape(N, K // 2, 2)[:, :, ::-1].reshape(N, K))
    ys, _ = oracle.linear(x, swapped, absmax, cb)
    assert not oracle.check_linear(ys, y, b)[0]
    # wrong block of scales (off by one block)
    yr, _ = oracle.linear(x, packed, np.roll(absmax, 1, axis=1), cb)
    assert not oracle.check_linear(yr, y, b)[0]
    # one element off by 2e-4 of its bound
    bad = y.copy()
    bad[1, 7] += 2e-4 * b[1, 7]
    assert not oracle.check_linear(bad, y, b)[0]
    # zero reference requires exact zeros
    z = np.zeros_like(y)
    assert oracle.check_linear(z, z, z)[0]
    assert not oracle.check_linear(z + 1e-30, z, z)[0]
