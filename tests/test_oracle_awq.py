"""Pins of the oracle's second format: asymmetric int4 in groups of 128
(vibevoice.c README, "Quantization" > "Weights", the AWQ/GPTQ paragraph: a
weight is (q - z) * s with an FP16 scale and an exact integer zero point per
group).  Each test checks the oracle against something other than its own
formulas: numpy's binary16 conversion, closed forms on exactly representable
groups, brute force over all 16 codes, and numpy's float64 matmul."""
import numpy as np
import pytest

import oracle
from bit_weight_only_amd import synth

G = oracle.GROUP


def test_round_fp16_matches_numpy_binary16():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.normal(0, 1, 20000) * 10.0 ** rng.integers(-9, 5, 20000),
        [0.0, -0.0, 1.0, 65504.0, 65519.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
         1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11)]])
    # every tie between neighbouring binary16 values, across the normal range
    h = np.arange(0x0400, 0x7BFF, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    nxt = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    vals = np.concatenate([vals, (h + nxt) / 2, -(h + nxt) / 2])
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).astype(np.float64)
    got = np.array([oracle.round_fp16(v) for v in vals])
    np.testing.assert_array_equal(got, want)


def test_group_on_grid_is_recovered_exactly():
    """A group holding (q - z) s for q = 0..15 (every code used) with an
    FP16-exact s gives back that s, z and q: the range is 15 s exactly."""
    rng = np.random.default_rng(2)
    for trial in range(50):
        s = float(np.float16(rng.uniform(1e-4, 0.05)))
        z = int(rng.integers(0, 16))
        q = np.concatenate([np.arange(16), rng.integers(0, 16, G - 16)])
        rng.shuffle(q)
        W = ((q - z) * s).astype(np.float32)[None, :]
        assert np.all(W.astype(np.float64) == (q - z) * s)        # exact in fp32
        codes, scales, zeros = oracle.awq_quantize(W)
        assert scales[0, 0] == np.float32(s) and zeros[0, 0] == z, (trial, scales, zeros)
        np.testing.assert_array_equal(codes[0], q)


@pytest.mark.parametrize("seed", [3, 4, 5])
def test_error_bound_and_nearest_code(seed):
    """For groups that straddle 0 (as N(0, sigma) groups of 128 do), every
    weight is the nearest of the 16 grid points (q' - z) s up to a tie, and
    the error is at most s/2 plus the FP16 rounding of the scale times the
    range (15 s 2^-11)."""
    W = synth.weights(0, 0, seed, 64, 1024)
    codes, scales, zeros = oracle.awq_quantize(W)
    N, K = W.shape
    s = np.repeat(scales.astype(np.float64), G, axis=1)
    z = np.repeat(zeros.astype(np.float64), G, axis=1)
    w = W.astype(np.float64)
    assert np.all(np.float16(scales).astype(np.float32) == scales)
    assert codes.max() <= 15 and zeros.max() <= 15
    err = np.abs(w - (codes - z) * s)
    assert np.all(err <= s * (0.5 + 15 * 2.0 ** -11) + 1e-12)
    grid = (np.arange(16)[None, None, :] - z[..., None]) * s[..., None]
    best = np.min(np.abs(w[..., None] - grid), axis=-1)
    assert np.all(err <= best * (1 + 1e-12) + 1e-15)


def test_zero_group_and_one_sided_group():
    """An all-zero group dequantizes to exact zeros; a group entirely above
    zero clamps z at 0, so its grid starts at 0 (the plain min-max form)."""
    W = np.zeros((2, G), np.float32)
    W[1] = np.linspace(1.0, 2.0, G, dtype=np.float32)
    codes, scales, zeros = oracle.awq_quantize(W)
    deq = oracle.awq_dequant(oracle.pack(codes), scales, zeros)
    assert np.all(deq[0] == 0.0) and zeros[0, 0] == 0
    assert zeros[1, 0] == 0 and scales[1, 0] == np.float32(oracle.round_fp16(1.0 / 15))
    assert np.all(codes[1] == 15)


def test_dequant_is_the_exact_product():
    """(q - z) * s is exact in binary32 for an FP16-exact s, so the oracle's
    fp32 multiply equals the double product."""
    W = synth.weights(0, 0, 6, 32, 512)
    codes, scales, zeros = oracle.awq_quantize(W)
    deq = oracle.awq_dequant(oracle.pack(codes), scales, zeros)
    want = (codes.astype(np.float64) - np.repeat(zeros, G, axis=1)) * \
        np.repeat(scales.astype(np.float64), G, axis=1)
    np.testing.assert_array_equal(deq.astype(np.float64), want)


@pytest.mark.parametrize("M", [1, 3])
def test_linear_matches_float64_matmul(M):
    N, K = 48, 384
    W = synth.weights(0, 0, 7, N, K)
    codes, scales, zeros = oracle.awq_quantize(W)
    packed = oracle.pack(codes)
    x = synth.activations(0, M, K, stream=2)
    y, b = oracle.awq_linear(x, packed, scales, zeros)
    xf = synth.bf16_bits_to_fp32(x).astype(np.float64)
    Wd = oracle.awq_dequant(packed, scales, zeros).astype(np.float64)
    np.testing.assert_allclose(y, xf @ Wd.T, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(b, np.abs(xf) @ np.abs(Wd).T, rtol=1e-12, atol=1e-15)
    y2, _ = oracle.awq_linear(x, packed, scales, zeros, rows=[5, 0, 47])
    np.testing.assert_array_equal(y2, y[:, [5, 0, 47]])


def test_codes_round_trip_through_the_canonical_packing():
    W = synth.weights(0, 0, 8, 16, 256)
    codes, _, _ = oracle.awq_quantize(W)
    np.testing.assert_array_equal(oracle.unpack(oracle.pack(codes)), codes)


def test_rejects_k_not_a_multiple_of_128():
    with pytest.raises(ValueError):
        oracle.awq_quantize(np.zeros((16, 192), np.float32))


# ------------------------------------------------------ act-order gather
def test_act_order_perm_sorts_channels_by_group_stably():
    g_idx = np.array([1, 0, 1, 0, 2, 1, 0, 2])
    perm = oracle.act_order_perm(g_idx)
    np.testing.assert_array_equal(perm, [1, 3, 6, 0, 2, 5, 4, 7])
    assert perm.dtype == np.int32


def test_act_order_perm_makes_groups_contiguous():
    rng = np.random.default_rng(11)
    K = 1024
    g_idx = rng.permutation(np.repeat(np.arange(K // G), G))  # scattered groups of 128
    perm = oracle.act_order_perm(g_idx)
    assert sorted(perm.tolist()) == list(range(K))
    np.testing.assert_array_equal(g_idx[perm], np.repeat(np.arange(K // G), G))
    for g in range(K // G):
        run = perm[g * G:(g + 1) * G]
        assert np.all(np.diff(run) > 0)  # ascending within a group


def test_gather_columns_by_hand_and_inverse():
    x = np.arange(12, dtype=np.uint16).reshape(2, 6)
    perm = np.array([5, 0, 3, 1, 4, 2], np.int32)
    np.testing.assert_array_equal(oracle.gather_columns(x, perm),
                                  [[5, 0, 3, 1, 4, 2], [11, 6, 9, 7, 10, 8]])
    rng = np.random.default_rng(12)
    x = rng.integers(0, 1 << 16, (3, 256), dtype=np.uint16)
    p = rng.permutation(256).astype(np.int32)
    inv = np.empty_like(p)
    inv[p] = np.arange(256, dtype=np.int32)
    np.testing.assert_array_equal(oracle.gather_columns(oracle.gather_columns(x, p), inv), x)
    ident = np.arange(256, dtype=np.int32)
    np.testing.assert_array_equal(oracle.gather_columns(x, ident), x)


def test_act_order_pipeline_computes_x_times_w():
    """Quantize the channel-sorted weight, gather x through the same order:
    the oracle's linear equals x @ W'^T with W' the dequantized weight put
    back into the checkpoint's channel order (numpy float64; only the order
    of the sum differs)."""
    rng = np.random.default_rng(13)
    N, K, M = 48, 512, 3
    g_idx = rng.permutation(np.repeat(np.arange(K // G), G))
    perm = oracle.act_order_perm(g_idx)
    W = synth.weights(0, 4, 1, N, K)
    codes, scales, zeros = oracle.awq_quantize(oracle.gather_columns(W, perm))
    packed = oracle.pack(codes)
    x = synth.activations(0, M, K, stream=4)
    y, _ = oracle.awq_linear(oracle.gather_columns(x, perm), packed, scales, zeros)
    deq_sorted = oracle.awq_dequant(packed, scales, zeros).astype(np.float64)
    Wp = np.empty_like(deq_sorted)
    Wp[:, perm] = deq_sorted
    xf = synth.bf16_bits_to_fp32(x).astype(np.float64)
    np.testing.assert_allclose(y, xf @ Wp.T, rtol=1e-12, atol=1e-12)
