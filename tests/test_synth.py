"""The seeded input generator (no part of the layer's arithmetic)."""
import numpy as np

from bit_weight_only_amd import synth


def test_splitmix64_published_vectors():
    # First outputs of SplitMix64 from state 0, as published with the algorithm.
    assert [int(v) for v in synth.splitmix64(0, 3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_c_generator_matches_numpy_restatement():
    """The threaded C generator equals the numpy restatement of the same
    definitions (draws bit for bit, normals to the last few ulps of libm)."""
    import ctypes
    raw = np.empty(1000, np.uint64)
    synth._c().synth_fill(3, 12345, 77, 1000, 1.0, raw.ctypes.data, 4)
    np.testing.assert_array_equal(raw, synth.splitmix64(12345, 1000, 77))
    np.testing.assert_allclose(synth.normal(99, 100_001, 5), synth.normal_numpy(99, 100_001, 5),
                               rtol=1e-13, atol=1e-13)


def test_normal_is_counter_based_and_standard():
    z = synth.normal(7, 300_001)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    np.testing.assert_array_equal(synth.normal(7, 11, 150_000), z[150_000:150_011])
    np.testing.assert_array_equal(synth.normal(7, 10, 3), z[3:13])


def test_weights_rows_regenerate():
    W = synth.weights(2, 5, synth.GATE, 40, 128)
    np.testing.assert_array_equal(synth.weights(2, 5, synth.GATE, 40, 128, rows=[39, 3]), W[[39, 3]])
    assert W.dtype == np.float32 and 0.015 < W.std() < 0.025


def test_activations_bf16_rounding():
    x = synth.activations(1, 3, 256)
    np.testing.assert_array_equal(synth.activations(1, 3, 256, rows=[2]), x[[2]])
    f = synth.bf16_bits_to_fp32(x)
    assert f.dtype == np.float32 and abs(f.std() - 1) < 0.1
    # ties to even on exact halfway patterns
    a = np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8)], np.float32)
    assert synth.bf16_bits_to_fp32(synth.fp32_to_bf16_bits(a)).tolist() == [1.0, 1.0 + 2**-6, -1.0]
