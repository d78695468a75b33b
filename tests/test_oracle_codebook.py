"""Pins of the oracle's codebook construction (CPU only).

The pages say the 4-bit codes index a non-uniform table (vibevoice.c README,
"Int8 activations: W8A8 and W4A8") kept with the quantization code, but never
print it.  The reading: normal quantiles normalised to [-1, 1] with an exact
zero, 7 negative and 8 positive levels, rounded to bfloat16.  These tests pin
the pieces against things other than the oracle itself: scipy's normal CDF
and quantile routines, the defining invariants, and neighbouring bf16 values.
"""
import math

import numpy as np
import pytest
from scipy import special

import oracle


@pytest.mark.parametrize("z", [-6.0, -2.5, -1.0, -0.3, 0.0, 0.2, 1.0, 1.959963984540054, 5.0])
def test_norm_cdf_matches_scipy(z):
    assert oracle.norm_cdf(z) == pytest.approx(special.ndtr(z), rel=1e-14, abs=1e-300)


@pytest.mark.parametrize("p", [1e-9, 0.025, 0.2, 0.5, 0.5 + 1e-6, 0.6, 0.75, 0.9, 0.9677083, 0.975, 0.999])
def test_norm_ppf_matches_scipy(p):
    assert oracle.norm_ppf(p) == pytest.approx(special.ndtri(p), rel=1e-12, abs=1e-15)


def test_norm_ppf_closed_forms():
    assert abs(oracle.norm_ppf(0.5)) < 1e-15
    # Phi(1) = (1 + erf(1/sqrt 2)) / 2
    assert oracle.norm_ppf(0.5 * (1.0 + math.erf(1.0 / math.sqrt(2.0)))) == pytest.approx(1.0, rel=1e-13)
    assert oracle.norm_ppf(0.975) == pytest.approx(1.959963984540054, rel=1e-13)
    assert math.isnan(oracle.norm_ppf(0.0)) and math.isnan(oracle.norm_ppf(1.0))


def _bf16_exact(v):
    return (np.float32(v).view(np.uint32) & np.uint32(0xFFFF)) == 0


def test_codebook_invariants():
    cb, unr = oracle.codebook()
    assert cb.dtype == np.float32 and cb.shape == (16,)
    assert np.all(np.diff(cb) > 0), "strictly increasing"
    assert cb[7] == 0.0 and not np.signbit(cb[7]), "index 7 is +0.0"
    assert cb[0] == -1.0 and cb[15] == 1.0, "endpoints are exactly -1 and +1"
    assert np.sum(cb < 0) == 7 and np.sum(cb > 0) == 8
    assert all(_bf16_exact(v) for v in cb), "every code is a bfloat16 value"
    nz = unr != 0
    assert np.all(np.abs(cb[nz] - unr[nz]) <= 2.0**-8 * np.abs(unr[nz]))


def test_codebook_quantiles_against_scipy():
    """Unrounded levels are Phi^-1 of equally spaced probabilities over
    Phi^-1(delta), computed here with scipy's ndtri."""
    d = oracle.DELTA
    _, unr = oracle.codebook()
    top = special.ndtri(d)
    pos = [special.ndtri(0.5 + (d - 0.5) * j / 8) / top for j in range(1, 9)]
    neg = [-special.ndtri(0.5 + (d - 0.5) * j / 7) / top for j in range(7, 0, -1)]
    np.testing.assert_allclose(unr, neg + [0.0] + pos, rtol=1e-12, atol=1e-15)


def test_codebook_equal_probability_mass():
    """Positive levels split (1/2, delta) into 8 equal probability steps and the
    negative levels split it into 7 (checked through scipy's CDF)."""
    d = oracle.DELTA
    _, unr = oracle.codebook()
    top = special.ndtri(d)
    mass_pos = np.diff(special.ndtr(np.concatenate([[0.0], unr[8:]]) * top))
    mass_neg = np.diff(special.ndtr(-np.concatenate([[0.0], unr[6::-1]]) * top))
    np.testing.assert_allclose(mass_pos, (d - 0.5) / 8, rtol=1e-10)
    np.testing.assert_allclose(mass_neg, (d - 0.5) / 7, rtol=1e-10)


def test_codebook_rounding_is_nearest_bf16():
    """Each code is the nearest bfloat16 to its level: neither bf16 neighbour
    is closer (ties to even)."""
    cb, unr = oracle.codebook()
    for c, u in zip(cb, unr):
        if c == 0:
            continue
        bits = np.float32(c).view(np.uint32)
        up = (bits + np.uint32(0x10000)).view(np.float32)
        dn = (bits - np.uint32(0x10000)).view(np.float32)
        e = abs(float(c) - u)
        assert e <= abs(float(up) - u) and e <= abs(float(dn) - u)


def test_round_bf16_examples():
    assert oracle.round_bf16(1.0) == 1.0
    assert oracle.round_bf16(1.0 + 2**-9) == 1.0              # below half an ulp (2^-7)
    assert oracle.round_bf16(1.0 + 2**-8) == 1.0              # exact tie -> even mantissa
    assert oracle.round_bf16(1.0 + 3 * 2**-8) == 1.0 + 2**-6  # exact tie -> even mantissa
    assert oracle.round_bf16(1.0 + 3 * 2**-9) == 1.0 + 2**-7  # above half an ulp
    assert oracle.round_bf16(-0.3) == -0.30078125


def test_codebook_fixture_matches():
    """The committed hex fixture is the oracle's codebook (regression guard)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "nf4_codebook.txt")
    vals = []
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            vals.append(float.fromhex(line))
    cb, _ = oracle.codebook()
    assert vals == [float(v) for v in cb]
