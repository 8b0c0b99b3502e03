"""Pins of the oracle's NF4 codebook and nearest-code rule.

Each check ties the oracle to something other than its own code: an
independent inverse-normal routine (scipy), the forward normal CDF (erfc),
exact rational brute force, and the qualitative properties the pages state
for NF4 ("A 65B fine-tune on the GPU you already have", figure 3; "QLoRA
Explained", "The three ideas behind QLoRA"; "QLoRA and Quantized Training",
"The idea").
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import nf4


def test_sixteen_levels_monotone_and_span_unit_interval():
    L = nf4.codebook()
    assert L.dtype == np.float32 and L.shape == (16,)
    assert np.all(np.diff(L) > 0)                      # 16 distinct, ascending
    assert L[0] == np.float32(-1.0) and L[15] == np.float32(1.0)  # max |level| = 1


def test_levels_antisymmetric_bitwise():
    L = nf4.codebook()
    assert np.array_equal((-L[::-1]).view(np.uint32), L.view(np.uint32))
    assert not np.any(L == 0)          # (i+1/2)/16 reading: no exact zero level


def test_levels_match_independent_inverse_normal():
    """scipy's ndtri is a different implementation of the normal quantile."""
    z = np.array([scipy.special.ndtri((i + 0.5) / 16) for i in range(16)])
    ref = (z / z[15]).astype(np.float32)
    assert np.array_equal(ref.view(np.uint32), nf4.codebook().view(np.uint32))


def test_levels_sit_at_equal_mass_quantiles():
    """Forward check with the normal CDF: level i carries probability (i+1/2)/16."""
    L = nf4.codebook().astype(np.float64)
    zstar = scipy.special.ndtri(15.5 / 16)
    for i, li in enumerate(L):
        p = 0.5 * math.erfc(-li * zstar / math.sqrt(2.0))
        assert abs(p - (i + 0.5) / 16) < 1e-7
    # equal mass per bin: consecutive levels are 1/16 of probability apart
    cdf = [0.5 * math.erfc(-li * zstar / math.sqrt(2.0)) for li in L]
    assert np.allclose(np.diff(cdf), 1 / 16, atol=2e-7)


def test_levels_dense_near_zero():
    L = nf4.codebook().astype(np.float64)
    gaps = np.diff(L[8:])              # positive half, moving outward
    assert np.all(np.diff(gaps) > 0)
    assert L[8] - L[7] < L[15] - L[14]


def test_occupancy_roughly_equal_on_normal_samples():
    """Each level used about equally often on N(0,1) data at its own scale.

    Reading of "roughly equal": every frequency within 1/16 +- 15%.
    """
    rng = np.random.Generator(np.random.PCG64(0))
    z = rng.standard_normal(1 << 22)
    zstar = scipy.special.ndtri(15.5 / 16)
    v = np.clip(z / zstar, -1, 1).astype(np.float32)
    freq = np.bincount(nf4.nearest_code(v), minlength=16) / v.size
    assert freq.min() > 0.053 and freq.max() < 0.072


def _brute_nearest(v, L):
    fv = Fraction(float(v))
    d = [abs(fv - Fraction(float(li))) for li in L]
    m = min(d)
    return d.index(m)                  # first index: ties to the lower one


def test_nearest_code_brute_force_random():
    L = nf4.codebook()
    rng = np.random.Generator(np.random.PCG64(7))
    v = rng.uniform(-1, 1, 3000).astype(np.float32)
    got = nf4.nearest_code(v)
    want = np.array([_brute_nearest(x, L) for x in v])
    assert np.array_equal(got, want)


def test_nearest_code_brute_force_around_every_midpoint():
    """+-300 fp32 ulps around each exact midpoint, plus the midpoints' own
    nearest fp32 neighbours: the tie rule and every boundary are exercised."""
    L = nf4.codebook()
    vals = []
    for j in range(15):
        m = (float(L[j]) + float(L[j + 1])) / 2
        c = np.float32(m)
        up, dn = c, c
        vals.append(c)
        for _ in range(300):
            up = np.nextafter(up, np.float32(2))
            dn = np.nextafter(dn, np.float32(-2))
            vals.extend([up, dn])
    vals = np.array(vals, dtype=np.float32)
    got = nf4.nearest_code(vals)
    want = np.array([_brute_nearest(x, L) for x in vals])
    assert np.array_equal(got, want)


def test_nearest_code_exact_ties_go_low():
    L = nf4.codebook()
    for j in range(15):
        m = (Fraction(float(L[j])) + Fraction(float(L[j + 1]))) / 2
        mf = np.float32(float(m))
        if Fraction(float(mf)) == m:           # midpoint representable in fp32
            assert nf4.nearest_code(np.array([mf]))[0] == j


def test_nearest_code_special_values():
    L = nf4.codebook()
    specials = np.array([0.0, -0.0, 1e-38, -1e-38, 1e-45, -1e-45, 1.0, -1.0,
                         0.5, -0.5], dtype=np.float32)
    got = nf4.nearest_code(specials)
    want = [_brute_nearest(x, L) for x in specials]
    assert list(got) == want
    assert got[0] == 7 and got[1] == 7         # zero ties to the lower level
    assert got[2] == 8 and got[3] == 7


@pytest.mark.parametrize("e", [0, 3, 7, 20])
def test_exact_levels_code_to_themselves(e):
    """A block holding L[c] * 2^-e (c cycling 0..15) has absmax 2^-e, the
    division is exact, and every weight codes to its own c."""
    L = nf4.codebook()
    c = np.tile(np.arange(16), 4 * 8)
    w = (L[c] * np.float32(2.0 ** -e)).astype(np.float32)
    packed, absmax = nf4.quantize(w)
    assert np.all(absmax == np.float32(2.0 ** -e))
    assert np.array_equal(nf4.unpack(packed), c.astype(np.uint8))
