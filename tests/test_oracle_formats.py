"""Pins of the INT4 / FP4 format variants of the oracle (oracle.formats).

Sources: "QLoRA Explained: ...", "The three ideas behind QLoRA" (NF4 beats the
standard 4-bit integer and float formats on normally distributed weights);
"A 65B fine-tune on the GPU you already have", figure 3 (uniform bins).

Pins used: the level tables against their closed forms (evenly spaced INT4;
the E2M1 value list), exact antisymmetry, brute-force nearest level in
rational arithmetic around every midpoint, the signed-zero rule of FP4, exact
levels coding to themselves, and the pages' claim that NF4 has the smallest
error of the three on N(0, 0.02) weights.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F, nf4


def test_int4_levels_closed_form():
    L = F.int4_levels()
    assert L.dtype == np.float32 and L.size == 16
    assert L[0] == -1.0 and L[15] == 1.0
    assert np.array_equal(L[::-1].view(np.uint32), (-L).view(np.uint32))
    assert np.allclose(np.diff(L.astype(np.float64)), 2.0 / 15.0, rtol=0, atol=2e-7)


def test_fp4_levels_are_e2m1_values_over_six():
    assert F.e2m1_values() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    L = F.fp4_levels()
    assert L.size == 16 and L[0] == -1.0 and L[15] == 1.0
    assert np.signbit(L[7]) and L[7] == 0.0 and not np.signbit(L[8]) and L[8] == 0.0
    assert np.array_equal(L[::-1].view(np.uint32), (-L).view(np.uint32))
    assert np.array_equal(L[8:] * np.float32(6.0), np.array(F.e2m1_values(), np.float32))


def _brute(v, L):
    """argmin |v - L_i| in exact rationals, ties to the lower index."""
    fv = Fraction(float(v))
    d = [abs(fv - Fraction(float(x))) for x in L]
    return min(range(16), key=lambda i: (d[i], i))


@pytest.mark.parametrize("fmt", [F.INT4, F.FP4])
def test_nearest_code_brute_force(fmt):
    L = F.levels(fmt)
    vals = []
    for m in nf4.level_midpoints(L):
        c = np.float32(m)
        for k in range(-3, 4):
            x = c
            for _ in range(abs(k)):
                x = np.nextafter(x, np.float32(np.sign(k) * 2.0), dtype=np.float32)
            vals.append(x)
    vals += list(np.random.Generator(np.random.PCG64(5)).uniform(-1, 1, 400).astype(np.float32))
    vals = np.array(vals, np.float32)
    codes = nf4.nearest_code(vals, L)
    for v, c in zip(vals, codes):
        b = _brute(v, L)
        if fmt == F.FP4 and b == 7 and v > 0:
            b = 8                                   # the signed-zero rule: v > 0 takes +0
        assert c == b, (v, c, b)


def test_fp4_signed_zero_rule():
    L = F.fp4_levels()
    v = np.array([-0.0, 0.0, 1e-30, -1e-30, 1 / 24, -1 / 24], np.float32)
    assert list(nf4.nearest_code(v, L)) == [7, 7, 8, 7, 8, 6]


@pytest.mark.parametrize("fmt", [F.INT4, F.FP4])
def test_exact_levels_code_to_themselves(fmt):
    L = F.levels(fmt)
    idx = [c for c in range(16) if not (fmt == F.FP4 and c == 8)]     # +0 codes as -0 (v = 0)
    w = np.zeros(64, np.float32)
    w[:len(idx)] = L[idx] * np.float32(0.5)
    w[63] = np.float32(0.5)                                            # absmax 0.5: exact division
    packed, a = nf4.quantize(w, L)
    codes = nf4.unpack(packed)
    assert a[0] == 0.5 and list(codes[:len(idx)]) == idx


def test_nf4_has_the_smallest_error_on_normal_weights():
    """The pages' claim, on seeded N(0, 0.02) weights, with and without double
    quantization."""
    w = (np.random.Generator(np.random.PCG64(11)).standard_normal(1 << 18) * 0.02).astype(np.float32)
    for dq in (True, False):
        e = {f: F.relative_error(w, f, dq) for f in (F.NF4, F.INT4, F.FP4)}
        assert e[F.NF4] < e[F.INT4] and e[F.NF4] < e[F.FP4], e
