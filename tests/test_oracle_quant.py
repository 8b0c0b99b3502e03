"""Pins of the oracle's block quantization, packing, double quantization and
dequantization.

Sources: "A 65B fine-tune on the GPU you already have", figure 4 (block of 64
with one 32-bit constant; 8-bit double quantization in blocks of 256) and
figure 2 (dequantize to bf16 right before the multiply); "QLoRA and Quantized
Training", "Worked example" (0.5 bytes per weight).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import nf4


def _brute_block_quantize(w):
    """Scalar, rational reference of one pass: absmax per 64-block, fp32
    quotient, exact nearest level with ties low, codes as a Python list."""
    L = [Fraction(float(x)) for x in nf4.codebook()]
    codes, amax = [], []
    for b in range(len(w) // 64):
        blk = [np.float32(x) for x in w[64 * b:64 * b + 64]]
        a = max(abs(x) for x in blk)
        amax.append(a)
        for x in blk:
            v = Fraction(0) if a == 0 else Fraction(float(np.float32(x) / np.float32(a)))
            d = [abs(v - li) for li in L]
            codes.append(d.index(min(d)))
    return codes, np.array(amax, dtype=np.float32)


def test_quantize_matches_rational_brute_force():
    rng = np.random.Generator(np.random.PCG64(3))
    w = (rng.standard_normal(64 * 12) * 0.02).astype(np.float32)
    w[64 * 5:64 * 6] = 0.0                          # an all-zero block
    w[64 * 7 + 3] = -0.3                             # a negative absmax element
    codes, amax = _brute_block_quantize(w)
    packed, absmax = nf4.quantize(w)
    assert np.array_equal(absmax.view(np.uint32), amax.view(np.uint32))
    assert list(nf4.unpack(packed)) == codes


def test_packing_closed_form():
    codes = np.tile(np.arange(16, dtype=np.uint8), 8)
    p = nf4.pack(codes)
    assert list(p[:8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert p.size == codes.size // 2                 # 0.5 byte per weight
    assert np.array_equal(nf4.unpack(p), codes)


def test_zero_block_codes_to_level_nearest_zero_from_below():
    packed, absmax = nf4.quantize(np.zeros(128, np.float32))
    assert np.all(absmax == 0)
    assert np.all(nf4.unpack(packed) == 7)


def test_absmax_element_codes_to_an_end_level():
    rng = np.random.Generator(np.random.PCG64(4))
    w = (rng.standard_normal(64 * 50) * 0.02).astype(np.float32)
    packed, absmax = nf4.quantize(w)
    codes = nf4.unpack(packed).reshape(-1, 64)
    wb = w.reshape(-1, 64)
    for b in range(50):
        i = int(np.argmax(np.abs(wb[b])))
        assert codes[b, i] == (15 if wb[b, i] > 0 else 0)


def test_bf16_input_equals_fp32_input_of_same_values():
    rng = np.random.Generator(np.random.PCG64(5))
    w32 = (rng.standard_normal(64 * 40) * 0.02).astype(np.float32)
    bits = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wide = torch.from_numpy(w32).to(torch.bfloat16).float().numpy()
    p1, a1 = nf4.quantize(bits)
    p2, a2 = nf4.quantize(wide)
    assert np.array_equal(p1, p2) and np.array_equal(a1, a2)


# --------------------------------------------------------------------------
# double quantization
# --------------------------------------------------------------------------
def _absmax_sample(nb, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.abs(rng.standard_normal(nb) * 0.05).astype(np.float32) + np.float32(1e-3)


@pytest.mark.parametrize("nb", [256, 1024, 1000, 7])
def test_dq_closed_forms(nb):
    a = _absmax_sample(nb, nb)
    q, step = nf4.double_quantize(a)
    ng = (nb + 255) // 256
    assert q.dtype == np.int8 and q.size == nb
    assert step.dtype == np.float32 and step.size == ng
    assert np.all(q >= 0)                            # constants are non-negative
    for g in range(ng):
        blk = a[256 * g:256 * g + 256]
        qg = q[256 * g:256 * g + 256].astype(np.int64)
        c2 = Fraction(float(blk.max()))
        d = Fraction(float(step[g]))
        # the step is the group max over 127, within half an fp32 ulp
        assert abs(d - c2 / 127) <= Fraction(float(np.spacing(step[g]))) / 2
        # the group's largest constant takes the top code
        assert qg[int(np.argmax(blk))] == 127
        # every code is the integer nearest to absmax / d (up to the fp32
        # rounding of the quotient before it is rounded to an integer)
        for ai, qi in zip(blk, qg):
            assert abs(Fraction(float(ai)) / d - qi) <= Fraction(1, 2) + Fraction(1, 1 << 16)


def test_dq_zero_group():
    a = np.zeros(300, np.float32)
    a[260] = 0.5
    q, step = nf4.double_quantize(a)
    assert step[0] == 0 and np.all(q[:256] == 0)
    assert q[260] == 127


def test_dq_relative_scale_error_is_small_on_gaussian_weights():
    """Quality guard (not parity): DQ loses about 1% of a typical constant."""
    rng = np.random.Generator(np.random.PCG64(9))
    w = (rng.standard_normal(64 * 4096) * 0.02).astype(np.float32)
    _, a = nf4.quantize(w)
    q, step = nf4.double_quantize(a)
    s = nf4.block_scales(q, step)
    rel = np.abs(s.astype(np.float64) - a) / a
    assert rel.max() < 0.03


# --------------------------------------------------------------------------
# dequantization
# --------------------------------------------------------------------------
def test_bf16_rounding_matches_torch():
    rng = np.random.Generator(np.random.PCG64(11))
    x = (rng.standard_normal(100000) * rng.uniform(1e-6, 1e3, 100000)).astype(np.float32)
    # add exact ties (low half == 0x8000) with both parities of the kept bit
    ties = (np.arange(2000, dtype=np.uint32) << 16 | 0x8000) + np.uint32(0x3F800000)
    x = np.concatenate([x, ties.view(np.float32), -ties.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(nf4.f32_to_bf16_bits(x), ref)


@pytest.mark.parametrize("e", [0, 5, 12])
def test_dequant_of_exact_levels(e):
    """Every block holds L[c] * 2^-e: all constants equal, so DQ gives q = 127
    and s = fl32(127 * fl32(2^-e / 127)); each output is bf16(L[c] * s)."""
    L = nf4.codebook()
    c = np.tile(np.arange(16), 4 * 300)
    w = (L[c] * np.float32(2.0 ** -e)).astype(np.float32)
    packed, q, step, _ = nf4.quantize_all(w)
    assert np.all(q == 127)
    out = nf4.bf16_bits_to_f32(nf4.dequantize(packed, q, step))
    # bf16 of a value within 1 fp32 ulp of L[c]*2^-e: within one bf16 ulp
    target = L[c].astype(np.float64) * 2.0 ** -e
    assert np.all(np.abs(out - target) <= np.abs(target) * 2.0 ** -8)
    # and the sign pattern and ordering of the 16 levels are preserved
    blk = out[:16]
    assert np.all(np.diff(blk) > 0)


def test_dequant_elementwise_bounds_and_reconstruction_quality():
    rng = np.random.Generator(np.random.PCG64(12))
    w = (rng.standard_normal(64 * 2048) * 0.02).astype(np.float32)
    packed, q, step, absmax = nf4.quantize_all(w)
    wd = nf4.bf16_bits_to_f32(nf4.dequantize(packed, q, step)).astype(np.float64)
    L = nf4.codebook().astype(np.float64)
    s = nf4.block_scales(q, step).astype(np.float64)
    codes = nf4.unpack(packed)
    exact = L[codes] * np.repeat(s, 64)
    # bf16 rounding (8-bit significand): unit roundoff 2^-8, plus fp32 slack
    assert np.all(np.abs(wd - exact) <= np.abs(exact) * (2.0 ** -8 + 2.0 ** -22))
    # quality guard (not parity): NF4 + DQ reconstructs N(0, s) to ~9%
    rel = np.linalg.norm(wd - w) / np.linalg.norm(w)
    assert 0.05 < rel < 0.15


def test_dequant_negative_zero_for_zero_constant():
    packed, q, step, _ = nf4.quantize_all(np.zeros(64, np.float32))
    out = nf4.dequantize(packed, q, step)
    assert np.all(out == 0x8000)                    # bf16(L[7] * 0) = -0


def test_dequantize_range_agrees_with_whole_array():
    rng = np.random.Generator(np.random.PCG64(13))
    w = (rng.standard_normal(64 * 700) * 0.02).astype(np.float32)
    packed, q, step, _ = nf4.quantize_all(w)
    full = nf4.dequantize(packed, q, step)
    for lo, hi in [(0, 64), (64 * 250, 64 * 260), (64 * 511, 64 * 700)]:
        assert np.array_equal(nf4.dequantize_range(packed, q, step, lo, hi), full[lo:hi])
