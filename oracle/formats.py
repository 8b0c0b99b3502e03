"""Other 16-level block formats the pages compare NF4 with -- oracle.

TEST INFRASTRUCTURE (see the package docstring).

Sources, cited by page title and section:
  [THREE]    "QLoRA Explained: ...", "The three ideas behind QLoRA", 1. 4-bit
             NormalFloat: NF4 beats the standard 4-bit integer and float
             formats on normally distributed weights.
  [FIG3]     "A 65B fine-tune on the GPU you already have", figure 3: uniform
             bins (INT4 / FP4) spend levels where weights rarely fall.

The pages name the formats but give no level tables. Readings:
  INT4: the 16 evenly spaced levels (2i - 15) / 15, i = 0..15, spanning
        [-1, 1] like NF4 (all 16 codes used, antisymmetric).
  FP4:  the values of a 1-sign / 2-exponent / 1-mantissa float (E2M1:
        0, 0.5, 1, 1.5, 2, 3, 4, 6), divided by 6 so they span [-1, 1]; the
        two zeros -0 and +0 are codes 7 and 8, and the code of v is the count
        of level midpoints strictly below v (so v <= 0 takes -0, v > 0 +0).
Both are used with the same block-64 absmax scaling and double quantization
as NF4 (``oracle.nf4`` with ``levels=``).
"""
import numpy as np

from . import nf4

NF4, INT4, FP4 = 0, 1, 2


def int4_levels():
    return np.array([(2 * i - 15) / 15 for i in range(16)], dtype=np.float64).astype(np.float32)


def e2m1_values():
    """Non-negative values of a float with 2 exponent bits (bias 1) and 1
    mantissa bit: exponent 0 is subnormal (m / 2), otherwise (1 + m/2) 2^(e-1)."""
    out = []
    for e in range(4):
        for m in range(2):
            out.append(m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return sorted(out)


def fp4_levels():
    mags = np.array(e2m1_values(), dtype=np.float64) / max(e2m1_values())
    neg = -mags[::-1]                                  # -1 .. -0 (the last is -0.0)
    return np.concatenate([neg, mags]).astype(np.float32)


def levels(fmt):
    return {NF4: nf4.codebook(), INT4: int4_levels(), FP4: fp4_levels()}[fmt]


def relative_error(w, fmt, double_quant=True):
    """||deq(W) - W|| / ||W|| of a weight stored in the given format."""
    L = levels(fmt)
    packed, absmax = nf4.quantize(w, L)
    if double_quant:
        q, step = nf4.double_quantize(absmax)
        deq = nf4.dequantize(packed, q, step, levels=L)
    else:
        deq = nf4.dequantize(packed, None, None, levels=L, absmax=absmax)
    d = nf4.bf16_bits_to_f32(deq).astype(np.float64)
    w64 = np.asarray(w, dtype=np.float64).reshape(-1)
    return float(np.linalg.norm(d - w64) / np.linalg.norm(w64))
