"""Storage rate and memory arithmetic of the format -- oracle.

TEST INFRASTRUCTURE (see the package docstring).

Everything here is computed from the byte counts of buffers that
``oracle.nf4`` actually produces, so the printed figures on the pages can be
checked against the format as built, not against a retyped formula.

Sources, cited by page title and section:
  [DQ-fig4]  "A 65B fine-tune on the GPU you already have", figure 4: half a
             bit per parameter of fp32 constants, cut to about 0.127 bits by
             8-bit double quantization in blocks of 256.
  [BILL]     same page, figure 5 (the 65B memory bill) and figure 1 (the
             memory wall: 16-bit weights, gradients, two Adam states).
  [WORKED]   "QLoRA and Quantized Training", section "Worked example" (7B).
  [SUMMARY]  "QLoRA > Summary" (70B; 0.5 -> 0.125 bits, "about 4.125").
  [THREE]    "QLoRA Explained: ...", "The three ideas behind QLoRA"
             (double quantization saves about 0.37 bits/param, ~3 GB at 65B).
  [NAME]     "QLoRA" (techbytebybyte), sections "Break the name into two
             parts" (1B) and "A concrete example, layered" (4 GB -> ~1 GB).
"""
import numpy as np

from . import nf4

GB = 1e9


def format_buffers(numel, double_quant=True, seed=0):
    """Quantize a synthetic weight of ``numel`` elements with the oracle and
    return the buffers the stored format consists of."""
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.standard_normal(numel, dtype=np.float32) * np.float32(0.02)
    packed, absmax = nf4.quantize(w)
    if not double_quant:
        return {"codes": packed, "absmax": absmax}
    q, step = nf4.double_quantize(absmax)
    return {"codes": packed, "qscale": q, "step": step}


def bytes_per_param(numel=1 << 16, double_quant=True):
    """Stored bytes per weight, from real buffers of a ``numel`` weight.

    ``numel`` should be a multiple of 64 * 256 so that no partial DQ group
    is present; the figure is then exact for any such matrix.
    """
    bufs = format_buffers(numel, double_quant)
    return sum(b.nbytes for b in bufs.values()) / numel


def bits_per_param(numel=1 << 16, double_quant=True):
    return 8.0 * bytes_per_param(numel, double_quant)


def scale_overhead_bits(numel=1 << 16, double_quant=True):
    """Bits per parameter spent on block constants (everything but the codes)."""
    bufs = format_buffers(numel, double_quant)
    return 8.0 * sum(b.nbytes for k, b in bufs.items() if k != "codes") / numel


def code_bits(numel=1 << 16):
    bufs = format_buffers(numel, True)
    return 8.0 * bufs["codes"].nbytes / numel


def frozen_base_gb(params, double_quant=True):
    """Frozen NF4 base of ``params`` weights, GB (1e9 bytes)."""
    return params * bytes_per_param(double_quant=double_quant) / GB


def breakdown_gb(params):
    """Component sizes in GB, as the pages list them for a model."""
    nodq = format_buffers(1 << 16, False)
    dq = format_buffers(1 << 16, True)
    n = float(1 << 16)
    return {
        "bf16": params * 2 / GB,
        "codes": params * nodq["codes"].nbytes / n / GB,
        "fp32_constants": params * nodq["absmax"].nbytes / n / GB,
        "dq_constants": params * (dq["qscale"].nbytes + dq["step"].nbytes) / n / GB,
        "total_dq": params * bytes_per_param(double_quant=True) / GB,
    }


def full_finetune_gb(params):
    """16-bit weights + 16-bit grads + two fp32 Adam states ([BILL] figure 1)."""
    return params * (2 + 2 + 4 + 4) / GB
