"""NF4 block quantization, double quantization and dequantization -- oracle.

TEST INFRASTRUCTURE (see the package docstring): plain numpy/stdlib code that
follows the pages step by step, with no blocking, fusion or reordering.

Sources, cited by page title and section:
  [NF4-fig3]  "A 65B fine-tune on the GPU you already have", figure 3
              (NF4 -- bins shaped like the weights): sixteen levels placed at
              quantiles of the zero-centred normal, equal mass per bin, dense
              near zero.
  [DQ-fig4]   same page, figure 4 (quantize the bookkeeping): one 32-bit
              constant per block of 64 weights; double quantization stores
              those constants in 8 bits, in blocks of 256.
  [ARCH-fig2] same page, figure 2 (the architecture): weights are
              dequantized block by block to bfloat16 right before the multiply.
  [IDEA]      "QLoRA and Quantized Training", section "The idea": 16 levels
              at normal quantiles, one scale per block, scales stored in
              8 bits; compute stays in bf16.
  [THREE]     "QLoRA Explained: 4-bit NF4, Double Quantization and Paged
              Optimizers", section "The three ideas behind QLoRA": levels at
              normal quantiles so each is used about equally often; the block
              constants are themselves quantized.

Readings where the pages leave a step open (each one is listed, with its
reason, in the design notes of the repository):
  R1 codebook: level i is the median of the i-th of 16 equal-mass bins of
     N(0,1), i.e. the quantile at probability (i + 1/2)/16, divided by the
     largest such quantile so the levels span [-1, 1]; fp64, rounded to fp32.
  R2 nearest code: a weight w in block b is normalised to v = fl32(w / absmax_b)
     (IEEE fp32 division); its code is the index of the level nearest to v in
     exact arithmetic, ties going to the lower index; a block whose absmax is
     0 is coded as v = 0.
  R3 packing: two codes per byte, the even element in the low nibble.
  R4 double quantization: groups of 256 consecutive blocks (flat block order,
     last group may be partial); step d = fl32(max_absmax / 127); code
     q = round-half-even(fl32(absmax / d)) clamped to [-127, 127], stored as
     int8; d == 0 gives q = 0.
  R5 dequantization: s = fl32(q * d); w' = bf16_rne(fl32(L[code] * s)).
"""
import statistics

import numpy as np

BLOCK = 64          # [DQ-fig4]: 64 weights share one 32-bit constant
DQ_GROUP = 256      # [DQ-fig4]: constants double-quantized in blocks of 256
DQ_QMAX = 127       # R4: symmetric signed 8-bit code


# --------------------------------------------------------------------------
# codebook
# --------------------------------------------------------------------------
def normal_quantile(p):
    """Inverse CDF of N(0,1) at probability p (Python stdlib, fp64)."""
    return statistics.NormalDist().inv_cdf(p)


def codebook():
    """The 16 NF4 levels, fp32, ascending ([NF4-fig3], [THREE], [IDEA]; R1)."""
    z = [normal_quantile((i + 0.5) / 16.0) for i in range(16)]
    top = z[15]
    return np.array([zi / top for zi in z], dtype=np.float64).astype(np.float32)


def level_midpoints(levels=None):
    """Exact real midpoints between adjacent fp32 levels, as fp64.

    Two fp32 numbers in [-1, 1] whose exponents differ by a few binades add
    exactly in fp64, and halving is exact, so these are the true midpoints.
    """
    L = codebook() if levels is None else levels
    L64 = L.astype(np.float64)
    return (L64[:-1] + L64[1:]) / 2.0


# --------------------------------------------------------------------------
# first-level quantization
# --------------------------------------------------------------------------
def block_absmax(w32):
    """Per-block max |w| over consecutive blocks of 64 ([DQ-fig4]); fp32, exact."""
    w = np.asarray(w32, dtype=np.float32).reshape(-1, BLOCK)
    return np.max(np.abs(w), axis=1).astype(np.float32)


def normalise(w32, absmax32):
    """v = fl32(w / absmax) per element (R2); v = 0 in blocks with absmax 0."""
    w = np.asarray(w32, dtype=np.float32).reshape(-1, BLOCK)
    a = np.asarray(absmax32, dtype=np.float32)
    zero = a == 0
    safe = np.where(zero, np.float32(1), a).astype(np.float32)
    v = (w / safe[:, None]).astype(np.float32)        # IEEE fp32 division
    v[zero, :] = np.float32(0)
    return v.reshape(-1)


def nearest_code(v32, levels=None):
    """Index of the level nearest each fp32 value, ties to the lower index (R2).

    For ascending levels, the nearest index equals the number of exact
    midpoints lying strictly below v (a value exactly on a midpoint stays on
    the lower side). v is widened to fp64 exactly, so every comparison is exact.
    """
    mids = level_midpoints(levels)
    v = np.asarray(v32, dtype=np.float32).astype(np.float64).reshape(-1)
    codes = np.zeros(v.shape, dtype=np.uint8)
    for m in mids:
        codes += (v > m).astype(np.uint8)
    return codes


def pack(codes):
    """Two 4-bit codes per byte, even element in the low nibble (R3)."""
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    assert c.size % 2 == 0
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def unpack(packed):
    """Inverse of ``pack``."""
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p & 0x0F
    out[1::2] = p >> 4
    return out


def quantize(w, levels=None):
    """Block-wise NF4 quantization of a flat weight array (``levels``: another
    16-level codebook, ascending, in [-1, 1]; see ``oracle.formats``).

    Accepts fp32 values, or bf16 given as uint16 bit patterns (widened to fp32
    exactly). Returns (packed uint8[numel/2], absmax fp32[numel/64]).
    """
    w = np.asarray(w)
    if w.dtype == np.uint16:
        w = bf16_bits_to_f32(w)
    w = w.astype(np.float32).reshape(-1)
    assert w.size % BLOCK == 0
    a = block_absmax(w)
    packed = np.empty(w.size // 2, dtype=np.uint8)
    chunk = 1 << 22                     # independent blocks, taken in slices
    for lo in range(0, w.size, chunk):  # only to bound the fp64 temporaries
        hi = min(lo + chunk, w.size)
        codes = nearest_code(normalise(w[lo:hi], a[lo // BLOCK:hi // BLOCK]), levels)
        packed[lo // 2:hi // 2] = pack(codes)
    return packed, a


# --------------------------------------------------------------------------
# double quantization of the block constants ([DQ-fig4]; R4)
# --------------------------------------------------------------------------
def double_quantize(absmax32):
    """absmax fp32[nb] -> (qscale int8[nb], step fp32[ceil(nb/256)])."""
    a = np.asarray(absmax32, dtype=np.float32).reshape(-1)
    nb = a.size
    ng = (nb + DQ_GROUP - 1) // DQ_GROUP
    q = np.zeros(nb, dtype=np.int8)
    step = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        blk = a[g * DQ_GROUP:(g + 1) * DQ_GROUP]
        c2 = np.float32(blk.max())
        d = np.float32(c2 / np.float32(DQ_QMAX))
        step[g] = d
        if d == 0:
            continue
        r = np.rint((blk / d).astype(np.float32))       # fp32 divide, RNE
        q[g * DQ_GROUP:(g + 1) * DQ_GROUP] = np.clip(r, -DQ_QMAX, DQ_QMAX).astype(np.int8)
    return q, step


def block_scales(qscale, step):
    """s_b = fl32(q_b * d_g) for every block b (R5)."""
    q = np.asarray(qscale, dtype=np.int8).astype(np.float32)
    d = np.asarray(step, dtype=np.float32)
    g = np.arange(q.size) // DQ_GROUP
    return (q * d[g]).astype(np.float32)


# --------------------------------------------------------------------------
# dequantization ([ARCH-fig2], [IDEA]; R5)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x32):
    """Round fp32 to bf16, nearest-even, on the integer bit pattern (finite input)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def dequantize(packed, qscale, step, numel=None, levels=None, absmax=None):
    """NF4 + double-quantized constants -> bf16 bit patterns (uint16[numel]).

    ``levels``: another codebook; ``absmax`` given (qscale, step None): the
    block constants stored in fp32 without double quantization (s = absmax).
    """
    codes = unpack(packed)
    if numel is not None:
        codes = codes[:numel]
    L = codebook() if levels is None else np.asarray(levels, dtype=np.float32)
    s = np.asarray(absmax, dtype=np.float32) if absmax is not None else block_scales(qscale, step)
    blk = np.arange(codes.size) // BLOCK
    prod = (L[codes] * s[blk]).astype(np.float32)       # fp32 product
    return f32_to_bf16_bits(prod)


def dequantize_range(packed, qscale, step, lo, hi):
    """Elements [lo, hi) of ``dequantize`` (lo, hi multiples of 64), computed
    from those elements' own codes, block constants and group steps only."""
    assert lo % BLOCK == 0 and hi % BLOCK == 0
    codes = unpack(np.asarray(packed)[lo // 2:hi // 2])
    blk = np.arange(lo, hi) // BLOCK
    q = np.asarray(qscale, dtype=np.int8)[blk].astype(np.float32)
    d = np.asarray(step, dtype=np.float32)[blk // DQ_GROUP]
    s = (q * d).astype(np.float32)
    prod = (codebook()[codes] * s).astype(np.float32)
    return f32_to_bf16_bits(prod)


def quantize_all(w, levels=None):
    """Convenience: the full storage format (packed, qscale, step, absmax)."""
    packed, absmax = quantize(w, levels)
    q, step = double_quantize(absmax)
    return packed, q, step, absmax


def n_groups(nblocks):
    return (nblocks + DQ_GROUP - 1) // DQ_GROUP


__all__ = [
    "BLOCK", "DQ_GROUP", "DQ_QMAX", "normal_quantile", "codebook",
    "level_midpoints", "block_absmax", "normalise", "nearest_code", "pack",
    "unpack", "quantize", "double_quantize", "block_scales",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "dequantize", "dequantize_range",
    "quantize_all",
    "n_groups",
]
