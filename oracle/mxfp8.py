"""MXFP8 (E4M3 elements, E8M0 block scales) for the CPU oracle.  TEST INFRASTRUCTURE.

The report pages fix only the payload size of the format: an MXFP8 row costs
33/32 bytes per value against 2 bytes for BF16 ("Supercharging Olmo-core ...",
Section 24: Conclusion, Evidence 10), i.e. one byte per element plus one
shared byte per 32 elements.  The element and scale encodings are those of the
public OCP Microscaling Formats (MX) v1.0 specification, which this module
restates from its definitions:

* E4M3 ("FN" variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
  subnormals when the exponent field is 0; no infinities; S.1111.111 is NaN;
  largest finite magnitude 1.75 * 2**8 = 448.
* E8M0 scale: an unsigned biased exponent, value 2**(code - 127); 255 is NaN.
* Block of 32 consecutive values along the contraction (K) axis; shared
  exponent floor(log2(amax)) - 8 (8 = largest E4M3 exponent), clamped to the
  E8M0 range; elements are v / 2**shared_exp rounded to nearest-even and
  saturated to +-448.  Readings the specification leaves to the implementer,
  taken here: an all-zero block gets the smallest scale 2**-127 (code 0), and
  a value that rounds to zero keeps its sign (negative -> code 0x80, -0).

Everything is computed in float64, where every step above is exact.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest E4M3 binade
E8M0_BIAS = 127


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (float64); NaN for S.1111.111."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e8m0_decode(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - E8M0_BIAS))


# magnitude -> code for the 127 finite non-negative E4M3 codes (0x00 .. 0x7E)
_POS_VALUES = e4m3_decode(np.arange(0x7F))


def e4m3_round(u) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value (ties to even), saturating at +-448.

    The spacing of E4M3 values is 2**(e-3) in the binade [2**e, 2**(e+1)) for
    e >= -6, and 2**-9 below 2**-6 (subnormals).
    """
    u = np.asarray(u, dtype=np.float64)
    a = np.abs(u)
    _, ex = np.frexp(a)                      # a = f * 2**ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)               # binade exponent, subnormal floor
    quantum_exp = e - 3
    q = np.ldexp(np.rint(np.ldexp(a, -quantum_exp)), quantum_exp)
    q = np.minimum(q, E4M3_MAX)
    return np.copysign(q, u)


def e4m3_encode(u) -> np.ndarray:
    """E4M3 code of float64 values (rounded to nearest-even, saturating); sign kept on zero."""
    q = e4m3_round(u)
    # codes 0x00..0x7E are in ascending order of magnitude, so the code of a
    # representable magnitude is its index in the sorted table
    mag_codes = np.searchsorted(_POS_VALUES, np.abs(q)).astype(np.uint8)
    sign = np.signbit(q).astype(np.uint8) << 7
    return (mag_codes | sign).astype(np.uint8)


def shared_exponent(amax) -> np.ndarray:
    """floor(log2(amax)) - 8, clamped to [-127, 127]; -127 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                   # amax = f * 2**ex, f in [0.5, 1) -> floor(log2) = ex - 1
    se = ex - 1 - E4M3_EMAX
    se = np.where(amax == 0, -E8M0_BIAS, se)
    return np.clip(se, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize(v, axis: int = -1):
    """MX-quantise along ``axis`` in blocks of 32.

    Returns (codes uint8, same shape as v; scales uint8, with ``axis`` shrunk by 32).
    """
    v = np.moveaxis(np.asarray(v, dtype=np.float64), axis, -1)
    n = v.shape[-1]
    if n % BLOCK:
        raise ValueError(f"length {n} along the block axis is not a multiple of {BLOCK}")
    blocks = v.reshape(v.shape[:-1] + (n // BLOCK, BLOCK))
    se = shared_exponent(np.max(np.abs(blocks), axis=-1))
    scaled = np.ldexp(blocks, -se[..., None])            # exact: power-of-two scaling in float64
    codes = e4m3_encode(scaled).reshape(v.shape)
    scales = (se + E8M0_BIAS).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def dequantize(codes, scales, axis: int = -1) -> np.ndarray:
    """Inverse of :func:`quantize` (exact): element value times its block's scale."""
    c = np.moveaxis(np.asarray(codes), axis, -1)
    s = np.moveaxis(np.asarray(scales), axis, -1)
    n = c.shape[-1]
    vals = e4m3_decode(c).reshape(c.shape[:-1] + (n // BLOCK, BLOCK))
    out = vals * e8m0_decode(s)[..., None]
    return np.moveaxis(out.reshape(c.shape), -1, axis)


def fake_quantize(v, axis: int = -1) -> np.ndarray:
    """deQ(Q(v)): the values an MXFP8 tensor actually holds."""
    codes, scales = quantize(v, axis)
    return dequantize(codes, scales, axis)
