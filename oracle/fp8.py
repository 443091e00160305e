"""fp8 E4M3 cache elements, written out from [P3-fmt] (see oracle/__init__).

[P3-fmt] names vLLM's fp8_e4m3 cache as an 8-bit floating point format with
a 4-bit exponent and a 3-bit mantissa, and its memory paragraph puts an 8-bit
cache at about 32-34 KiB per token where 16-bit takes 64 KiB: one byte per
element, with no per-group scales for the fp8 variant (the 2 extra KiB are
the 32-element block scales of the integer q8_0 format). Everything else is a
reading, each also listed in the design notes:

  * Bit layout (the OCP 8-bit floating point E4M3 layout): sign bit 7,
    exponent bits 6..3 with bias 7, mantissa bits 2..0. Exponent field 0
    holds the subnormals m * 2^-9; there are no infinities; S.1111.111 is NaN,
    so the largest finite magnitude is 1.75 * 2^8 = 448.
  * One fp32 scale per cache for keys and one for values (the per-tensor
    scales of serving engines; 1.0 when the data already fits the range):
    code = e4m3(x / scale) with x / scale an IEEE fp32 division, and
    x_hat = scale * value(code).
  * e4m3() rounds to nearest with ties to the even code (the one whose
    mantissa is even) and saturates magnitudes above 448 to 448; the sign is
    kept, so a negative value that rounds to zero is -0 (code 0x80).
  * Dequantized fp16 (what kvq_dequantize writes): the fp32 product
    scale * value(code), rounded to fp16 (round to nearest even).
"""
import numpy as np

F16 = np.float16
F32 = np.float32

E4M3_MAX = 448.0
BIAS = 7


def e4m3_value(codes):
    """float64 value of each code (uint8 array), from the bit layout:
    (-1)^s * 2^(e-7) * (1 + m/8) for e > 0, (-1)^s * m * 2^-9 for e = 0, and
    NaN for S.1111.111."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** (1 - BIAS - 3),
                   (1.0 + m / 8.0) * np.exp2((e - BIAS).astype(np.float64)))
    val = s * mag
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)


# the 127 finite non-negative magnitudes, in code order (codes 0x00..0x7E);
# they increase with the code
_MAGS = e4m3_value(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x):
    """Code of each fp32 value: nearest magnitude, ties to the even code,
    saturating at 448, sign kept. Finite inputs only."""
    x = np.asarray(x, F32)
    a = np.abs(x.astype(np.float64))
    i = np.searchsorted(_MAGS, a)            # _MAGS[i-1] < a <= _MAGS[i]
    hi = np.minimum(i, 0x7E)
    lo = np.maximum(i - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)          # saturate (and exactly 448)
    code = np.where(a == 0, 0, code)
    sign = np.signbit(x)
    return (code | np.where(sign, 0x80, 0)).astype(np.uint8)


def quantize(x16, scale):
    """fp16 values -> fp8 codes: e4m3(fp32(x) / fp32(scale))."""
    q = np.asarray(x16, F16).astype(F32) / F32(scale)
    return e4m3_encode(q)


def dequantize_f64(codes, scale):
    """x_hat = scale * value(code), exact in float64."""
    return float(np.float64(F32(scale))) * e4m3_value(codes)


def dequantize_f16(codes, scale):
    """fp16 of the fp32 product scale * value(code) (each step rounded to
    nearest even)."""
    v = e4m3_value(codes).astype(F32)          # exact: 4 significant bits
    return (F32(scale) * v).astype(F16)
