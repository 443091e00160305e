"""Affine group quantization, written out from [P2-int] (see oracle/__init__).

A *group* is a set of fp16 values that share one scale and one zero-point:
one token's channel vector (per-token), or one channel over 32 consecutive
tokens (per-channel keys). Everything below is elementwise IEEE fp32 numpy
arithmetic with round-half-to-even, done in the order the formulas give:

    scale      = (x_max - x_min) / (q_max - q_min)
    zero_point = q_min - round(x_min / scale)
    q          = round(x / scale) + zero_point
    x_hat      = scale * (q - zero_point)

Readings where the page is silent (each is also listed in the design notes):
  * round() is round-half-to-even (numpy.rint).
  * The scale is stored as fp16 rounded toward +inf: the smallest fp16 >= the
    fp32 quotient. With round-to-nearest the stored scale can be slightly
    below the quotient and the top code then lands past q_max, breaking the
    page's error bound of scale/2; rounding up keeps the bound.
  * q is clamped to [q_min, q_max] (needed at half-way ties).
  * A constant group (x_max == x_min) would divide by zero; it takes scale =
    |x_min| (or 1 when x_min == 0), which reconstructs every element exactly.
  * The zero-point is stored as fp16, which holds every integer in
    [-2048, 2048] exactly; codes are stored unsigned (q - q_min), so the zero
    point in those units, z - q_min = -round(x_min / scale), must be an exact
    fp16 integer too. Both hold while |round(x_min / scale)| <= 2048 + q_min.
    A group lying far from zero compared with its spread breaks that; such a
    group instead takes the smallest fp16 scale >= |x_min| / (2048 + q_min),
    which brings round(x_min / scale) back inside. The codes then still use at
    most the q_max - q_min steps of the range, so every element stays within
    scale/2 of its reconstruction at the stored (wider) scale.
  * int2 uses [-2, 1] (two's complement, the four levels of [P1-kivi]).

Symmetric groups ([P2-int] "Symmetric vs asymmetric") force the zero point to
zero: scale = max|x| / q_max (the range [-q_max, q_max] centred on zero),
stored as fp16 rounded up, q = clamp(round(x / scale), -q_max, q_max) and
x_hat = scale * q; an all-zero group takes scale 1.
"""
import numpy as np

F16 = np.float16
F32 = np.float32

F16_INT_LIMIT = 2048  # every integer of magnitude <= 2048 is an exact fp16


def qrange(bits):
    """Signed integer range of a b-bit code: int8 [-128,127], int4 [-8,7]
    ([P2-int]); int2 [-2,1] (reading)."""
    if bits not in (2, 4, 8):
        raise ValueError("bits must be 2, 4 or 8")
    return -(1 << (bits - 1)), (1 << (bits - 1)) - 1


def f16_bits(a):
    """fp16 array -> its uint16 bit patterns."""
    return np.ascontiguousarray(a, dtype=F16).view(np.uint16)


def bits_f16(b):
    """uint16 bit patterns -> fp16 array."""
    return np.ascontiguousarray(b, dtype=np.uint16).view(F16)


def f32_to_f16_up(x):
    """Smallest fp16 >= x for finite non-negative fp32 x: round to nearest,
    then step one fp16 ulp up when that landed below x."""
    x = np.asarray(x, dtype=F32)
    h = x.astype(F16)
    below = h.astype(F32) < x
    hb = f16_bits(h).copy()
    hb[below] += 1  # positive fp16 patterns are ordered like their values
    return bits_f16(hb)


def group_scale_zero(xmin, xmax, bits):
    """Scale and zero-point of groups with the given fp32 extremes.

    Returns (s16, z16) as fp16 arrays; s = float(s16) is the scale the codes
    use. [P2-int] formulas with the readings listed in the module docstring.
    """
    qmin, qmax = qrange(bits)
    xmin = np.asarray(xmin, dtype=F32)
    xmax = np.asarray(xmax, dtype=F32)
    n_lev = F32(qmax - qmin)
    with np.errstate(divide="ignore", invalid="ignore"):
        s32 = (xmax - xmin) / n_lev                      # fp32 range / levels
        s16 = f32_to_f16_up(s32)                         # stored scale, rounded up
        const = xmax == xmin
        s_const = np.where(xmin != 0, np.abs(xmin), F32(1.0)).astype(F16)
        s16 = np.where(const, s_const, s16)
        s = s16.astype(F32)
        r = np.rint(xmin / s)                            # round(x_min / scale)
        # zero points that fp16 would not hold exactly: widen the scale instead
        lim = F32(F16_INT_LIMIT + qmin)
        wide = np.abs(r) > lim
        if np.any(wide):
            s16 = np.where(wide, f32_to_f16_up(np.abs(xmin) / lim), s16)
            s = s16.astype(F32)
            r = np.rint(xmin / s)
        z = F32(qmin) - r                                # zero_point, fp32
    assert np.all(np.abs(r) <= lim) and np.all(np.abs(z) <= F16_INT_LIMIT)
    return s16, z.astype(F16)


def quantize_groups(x16, bits):
    """Quantize groups laid out along the last axis of an fp16 array.

    x16: fp16 array [..., n]; each row of n values is one group.
    Returns (q int8 [..., n], s16 fp16 [...], z16 fp16 [...]).
    """
    x16 = np.asarray(x16, dtype=F16)
    qmin, qmax = qrange(bits)
    x = x16.astype(F32)
    xmin = x.min(axis=-1)
    xmax = x.max(axis=-1)
    s16, z16 = group_scale_zero(xmin, xmax, bits)
    s = s16.astype(F32)[..., None]
    z = z16.astype(F32)[..., None]
    q = np.rint(x / s) + z                               # round(x/scale) + zp
    q = np.clip(q, F32(qmin), F32(qmax))
    return q.astype(np.int8), s16, z16


def dequantize(q, s16, z16):
    """x_hat = scale * (q - zero_point) in fp32 ([P2-int]). Exact: |q - z| has at
    most 12 significant bits and the fp16 scale 11, so the product fits fp32's
    24-bit significand. Broadcasting: s16/z16 must broadcast against q."""
    return np.asarray(s16, dtype=F16).astype(F32) * (
        np.asarray(q).astype(F32) - np.asarray(z16, dtype=F16).astype(F32))


def dequantize_f64(q, s16, z16):
    """The same value as dequantize(), computed in float64."""
    return np.asarray(s16, dtype=F16).astype(np.float64) * (
        np.asarray(q).astype(np.float64) - np.asarray(z16, dtype=F16).astype(np.float64))


def sym_qmax(bits):
    """Largest code of the symmetric range [-q_max, q_max] centred on zero:
    127, 7, 1 for 8, 4, 2 bits."""
    return qrange(bits)[1]


def sym_scale(amax, bits):
    """Scale of symmetric groups ([P2-int] "Symmetric vs asymmetric": zero
    point forced to zero, the integer range centred on real zero), with the
    readings: scale = max|x| / q_max rounded up to fp16 (as for the affine
    scale, so that every element stays within scale/2), and scale 1 for an
    all-zero group. Returns fp16 scales."""
    amax = np.asarray(amax, dtype=F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        s16 = f32_to_f16_up(amax / F32(sym_qmax(bits)))
    return np.where(amax == 0, F16(1.0), s16).astype(F16)


def quantize_sym_groups(x16, bits):
    """Symmetric quantization of groups along the last axis: q =
    clamp(round(x / scale), -q_max, q_max), no zero point.
    Returns (q int8 [..., n], s16 fp16 [...])."""
    x = np.asarray(x16, dtype=F16).astype(F32)
    qm = F32(sym_qmax(bits))
    s16 = sym_scale(np.abs(x).max(axis=-1), bits)
    q = np.clip(np.rint(x / s16.astype(F32)[..., None]), -qm, qm)
    return q.astype(np.int8), s16


def dequantize_sym(q, s16):
    """x_hat = scale * q: one multiply, exact in fp32 (at most 8 + 11
    significant bits)."""
    return np.asarray(s16, dtype=F16).astype(F32) * np.asarray(q).astype(F32)


def split_sparse(x16, k):
    """Dense-and-sparse split of key vectors ([P1-kivi], KVQuant's per-vector
    outlier isolation), with the reading: per vector keep the k entries of
    largest |x| (ties to the lower channel) in fp16, listed by ascending
    channel, and set them to +0 in the dense copy.

    x16: fp16 [..., D]. Returns (dense fp16 [..., D], cols int [..., k],
    vals fp16 [..., k]). Magnitudes are compared as fp16 absolute-value bit
    patterns, which order finite fp16 magnitudes exactly.
    """
    x16 = np.asarray(x16, dtype=F16)
    mag = (f16_bits(x16) & 0x7FFF).astype(np.int32)
    order = np.argsort(-mag, axis=-1, kind="stable")     # stable: ties keep lower channel first
    cols = np.sort(order[..., :k], axis=-1)
    vals = np.take_along_axis(x16, cols, axis=-1)
    dense = x16.copy()
    np.put_along_axis(dense, cols, F16(0.0), axis=-1)
    return dense, cols, vals
