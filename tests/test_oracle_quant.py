"""Pins of the oracle's group quantizer against what the pages and arithmetic
fix: hand-worked examples, the scale/2 error bound, round-trip identity on
grid values, closed-form special cases, and the axis-choice effect the pages
describe. CPU only."""
import json
import os
import struct

import numpy as np
import pytest

from oracle import quant

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    with open(os.path.join(GOLD, "quant_hand_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"int{c['bits']}-{c['x'][0]}")
def test_hand_cases(case):
    x = np.array(case["x"], np.float16)[None]
    q, s, z = quant.quantize_groups(x, case["bits"])
    assert float(s[0]) == case["scale"]
    assert float(z[0]) == case["zero"]
    assert q[0].tolist() == case["q"]
    xh = quant.dequantize(q, s[:, None], z[:, None])[0]
    assert xh.tolist() == case["x_hat"]


def test_ranges():
    # int8 [-128,127] and int4 [-8,7] as printed; int2 [-2,1] (four levels)
    assert quant.qrange(8) == (-128, 127)
    assert quant.qrange(4) == (-8, 7)
    assert quant.qrange(2) == (-2, 1)
    with pytest.raises(ValueError):
        quant.qrange(3)


def _half_up_reference(v):
    """Smallest fp16 >= v by brute force over fp16 bit patterns, using the
    standard library's IEEE half decoding."""
    pats = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = np.array([struct.unpack("<e", struct.pack("<H", int(p)))[0] for p in pats])
    i = np.searchsorted(vals, v, side="left")
    return vals[i]


def test_scale_rounds_up_brute_force():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.random(300, dtype=np.float32) * 50,
                         rng.random(100, dtype=np.float32) * 1e-4,
                         np.float32([2.0 ** -30, 1.0, 0.2, 65504.0])]).astype(np.float32)
    got = quant.f32_to_f16_up(xs).astype(np.float64)
    want = np.array([_half_up_reference(float(v)) for v in xs])
    assert np.array_equal(got, want)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("n", [32, 128])
def test_error_bound(bits, n):
    """|x - x_hat| <= scale/2 per element ("Integer quantization in one
    screen"), plus 2^-12 * scale for the fp32 rounding of x/scale."""
    rng = np.random.default_rng(bits * 1000 + n)
    x = rng.standard_normal((4000, n), dtype=np.float32)
    x[::7, 3] *= 20
    x[::11] *= 1e-3
    x[::13] += 5
    # groups far from zero compared with their spread (widened scale)
    x[1::17] = x[1::17] * 1e-2 + 300
    x[2::19] = x[2::19] * 1e-3 - 40
    x = x.astype(np.float16)
    q, s, z = quant.quantize_groups(x, bits)
    xf = x.astype(np.float32)
    qmin, qmax = quant.qrange(bits)
    s_formula = quant.f32_to_f16_up((xf.max(1) - xf.min(1)) / np.float32(qmax - qmin))
    widened = s.astype(np.float32) > s_formula.astype(np.float32)
    assert widened.sum() >= 100
    # every zero point is an integer fp16 holds exactly
    zf = z.astype(np.float64)
    assert np.all(np.abs(zf) <= 2048) and np.all(zf == np.rint(zf))
    xh = quant.dequantize(q, s[:, None], z[:, None]).astype(np.float64)
    err = np.abs(x.astype(np.float64) - xh)
    bound = s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -12)
    assert np.all(err <= bound)
    assert np.all(err[widened] <= bound[widened])
    # the bound is attained (up to the slack) on some element: it is tight
    assert np.max(err / bound) > 0.9


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_round_trip_on_grid(bits):
    """Values already on a grid s*(q - z) with an exact power-of-two s come
    back with the same q, s, z and bit-identical reconstruction."""
    qmin, qmax = quant.qrange(bits)
    rng = np.random.default_rng(bits)
    n, G = 128, 500
    q = rng.integers(qmin, qmax, size=(G, n), endpoint=True)
    q[:, 0], q[:, 1] = qmin, qmax
    z = rng.integers(qmin, qmax, size=G, endpoint=True)
    s = 2.0 ** -4
    x = (s * (q - z[:, None])).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), s * (q - z[:, None]))
    q2, s2, z2 = quant.quantize_groups(x, bits)
    assert np.all(s2 == np.float16(s))
    assert np.array_equal(z2.astype(np.int64), z)
    assert np.array_equal(q2.astype(np.int64), q)
    xh = quant.dequantize(q2, s2[:, None], z2[:, None]).astype(np.float16)
    assert np.array_equal(quant.f16_bits(xh), quant.f16_bits(x))
    # idempotence: quantizing the reconstruction changes nothing
    q3, s3, z3 = quant.quantize_groups(xh, bits)
    assert np.array_equal(q3, q2) and np.array_equal(s3, s2) and np.array_equal(z3, z2)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_closed_form_specials(bits):
    qmin, qmax = quant.qrange(bits)
    rng = np.random.default_rng(7 + bits)
    x = rng.standard_normal((2000, 32), dtype=np.float32).astype(np.float16)
    q, s, z = quant.quantize_groups(x, bits)
    xf = x.astype(np.float32)
    # the group minimum always lands on q_min; the maximum on q_max, or one
    # below it when rounding the scale up shrank max/scale below the top level
    assert np.all(q[np.arange(2000), xf.argmin(1)] == qmin)
    top = q[np.arange(2000), xf.argmax(1)]
    assert np.all((top == qmax) | (top == qmax - 1))
    assert np.mean(top == qmax) > 0.5
    # zero (inside every one of these ranges) codes to z and reconstructs to 0
    x0 = x.copy()
    x0[:, 5] = 0
    q0, s0, z0 = quant.quantize_groups(x0, bits)
    assert np.array_equal(q0[:, 5].astype(np.float32), z0.astype(np.float32))
    assert np.all(quant.dequantize(q0, s0[:, None], z0[:, None])[:, 5] == 0)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_constant_groups_exact(bits):
    qmin, _ = quant.qrange(bits)
    vals = np.float16([0.0, 1.5, -3.25, 6e-8, -65504.0, 1000.0])
    x = np.repeat(vals[:, None], 16, axis=1)
    q, s, z = quant.quantize_groups(x, bits)
    assert np.all(q == qmin)
    xh = quant.dequantize(q, s[:, None], z[:, None])
    assert np.array_equal(xh, x.astype(np.float32))


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_offset_groups_keep_the_bound(bits):
    """Groups far from zero compared with their spread would need a zero point
    fp16 cannot hold; the widened scale keeps |z| <= 2048, the minimum on
    q_min, no code past q_max, and the scale/2 bound. Offsets of both signs
    and sizes up to the fp16 range."""
    qmin, qmax = quant.qrange(bits)
    rng = np.random.default_rng(40 + bits)
    off = np.concatenate([10.0 ** rng.uniform(1, 4.5, 500), -(10.0 ** rng.uniform(1, 4.5, 500))])
    x = (off[:, None] + rng.standard_normal((1000, 32)) * np.abs(off[:, None]) * 1e-3)
    x = np.clip(x, -65504, 65504).astype(np.float16)
    q, s, z = quant.quantize_groups(x, bits)
    assert np.all(np.abs(z.astype(np.float64)) <= 2048)
    # the zero point in stored-code units (z - q_min) is an exact fp16 integer too
    assert np.all(np.abs(z.astype(np.float64) - qmin) <= 2048 + qmin)
    xf = x.astype(np.float64)
    assert np.all(q[np.arange(1000), xf.argmin(1)] == qmin)
    assert np.all(q <= qmax)
    xh = quant.dequantize(q, s[:, None], z[:, None]).astype(np.float64)
    assert np.all(np.abs(xf - xh) <= s.astype(np.float64)[:, None] * (0.5 + 2.0 ** -12))


def test_symmetric_data_int8_zero():
    """For data spanning [-a, a] at int8 the zero-point is 0 or -1."""
    a = np.float16([0.1, 1.0, 3.0, 17.0, 250.0])
    x = np.stack([-a, a, np.zeros_like(a)], axis=1)
    _, _, z = quant.quantize_groups(x, 8)
    assert set(z.astype(int).tolist()) <= {0, -1}


def test_outlier_channel_coarsens_per_token_step():
    """Outlier section: a per-token scale must cover the largest value, so one
    large channel coarsens the step of every ordinary channel. With ordinary
    channels spanning [-1, 1] and one channel at 20 the asymmetric range grows
    from 2 to 21, so the int4 step grows 10.5x (a symmetric scale, max|x|/q_max,
    would grow exactly 20x, the page's figure)."""
    x = np.zeros((2, 128), np.float32)
    x[:, :] = np.linspace(-1, 1, 128, dtype=np.float32)
    x[1, 64] = 20.0
    _, s, _ = quant.quantize_groups(x.astype(np.float16), 4)
    ratio = float(s[1]) / float(s[0])
    assert abs(ratio - 10.5) < 0.01
    # on the synthetic keys (four N(0,1) channels x20) the step grows several-fold
    rng = np.random.default_rng(3)
    base = rng.standard_normal((2000, 128), dtype=np.float32)
    out = base.copy()
    out[:, [3, 17, 64, 101]] *= 20
    _, s0, _ = quant.quantize_groups(base.astype(np.float16), 4)
    _, s1, _ = quant.quantize_groups(out.astype(np.float16), 4)
    assert np.median(s1.astype(np.float64) / s0.astype(np.float64)) > 5


def test_per_channel_keys_beat_per_token():
    """Keys with outlier channels: grouping along channels (over tokens) gives a
    far smaller error on the ordinary channels than grouping per token; for
    values (no outlier channels) the two axes are comparable."""
    rng = np.random.default_rng(4)
    k = rng.standard_normal((256, 128), dtype=np.float32)
    k[:, [3, 17, 64, 101]] *= 20
    k = k.astype(np.float16)
    ordinary = np.setdiff1d(np.arange(128), [3, 17, 64, 101])

    def mse_token(x):
        q, s, z = quant.quantize_groups(x, 4)
        return (quant.dequantize(q, s[:, None], z[:, None]) - x.astype(np.float32)) ** 2

    def mse_channel(x):
        g = x.reshape(8, 32, 128).transpose(0, 2, 1)
        q, s, z = quant.quantize_groups(g, 4)
        xh = quant.dequantize(q, s[..., None], z[..., None]).transpose(0, 2, 1).reshape(256, 128)
        return (xh - x.astype(np.float32)) ** 2

    assert mse_channel(k)[:, ordinary].mean() * 20 < mse_token(k)[:, ordinary].mean()
    v = rng.standard_normal((256, 128), dtype=np.float32).astype(np.float16)
    r = mse_channel(v).mean() / mse_token(v).mean()
    assert 0.3 < r < 3


def test_sparse_split_hand_case():
    x = np.zeros((3, 8), np.float16)
    x[0] = [1, -9, 3, 9, 0, 2, -2, 5]          # |-9| == |9|: both kept
    x[1] = [4, 4, 4, 4, 1, 1, 1, 1]            # ties: lowest channels 0,1
    x[2] = [0, 0, 0, 0, 0, 0, 0, -7]           # one non-zero, then a zero tie -> channel 0
    dense, cols, vals = quant.split_sparse(x, 2)
    assert cols.tolist() == [[1, 3], [0, 1], [0, 7]]
    assert vals.astype(float).tolist() == [[-9, 9], [4, 4], [0, -7]]
    assert dense[0].astype(float).tolist() == [1, 0, 3, 0, 0, 2, -2, 5]
    assert quant.f16_bits(dense[2, 7]) == 0   # +0, not -0


def test_sparse_brute_force():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((300, 16)) * 3).round(0).astype(np.float16)
    dense, cols, vals = quant.split_sparse(x, 2)
    for r in range(300):
        mags = [abs(float(v)) for v in x[r]]
        pick = sorted(range(16), key=lambda c: (-mags[c], c))[:2]
        assert sorted(pick) == cols[r].tolist()
        rest = [mags[c] for c in range(16) if c not in pick]
        assert min(mags[c] for c in pick) >= max(rest)
