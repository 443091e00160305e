"""Pins of the fp8 E4M3 oracle (oracle/fp8.py).

The pages name the format only ("KV Cache Quantization Benchmarked: 8-bit Is
Nearly Lossless, How Much Does 4-bit Cost?": an 8-bit float with a 4-bit
exponent and a 3-bit mantissa, about 32-34 KiB per token where 16 bits take
64 KiB). The decoding is pinned by closed-form values and by PyTorch's own
float8_e4m3fn type (an independent implementation of the same layout); the
encoding by PyTorch's rounding cast inside the finite range, by an exact
rational brute force, and by closed forms for ties and saturation; the cache
level by brute-force attention and by the pages' 8-bit size figures."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import fp8, sizes
from oracle.cache import Config, RefCache

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_closed_forms():
    v = lambda c: float(fp8.e4m3_value(np.array([c], np.uint8))[0])
    assert v(0x00) == 0.0 and math.copysign(1, v(0x80)) == -1.0
    assert v(0x01) == 2.0 ** -9            # smallest subnormal
    assert v(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert v(0x08) == 2.0 ** -6            # smallest normal
    assert v(0x38) == 1.0                  # exponent field 7 = bias
    assert v(0x3F) == 1.875
    assert v(0x40) == 2.0
    assert v(0x7E) == 448.0 == fp8.E4M3_MAX
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert v(0xFE) == -448.0
    finite = fp8.e4m3_value(np.arange(256, dtype=np.uint8))
    assert np.isnan(finite).sum() == 2
    # positive codes are ordered like their values
    assert np.all(np.diff(finite[:0x7F]) > 0)


def test_decode_matches_torch_float8():
    torch = pytest.importorskip("torch")
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    tv = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(tv, fp8.e4m3_value(np.arange(256, dtype=np.uint8)), equal_nan=True)


def _probe_values():
    """fp32 inputs: every finite value, every midpoint between neighbours and
    its two fp32 neighbours, and random values over the whole range."""
    mags = fp8.e4m3_value(np.arange(0x7F, dtype=np.uint8))
    mids = (mags[:-1] + mags[1:]) / 2
    m32 = mids.astype(np.float32)
    near = np.concatenate([np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(1e9))])
    rng = np.random.default_rng(5)
    rnd = (rng.standard_normal(4000) * np.exp2(rng.uniform(-12, 9, 4000))).astype(np.float32)
    x = np.concatenate([mags.astype(np.float32), near, rnd])
    return np.concatenate([x, -x]).astype(np.float32)


def test_encode_matches_torch_cast_in_range():
    torch = pytest.importorskip("torch")
    x = _probe_values()
    x = x[np.abs(x) < 464]                  # torch's cast gives NaN above the range
    got = fp8.e4m3_encode(x)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, want)


def _nearest_exact(x):
    """Brute force in exact rational arithmetic: the nearest finite magnitude,
    ties to the even code, saturating at 448."""
    a = abs(Fraction(float(x)))
    best = None
    for c in range(0x7F):
        d = abs(a - Fraction(float(fp8.e4m3_value(np.array([c], np.uint8))[0])))
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    c = 0x7E if a >= 448 else best[1]
    return c | (0x80 if math.copysign(1.0, float(x)) < 0 else 0)


def test_encode_brute_force_exact():
    x = _probe_values()
    rng = np.random.default_rng(6)
    pick = np.concatenate([rng.choice(len(x), 600, replace=False),
                           np.arange(0, 381)])          # all grid values and midpoints
    xs = x[pick]
    got = fp8.e4m3_encode(xs)
    want = np.array([_nearest_exact(v) for v in xs], np.uint8)
    assert np.array_equal(got, want)


def test_round_trip_on_the_grid():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = fp8.e4m3_value(codes).astype(np.float32)
    assert np.array_equal(fp8.e4m3_encode(vals), codes)


def test_ties_and_saturation():
    enc = lambda v: int(fp8.e4m3_encode(np.array([v], np.float32))[0])
    assert enc(1.0625) == 0x38       # between 1 (0x38) and 1.125 (0x39): even code
    assert enc(1.1875) == 0x3A       # between 1.125 and 1.25 (0x3A): even code
    assert enc(2.0 ** -10) == 0x00   # half the smallest subnormal: ties to 0
    assert enc(3 * 2.0 ** -10) == 0x02
    assert enc(-1e-9) == 0x80        # negative underflow keeps the sign
    for big in (448.0, 460.0, 464.0, 500.0, 1e30):
        assert enc(big) == 0x7E and enc(-big) == 0xFE


def test_error_at_most_half_spacing():
    x = _probe_values()
    x = x[np.abs(x) <= 448]
    err = np.abs(x.astype(np.float64) - fp8.e4m3_value(fp8.e4m3_encode(x)))
    a = np.abs(x.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    spacing = np.exp2(e - 3)                 # 3 mantissa bits; 2^-9 below 2^-6
    assert np.all(err <= spacing / 2)


def test_scale_divides_before_rounding():
    x = np.array([1.0, -3.0, 100.0, 0.01], np.float16)
    for s in (1.0, 0.25, 3.0):
        codes = fp8.quantize(x, s)
        assert np.array_equal(codes, fp8.e4m3_encode(x.astype(np.float32) / np.float32(s)))
        # exact values on the grid come back exactly
    grid = fp8.e4m3_value(np.array([0x38, 0x40, 0xC0, 0x50], np.uint8))
    assert np.array_equal(fp8.dequantize_f64(fp8.quantize((grid * 0.5).astype(np.float16), 0.5), 0.5),
                          grid * 0.5)


def _fp8_cfg(H=2, g=2):
    return Config(128, H, H * g, 8, 8, "token", 0, 0, 0, k_format="fp8", v_format="fp8",
                  k_scale=0.5, v_scale=2.0)


def test_cache_attention_brute_force():
    cfg = _fp8_cfg()
    rng = np.random.default_rng(7)
    c = RefCache(cfg, 2, 64)
    n = [5, 9]
    k = (rng.standard_normal((sum(n), 2, 128)) * 3).astype(np.float16)
    v = rng.standard_normal((sum(n), 2, 128)).astype(np.float16)
    c.append(k, v, n)
    q = rng.standard_normal((2, 4, 128)).astype(np.float16)
    out = c.attention(q, 0.125)
    off = 0
    for b in range(2):
        kb, vb = k[off:off + n[b]], v[off:off + n[b]]
        off += n[b]
        for hq in range(4):
            h = hq // 2
            kh = [[0.5 * float(fp8.e4m3_value(np.array([fp8.e4m3_encode(np.float32(x) / np.float32(0.5))[()]], np.uint8))[0])
                   for x in row] for row in kb[:, h].astype(np.float32)]
            vh = 2.0 * fp8.e4m3_value(fp8.e4m3_encode(vb[:, h].astype(np.float32) / np.float32(2.0)))
            sc = [0.125 * sum(a * float(qq) for a, qq in zip(row, q[b, hq])) for row in kh]
            m = max(sc)
            p = [math.exp(s - m) for s in sc]
            want = sum(pi * vh[t] for t, pi in enumerate(p)) / sum(p)
            assert np.max(np.abs(out[b, hq] - want)) < 1e-12


def test_cache_layout_and_sizes():
    cfg = _fp8_cfg()
    c = RefCache(cfg, 1, 64)
    rng = np.random.default_rng(8)
    k = rng.standard_normal((40, 2, 128)).astype(np.float16)
    v = rng.standard_normal((40, 2, 128)).astype(np.float16)
    c.append(k, v, [40])
    pk = c.pack()
    assert set(pk) == {"k_codes", "v_codes"}              # no metadata arrays
    # keys: token-major rows of the raw codes; values: per-block channel records
    assert np.array_equal(pk["k_codes"][0, 1, 7], fp8.quantize(k[7, 1], 0.5))
    assert np.array_equal(pk["v_codes"][0, 1, 1, 5, :8], fp8.quantize(v[32:40, 1, 5], 2.0))
    a = sizes.actual_bytes(cfg, 1, 64)
    assert a["k_meta"] == a["v_meta"] == 0
    assert (a["k_codes"] + a["v_codes"]) == a["nominal_bytes"] == 2 * 2 * 64 * 128


def test_pages_8bit_size_figures():
    g = json.load(open(os.path.join(GOLD, "sizes_worked_example.json")))
    base, c8 = g["context_64k"], g["context_64k_8bit"]
    per16 = base["fp16_KiB_per_token"] * 1024
    fp8_tok = per16 // 2                                   # one byte per element, no scales
    q8_tok = fp8_tok + (per16 // 2) // c8["block_elements_q8_0"] * 2   # + an fp16 scale per 32
    lo, hi = c8["KiB_per_token_printed_range"]
    assert fp8_tok == lo * 1024 and q8_tok == hi * 1024
    assert round(fp8_tok * base["tokens"] / 2 ** 30) == c8["GiB_printed"]
