"""Pins of the symmetric quantizer and the symmetric 32-element block format
(oracle/quant.py sym_*, oracle/cache.py "sym32").

Sources: "KV Cache Quantization — 8-bit and 4-bit", "Symmetric vs asymmetric"
(zero point forced to zero, range centred on real zero, x_hat = scale * q, and
its example: data in [-0.1, 3.0] make a symmetric range stretch to +-3 and
waste half the codes); "KV Cache Quantization Benchmarked: 8-bit Is Nearly
Lossless, How Much Does 4-bit Cost?" (q8_0 / q4_0: 32 elements share a scale;
about 34 and 18 KiB per token where 16 bits take 64 KiB)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import quant, sizes
from oracle.cache import Config, RefCache

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f16_up(r):
    """Smallest fp16 >= the positive rational r, by exhaustive search over
    positive fp16 patterns (decoded with the stdlib)."""
    import struct
    best = None
    for bits in range(0x0001, 0x7C00):
        v = Fraction(struct.unpack("<e", struct.pack("<H", bits))[0])
        if v >= r:
            best = v
            break
    return best


@pytest.mark.parametrize("bits,xs", [(4, [-1.0, 0.5, 3.0]), (8, [-3.0, 3.0, 0.0, 1.0]), (2, [-0.5, 0.2, 1.0])])
def test_hand_cases_exact(bits, xs):
    qmax = 2 ** (bits - 1) - 1
    amax = max(abs(Fraction(x)) for x in xs)
    s = _f16_up(amax / qmax)
    want_q = []
    for x in xs:
        r = Fraction(x) / s
        fl = math.floor(r)
        q = fl + 1 if (r - fl > Fraction(1, 2) or (r - fl == Fraction(1, 2) and fl % 2 == 1)) else fl
        want_q.append(max(-qmax, min(qmax, q)))
    q, s16 = quant.quantize_sym_groups(np.array([xs], np.float16), bits)
    assert Fraction(float(s16[0])) == s
    assert q[0].tolist() == want_q
    xh = quant.dequantize_sym(q, s16[:, None])
    assert [Fraction(float(v)) for v in xh[0]] == [s * qq for qq in want_q]     # one exact multiply


def test_int4_case_values():
    # worked by hand: 3/7 rounds up to the fp16 0.4287109375; codes -2, 1, 7
    q, s16 = quant.quantize_sym_groups(np.array([[-1.0, 0.5, 3.0]], np.float16), 4)
    assert float(s16[0]) == 0.4287109375
    assert q.tolist() == [[-2, 1, 7]]


def test_lopsided_data_wastes_half_the_codes():
    x = np.linspace(-0.1, 3.0, 4001).astype(np.float16)[None, :]
    qs, _ = quant.quantize_sym_groups(x, 4)
    used_sym = np.unique(qs)
    assert used_sym.tolist() == list(range(0, 8))          # 8 of the 15 symmetric levels
    qa, _, _ = quant.quantize_groups(x, 4)
    assert len(np.unique(qa)) == 16                        # the affine grid uses all 16
    # and its step is about half the symmetric one
    _, sa, _ = quant.quantize_groups(x, 4)
    _, ss = quant.quantize_sym_groups(x, 4)
    assert 1.8 < float(ss[0]) / float(sa[0]) < 2.1


def test_error_within_half_a_step():
    rng = np.random.default_rng(12)
    for bits in (2, 4, 8):
        x = (rng.standard_normal((500, 32)) * np.exp2(rng.uniform(-6, 6, (500, 1)))).astype(np.float16)
        q, s16 = quant.quantize_sym_groups(x, bits)
        err = np.abs(x.astype(np.float64) - quant.dequantize_sym(q, s16[:, None]).astype(np.float64))
        assert np.all(err <= s16.astype(np.float64)[:, None] / 2)
        assert np.abs(q).max() <= 2 ** (bits - 1) - 1


def test_zero_and_constant_groups():
    q, s16 = quant.quantize_sym_groups(np.zeros((1, 32), np.float16), 4)
    assert float(s16[0]) == 1.0 and not q.any()
    c = np.full((1, 32), -2.5, np.float16)
    q, s16 = quant.quantize_sym_groups(c, 8)
    assert np.all(q == -127)
    assert np.all(np.abs(quant.dequantize_sym(q, s16[:, None]) + 2.5) <= float(s16[0]) / 2)


def test_symmetric_step_versus_affine_on_centred_data():
    # data spanning [-a, a]: affine step 2a/(2^b - 1), symmetric a/(2^(b-1) - 1);
    # both are then rounded up to fp16
    for bits in (4, 8):
        a = 3.0
        x = np.linspace(-a, a, 257).astype(np.float16)[None, :]
        _, sa, _ = quant.quantize_groups(x, bits)
        _, ss = quant.quantize_sym_groups(x, bits)
        assert Fraction(float(sa[0])) == _f16_up(Fraction(2 * 3, 2 ** bits - 1))
        assert Fraction(float(ss[0])) == _f16_up(Fraction(3, 2 ** (bits - 1) - 1))


def _cfg(bits=8):
    return Config(128, 2, 4, bits, bits, "token", k_format="sym32", v_format="sym32")


def test_blocks_keep_an_outlier_to_its_own_block():
    c = RefCache(_cfg(4), 1, 32)
    rng = np.random.default_rng(13)
    k = rng.standard_normal((1, 2, 128)).astype(np.float16)
    k[0, 0, 5] = 100.0                                     # outlier in block 0
    c.append(k, k, [1])
    s = c.ks[0, 0, 0].astype(np.float32)                   # 4 block scales of that token
    assert s[0] >= 100 / 7 and np.all(s[1:] < 1.0)
    kh = c.k_hat(0, 0)[0]
    assert np.max(np.abs(kh[32:] - k[0, 0, 32:].astype(np.float64))) <= float(s[1:].max()) / 2


def test_cache_attention_brute_force_and_layout():
    cfg = _cfg(4)
    rng = np.random.default_rng(14)
    c = RefCache(cfg, 2, 64)
    n = [7, 3]
    k = (rng.standard_normal((10, 2, 128)) * 2).astype(np.float16)
    v = rng.standard_normal((10, 2, 128)).astype(np.float16)
    c.append(k, v, n)
    q = rng.standard_normal((2, 4, 128)).astype(np.float16)
    out = c.attention(q, 0.125)
    off = 0
    for b in range(2):
        for hq in range(4):
            h = hq // 2
            K = []
            for t in range(n[b]):
                qq, ss = quant.quantize_sym_groups(k[off + t, h].reshape(4, 32), 4)
                K.append((ss.astype(np.float64)[:, None] * qq).reshape(128))
            V = []
            for t in range(n[b]):
                qq, ss = quant.quantize_sym_groups(v[off + t, h].reshape(4, 32), 4)
                V.append((ss.astype(np.float64)[:, None] * qq).reshape(128))
            sc = [0.125 * float(np.dot(Kt, q[b, hq].astype(np.float64))) for Kt in K]
            m = max(sc)
            p = [math.exp(x - m) for x in sc]
            want = sum(pi * Vt for pi, Vt in zip(p, V)) / sum(p)
            assert np.max(np.abs(out[b, hq] - want)) < 1e-12
        off += n[b]
    pk = c.pack()
    assert pk["k_meta"].shape == (2, 2, 64, 4) and pk["v_meta"].shape == (2, 2, 64, 4)
    # stored codes: u = q - q_min, the 4-bit layout (channel c in bits 4(c%2) of byte c/2)
    u = pk["k_codes"][0, 1, 2]
    qq, ss = quant.quantize_sym_groups(k[2, 1].reshape(4, 32), 4)
    want_u = (qq.reshape(128).astype(np.int16) + 8).astype(np.uint8)
    assert np.array_equal(u & 0xF, want_u[0::2]) and np.array_equal(u >> 4, want_u[1::2])
    assert np.array_equal(pk["k_meta"][0, 1, 2], quant.f16_bits(ss))


@pytest.mark.parametrize("bits,key", [(8, "context_64k_8bit"), (4, "context_64k_4bit")])
def test_pages_block_sizes(bits, key):
    g = json.load(open(os.path.join(GOLD, "sizes_worked_example.json")))
    base, blk = g["context_64k"], g[key]
    # one layer of an architecture whose fp16 KV takes 64 KiB per token: scale it
    cfg = Config(128, 8, 32, bits, bits, "token", k_format="sym32", v_format="sym32")
    a = sizes.actual_bytes(cfg, 1, 32)
    per_tok_head = (a["k_codes"] + a["k_meta"] + a["v_codes"] + a["v_meta"]) / (8 * 32)
    fp16_tok_head = 2 * 128 * 2
    ratio = Fraction(int(per_tok_head), fp16_tok_head)
    kib = ratio * base["fp16_KiB_per_token"]
    printed = blk.get("KiB_per_token_printed", blk.get("KiB_per_token_printed_range", [0, 0])[-1])
    assert kib == printed                                  # 34 (q8_0-like), 18 (q4_0-like)
    if "GiB_printed" in blk and bits == 4:
        # 18 KiB x 65536 = 1.125 GiB, printed rounded half up as 1.13
        assert abs(float(kib) * 1024 * base["tokens"] / 2 ** 30 - blk["GiB_printed"]) <= 0.005
