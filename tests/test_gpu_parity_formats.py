"""GPU parity of the two extra element formats against the oracle:
* fp8 E4M3 bytes with one scale per cache side ("KV Cache Quantization
  Benchmarked: 8-bit Is Nearly Lossless, How Much Does 4-bit Cost?", glossary
  paragraph: vLLM's fp8_e4m3 cache);
* symmetric 32-channel blocks with one fp16 scale each (same page, llama.cpp's
  q8_0 / q4_0 blocks of 32 elements sharing a scale; "KV Cache Quantization —
  8-bit and 4-bit", "Symmetric vs asymmetric").
Both on the token axis for keys, on the structure of the 32-layer int8
workload (per-token keys with outlier channels) cut to a few ragged
sequences. Codes and scales byte-equal, dequantized fp16 equal, attention
within 2e-3 of the float64 oracle; every finite E4M3 code round-trips and
reaches the output (to 1e-6 relative); all-zero blocks take scale 1; the split of the
work over workgroups does not change the result."""
import numpy as np
import pytest

from oracle import fp8 as ofp8
from quantized_decode_attention_03_amd import workloads as W
from harness import ATOL, Pair, prefill_inputs, max_abs, f16_equal

pytestmark = pytest.mark.gpu

F16 = np.float16

# (format, key bits, value bits, key scale, value scale)
CASES = [
    ("fp8", 8, 8, 1.0, 1.0),
    ("fp8", 8, 8, 0.25, 2.0),      # outlier keys / 0.25 pass 112: some saturate at 448
    ("sym32", 8, 8, 1.0, 1.0),
    ("sym32", 4, 4, 1.0, 1.0),
    ("sym32", 2, 2, 1.0, 1.0),
    ("sym32", 8, 4, 1.0, 1.0),
    ("sym32", 4, 2, 1.0, 1.0),
    ("sym32", 2, 8, 1.0, 1.0),
]
IDS = [f"{f}-k{kb}v{vb}-s{ks}" for f, kb, vb, ks, _ in CASES]


def _spec(fmt, kb, vb, ks, vs, **kw):
    base = dict(layers=1, batch=3, seq_len=300, min_len=60)
    base.update(kw)
    return W.spec(3, k_bits=kb, v_bits=vb, fmt=fmt, k_scale=ks, v_scale=vs, **base)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_format_prefill_state_and_dequant(case):
    s = _spec(*case)
    k, v, lens = prefill_inputs(s)
    print(f"{case} lens {lens}", flush=True)
    p = Pair(s, s.max_tokens(8))
    p.append(k, v, lens)
    p.assert_state_equal()
    kd, vd = p.dequantize()
    kr, vr = p.ref.dequantize_f16()
    assert f16_equal(kd, kr)
    assert f16_equal(vd, vr)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_format_decode_attention(case):
    s = _spec(*case)
    k, v, lens = prefill_inputs(s)
    print(f"{case} lens {lens}", flush=True)
    p = Pair(s, s.max_tokens(8))
    p.append(k, v, lens)
    worst = 0.0
    for i in range(4):
        q, kn, vn = W.step(s, 0, i)
        p.append(kn, vn, [1] * s.batch)
        out, scale = p.attend(q)
        err = max_abs(out, p.ref.attention(q, scale))
        worst = max(worst, err)
        assert err <= ATOL, (case, i, err)
    p.assert_state_equal()
    print(f"{case}: worst attention max-abs {worst:.3e}", flush=True)


def test_fp8_every_code():
    """Keys and values holding every finite E4M3 value (and -0): the codes
    round-trip byte for byte, and with one token per sequence the output is
    that token's value vector (to 1e-6 relative: the softmax weight of the
    sole token is 1 up to the rounding of its score; a misread code would be
    off by at least 1/16)."""
    s = W.spec(3, layers=1, batch=2, seq_len=1, min_len=1, fmt="fp8")
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] + [0x00, 0x80], np.uint8)
    vals = ofp8.e4m3_value(codes).astype(F16)               # exact: E4M3 values are fp16 values
    assert np.array_equal(ofp8.quantize(vals, 1.0), codes)
    H, D = s.n_kv_heads, s.d_head
    rng = np.random.default_rng(3)
    k = rng.standard_normal((2, H, D), dtype=np.float32).astype(F16)
    v = rng.standard_normal((2, H, D), dtype=np.float32).astype(F16)
    for h in range(H):                                       # every head, rotated
        rot = np.roll(vals, 37 * h).reshape(2, D)
        k[:, h] = rot
        v[:, h] = rot[::-1]
    p = Pair(s, 32)
    p.append(k, v, [1, 1])
    p.assert_state_equal()
    q = rng.standard_normal((2, s.n_q_heads, D), dtype=np.float32).astype(F16)
    out, scale = p.attend(q)
    want = np.repeat(v.astype(np.float64), s.group, axis=1)   # query head h reads KV head h // g
    bad = np.abs(out - want) > 1e-6 * np.abs(want)
    assert not bad.any(), (np.argwhere(bad)[:5].tolist(), max_abs(out, want))


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_sym32_zero_blocks(bits):
    """Whole-zero 32-channel blocks in keys and values (scale 1, every code at
    -q_min) next to ordinary blocks of the same tokens."""
    s = _spec("sym32", bits, bits, 1.0, 1.0, batch=2, seq_len=90, min_len=90)
    k, v, lens = prefill_inputs(s)
    k[::3, :, 32:64] = 0
    v[1::4, :, 96:128] = 0
    v[2::5] = 0
    p = Pair(s, s.max_tokens(8))
    p.append(k, v, lens)
    p.assert_state_equal()
    q, kn, vn = W.step(s, 0, 0)
    p.append(kn, vn, [1] * s.batch)
    out, scale = p.attend(q)
    assert max_abs(out, p.ref.attention(q, scale)) <= ATOL


@pytest.mark.parametrize("fmt,bits", [("fp8", 8), ("sym32", 4)])
def test_format_split_varied(monkeypatch, fmt, bits):
    """Long sequences attended with the work cut into ranges of 8 tiles up to
    one workgroup for everything: the merged partials (which carry the fp8
    value scale) agree with the oracle and with each other."""
    s = _spec(fmt, bits, bits, 0.5, 1.5, batch=3, seq_len=1200, min_len=900)
    k, v, lens = prefill_inputs(s)
    p = Pair(s, s.max_tokens(8))
    p.append(k, v, lens)
    q = np.random.default_rng(12).standard_normal((3, s.n_q_heads, s.d_head), dtype=np.float32).astype(F16)
    want = None
    outs = []
    for tokens in (256, 512, 1024, 1 << 20):
        monkeypatch.setenv("KVQ_SPLIT_TOKENS", str(tokens))
        out, scale = p.attend(q)
        if want is None:
            want = p.ref.attention(q, scale)
        err = max_abs(out, want)
        print(f"{fmt} split length {tokens}: max-abs {err:.3e}", flush=True)
        assert err <= ATOL, tokens
        outs.append(out)
    monkeypatch.delenv("KVQ_SPLIT_TOKENS")
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= ATOL
