"""GPU parity of pre-RoPE key quantization with the rotary embedding applied
inside attention (KVQuant's pre-RoPE keys: "Sub-8-Bit KV Cache Quantization
Is Not a Free Lever for an RDNA4 Agent Swarm", "What the low-bit numbers
actually cost"; the embedding is the textbook one, oracle/rope.py, so parity
of the rotation rests on that definition, not on the pages). Channel-axis
keys at 8, 4 and 2 bits and mixed widths, two frequency bases, ragged
sequences with residual-only ones, decode steps crossing residual flushes,
positions up to about 30k, and several work splits: codes byte-equal (the
cache holds the keys before rotation) and attention within 2e-3 of the float64
oracle."""
import numpy as np
import pytest

from quantized_decode_attention_03_amd import workloads as W
from harness import ATOL, Pair, prefill_inputs, max_abs

pytestmark = pytest.mark.gpu

CASES = [
    (2, 4, 4, 10000.0, dict(batch=3, seq_len=333, min_len=1)),      # KIVI int4, R = 32, ragged
    (4, 2, 2, 10000.0, dict(batch=3, seq_len=400, min_len=100)),    # KIVI int2, R = 128, spikes
    (2, 8, 8, 500000.0, dict(batch=2, seq_len=300, min_len=200)),   # int8 channel-axis keys
    (2, 8, 4, 10000.0, dict(batch=2, seq_len=260, min_len=90)),     # keys at more bits than values
    (4, 4, 2, 500000.0, dict(batch=2, seq_len=500, min_len=300)),
]
IDS = [f"w{c}-k{kb}v{vb}-base{int(b)}" for c, kb, vb, b, _ in CASES]


def _spec(cid, kb, vb, base, kw):
    return W.spec(cid, k_bits=kb, v_bits=vb, k_rope=1, rope_theta=base, **kw)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_rope_decode_attention(case):
    s = _spec(*case)
    k, v, lens = prefill_inputs(s)
    print(f"{case[:4]} lens {lens}", flush=True)
    p = Pair(s, s.max_tokens(40))
    p.append(k, v, lens)
    p.assert_state_equal()
    worst = 0.0
    for i in range(34):                  # crosses a residual flush of every sequence when R = 32
        q, kn, vn = W.step(s, 0, i)
        p.append(kn, vn, [1] * s.batch)
        if i % 3 == 0 or i == 33:
            out, scale = p.attend(q)
            err = max_abs(out, p.ref.attention(q, scale))
            worst = max(worst, err)
            assert err <= ATOL, (case[:4], i, err)
    p.assert_state_equal()
    print(f"{case[:4]}: worst attention max-abs {worst:.3e}", flush=True)


def test_rope_long_positions():
    """One sequence of 30000 tokens (angles up to 30000 rad on the fastest
    frequency) plus a short one; all pairs checked against the oracle."""
    s = W.spec(2, batch=2, seq_len=30000, min_len=30000, k_rope=1)
    lens = [30000, 77]
    k, v, _ = prefill_inputs(s, lens=np.array(lens))
    p = Pair(s, s.max_tokens(8))
    p.append(k, v, lens)
    q, kn, vn = W.step(s, 0, 0)
    p.append(kn, vn, [1, 1])
    out, scale = p.attend(q)
    err = max_abs(out, p.ref.attention(q, scale))
    print(f"long positions: max-abs {err:.3e}", flush=True)
    assert err <= ATOL


def test_rope_split_varied(monkeypatch):
    s = W.spec(2, batch=3, seq_len=1200, min_len=900, k_rope=1)
    k, v, lens = prefill_inputs(s)
    p = Pair(s, s.max_tokens(8))
    p.append(k, v, lens)
    q = np.random.default_rng(13).standard_normal((3, 32, 128), dtype=np.float32).astype(np.float16)
    want = None
    for tokens in (256, 1024, 1 << 20):
        monkeypatch.setenv("KVQ_SPLIT_TOKENS", str(tokens))
        out, scale = p.attend(q)
        want = p.ref.attention(q, scale) if want is None else want
        assert max_abs(out, want) <= ATOL, tokens
    monkeypatch.delenv("KVQ_SPLIT_TOKENS")


def test_rope_changes_the_result():
    """The same cache attended with and without the rotation differs by far
    more than the tolerance (the rotation is really applied)."""
    s = W.spec(2, batch=2, seq_len=200, min_len=200, k_rope=1)
    k, v, lens = prefill_inputs(s)
    p = Pair(s, s.max_tokens(8))
    p.append(k, v, lens)
    q, _, _ = W.step(s, 0, 0)
    out, scale = p.attend(q)
    p.ref.cfg.k_rope = 0
    assert max_abs(out, p.ref.attention(q, scale)) > 50 * ATOL
