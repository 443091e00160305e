"""GPU parity: the HIP path against the oracle on identical seeded inputs.

Codes, metadata, sparse entries, residual keys and dequantized fp16 values
must be byte-equal; attention must be within 2e-3 max-abs of the float64
oracle. Shapes are the five workloads' structures at sizes the oracle runs in
seconds, spanning several 32-token tiles and ragged tails."""
import numpy as np
import pytest

from quantized_decode_attention_03_amd import workloads as W
from harness import ATOL, Pair, prefill_inputs, max_abs, f16_equal

pytestmark = pytest.mark.gpu

SMALL = {
    1: dict(),                                                     # full size: B=1, S=256
    2: dict(batch=3, seq_len=333, min_len=1),                      # ragged lengths, R = 32
    3: dict(seq_len=300, min_len=300, layers=2),
    4: dict(batch=3, seq_len=400, min_len=100),                    # int2, R = 128
    5: dict(batch=4, seq_len=700, min_len=30, steps=40),           # sparse + streaming
}


def _small(cid):
    return W.spec(cid, **SMALL[cid])


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_prefill_state_and_dequant(cid):
    s = _small(cid)
    layer = s.layers - 1
    k, v, lens = prefill_inputs(s, layer)
    p = Pair(s, s.max_tokens(8))
    print(f"workload {cid} lens {lens}", flush=True)
    p.append(k, v, lens)
    p.assert_state_equal()
    kd, vd = p.dequantize()
    kr, vr = p.ref.dequantize_f16()
    assert f16_equal(kd, kr)
    assert f16_equal(vd, vr)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_decode_steps_attention(cid):
    s = _small(cid)
    layer = s.layers - 1
    k, v, lens = prefill_inputs(s, layer)
    p = Pair(s, s.max_tokens(8))
    p.append(k, v, lens)
    worst = 0.0
    for i in range(s.steps if s.steps > 1 else 3):
        q, kn, vn = W.step(s, layer, i)
        p.append(kn.reshape(s.batch, s.n_kv_heads, s.d_head), vn, [1] * s.batch)
        out, scale = p.attend(q)
        ref = p.ref.attention(q, scale)
        err = max_abs(out, ref)
        worst = max(worst, err)
        assert err <= ATOL, (cid, i, err)
    print(f"workload {cid}: worst attention max-abs {worst:.3e}")
    p.assert_state_equal()


@pytest.mark.parametrize("cid", [2, 4, 5])
def test_multi_token_appends_cross_flushes(cid):
    """Appends of several tokens that fill the residual window once, twice or
    not at all, mixed per sequence, including empty appends."""
    s = _small(cid)
    rng = np.random.default_rng(100 + cid)
    p = Pair(s, 1024)
    chunks = [[5, 0, 32, 1], [27, 33, 0, 64], [1, 95, 129, 3], [0, 0, 0, 0], [200, 1, 31, 60]]
    for ci, n in enumerate(chunks):
        n = n[:s.batch]
        tot = sum(n)
        k = rng.standard_normal((tot, s.n_kv_heads, s.d_head), dtype=np.float32)
        k[..., [3, 17, 64, 101]] *= 20
        k = k.astype(np.float16)
        v = rng.standard_normal((tot, s.n_kv_heads, s.d_head), dtype=np.float32).astype(np.float16)
        if tot:
            p.append(k, v, n)
        p.assert_state_equal()
        q = rng.standard_normal((s.batch, s.n_q_heads, s.d_head), dtype=np.float32).astype(np.float16)
        out, scale = p.attend(q)
        assert max_abs(out, p.ref.attention(q, scale)) <= ATOL, ci


def test_empty_and_single_token_sequences():
    s = W.spec(2, batch=4, seq_len=64, min_len=64)
    p = Pair(s, 64)
    rng = np.random.default_rng(7)
    n = [0, 1, 31, 32]
    k = rng.standard_normal((sum(n), 8, 128), dtype=np.float32).astype(np.float16)
    v = rng.standard_normal((sum(n), 8, 128), dtype=np.float32).astype(np.float16)
    p.append(k, v, n)
    p.assert_state_equal()
    q = rng.standard_normal((4, 32, 128), dtype=np.float32).astype(np.float16)
    out, scale = p.attend(q)
    assert np.all(out[0] == 0)
    assert max_abs(out, p.ref.attention(q, scale)) <= ATOL
    # a single token: every query head returns that token's value row
    for h in range(32):
        assert max_abs(out[1, h], p.ref.v_hat(1, h // 4)[0]) <= ATOL


def test_fill_to_capacity():
    s = W.spec(4, batch=2, seq_len=256, min_len=256)
    p = Pair(s, 256)
    k, v, lens = prefill_inputs(s, 0)
    p.append(k, v, lens)
    p.assert_state_equal()
    q = np.random.default_rng(8).standard_normal((2, 32, 128), dtype=np.float32).astype(np.float16)
    out, scale = p.attend(q)
    assert max_abs(out, p.ref.attention(q, scale)) <= ATOL
    import quantized_decode_attention_03_amd as K
    with pytest.raises(K.KVQError):
        p.append(k[:2], v[:2], [1, 1])


@pytest.mark.parametrize("cid", [2, 3])
def test_attention_deterministic(cid):
    s = _small(cid)
    k, v, lens = prefill_inputs(s, s.layers - 1)
    p = Pair(s, s.max_tokens(8), with_ref=False)
    p.append(k, v, lens)
    q, _, _ = W.step(s, 0, 0)
    first, _ = p.attend(q)
    for _ in range(9):                     # 10 runs in all
        again, _ = p.attend(q)
        assert np.array_equal(first, again)


def test_workspace_shared_by_two_caches():
    """One zero-filled workspace serves attention calls on two caches of
    different shapes and split counts, alternating; every call matches the
    oracle (whatever a call leaves in the workspace must not disturb the next)."""
    import torch
    import quantized_decode_attention_03_amd as K
    pairs = []
    for cid, kw in ((2, dict(batch=3, seq_len=900, min_len=300)),
                    (4, dict(batch=2, seq_len=640, min_len=200))):
        s = W.spec(cid, **kw)
        k, v, lens = prefill_inputs(s, 0)
        p = Pair(s, s.max_tokens(8))
        p.append(k, v, lens)
        pairs.append(p)
    n = max(K.kvq_workspace_bytes(p.gpu.cfg, p.B, p.T) for p in pairs)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(9)
    for rep in range(3):
        for p in pairs:
            q = rng.standard_normal((p.B, p.s.n_q_heads, p.s.d_head), dtype=np.float32).astype(np.float16)
            out, scale = p.attend(q, ws=ws)
            assert max_abs(out, p.ref.attention(q, scale)) <= ATOL, (p.s.cid, rep)


def test_split_length_varied_on_one_input(monkeypatch):
    """The same cache and queries attended with the work cut into ranges of
    8 tiles (256 tokens, the shortest allowed: pairs split over up to 5
    workgroups here) up to a single workgroup for everything: every result
    within 2e-3 of the oracle, and of each other."""
    s = W.spec(2, batch=3, seq_len=1200, min_len=900)
    k, v, lens = prefill_inputs(s, 0)
    p = Pair(s, s.max_tokens(8))
    p.append(k, v, lens)
    q = np.random.default_rng(10).standard_normal((3, 32, 128), dtype=np.float32).astype(np.float16)
    outs = []
    for tokens in (256, 512, 1024, 1 << 20):
        monkeypatch.setenv("KVQ_SPLIT_TOKENS", str(tokens))
        out, scale = p.attend(q)
        print(f"split length {tokens}: max-abs {max_abs(out, p.ref.attention(q, scale)):.3e}", flush=True)
        assert max_abs(out, p.ref.attention(q, scale)) <= ATOL, tokens
        outs.append(out)
    monkeypatch.delenv("KVQ_SPLIT_TOKENS")
    for o in outs[1:]:
        assert max_abs(o, outs[0]) <= ATOL
