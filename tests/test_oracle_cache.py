"""Pins of the oracle's cache state machine, packed layout and float64
attention: the residual-window invariant, bulk vs token-by-token appends,
dense-and-sparse exactness, attention special cases and brute force against
an independent pure-Python softmax. CPU only."""
import math
import struct

import numpy as np
import pytest

from oracle import quant
from oracle.cache import Config, RefCache, pack_fields, unpack_fields
from quantized_decode_attention_03_amd import workloads as W


def _cfg(kind, H=2, Hq=4):
    if kind == "token8":
        return Config(128, H, Hq, 8, 8, "token")
    if kind == "chan4":
        return Config(128, H, Hq, 4, 4, "channel", 32, 32, 0)
    if kind == "chan2r128":
        return Config(128, H, Hq, 2, 2, "channel", 32, 128, 0)
    if kind == "chan4sp":
        return Config(128, H, Hq, 4, 4, "channel", 32, 32, 2)
    if kind == "fp8":
        return Config(128, H, Hq, 8, 8, "token", k_format="fp8", v_format="fp8",
                      k_scale=0.5, v_scale=2.0)
    if kind.startswith("sym"):
        b = int(kind[3:])
        return Config(128, H, Hq, b, b, "token", k_format="sym32", v_format="sym32")
    raise KeyError(kind)


def _rand_kv(rng, n, H):
    k = rng.standard_normal((n, H, 128), dtype=np.float32)
    k[..., [3, 17, 64, 101]] *= 20
    v = rng.standard_normal((n, H, 128), dtype=np.float32)
    return k.astype(np.float16), v.astype(np.float16)


@pytest.mark.parametrize("kind", ["token8", "chan4", "chan2r128", "chan4sp", "fp8", "sym8", "sym4", "sym2"])
def test_bulk_append_equals_single_appends(kind):
    """Appending n keys at once reaches the same state as n single-token
    appends (the residual window fills and flushes the same way)."""
    cfg = _cfg(kind)
    rng = np.random.default_rng(11)
    B, T = 3, 384
    lens = [0, 77, 300]
    a, b = RefCache(cfg, B, T), RefCache(cfg, B, T)
    ks, vs = zip(*[_rand_kv(rng, n, cfg.n_kv_heads) for n in lens])
    a.append(np.concatenate(ks), np.concatenate(vs), lens)
    for t in range(max(lens)):
        n = [1 if t < L else 0 for L in lens]
        kk = np.stack([ks[i][t] for i in range(B) if n[i]])
        vv = np.stack([vs[i][t] for i in range(B) if n[i]])
        b.append(kk, vv, n)
    pa, pb = a.pack(), b.pack()
    for key in pa:
        if key == "k_resid":
            for i in range(B):
                r = lens[i] - a.n_quantized(i)
                assert np.array_equal(pa[key][i, :, :r], pb[key][i, :, :r])
        else:
            assert np.array_equal(pa[key], pb[key]), key


@pytest.mark.parametrize("kind", ["chan4", "chan2r128"])
def test_residual_window_invariant(kind):
    cfg = _cfg(kind)
    R = cfg.k_residual_tokens
    rng = np.random.default_rng(12)
    c = RefCache(cfg, 1, 512)
    total = 0
    for n in [5, 27, 1, 31, 100, 0, 64, 129]:
        k, v = _rand_kv(rng, n, cfg.n_kv_heads)
        c.append(k, v, [n])
        total += n
        L = int(c.length[0])
        assert L == total
        assert c.n_quantized(0) == L - L % R
        r = L % R
        # the residual holds the last r keys verbatim
        kh = c.k_hat(0, 1)
        assert np.array_equal(kh[L - r:], c.kres[0, 1, :r].astype(np.float64))
        if r and n >= r:
            assert np.array_equal(c.kres[0, 1, :r], k[n - r:, 1])


def test_sparse_entries_reconstruct_exactly():
    cfg = _cfg("chan4sp")
    rng = np.random.default_rng(13)
    k, v = _rand_kv(rng, 96, 2)
    c = RefCache(cfg, 1, 128)
    c.append(k, v, [96])
    kh = c.k_hat(0, 0)
    for t in range(96):
        cols = c.sp_col[0, 0, t]
        assert np.array_equal(kh[t, cols], k[t, 0, cols].astype(np.float64))
        # the kept entries are the two largest magnitudes of that key vector
        mags = np.abs(k[t, 0].astype(np.float64))
        assert mags[cols].min() >= np.delete(mags, cols).max()
    # every other entry is within the bound of its own channel group
    dense = k[:, 0].astype(np.float64).copy()
    for t in range(96):
        dense[t, c.sp_col[0, 0, t]] = 0
    blk = np.arange(96) // 32
    s = c.ks[0, 0, blk].astype(np.float64)
    err = np.abs(kh - k[:, 0].astype(np.float64))
    for t in range(96):
        err[t, c.sp_col[0, 0, t]] = 0
    assert np.all(err <= s * (0.5 + 2 ** -12))


def test_dequantize_f16_matches_stdlib_half_rounding():
    """kvq_dequantize's values: the exact reconstruction rounded to fp16, here
    through the standard library's IEEE half conversion."""
    cfg = _cfg("chan4")
    rng = np.random.default_rng(14)
    k, v = _rand_kv(rng, 70, 2)
    c = RefCache(cfg, 1, 96)
    c.append(k, v, [70])
    kd, vd = c.dequantize_f16()
    v32 = c.v_hat(0, 1, np.float64)
    for t in range(0, 70, 7):
        for ch in range(0, 128, 5):
            want = struct.unpack("<e", struct.pack("<e", float(v32[t, ch])))[0]
            assert float(vd[0, t, 1, ch]) == want
    assert np.all(kd[0, 70:] == 0) and np.all(vd[0, 70:] == 0)
    # residual keys (64..69) come back verbatim
    assert np.array_equal(quant.f16_bits(kd[0, 64:70]), quant.f16_bits(k[64:70]))


def test_dequantize_f16_of_blocks_matches_stdlib_half_rounding():
    """The symmetric blocks' fp16 values: s * q (exact) rounded to fp16 by the
    standard library's IEEE half conversion."""
    c = RefCache(_cfg("sym4"), 1, 64)
    rng = np.random.default_rng(15)
    k, v = _rand_kv(rng, 40, 2)
    c.append(k, v, [40])
    kd, vd = c.dequantize_f16()
    k64 = c.k_hat(0, 0, np.float64)
    for t in range(0, 40, 3):
        for ch in range(0, 128, 7):
            want = struct.unpack("<e", struct.pack("<e", float(k64[t, ch])))[0]
            assert float(kd[0, t, 0, ch]) == want
    assert np.all(kd[0, 40:] == 0) and np.all(vd[0, 40:] == 0)


def test_pack_unpack_identity():
    rng = np.random.default_rng(15)
    for bits in (2, 4, 8):
        u = rng.integers(0, 1 << bits, size=(3, 5, 64)).astype(np.uint8)
        p = pack_fields(u, bits)
        assert p.shape[-1] == 64 * bits // 8
        assert np.array_equal(unpack_fields(p, bits), u)
    # little-endian fields: int4 codes 1,2 -> 0x21; int2 codes 1,2,3,0 -> 0b00111001
    assert pack_fields(np.uint8([[1, 2]]), 4).tolist() == [[0x21]]
    assert pack_fields(np.uint8([[1, 2, 3, 0]]), 2).tolist() == [[0b00111001]]


def test_pack_layout_shapes_and_unused_slots():
    cfg = _cfg("chan4sp")
    rng = np.random.default_rng(16)
    k, v = _rand_kv(rng, 45, 2)
    c = RefCache(cfg, 1, 64)
    c.append(k, v, [45])
    p = c.pack()
    assert p["k_codes"].shape == (1, 2, 64, 64)
    assert p["v_codes"].shape == (1, 2, 2, 128, 16)
    assert p["k_meta"].shape == (1, 2, 2, 128)
    assert p["v_meta"].shape == (1, 2, 64)
    assert p["k_sparse"].shape == (1, 2, 64, 2)
    Q = c.n_quantized(0)
    assert Q == 32
    assert np.all(p["k_codes"][0, :, Q:] == 0) and np.all(p["k_meta"][0, :, 1:] == 0)
    assert np.all(p["k_sparse"][0, :, Q:] == 0)
    # value codes of tokens >= 45 are zero bits inside block 1
    u = unpack_fields(p["v_codes"][0, :, 1], 4)     # [H, D, 32]
    assert np.all(u[..., 45 - 32:] == 0)
    assert np.all(p["v_meta"][0, :, 45:] == 0)
    # a value record really is token-ordered: re-derive from logical codes
    qv = c.vq[0, 1, :32, 9].astype(np.int16) + 8
    assert np.array_equal(unpack_fields(p["v_codes"][0, 1, 0, 9][None], 4)[0], qv)


# ---------------------------------------------------------------- attention

def _py_attention(qv, K, V, scale):
    """Independent pure-Python float64 softmax attention for tiny inputs."""
    sc = [scale * sum(a * b for a, b in zip(qv, row)) for row in K]
    m = max(sc)
    e = [math.exp(s - m) for s in sc]
    tot = math.fsum(e)
    return [math.fsum(e[t] * V[t][c] for t in range(len(K))) / tot for c in range(len(V[0]))]


@pytest.mark.parametrize("kind", ["token8", "chan4", "chan4sp"])
def test_attention_brute_force(kind):
    cfg = _cfg(kind, H=2, Hq=4)
    rng = np.random.default_rng(17)
    lens = [40, 7, 1]
    k, v = zip(*[_rand_kv(rng, n, 2) for n in lens])
    c = RefCache(cfg, 3, 64)
    c.append(np.concatenate(k), np.concatenate(v), lens)
    q = rng.standard_normal((3, 4, 128), dtype=np.float32).astype(np.float16)
    scale = 1 / math.sqrt(128)
    out = c.attention(q, scale)
    for b in range(3):
        for hq in range(4):
            kv = hq // 2
            K = c.k_hat(b, kv).tolist()
            V = c.v_hat(b, kv).tolist()
            ref = _py_attention(q[b, hq].astype(np.float64).tolist(), K, V,
                                float(np.float32(scale)))
            assert np.allclose(out[b, hq], ref, rtol=0, atol=1e-12)


def test_attention_special_cases():
    cfg = _cfg("token8", H=1, Hq=2)
    rng = np.random.default_rng(18)
    # S = 1: the output is the single value row
    c = RefCache(cfg, 1, 32)
    k, v = _rand_kv(rng, 1, 1)
    c.append(k, v, [1])
    q = rng.standard_normal((1, 2, 128), dtype=np.float32).astype(np.float16)
    out = c.attention(q, 0.1)
    assert np.array_equal(out[0, 0], c.v_hat(0, 0)[0])
    # q = 0: uniform weights, the mean of the value rows
    c = RefCache(cfg, 1, 64)
    k, v = _rand_kv(rng, 50, 1)
    c.append(k, v, [50])
    out = c.attention(np.zeros((1, 2, 128), np.float16), 0.1)
    assert np.allclose(out[0, 1], c.v_hat(0, 0).mean(0), atol=1e-13)
    # identical keys: uniform weights too
    c = RefCache(cfg, 1, 64)
    kk = np.repeat(k[:1], 50, axis=0)
    c.append(kk, v, [50])
    out = c.attention(q, 0.1)
    assert np.allclose(out[0, 0], c.v_hat(0, 0).mean(0), atol=1e-13)
    # a sequence with no tokens gives zeros
    c = RefCache(cfg, 2, 32)
    c.append(k[:3], v[:3], [0, 3])
    out = c.attention(np.ones((2, 2, 128), np.float16), 0.1)
    assert np.all(out[0] == 0) and np.any(out[1] != 0)


def test_attention_head_grouping():
    """Query head h reads KV head h // (Hq/H): swapping the KV heads' data
    swaps the query-head groups' outputs."""
    cfg = _cfg("token8", H=2, Hq=4)
    rng = np.random.default_rng(19)
    k, v = _rand_kv(rng, 30, 2)
    q = rng.standard_normal((1, 4, 128), dtype=np.float32).astype(np.float16)
    a = RefCache(cfg, 1, 32)
    a.append(k, v, [30])
    b = RefCache(cfg, 1, 32)
    b.append(k[:, ::-1].copy(), v[:, ::-1].copy(), [30])
    qa = a.attention(q, 0.09)
    qb = b.attention(q[:, [2, 3, 0, 1]].copy(), 0.09)
    assert np.allclose(qa, qb[:, [2, 3, 0, 1]], atol=1e-14)


def test_workload_generator_structure():
    s = W.spec(2, batch=2, seq_len=64, min_len=64)
    k, v = W.prefill(s, 0, 1)
    assert k.shape == (64, 8, 128) and k.dtype == np.float16
    ch = W.outlier_channels(s, 0)
    big = np.abs(k.astype(np.float32)).mean(0)          # [H, D]
    for h in range(8):
        assert set(np.argsort(-big[h])[:4]) == set(ch[h])
    k2, _ = W.prefill(s, 0, 1)
    assert np.array_equal(k, k2)                         # seeded
    s5 = W.spec(5)
    L = W.seq_lengths(s5)
    assert L.min() >= 1024 and L.max() <= 32768 and len(set(L.tolist())) > 100


def test_split_merge_equals_unsplit():
    # closed form of the split-K merge: any split of the tokens, merged with
    # the log-sum-exp rule, reproduces the unsplit softmax result
    from oracle.cache import softmax_partial, merge_partials
    rng = np.random.default_rng(7)
    for trial in range(40):
        S = int(rng.integers(1, 300))
        sc = rng.standard_normal(S) * rng.choice([0.5, 5.0, 60.0])
        V = rng.standard_normal((S, 16))
        p = np.exp(sc - sc.max())
        want = (p @ V) / p.sum()
        cuts = np.sort(rng.integers(0, S + 1, size=int(rng.integers(0, 6))))
        bounds = [0] + cuts.tolist() + [S]
        parts = [softmax_partial(sc[a:b], V[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
        got = merge_partials(parts)
        assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def test_split_merge_degenerate_cases():
    from oracle.cache import softmax_partial, merge_partials
    V = np.arange(12, dtype=np.float64).reshape(3, 4)
    empty = softmax_partial(np.zeros(0), np.zeros((0, 4)))
    assert empty[0] == -np.inf and empty[1] == 0.0 and not np.any(empty[2])
    # every range empty -> 0 (the empty-sequence convention)
    assert not np.any(merge_partials([empty, empty]))
    # one token per range: weights exp(s_t - max) / sum
    sc = np.array([1.0, 3.0, 2.0])
    parts = [softmax_partial(sc[i:i + 1], V[i:i + 1]) for i in range(3)] + [empty]
    w = np.exp(sc - 3.0) / np.exp(sc - 3.0).sum()
    assert np.allclose(merge_partials(parts), w @ V, rtol=0, atol=1e-13)
