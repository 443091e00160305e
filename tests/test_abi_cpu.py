"""The C-ABI library without a GPU: it loads, exports every entry point that
include/kvq.h declares, computes sizes, and rejects bad arguments before it
launches anything (every case here returns before any HIP call)."""
import ctypes
import os
import re

import pytest

from quantized_decode_attention_03_amd import _native as N
from quantized_decode_attention_03_amd import Config, kvq_cache_sizes, kvq_workspace_bytes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(N.EXPORTS)
    L = N.lib()
    for n in names:
        assert hasattr(L, n), n


def _cfg(**kw):
    base = dict(n_kv_heads=8, n_q_heads=32, k_bits=4, v_bits=4, k_axis="channel",
                k_group_tokens=32, k_residual_tokens=32, k_sparse_per_vector=0)
    base.update(kw)
    return Config(**base)


TOKEN_AXIS = dict(k_axis="token", k_group_tokens=0, k_residual_tokens=0)


def test_sizes_match_oracle_formula():
    from oracle import sizes
    from oracle.cache import Config as RC
    for kw in [dict(), dict(k_bits=2, v_bits=2, k_residual_tokens=128),
               dict(k_sparse_per_vector=2),
               dict(TOKEN_AXIS, k_bits=8, v_bits=8),
               dict(TOKEN_AXIS, k_bits=8, v_bits=8, k_format="fp8", k_scale=0.5, v_scale=2.0),
               dict(TOKEN_AXIS, k_bits=8, v_bits=8, k_format="sym32"),
               dict(TOKEN_AXIS, k_bits=4, v_bits=2, k_format="sym32")]:
        c = _cfg(**kw)
        got = kvq_cache_sizes(c, 3, 4096)
        rc = RC(128, c.n_kv_heads, c.n_q_heads, c.k_bits, c.v_bits, c.k_axis, c.k_group_tokens,
                c.k_residual_tokens, c.k_sparse_per_vector, k_format=c.k_format,
                v_format=c.v_format, k_scale=c.k_scale, v_scale=c.v_scale)
        want = sizes.actual_bytes(rc, 3, 4096)
        for k, v in want.items():
            assert got[k] == v, (kw, k)


def test_block_format_sizes_per_token():
    # 8-bit caches: one byte per element plus, for the 32-element blocks, one
    # fp16 scale per block (34 B per 32 elements, the 2 extra KiB per 64 KiB of
    # the glossary's q8_0); fp8 carries no per-element metadata at all
    D, H = 128, 8
    per_tok = lambda c: (kvq_cache_sizes(c, 1, 4096)["total_bytes"] - 4) / 4096
    fp8 = _cfg(**TOKEN_AXIS, k_bits=8, v_bits=8, k_format="fp8")
    q8 = _cfg(**TOKEN_AXIS, k_bits=8, v_bits=8, k_format="sym32")
    q4 = _cfg(**TOKEN_AXIS, k_bits=4, v_bits=4, k_format="sym32")
    assert per_tok(fp8) == 2 * H * D
    assert per_tok(q8) == 2 * H * D * 34 / 32
    assert per_tok(q4) == 2 * H * D * 18 / 32


def test_worked_example_nominal():
    # 8 KV heads, d 128, 32768 tokens, one layer: 32 layers give the page's 2^31 B at int8
    c = _cfg(k_axis="token", k_group_tokens=0, k_residual_tokens=0, k_bits=8, v_bits=8)
    assert kvq_cache_sizes(c, 1, 32768)["nominal_bytes"] * 32 == 2 ** 31
    c4 = _cfg(k_bits=4, v_bits=4)
    assert kvq_cache_sizes(c4, 1, 32768)["nominal_bytes"] * 32 == 2 ** 30


@pytest.mark.parametrize("kw,status", [
    (dict(k_bits=3), N.KVQ_EUNSUPPORTED),
    (dict(v_bits=16), N.KVQ_EUNSUPPORTED),
    (dict(d_head=64), N.KVQ_EUNSUPPORTED),
    (dict(n_q_heads=12), N.KVQ_EINVAL),
    (dict(n_q_heads=8 * 16), N.KVQ_EUNSUPPORTED),
    (dict(k_residual_tokens=48), N.KVQ_EINVAL),
    (dict(k_residual_tokens=0), N.KVQ_EINVAL),
    (dict(k_group_tokens=64), N.KVQ_EUNSUPPORTED),
    (dict(k_sparse_per_vector=3), N.KVQ_EUNSUPPORTED),
    (dict(k_axis="token"), N.KVQ_EINVAL),
    # formats: fp8 is 8-bit, token axis; one format for keys and values
    (dict(TOKEN_AXIS, k_format="fp8"), N.KVQ_EINVAL),
    (dict(k_bits=8, v_bits=8, k_format="fp8"), N.KVQ_EUNSUPPORTED),
    (dict(k_format="sym32"), N.KVQ_EUNSUPPORTED),
    (dict(TOKEN_AXIS, k_format="sym32", v_format="int"), N.KVQ_EUNSUPPORTED),
    (dict(TOKEN_AXIS, k_bits=8, v_bits=8, k_format="fp8", k_scale=0.0), N.KVQ_EINVAL),
    (dict(TOKEN_AXIS, k_bits=8, v_bits=8, k_format="fp8", v_scale=float("inf")), N.KVQ_EINVAL),
    (dict(TOKEN_AXIS, k_bits=8, v_bits=8, k_format="fp8", v_scale=float("nan")), N.KVQ_EINVAL),
    # pre-RoPE keys: channel-axis affine keys without sparse entries, a base above 1
    (dict(k_rope=2), N.KVQ_EINVAL),
    (dict(k_rope=1, rope_theta=1.0), N.KVQ_EINVAL),
    (dict(k_rope=1, rope_theta=float("nan")), N.KVQ_EINVAL),
    (dict(TOKEN_AXIS, k_rope=1), N.KVQ_EUNSUPPORTED),
    (dict(k_rope=1, k_sparse_per_vector=2), N.KVQ_EUNSUPPORTED),
])
def test_bad_config(kw, status):
    c = _cfg(**kw)
    with pytest.raises(N.KVQError) as e:
        kvq_cache_sizes(c, 2, 256)
    assert e.value.status == status
    assert kvq_workspace_bytes(c, 2, 256) == 0


def test_rope_config_accepted():
    for kw in (dict(k_rope=1), dict(k_rope=1, k_bits=2, v_bits=2, k_residual_tokens=128, rope_theta=5e5)):
        c = _cfg(**kw)
        assert kvq_cache_sizes(c, 2, 256) == kvq_cache_sizes(_cfg(**{**kw, "k_rope": 0}), 2, 256)


def test_unknown_format_code():
    c = _cfg(**TOKEN_AXIS).c()
    c.k_format = c.v_format = 7
    out = N.kvq_sizes()
    assert N.lib().kvq_cache_sizes(ctypes.byref(c), 2, 256, ctypes.byref(out)) == N.KVQ_EINVAL


def test_fp8_cache_needs_no_meta_pointers():
    L = N.lib()
    pc = _cfg(**TOKEN_AXIS, k_bits=8, v_bits=8, k_format="fp8")
    cfg = pc.c()
    c, lh = _fake_cache(pc, 2, 64, [60, 0])
    c.k_meta = c.v_meta = None
    cu = ctypes.cast(ctypes.c_void_p(1 << 20), ctypes.POINTER(ctypes.c_int32))
    fake = ctypes.c_void_p(1 << 20)
    n = (ctypes.c_int32 * 2)(5, 1)               # reaches the capacity check: the cache itself is valid
    assert L.kvq_append(ctypes.byref(cfg), ctypes.byref(c), fake, fake, cu, n, None) == N.KVQ_ECAPACITY
    # an affine cache without metadata is invalid
    pi = _cfg(**TOKEN_AXIS, k_bits=8, v_bits=8)
    ci = pi.c()
    assert L.kvq_append(ctypes.byref(ci), ctypes.byref(c), fake, fake, cu, n, None) == N.KVQ_EINVAL


def _fake_cache(cfg, batch, max_tokens, lens):
    fake = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced on these paths
    lh = (ctypes.c_int32 * batch)(*lens)
    c = N.kvq_cache(batch, max_tokens, fake, fake, fake, fake, fake, fake,
                    ctypes.cast(fake, ctypes.POINTER(ctypes.c_int32)),
                    ctypes.cast(lh, ctypes.POINTER(ctypes.c_int32)))
    return c, lh


def test_append_errors_before_launch():
    L = N.lib()
    cfg = _cfg().c()
    c, lh = _fake_cache(_cfg(), 2, 64, [60, 0])
    cu = ctypes.cast(ctypes.c_void_p(1 << 20), ctypes.POINTER(ctypes.c_int32))
    fake = ctypes.c_void_p(1 << 20)
    n = (ctypes.c_int32 * 2)(5, 1)               # 60 + 5 > 64
    assert L.kvq_append(ctypes.byref(cfg), ctypes.byref(c), fake, fake, cu, n, None) == N.KVQ_ECAPACITY
    n = (ctypes.c_int32 * 2)(-1, 1)
    assert L.kvq_append(ctypes.byref(cfg), ctypes.byref(c), fake, fake, cu, n, None) == N.KVQ_EINVAL
    n = (ctypes.c_int32 * 2)(1, 1)
    assert L.kvq_append(ctypes.byref(cfg), ctypes.byref(c), fake, fake, None, n, None) == N.KVQ_EINVAL
    mis = ctypes.c_void_p((1 << 20) + 2)
    assert L.kvq_append(ctypes.byref(cfg), ctypes.byref(c), mis, fake, cu, n, None) == N.KVQ_EINVAL
    # nothing to append is a no-op that touches no device memory
    n = (ctypes.c_int32 * 2)(0, 0)
    assert L.kvq_append(ctypes.byref(cfg), ctypes.byref(c), None, None, cu, n, None) == N.KVQ_OK
    assert list(lh) == [60, 0]
    # capacity not a multiple of 32
    c2, _ = _fake_cache(_cfg(), 2, 70, [0, 0])
    assert L.kvq_append(ctypes.byref(cfg), ctypes.byref(c2), fake, fake, cu, n, None) == N.KVQ_EINVAL
    # a residual buffer is required for channel-axis keys
    c.k_resid = None
    assert L.kvq_append(ctypes.byref(cfg), ctypes.byref(c), fake, fake, cu, n, None) == N.KVQ_EINVAL


def test_attention_errors_before_launch():
    L = N.lib()
    pc = _cfg()
    cfg = pc.c()
    c, _ = _fake_cache(pc, 2, 256, [10, 20])
    fake = ctypes.c_void_p(1 << 20)
    need = kvq_workspace_bytes(pc, 2, 256)
    assert need > 0
    assert L.kvq_decode_attention(ctypes.byref(cfg), ctypes.byref(c), fake, fake, ctypes.c_float(0.1),
                                  fake, need - 1, None) == N.KVQ_EWORKSPACE
    assert L.kvq_decode_attention(ctypes.byref(cfg), ctypes.byref(c), None, fake, ctypes.c_float(0.1),
                                  fake, need, None) == N.KVQ_EINVAL
    c.len_host[0] = 300                         # > max_tokens
    assert L.kvq_decode_attention(ctypes.byref(cfg), ctypes.byref(c), fake, fake, ctypes.c_float(0.1),
                                  fake, need, None) == N.KVQ_EINVAL
    assert L.kvq_dequantize(ctypes.byref(cfg), ctypes.byref(c), fake, fake, None) == N.KVQ_EINVAL
    # the entry point without a workspace validates the same way, before any HIP call
    assert L.kvq_decode_attention_noalloc(ctypes.byref(cfg), ctypes.byref(c), fake, fake,
                                          ctypes.c_float(0.1), None) == N.KVQ_EINVAL
    c.len_host[0] = 10
    assert L.kvq_decode_attention_noalloc(ctypes.byref(cfg), ctypes.byref(c), None, fake,
                                          ctypes.c_float(0.1), None) == N.KVQ_EINVAL
    mis = ctypes.c_void_p((1 << 20) + 4)
    assert L.kvq_decode_attention_noalloc(ctypes.byref(cfg), ctypes.byref(c), fake, mis,
                                          ctypes.c_float(0.1), None) == N.KVQ_EINVAL


def test_workspace_bound():
    # two partial slots of G query heads per workgroup, at most 2048
    # workgroups, each taking at least 8 tiles
    slot = 132 * 4
    assert kvq_workspace_bytes(_cfg(), 128, 32800) == 2 * 2048 * 4 * slot     # ragged int4 workload
    assert kvq_workspace_bytes(_cfg(n_q_heads=64), 1, 4096) == 2 * (8 * 128 // 8) * 8 * slot
    assert kvq_workspace_bytes(_cfg(n_kv_heads=1, n_q_heads=1), 1, 32) == 2 * 1 * 1 * slot
    assert kvq_workspace_bytes(_cfg(n_q_heads=64), 128, 1 << 20) <= 17_301_504  # the scratch held for the no-allocation call


def test_status_strings():
    for s in range(6):
        assert N.status_string(s)
    assert N.status_string(N.KVQ_ECAPACITY) == "append exceeds cache capacity"


def test_sizes_take_64_bit_token_counts():
    # the sizing calls take int64_t max_tokens: values past int32 reach the
    # library intact and are refused as unsupported, not truncated
    c = _cfg()
    L = N.lib()
    out = N.kvq_sizes()
    for big in (1 << 31, (1 << 32) + 32, 1 << 40):
        assert L.kvq_cache_sizes(ctypes.byref(c.c()), 1, big, ctypes.byref(out)) == N.KVQ_EUNSUPPORTED
        assert kvq_workspace_bytes(c, 1, big) == 0
    # the largest capacity a cache can describe is still accepted
    assert kvq_cache_sizes(c, 1, 1 << 24)["k_codes"] == 8 * (1 << 24) * 64
    assert kvq_workspace_bytes(c, 1, 1 << 24) > 0
    assert L.kvq_cache_sizes(ctypes.byref(c.c()), 1, (1 << 24) + 32, ctypes.byref(out)) == N.KVQ_EUNSUPPORTED


def test_binding_rejects_bad_tensors():
    """The binding checks dtype, device, contiguity and exact shape of every
    tensor before any pointer crosses the ABI (CPU tensors are refused as not
    on the device, so nothing here launches)."""
    import torch
    import quantized_decode_attention_03_amd as K

    class _Cache:  # the attributes the binding reads
        batch, max_tokens = 2, 64
        cfg = _cfg()
        device = torch.device("cuda", 0)

    cache = _Cache()
    k = torch.zeros((3, 8, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="device tensor"):
        K.kvq_append(cache, k, k, None, [2, 1])
    with pytest.raises(ValueError, match="counts for a batch"):
        K.kvq_append(cache, k, k, None, [3])
    with pytest.raises(ValueError, match="negative"):
        K.kvq_append(cache, k, k, None, [4, -1])
    q = torch.zeros((2, 32, 128), dtype=torch.float16)
    with pytest.raises(ValueError, match="device tensor"):
        K.kvq_decode_attention(cache, q, q.float(), 0.1, torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="device tensor"):
        K.kvq_dequantize(cache, q, q)
    # the checks themselves, on tensors that pass the device test
    chk = K._check
    with pytest.raises(ValueError, match="torch tensor"):
        chk(3, "x", torch.float16)


def test_binding_check_rules(monkeypatch):
    """Dtype, contiguity, shape and device rules of the binding's tensor check,
    exercised with CPU tensors that pretend to be on the device."""
    import torch
    import quantized_decode_attention_03_amd as K

    class _Dev(torch.Tensor):
        pass

    def dev(t):
        d = t.as_subclass(_Dev)
        return d

    monkeypatch.setattr(_Dev, "is_cuda", property(lambda self: True))
    monkeypatch.setattr(_Dev, "device", property(lambda self: torch.device("cuda", 0)))
    t = dev(torch.zeros((4, 8, 128), dtype=torch.float16))
    K._check(t, "t", torch.float16, (4, 8, 128), torch.device("cuda", 0))
    with pytest.raises(ValueError, match="dtype"):
        K._check(t, "t", torch.float32, (4, 8, 128))
    with pytest.raises(ValueError, match="shape"):
        K._check(t, "t", torch.float16, (5, 8, 128))
    with pytest.raises(ValueError, match="contiguous"):
        K._check(dev(torch.zeros((8, 4, 128), dtype=torch.float16)).transpose(0, 1), "t", torch.float16)
    with pytest.raises(ValueError, match="the cache is on"):
        K._check(t, "t", torch.float16, None, torch.device("cuda", 1))


def test_append_binding_passes_current_counts(monkeypatch):
    """The binding keeps the C array of host counts while the counts repeat
    (every decode step); a change of counts, also in place in the same list,
    reaches the library."""
    import quantized_decode_attention_03_amd as K
    seen = []

    class Lib:
        def kvq_append(self, cfg, cache, k, v, cu, n, stream):
            seen.append(list(n))
            return N.KVQ_OK

    monkeypatch.setattr(N, "lib", lambda: Lib())
    monkeypatch.setattr(K, "_check", lambda *a, **k: None)

    class Stream:
        cuda_stream = 0

    class Cache:
        batch, cfg, device = 3, _cfg(), None
        _cfg, _c = None, None
        _n_prev, _n_arr = None, None

    class Buf:  # stands for a device tensor: only its address is read
        def data_ptr(self):
            return 1 << 20

    c = Cache()
    c._cfg, c._c = c.cfg.c(), N.kvq_cache()
    counts = [1, 1, 1]
    K.kvq_append(c, None, None, Buf(), counts, Stream())
    K.kvq_append(c, None, None, Buf(), counts, Stream())
    counts[1] = 5
    K.kvq_append(c, None, None, Buf(), counts, Stream())
    K.kvq_append(c, None, None, Buf(), (2, 0, 7), Stream())
    assert seen == [[1, 1, 1], [1, 1, 1], [1, 5, 1], [2, 0, 7]]
    with pytest.raises(ValueError):
        K.kvq_append(c, None, None, Buf(), [1, -1, 1], Stream())
    with pytest.raises(ValueError):
        K.kvq_append(c, None, None, Buf(), [1, 1], Stream())
