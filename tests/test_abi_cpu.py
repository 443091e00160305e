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


def test_sizes_match_oracle_formula():
    from oracle import sizes
    from oracle.cache import Config as RC
    for kw in [dict(), dict(k_bits=2, v_bits=2, k_residual_tokens=128),
               dict(k_sparse_per_vector=2),
               dict(k_axis="token", k_group_tokens=0, k_residual_tokens=0, k_bits=8, v_bits=8)]:
        c = _cfg(**kw)
        got = kvq_cache_sizes(c, 3, 4096)
        rc = RC(128, c.n_kv_heads, c.n_q_heads, c.k_bits, c.v_bits, c.k_axis, c.k_group_tokens,
                c.k_residual_tokens, c.k_sparse_per_vector)
        want = sizes.actual_bytes(rc, 3, 4096)
        for k, v in want.items():
            assert got[k] == v, k


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
])
def test_bad_config(kw, status):
    c = _cfg(**kw)
    with pytest.raises(N.KVQError) as e:
        kvq_cache_sizes(c, 2, 256)
    assert e.value.status == status
    assert kvq_workspace_bytes(c, 2, 256) == 0


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


def test_status_strings():
    for s in range(6):
        assert N.status_string(s)
    assert N.status_string(N.KVQ_ECAPACITY) == "append exceeds cache capacity"
