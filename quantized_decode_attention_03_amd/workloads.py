"""Seeded synthetic workloads: shapes and inputs only, none of the method's
arithmetic. Shared by the tests, the bench and the oracle checks.

Value recipe (stand-ins for real model activations, which the pages study on
trained models and datasets that are not used here):
  * keys and values are fp32 N(0, 1) draws rounded to fp16 (round to nearest
    even); four channels of every key head are multiplied by 20 before the
    rounding — the outlier-channel structure the pages describe for keys
    ("KV Cache Quantization — 8-bit and 4-bit", "The outlier problem: keys have
    outlier channels", whose example is a channel 20x larger than the rest).
    Values have no outlier channels ("Why keys and values want different
    treatment").
  * the int2 workload also multiplies each key entry by 50 with probability
    0.001 (isolated spikes);
  * queries are N(0, 1) in fp16.
Streams: numpy PCG64 seeded by SeedSequence(seed, spawn_key=(layer, kind, i)),
so any one sequence, layer or step can be regenerated alone.
"""
from dataclasses import dataclass, replace

import numpy as np

# kinds of spawned streams
_OUTLIERS, _LENGTHS, _PREFILL, _STEP = 0, 1, 2, 3

FIXED_OUTLIERS = (3, 17, 64, 101)


@dataclass(frozen=True)
class Spec:
    cid: int                 # workload number 1..5
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int             # prefill length (upper bound when ragged)
    min_len: int             # == seq_len unless lengths are ragged
    layers: int
    k_bits: int
    v_bits: int
    k_axis: str              # "token" or "channel"
    k_group: int             # G
    k_residual: int          # R
    k_sparse: int            # entries per key vector kept in fp16
    spike_prob: float
    fixed_outliers: bool
    steps: int               # decode steps (append 1 token + attend)
    seed: int
    d_head: int = 128
    fmt: str = "int"         # element format: "int" (affine), "fp8" or "sym32"
    k_scale: float = 1.0     # fp8 per-cache scales
    v_scale: float = 1.0
    k_rope: int = 0          # 1: keys cached before the rotary embedding
    rope_theta: float = 10000.0

    @property
    def ragged(self):
        return self.min_len != self.seq_len

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    def max_tokens(self, extra_steps=0):
        """Capacity for the prefill plus decode steps, rounded up to 32."""
        t = self.seq_len + self.steps + extra_steps
        return (t + 31) // 32 * 32


SPECS = {
    1: Spec(1, "int8 per-token K/V, B=1, Hq=Hkv=1, S=256", 1, 1, 1, 256, 256, 1,
            8, 8, "token", 0, 0, 0, 0.0, True, 1, 1001),
    2: Spec(2, "KIVI int4 (K per-channel G=32 R=32, V per-token), B=16, Hq=32, Hkv=8, S=4096",
            16, 32, 8, 4096, 4096, 1, 4, 4, "channel", 32, 32, 0, 0.0, False, 1, 1002),
    3: Spec(3, "int8 per-token K/V, 32 layers, B=1, Hq=32, Hkv=8, S=32768",
            1, 32, 8, 32768, 32768, 32, 8, 8, "token", 0, 0, 0, 0.0, False, 1, 1003),
    4: Spec(4, "KIVI int2 (K per-channel G=32 R=128, V per-token), B=64, Hq=32, Hkv=8, S=8192",
            64, 32, 8, 8192, 8192, 1, 2, 2, "channel", 32, 128, 0, 0.001, False, 1, 1004),
    5: Spec(5, "streaming int4 per-channel K + top-2 sparse, B=128, S~U[1024,32768], Hq=32, Hkv=8",
            128, 32, 8, 32768, 1024, 1, 4, 4, "channel", 32, 32, 2, 0.0, False, 64, 1005),
}


def spec(cid, **overrides):
    """The workload spec, optionally resized (tests use smaller shapes of the
    same structure)."""
    s = SPECS[cid]
    return replace(s, **overrides) if overrides else s


def _rng(s, layer, kind, i):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(s.seed, spawn_key=(layer, kind, i))))


def outlier_channels(s, layer):
    """[n_kv_heads, 4] outlier channel indices of one layer."""
    if s.fixed_outliers:
        return np.array([FIXED_OUTLIERS] * s.n_kv_heads, np.int64)
    rng = _rng(s, layer, _OUTLIERS, 0)
    return np.stack([np.sort(rng.choice(s.d_head, 4, replace=False))
                     for _ in range(s.n_kv_heads)])


def seq_lengths(s):
    """Prefill lengths [batch]: all seq_len, or uniform integers in
    [min_len, seq_len] when ragged."""
    if not s.ragged:
        return np.full(s.batch, s.seq_len, np.int64)
    return _rng(s, 0, _LENGTHS, 0).integers(s.min_len, s.seq_len, size=s.batch,
                                            endpoint=True).astype(np.int64)


def _keys(s, rng, shape, chans):
    z = rng.standard_normal(shape, dtype=np.float32)
    for h in range(s.n_kv_heads):
        z[..., h, chans[h]] *= np.float32(20.0)
    if s.spike_prob > 0:
        spikes = rng.random(shape, dtype=np.float32) < s.spike_prob
        z[spikes] *= np.float32(50.0)
    return z.astype(np.float16)


def prefill(s, layer, b, length=None):
    """Prefill keys and values of sequence b: fp16 [len, n_kv_heads, d_head]."""
    n = int(seq_lengths(s)[b]) if length is None else length
    rng = _rng(s, layer, _PREFILL, b)
    shape = (n, s.n_kv_heads, s.d_head)
    k = _keys(s, rng, shape, outlier_channels(s, layer))
    v = rng.standard_normal(shape, dtype=np.float32).astype(np.float16)
    return k, v


def step(s, layer, i):
    """Inputs of decode step i: q fp16 [B, Hq, D]; new key/value fp16
    [B, Hkv, D] (one token per sequence)."""
    rng = _rng(s, layer, _STEP, i)
    q = rng.standard_normal((s.batch, s.n_q_heads, s.d_head), dtype=np.float32).astype(np.float16)
    shape = (s.batch, s.n_kv_heads, s.d_head)
    k = _keys(s, rng, shape, outlier_channels(s, layer))
    v = rng.standard_normal(shape, dtype=np.float32).astype(np.float16)
    return q, k, v
