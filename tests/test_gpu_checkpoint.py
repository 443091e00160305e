"""Checkpoint and resume on the ragged streaming workload (int4 channel-axis
keys with top-2 sparse entries, R = 32): a cache run for 10 decode steps,
copied to host memory, loaded into a fresh cache and run for 30 more steps
(crossing a residual flush of every sequence) gives, step for step, the same
attention outputs and in the end the same cache bytes as an uninterrupted run
of 40 steps."""
import numpy as np
import pytest

from quantized_decode_attention_03_amd import workloads as W
from harness import Pair, prefill_inputs

pytestmark = pytest.mark.gpu


def test_checkpoint_resume_bit_exact():
    import quantized_decode_attention_03_amd as K
    s = W.spec(5, batch=16, seq_len=4096, min_len=1024, steps=40)
    k, v, lens = prefill_inputs(s)
    T = s.max_tokens()
    a = Pair(s, T, with_ref=False)
    b = Pair(s, T, with_ref=False)
    a.append(k, v, lens)
    b.append(k, v, lens)
    for i in range(10):
        q, kn, vn = W.step(s, 0, i)
        a.append(kn, vn, [1] * s.batch)
        b.append(kn, vn, [1] * s.batch)
        oa, _ = a.attend(q)
        ob, _ = b.attend(q)
        assert np.array_equal(oa, ob)
    st = b.gpu.state()                       # checkpoint to host memory
    b.gpu = K.KVCache(K.Config.from_spec(s), s.batch, T)
    b.gpu.load_state(st)                     # resume in a fresh cache
    del st
    for i in range(10, 40):
        q, kn, vn = W.step(s, 0, i)
        a.append(kn, vn, [1] * s.batch)
        b.append(kn, vn, [1] * s.batch)
        oa, _ = a.attend(q)
        ob, _ = b.attend(q)
        assert np.array_equal(oa, ob), i
    sa, sb = a.gpu.state(), b.gpu.state()
    for name in sa:
        assert np.array_equal(sa[name], sb[name]), name
    print(f"resumed run equal to the uninterrupted one; lengths {list(sa['len_host'][:4])} ...", flush=True)
