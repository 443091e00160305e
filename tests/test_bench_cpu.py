"""Host logic of bench.py, on the CPU.

The roofline figure divides bench.algorithmic_bytes by the measured time, so
that count is checked against the oracle's own array sizes (oracle/sizes.py,
itself pinned to the pages' worked sizing example): for caches that are full
(every token held, no residual keys) the bytes one attention launch must read
are exactly the cache arrays, plus fp16 queries in and fp32 outputs out.
"""
import os
import subprocess
import sys
from dataclasses import replace

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle.sizes import actual_bytes  # noqa: E402
from harness import ref_config  # noqa: E402
from quantized_decode_attention_03_amd import workloads as W  # noqa: E402


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_algorithmic_bytes_match_oracle_sizes_on_full_caches(cid):
    s = W.spec(cid)
    T = 256 if cid != 4 else 512          # multiples of 32 and of every R
    s = replace(s, batch=3)
    sz = actual_bytes(ref_config(s), s.batch, T)
    cache = sz["k_codes"] + sz["k_meta"] + sz["k_sparse"] + sz["v_codes"] + sz["v_meta"]
    q_out = s.batch * s.n_q_heads * s.d_head * (2 + 4)
    assert bench.algorithmic_bytes(s, [T] * s.batch) == cache + q_out


@pytest.mark.parametrize("fmt,kb,vb", [("fp8", 8, 8), ("sym32", 8, 8), ("sym32", 4, 2)])
def test_algorithmic_bytes_of_element_formats(fmt, kb, vb):
    s = replace(W.spec(3), batch=2, fmt=fmt, k_bits=kb, v_bits=vb)
    T = 256
    sz = actual_bytes(ref_config(s), s.batch, T)
    cache = sz["k_codes"] + sz["k_meta"] + sz["v_codes"] + sz["v_meta"]
    assert bench.algorithmic_bytes(s, [T] * s.batch) == cache + s.batch * s.n_q_heads * s.d_head * 6


def test_algorithmic_bytes_count_residual_keys_as_fp16():
    s = replace(W.spec(2), batch=1)
    D, H = s.d_head, s.n_kv_heads
    full = bench.algorithmic_bytes(s, [4096])
    # one more token: its key waits in the fp16 residual (256 B), its value
    # is quantized (64 B of codes + a 4 B scale word)
    assert bench.algorithmic_bytes(s, [4097]) - full == H * (D * 2 + D * s.v_bits // 8 + 4)


def test_per_token_figures():
    # bytes per (token, KV head) of the documented layout
    def per_token(cid):
        s = replace(W.spec(cid), batch=1)
        q_out = s.n_q_heads * s.d_head * 6
        return (bench.algorithmic_bytes(s, [1024]) - q_out) // (1024 * s.n_kv_heads)
    assert per_token(2) == 148   # int4 KIVI: 64 + 16 (K) + 64 + 4 (V)
    assert per_token(4) == 84    # int2 KIVI: 32 + 16 + 32 + 4
    assert per_token(1) == 264   # int8 per token: 128 + 4 + 128 + 4
    assert per_token(5) == 156   # int4 KIVI + 2 sparse entries (8 B)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


@pytest.mark.parametrize("cid", [2, 4, 5])
def test_prefill_bytes_are_fp16_read_plus_cache_written(cid):
    # a whole-context append reads every fp16 key and value once and writes
    # the cache arrays once (full caches: no residual keys left)
    s = replace(W.spec(cid), batch=2)
    T = 512
    sz = actual_bytes(ref_config(s), s.batch, T)
    cache = sz["k_codes"] + sz["k_meta"] + sz["k_sparse"] + sz["v_codes"] + sz["v_meta"]
    fp16_in = s.batch * T * s.n_kv_heads * s.d_head * 2 * 2
    assert bench.prefill_bytes(s, [T] * s.batch) == fp16_in + cache


class _Event:
    """Stand-in for torch.cuda.Event: record() stamps a fake clock 10 us ahead."""
    clock = 0.0

    def __init__(self, enable_timing=False):
        self.t = None

    def record(self, stream=None):
        _Event.clock += 0.01
        self.t = _Event.clock

    def elapsed_time(self, other):
        return other.t - self.t


class _Cache:
    def __init__(self, cfg, batch, max_tokens, device="cuda"):
        self.batch, self.max_tokens = batch, max_tokens
        self.len_host = [0] * batch

    def copy_from(self, other):
        self.len_host = list(other.len_host)


def _stub_gpu(monkeypatch):
    import torch
    import quantized_decode_attention_03_amd as K

    monkeypatch.setattr(torch.cuda, "Event", _Event)
    monkeypatch.setattr(torch.cuda, "synchronize", lambda *a, **k: None)
    monkeypatch.setattr(torch.cuda, "empty_cache", lambda *a, **k: None)
    monkeypatch.setattr(torch.cuda, "set_device", lambda *a, **k: None)
    monkeypatch.setattr(torch.cuda, "current_stream", lambda *a, **k: None)
    monkeypatch.setattr(torch.Tensor, "to", lambda self, *a, **k: self)
    for fn in ("zeros", "empty", "tensor", "arange"):
        orig = getattr(torch, fn)
        monkeypatch.setattr(torch, fn, (lambda o: lambda *a, **k: o(*a, **{x: y for x, y in k.items()
                                                                             if x != "device"}))(orig))

    def append(c, k, v, cu, n, stream=None):
        c.len_host = [a + int(b) for a, b in zip(c.len_host, n)]

    monkeypatch.setattr(K, "KVCache", _Cache)
    monkeypatch.setattr(K, "kvq_append", append)
    monkeypatch.setattr(K, "kvq_decode_attention", lambda *a, **k: None)


def test_bench_default_runs_three_workloads_headline_last(monkeypatch, capsys):
    """With no --config, workloads 2, 4 and 5 run in turn (shrunk here so the
    host generation stays small) and the headline fields are workload 5's."""
    import json
    _stub_gpu(monkeypatch)
    small = {2: dict(batch=2, seq_len=300, min_len=300), 4: dict(batch=2, seq_len=400, min_len=400),
             5: dict(batch=4, seq_len=600, min_len=100)}
    specs = {cid: replace(W.SPECS[cid], **kw) for cid, kw in small.items()}
    monkeypatch.setattr(W, "SPECS", {**W.SPECS, **specs})
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "3", "--warmup", "1", "--cpu-seqs", "2",
                                      "--cpu-steps", "1", "--settle-ms", "0"])
    bench.main()
    d = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert [w["workload"] for w in d["workloads"]] == [specs[c].name for c in (2, 4, 5)]
    assert d["config"]["workload"] == specs[5].name and d["value"] == d["workloads"][-1]["value"]
    assert d["roofline"] == d["workloads"][-1]["roofline"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["host_cores"] >= 1 and cb["value"] > 0


@pytest.mark.parametrize("argv", [["--config", "1", "--steps", "5", "--warmup", "2", "--cpu-steps", "1"],
                                  ["--config", "2", "--steps", "3", "--warmup", "2", "--no-cpu-baseline"]])
def test_bench_main_with_gpu_calls_stubbed(argv, monkeypatch, capsys):
    """bench.main() end to end on the CPU, every GPU call replaced by a stub:
    the data flow (replicas, lengths, events, byte counts) and the JSON line."""
    import json
    _stub_gpu(monkeypatch)
    argv = argv + ["--settle-ms", "0"]

    monkeypatch.setattr(sys, "argv", ["bench.py"] + argv)
    bench.main()
    line = capsys.readouterr().out.strip().splitlines()[-1]
    d = json.loads(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["unit"] == "tokens/s" and d["value"] > 0
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"])
    s = W.spec(int(argv[1]))
    assert r["algorithmic_bytes_per_launch"] >= bench.algorithmic_bytes(s, [int(x) for x in W.seq_lengths(s)])
    assert d["append"]["prefill_bytes"] == bench.prefill_bytes(s, [int(x) for x in W.seq_lengths(s)])
    assert ("cpu_baseline" in d) == ("--no-cpu-baseline" not in argv)
    if "cpu_baseline" in d:
        assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["value"] > 0
    assert len(d["workloads"]) == 1 and d["workloads"][0]["value"] == d["value"]


def test_bench_formats_mode(monkeypatch, capsys):
    """--formats runs the 8-bit per-token shape in the four element formats
    (shrunk here) and reports each one's bytes and roofline."""
    import json
    _stub_gpu(monkeypatch)
    monkeypatch.setattr(W, "SPECS", {**W.SPECS, 3: replace(W.SPECS[3], seq_len=640, min_len=640),
                                     2: replace(W.SPECS[2], batch=2, seq_len=300, min_len=300)})
    monkeypatch.setattr(sys, "argv", ["bench.py", "--formats", "--steps", "2", "--warmup", "1",
                                      "--settle-ms", "0"])
    bench.main()
    d = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    ws = d["workloads"]
    assert len(ws) == 5 and "cpu_baseline" not in d and "pre-RoPE" in ws[4]["workload"]
    assert d["roofline"] == ws[0]["roofline"]
    # bytes per (token, KV head): int8 128+4+128+4, fp8 128+128, 8-bit blocks
    # 128+8+128+8, 4-bit blocks 64+8+64+8
    b = [w["roofline"]["algorithmic_bytes_per_launch"] for w in ws]
    assert b[1] < b[0] < b[2] and b[3] < b[1]
    assert "fp8" in ws[1]["dtype"] and "symmetric" in ws[3]["dtype"]
