#!/usr/bin/env python3
"""Decode benchmark on one MI355X.

One step = one pass of the hot path over one batch: quantize-on-append of one
new key/value token per sequence (with the residual flush when a window fills)
followed by fused-dequant decode attention for one query token per sequence,
in every layer of the workload (the 32-layer worked-example shape runs all
32 layers per step; the roofline entry is per attention launch, one layer).
Inputs are resident in HBM before timing starts. Cache replicas are rotated so
each step reads a cache that is not resident in the 256 MB last-level cache.

By default the int4 and int2 KIVI workloads (2 and 4) and the ragged int4 +
sparse streaming workload (5) run in turn; the JSON line's headline fields
(value, ms_per_step, config, roofline) are workload 5's, the largest, and a
"workloads" array carries each one's figures. --config N runs one workload.

For each workload: tokens/s over the whole decode step, ms per step, and for
the attention call a roofline entry (algorithmic bytes per launch / measured
launch time against 8 TB/s HBM, with the HBM traffic recorded by rocprofv3
counters when they were taken on the current kernel sources), plus an "append"
entry for the quantize-on-append path on its own: a whole-context prefill (GB/s
over its algorithmic bytes) and the per-step append of one token per sequence.
The float64 oracle is timed on the host on a bounded sample of the headline
workload as a reported baseline.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn tokens/s + achieved HBM GB/s (% of peak), int4/int2 KV, 1 MI355X"
PEAK_GBS = 8000.0


def algorithmic_bytes(s, lens):
    """Bytes one attention launch must move: every held token's codes and
    metadata (plus residual fp16 keys and sparse entries), the fp16 queries and
    the fp32 outputs. Per (sequence, KV head) with L tokens of which Q are
    quantized keys."""
    H, D = s.n_kv_heads, s.d_head
    # metadata bytes per token of a token-axis side: one word (affine codes),
    # four fp16 block scales (symmetric blocks), none (fp8)
    meta_tok = {"int": 4, "sym32": 8, "fp8": 0}[s.fmt]
    tot = 0
    for L in lens:
        Q = L if s.k_axis == "token" else L - L % s.k_residual
        k = Q * D * s.k_bits // 8
        k += (Q // 32) * D * 4 if s.k_axis == "channel" else Q * meta_tok
        k += (L - Q) * D * 2
        k += Q * 8 if s.k_sparse else 0
        v = L * D * s.v_bits // 8 + L * meta_tok
        tot += H * (k + v)
    tot += s.batch * s.n_q_heads * D * (2 + 4)
    return tot


def attention_source_hash():
    """Hash of the attention kernel sources; HBM traffic figures recorded under
    profiles/ apply only while it is unchanged."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "quantized_decode_attention_03_amd", "csrc")
    for f in ("kvq_attention.hip", "kvq_device.h", "kvq_internal.h"):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(cid):
    """Calibrated HBM bytes per attention launch from the rocprofv3 counter runs
    recorded in profiles/traffic.json (FETCH_SIZE and WRITE_SIZE, each scaled by
    the same counter's reading for a plain copy of known size), or None when
    there is no record for this workload or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(str(cid))
    if not rec or rec.get("source_sha256_16") != attention_source_hash():
        return None
    return rec["traffic_bytes_per_dispatch"]


def progress(msg):
    """A line on stderr per stage (stdout carries only the result line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def prefill_bytes(s, lens):
    """Algorithmic bytes of quantizing a whole context on append: the fp16
    keys and values read once, the packed cache (codes, metadata, residual
    keys, sparse entries) written once."""
    read = sum(lens) * s.n_kv_heads * s.d_head * 2 * 2
    written = algorithmic_bytes(s, lens) - s.batch * s.n_q_heads * s.d_head * (2 + 4)
    return read + written


def append_report(s, lens, prefill_ms, step_ms):
    """Quantize-on-append timings (HIP events on the launch stream): a whole
    prefill of the workload's context, and the append of one token per
    sequence inside each timed decode step (flushes included)."""
    nbytes = prefill_bytes(s, lens)
    pre_s = float(np.mean(prefill_ms)) / 1e3
    return {"prefill_tokens": int(sum(lens)), "prefill_bytes": nbytes,
            "prefill_us": pre_s * 1e6, "prefill_GBps": nbytes / pre_s / 1e9,
            "decode_step_append_us": float(np.mean(step_ms)) * 1e3}


def host_cpu():
    """(usable cores, CPU model) of the host this process runs on."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def cpu_baseline(s, n_seq, steps):
    """The oracle's decode step (append + float64 attention) on the n_seq
    sequences closest to the median length, timed on the host with numpy's
    BLAS pool held to one thread. Returns (tokens/s, seconds, the sample's
    lengths)."""
    from dataclasses import replace
    from threadpoolctl import threadpool_limits
    from oracle.cache import Config as RC, RefCache
    from quantized_decode_attention_03_amd import workloads as W
    lens_all = [int(x) for x in W.seq_lengths(s)]
    order = sorted(range(s.batch), key=lambda b: lens_all[b])
    lo = max(0, min(len(order) - n_seq, len(order) // 2 - n_seq // 2))
    pick = sorted(order[lo:lo + n_seq])
    lens = [lens_all[b] for b in pick]
    sub = replace(s, batch=len(pick))
    with threadpool_limits(1):
        ref = RefCache(RC(s.d_head, s.n_kv_heads, s.n_q_heads, s.k_bits, s.v_bits, s.k_axis,
                          s.k_group, s.k_residual, s.k_sparse), len(pick),
                       ((max(lens) + steps + 31) // 32) * 32)
        ks, vs = zip(*[W.prefill(s, 0, b, lens_all[b]) for b in pick])
        ref.append(np.concatenate(ks), np.concatenate(vs), lens)
        scale = 1.0 / math.sqrt(s.d_head)
        inputs = []
        for i in range(steps):
            q, kn, vn = W.step(s, 0, i)
            inputs.append((q[pick], kn[pick], vn[pick]))
        t0 = time.perf_counter()
        for q, kn, vn in inputs:
            ref.append(kn, vn, [1] * len(pick))
            ref.attention(q, scale)
        dt = time.perf_counter() - t0
    del sub
    return len(pick) * steps / dt, dt, lens


def copy_probe():
    """A plain copy of known size: reads and writes 1 GiB per launch. Its HBM
    counters calibrate the attention kernel's, and its rate is the attainable
    copy bandwidth on this device."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    reps = 10
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "avg_ms": ms,
                      "read_plus_write_GBps": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


DEFAULT_WORKLOADS = (2, 4, 5)   # int4 KIVI, int2 KIVI, ragged int4 + sparse (headline: the largest)


def format_specs():
    """The 8-bit per-token workload's shape (B=1, Hq=32, Hkv=8, S=32768), one
    layer, in each element format: affine int8 (the workload's own), fp8 E4M3
    with per-cache scales, and symmetric 32-channel blocks at 8 and 4 bits
    (llama.cpp's q8_0 / q4_0 block shapes); then the int4 KIVI workload with
    its keys cached before the rotary embedding (rotated inside attention),
    to compare with the default run's plain one."""
    from dataclasses import replace
    from quantized_decode_attention_03_amd import workloads as W
    base = W.spec(3, layers=1)
    shape = "B=1, Hq=32, Hkv=8, S=32768, one layer"
    return [
        (3, replace(base, name=f"int8 per-token K/V (affine), {shape}")),
        ("3-fp8", replace(base, fmt="fp8", name=f"fp8 E4M3 K/V (per-cache scales 1.0), {shape}")),
        ("3-sym8", replace(base, fmt="sym32", name=f"int8 symmetric 32-channel blocks K/V, {shape}")),
        ("3-sym4", replace(base, fmt="sym32", k_bits=4, v_bits=4,
                           name=f"int4 symmetric 32-channel blocks K/V, {shape}")),
        # the int4 KIVI workload with keys cached before the rotary embedding
        ("2-rope", replace(W.spec(2), k_rope=1, name=W.spec(2).name + ", keys pre-RoPE")),
    ]


def run_workload(key, args, s=None):
    """Prefill, settle, warm up and time one workload (workload number key, or
    the spec s recorded under key); returns its result entry (everything but
    the host baseline)."""
    import torch
    import quantized_decode_attention_03_amd as K
    from quantized_decode_attention_03_amd import workloads as W

    s = W.spec(key) if s is None else s
    dev = "cuda"
    lens0 = [int(x) for x in W.seq_lengths(s)]
    cache_bytes = algorithmic_bytes(s, lens0)
    nlay = s.layers
    # single-layer workloads rotate cache replicas so that each step misses
    # the last-level cache; a multi-layer workload visits every layer's cache
    # in each step, which already exceeds it
    nrep = 1 if nlay > 1 else (args.replicas or max(1, min(16, math.ceil(1.25e9 / cache_bytes))))
    total_steps = args.warmup + args.steps
    per_rep = math.ceil(total_steps / nrep)
    T = ((max(lens0) + per_rep + 31) // 32) * 32
    cfg = K.Config.from_spec(s)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens0)]).astype(np.int32), device=dev)

    def prefill_inputs(layer):
        ks, vs = zip(*[W.prefill(s, layer, b, lens0[b]) for b in range(s.batch)])
        return (torch.from_numpy(np.concatenate(ks)).to(dev),
                torch.from_numpy(np.concatenate(vs)).to(dev))

    # prefill layer 0's cache (untimed: first launches), then two more timed
    # prefills into fresh caches (quantize-on-append of the whole context);
    # the replicas are those caches and clones of the first; further layers
    # get caches of their own
    progress(f"workload {key}: generating {sum(lens0)} prefill tokens x {nlay} layer(s)")
    kd, vd = prefill_inputs(0)
    base = K.KVCache(cfg, s.batch, T)
    K.kvq_append(base, kd, vd, cu, lens0)
    reps = [base]
    prefill_ms = []
    for _ in range(2):
        r = K.KVCache(cfg, s.batch, T)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        K.kvq_append(r, kd, vd, cu, lens0)
        b.record()
        torch.cuda.synchronize()
        prefill_ms.append(a.elapsed_time(b))
        if len(reps) < nrep:
            reps.append(r)
        else:
            del r
    del kd, vd
    while len(reps) < nrep:
        r = K.KVCache(cfg, s.batch, T)
        r.copy_from(base)
        reps.append(r)
    layer_caches = [base]
    for layer in range(1, nlay):
        kd, vd = prefill_inputs(layer)
        c = K.KVCache(cfg, s.batch, T)
        K.kvq_append(c, kd, vd, cu, lens0)
        layer_caches.append(c)
        del kd, vd
        torch.cuda.synchronize()
    progress(f"{nrep} cache replica(s) x {nlay} layer(s) ready; prefill {np.mean(prefill_ms) * 1e3:.1f} us")

    # per-step inputs resident on the device, per layer
    pool = 16 if nlay == 1 else 4
    inputs = []
    for layer in range(nlay):
        qs, kn, vn = [], [], []
        for i in range(pool):
            q, k, v = W.step(s, layer, i)
            qs.append(torch.from_numpy(q).to(dev))
            kn.append(torch.from_numpy(k).to(dev))
            vn.append(torch.from_numpy(v).to(dev))
        inputs.append((qs, kn, vn))
    cu1 = torch.arange(s.batch + 1, dtype=torch.int32, device=dev)
    ones = [1] * s.batch
    out = torch.empty((s.batch, s.n_q_heads, s.d_head), dtype=torch.float32, device=dev)
    ws = torch.zeros(K.kvq_workspace_bytes(cfg, s.batch, T), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(s.d_head)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step_caches(i):
        """(layer, cache) pairs one decode step visits, in order."""
        if nlay > 1:
            return list(enumerate(layer_caches))
        return [(0, reps[i % nrep])]

    def run(i, evs=None):
        for u, (layer, r) in enumerate(step_caches(i)):
            qs, kn, vn = inputs[layer]
            if evs is not None:
                evs[u][2].record(stream)
            K.kvq_append(r, kn[i % pool], vn[i % pool], cu1, ones, stream)
            if evs is not None:
                evs[u][0].record(stream)
            K.kvq_decode_attention(r, qs[i % pool], out, scale, ws, stream)
            if evs is not None:
                evs[u][1].record(stream)

    # Bring the device to its steady clocks before the warmup steps: attention
    # launches on cache 0 (they leave every cache unchanged) for at least
    # --settle-ms of wall time. The first launches after the host-side input
    # generation run measurably slower (clock ramp) for about 10 ms.
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for layer, r in step_caches(0):
            K.kvq_decode_attention(r, inputs[layer][0][0], out, scale, ws, stream)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    # lengths seen by the timed attention launches (every layer of a step
    # holds the same lengths)
    lens_timed = []
    step_lens = [list(r.len_host) for r in reps]
    for i in range(args.warmup, total_steps):
        rr = i % nrep
        step_lens[rr] = [x + 1 for x in step_lens[rr]]
        lens_timed += [list(step_lens[rr])] * nlay
    # per attention launch: attention start, attention end, append start
    events = [[tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(nlay)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        run(args.warmup + j, events[j])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launches = [e for step in events for e in step]
    attn_ms = [a.elapsed_time(b) for a, b, _ in launches]
    append_ms = [c.elapsed_time(a) for a, _, c in launches]
    attn_avg_s = float(np.mean(attn_ms)) / 1e3
    bytes_avg = float(np.mean([algorithmic_bytes(s, L) for L in lens_timed]))
    achieved = bytes_avg / attn_avg_s / 1e9
    progress(f"workload {key}: {args.steps} timed steps in {wall:.3f} s, attention {attn_avg_s * 1e6:.1f} us")
    return {
        "workload": s.name,
        "value": s.batch * args.steps / wall,
        "unit": "tokens/s",
        "ms_per_step": wall / args.steps * 1e3,
        "dtype": "f16 MFMA, f32 accumulate (" + (
            "fp8 E4M3 codes" if s.fmt == "fp8" else
            f"int{s.k_bits}/int{s.v_bits} {'symmetric block' if s.fmt == 'sym32' else 'affine'} codes") + ")",
        "config": {"workload": s.name, "batch": s.batch, "n_q_heads": s.n_q_heads,
                   "n_kv_heads": s.n_kv_heads, "d_head": s.d_head, "seq_len": s.seq_len,
                   "min_len": s.min_len, "k_bits": s.k_bits, "v_bits": s.v_bits,
                   "k_axis": s.k_axis, "k_group": s.k_group, "k_residual": s.k_residual,
                   "k_sparse": s.k_sparse, "format": s.fmt, "k_rope": s.k_rope, "layers": nlay,
                   "cache_replicas": nrep},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_GBS, "traffic": recorded_traffic(key),
                     "kernel": "kvq_decode_attention (attention kernel + partial merge)",
                     "avg_launch_us": attn_avg_s * 1e6,
                     "p10_p90_us": [float(np.percentile(attn_ms, 10)) * 1e3,
                                    float(np.percentile(attn_ms, 90)) * 1e3],
                     "algorithmic_bytes_per_launch": bytes_avg},
        "append": append_report(s, lens0, prefill_ms, append_ms),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=0,
                    help="one workload 1..5 (default: workloads 2, 4 and 5, headline 5)")
    ap.add_argument("--replicas", type=int, default=0, help="cache copies rotated (0: auto)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed attention launches before the warmup steps (device clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=4)
    ap.add_argument("--cpu-steps", type=int, default=4)
    ap.add_argument("--copy-probe", action="store_true",
                    help="time a plain 1 GiB device copy (HBM reference and counter calibration)")
    ap.add_argument("--formats", action="store_true",
                    help="compare the element formats (affine int8, fp8, symmetric blocks at 8 "
                         "and 4 bits) on the 8-bit per-token workload's shape, one layer, and "
                         "pre-RoPE keys on the int4 KIVI workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              "(the decode path shards by sequence or KV head with no communication, "
              "so one GPU's throughput is the per-GPU figure)", file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_decode_attention_03_amd import workloads as W
    from quantized_decode_attention_03_amd import _native

    _native.lib()
    if args.copy_probe:
        copy_probe()
        return
    torch.cuda.set_device(0)
    if args.formats:
        runs = format_specs()
        args.no_cpu_baseline = True
    else:
        runs = [(c, None) for c in ([args.config] if args.config else list(DEFAULT_WORKLOADS))]
    results = []
    for key, spec in runs:
        results.append(run_workload(key, args, spec))
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    # headline: the largest workload (the affine int8 one in the format comparison)
    head = results[0] if args.formats else results[-1]
    s = W.spec(runs[-1][0]) if not args.formats else runs[0][1]
    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "append": head["append"],
        "workloads": [{k: r[k] for k in ("workload", "value", "unit", "ms_per_step", "dtype", "roofline",
                                         "append")} for r in results],
    }
    if not args.no_cpu_baseline:
        progress("timing the oracle on the host")
        n_seq = min(args.cpu_seqs, s.batch)
        tps, dt, lens = cpu_baseline(s, n_seq, args.cpu_steps)
        cores, model = host_cpu()
        per_layer = f", one of {s.layers} layers, rate divided by {s.layers}" if s.layers > 1 else ""
        res["cpu_baseline"] = {
            "value": tps / s.layers, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_seq} of {s.batch} sequences (lengths {lens}, the median ones) x "
                      f"{args.cpu_steps} decode steps (append + float64 attention){per_layer}, "
                      f"{dt:.1f} s, numpy BLAS held to 1 thread",
            "host_cores": cores, "host_cpu": model}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
