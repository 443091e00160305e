"""A CPU replica of the attention kernel's work split and load addressing,
run on every workload's full shape (and the element-format variants) for
several workgroup counts, without a GPU.

It follows the kernel step by step: workgroup i of n takes units
[i U / n, (i+1) U / n) of the 32-token tiles of all (sequence, KV head)
pairs; it walks the pairs' segments; each of its four wavefronts takes every
fourth tile of a segment and loads, per tile, the key codes, the value block
and the metadata pieces straight into its LDS slots through a buffer
descriptor over the pair's slice of each cache array; the pair's last segment
also loads the fp16 residual key tiles. For every load the replica checks that
the bytes read lie inside the tile (or residual tile) being processed and
inside the descriptor's range, and that every descriptor's range lies inside
its cache array as kvq_cache_sizes sizes it. It then checks the coverage: every
quantized tile of every pair is processed exactly once, residual keys exactly
once, empty sequences never; and the partial-result protocol: pieces of a
pair that spans several workgroups land in distinct workspace slots, which are
exactly the slots the merge kernel reads back (the workgroup's first segment
in slot 2i, its last in slot 2i + 1).
"""
import math
from dataclasses import replace

import pytest

from oracle.sizes import actual_bytes
from harness import ref_config
from quantized_decode_attention_03_amd import workloads as W

D = 128
BLOCK = 32


def units_of(s, L):
    Q = L - L % s.k_residual if s.k_axis == "channel" else L
    return (Q + BLOCK - 1) // BLOCK if Q > 0 else (1 if L > 0 else 0)


def geometry(s):
    """Per-tile byte sizes of the loads (the kernel's tile geometry)."""
    meta_tok = {"int": 4, "sym32": 8, "fp8": 0}[s.fmt]
    g = dict(row_k=16 * s.k_bits, v=512 * s.v_bits, meta_tok=meta_tok, vm=32 * meta_tok,
             km=512 if s.k_axis == "channel" else 32 * meta_tok, sp=256 if s.k_sparse else 0)
    g["k"] = 32 * g["row_k"]
    return g


def wg_of_unit(u, U, n):
    return ((u + 1) * n + U - 1) // U - 1


def walk(s, lens, n):
    """Segments of every workgroup, as the kernel walks them:
    (wg, b, h, k0, k1, first_segment)."""
    H = s.n_kv_heads
    units = [H * units_of(s, L) for L in lens]
    U = sum(units)
    cum = [0]
    for x in units:
        cum.append(cum[-1] + x)
    segs = []
    for i in range(n):
        u, u1 = i * U // n, (i + 1) * U // n
        # locate_unit: the first sequence whose units reach past u
        b = next((bb for bb in range(len(lens)) if u < cum[bb + 1]), len(lens))
        base = cum[b] if b < len(lens) else U
        first = True
        while u < u1 and b < len(lens):
            nt = units_of(s, lens[b])
            rel = u - base
            h, k0 = rel // nt, rel % nt
            k1 = min(nt, k0 + (u1 - u))
            segs.append((i, b, h, k0, k1, first))
            first = False
            u += k1 - k0
            if k1 == nt and h == H - 1:
                base += H * nt
                b += 1
                while b < len(lens) and lens[b] == 0:
                    b += 1
    return segs, U


def check(s, lens, T, n):
    H, G = s.n_kv_heads, s.group
    g = geometry(s)
    sizes = actual_bytes(ref_config(s), s.batch, T)
    # descriptor ranges: the pair's slice of each array
    rng = {"k": T * g["row_k"], "v": (T // BLOCK) * g["v"], "vm": T * g["meta_tok"],
           "km": (T // BLOCK) * D * 4 if s.k_axis == "channel" else T * g["meta_tok"],
           "sp": T * 8, "res": s.k_residual * D * 2}
    arrays = {"k": "k_codes", "v": "v_codes", "vm": "v_meta", "km": "k_meta", "sp": "k_sparse",
              "res": "k_resid"}
    for key, arr in arrays.items():
        if sizes[arr]:
            assert H * s.batch * rng[key] == sizes[arr], (key, arr)

    segs, U = walk(s, lens, n)
    assert sum(k1 - k0 for _, _, _, k0, k1, _ in segs) == U      # every unit exactly once
    done = {}                                                    # (b, h) -> tiles seen
    res_done = {}
    written = {}                                                 # workspace slot -> (b, h)
    for i, b, h, k0, k1, first in segs:
        L = lens[b]
        Q = L - L % s.k_residual if s.k_axis == "channel" else L
        nt = units_of(s, L)
        assert L > 0 and 0 <= k0 < k1 <= nt
        ts0, ts1 = min(k0 * BLOCK, Q), min(k1 * BLOCK, Q)
        ntiles = (ts1 - ts0 + BLOCK - 1) // BLOCK
        for w in range(4):
            nw = (ntiles - w + 3) // 4 if w < ntiles else 0
            for t in range(nw):
                tw = ts0 + (w + 4 * t) * BLOCK
                assert tw % BLOCK == 0 and ts0 <= tw < ts1 and tw + BLOCK <= T
                done.setdefault((b, h), []).append(tw)
                # key codes: tw * row + lane * 16 + x * 1024, lane < 64, x < k / 1024
                lo, hi = tw * g["row_k"], tw * g["row_k"] + 63 * 16 + (g["k"] // 1024 - 1) * 1024 + 16
                assert lo >= 0 and hi == (tw + BLOCK) * g["row_k"] <= rng["k"]
                # value block of the tile
                lo, hi = (tw // BLOCK) * g["v"], (tw // BLOCK) * g["v"] + 63 * 16 + (g["v"] // 1024 - 1) * 1024 + 16
                assert hi == (tw // BLOCK + 1) * g["v"] <= rng["v"]
                # value metadata: lanes 0 .. vm/16 - 1
                if g["vm"]:
                    hi = tw * g["meta_tok"] + (g["vm"] // 16 - 1) * 16 + 16
                    assert hi == (tw + BLOCK) * g["meta_tok"] <= rng["vm"]
                # key metadata: the next km/16 lanes
                if g["km"]:
                    if s.k_axis == "channel":
                        lo = (tw // BLOCK) * D * 4
                        hi = lo + (g["km"] // 16 - 1) * 16 + 16
                        assert hi == lo + D * 4 <= rng["km"]
                    else:
                        hi = tw * g["meta_tok"] + (g["km"] // 16 - 1) * 16 + 16
                        assert hi == (tw + BLOCK) * g["meta_tok"] <= rng["km"]
                if g["sp"]:
                    hi = tw * 8 + (g["sp"] // 16 - 1) * 16 + 16
                    assert hi == (tw + BLOCK) * 8 <= rng["sp"]
        if k1 == nt and L > Q:                                   # residual keys with the last unit
            nres = (L - Q + BLOCK - 1) // BLOCK
            for jr in range(nres):
                t0 = Q + jr * BLOCK
                assert t0 + BLOCK <= T
                # residual rows t0 - Q + (0..31): 256 B each
                assert (t0 - Q + BLOCK) * D * 2 <= rng["res"]
                assert (t0 // BLOCK + 1) * g["v"] <= rng["v"] and (t0 + BLOCK) * 4 <= rng["vm"]
                res_done[(b, h)] = res_done.get((b, h), 0) + 1
        if not (k0 == 0 and k1 == nt):                           # a piece: a partial slot
            slot = 2 * i + (0 if first else 1)
            assert slot not in written, ("slot written twice", slot)
            written[slot] = (b, h)

    for b, L in enumerate(lens):
        Q = L - L % s.k_residual if s.k_axis == "channel" else L
        for h in range(H):
            tiles = sorted(done.get((b, h), []))
            assert tiles == list(range(0, Q, BLOCK)), (b, h)
            assert res_done.get((b, h), 0) == ((L - Q + BLOCK - 1) // BLOCK if L > Q else 0)

    # the merge kernel's view: slots of each pair that spans workgroups
    H_units = [H * units_of(s, L) for L in lens]
    read = {}
    for b, L in enumerate(lens):
        if L == 0:
            continue
        nt = units_of(s, L)
        for h in range(H):
            s0 = sum(H_units[:b]) + h * nt
            first, last = wg_of_unit(s0, U, n), wg_of_unit(s0 + nt - 1, U, n)
            if last == first:
                continue
            mid_start = s0 != first * U // n
            for j in range(last - first + 1):
                slot = 2 * (first + j) + (1 if (j == 0 and mid_start) else 0)
                read[slot] = (b, h)
    assert read == written


CASES = [(c, None) for c in (1, 2, 3, 4, 5)] + [
    (3, dict(fmt="fp8")), (3, dict(fmt="sym32")), (3, dict(fmt="sym32", k_bits=4, v_bits=2)),
    (2, dict(k_bits=8, v_bits=2))]


@pytest.mark.parametrize("cid,kw", CASES)
def test_dma_addresses_and_coverage(cid, kw):
    s = W.spec(cid, **(kw or {}))
    s = replace(s, layers=1)
    lens = [int(x) + 1 for x in W.seq_lengths(s)]          # after one decode step
    T = s.max_tokens(64)
    U = s.n_kv_heads * sum(units_of(s, L) for L in lens)
    for n in sorted({1, 3, 7, 512, 1024, min(2048, max(1, U // 8)), min(U, 2048)}):
        if n <= U:
            check(s, lens, T, n)


def test_ragged_with_empty_and_residual_only_sequences():
    s = W.spec(2, batch=6, seq_len=200, min_len=1)
    lens = [0, 31, 32, 0, 200, 65]                         # empty, residual only (R = 32), full
    T = 256
    U = s.n_kv_heads * sum(units_of(s, L) for L in lens)
    for n in range(1, U + 1, 3):
        check(s, lens, T, n)
