"""Pins of the oracle's size formulas against the pages' printed arithmetic."""
import json
import os

from oracle import sizes
from oracle.cache import Config

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "sizes_worked_example.json")) as f:
        return json.load(f)


def test_worked_example():
    g = _gold()["worked_example"]
    L, H, D, S = g["layers"], g["n_kv"], g["d_head"], g["seq_len"]
    assert 2 * L * H * D == g["elements_per_token"]
    assert sizes.nominal_bytes(L, H, D, 1, 16) == g["fp16_bytes_per_token"]
    assert sizes.nominal_bytes(L, H, D, S, 16) == g["fp16_bytes_sequence"]
    assert sizes.nominal_bytes(L, H, D, S, 8) == g["int8_bytes_sequence"]
    assert sizes.nominal_bytes(L, H, D, S, 4) == g["int4_bytes_sequence"]
    # the page's rounded decimal figures
    for key, bits in (("fp16_GB", 16), ("int8_GB", 8), ("int4_GB", 4)):
        gb = sizes.nominal_bytes(L, H, D, S, bits) / 1e9
        assert round(gb, 1) == g["printed"][key]


def test_precision_table_halves():
    t = _gold()["kv_precision_table"]
    # an architecture with 160 KiB of fp16 KV per token: 2*L*n_kv*d = 81920
    L, H, D = 40, 8, 128
    assert sizes.nominal_bytes(L, H, D, 1, 16) == t["fp16_KiB_per_token"] * 1024
    for row in t["rows"]:
        per_tok = sizes.nominal_bytes(L, H, D, 1, row["bits"])
        assert per_tok == row["KiB"] * 1024
        turn = sizes.nominal_bytes(L, H, D, t["turn_tokens"], row["bits"]) / 2 ** 30
        assert round(turn, 2) == row["GiB_turn"]


def test_context_64k():
    c = _gold()["context_64k"]
    assert c["fp16_KiB_per_token"] * 1024 * c["tokens"] / 2 ** 30 == c["fp16_GiB"]


def test_actual_bytes_per_token_head():
    # KIVI int4, G=32: K 64 B codes + 16 B per-channel meta, V 64 B + 4 B
    cfg = Config(128, 8, 32, 4, 4, "channel", 32, 32, 0)
    a = sizes.actual_bytes(cfg, 1, 4096)
    per = (a["k_codes"] + a["k_meta"] + a["v_codes"] + a["v_meta"]) / (8 * 4096)
    assert per == 148
    # int8 per-token K and V: 128 + 4 twice
    cfg8 = Config(128, 8, 32, 8, 8, "token")
    a8 = sizes.actual_bytes(cfg8, 1, 4096)
    assert (a8["k_codes"] + a8["k_meta"] + a8["v_codes"] + a8["v_meta"]) / (8 * 4096) == 264
    # int2 KIVI: 32 + 16 and 32 + 4
    cfg2 = Config(128, 8, 32, 2, 2, "channel", 32, 128, 0)
    a2 = sizes.actual_bytes(cfg2, 1, 4096)
    assert (a2["k_codes"] + a2["k_meta"] + a2["v_codes"] + a2["v_meta"]) / (8 * 4096) == 84
    # nominal = codes only
    assert a["nominal_bytes"] == a["k_codes"] + a["v_codes"]
