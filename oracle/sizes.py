"""Cache sizes. Test infrastructure only (see oracle/__init__).

nominal_bytes follows [P2-size]: bytes = 2 * L * n_kv * d_head * S *
bytes_per_elem, the K and V codes alone. actual_bytes adds what the pages say
the nominal figure leaves out (the group scales, [P2-gran] last sentences;
the sparse outlier store, [P1-kivi] table note): one 4-byte scale+zero word
per group, the fp16 residual window and the sparse entries. fp8 E4M3 codes
([P3-fmt]) have no groups and so no metadata: their actual size is the
nominal one. Symmetric 32-element blocks carry one fp16 scale per block
(2 bytes per 32 elements).
"""

BLOCK = 32


def nominal_bytes(layers, n_kv, d_head, seq_len, bits):
    """2 * L * n_kv * d_head * S * bits/8, exact integer arithmetic."""
    return 2 * layers * n_kv * d_head * seq_len * bits // 8


def nominal_bytes_mixed(layers, n_kv, d_head, seq_len, k_bits, v_bits):
    return layers * n_kv * d_head * seq_len * (k_bits + v_bits) // 8


def actual_bytes(cfg, batch, max_tokens):
    """Byte sizes of every array of one layer's cache in the layout of
    include/kvq.h, for a cache of the given capacity."""
    H, D, T = cfg.n_kv_heads, cfg.d_head, max_tokens
    n = batch * H
    fp8_k, fp8_v = cfg.k_fp8, cfg.v_fp8
    blocks = D // BLOCK                           # sym32: one fp16 scale per 32 channels
    out = {
        "k_codes": n * T * D * cfg.k_bits // 8,
        "v_codes": n * T * D * cfg.v_bits // 8,
        "v_meta": 0 if fp8_v else (n * T * blocks * 2 if cfg.v_sym else n * T * 4),
        "seq_len": batch * 4,
    }
    if cfg.per_channel:
        out["k_meta"] = n * (T // BLOCK) * D * 4
        out["k_resid"] = n * cfg.k_residual_tokens * D * 2
        out["k_sparse"] = n * T * 8 if cfg.k_sparse_per_vector else 0
    else:
        out["k_meta"] = 0 if fp8_k else (n * T * blocks * 2 if cfg.k_sym else n * T * 4)
        out["k_resid"] = 0
        out["k_sparse"] = 0
    out["nominal_bytes"] = batch * nominal_bytes_mixed(1, H, D, T, cfg.k_bits, cfg.v_bits)
    out["total_bytes"] = sum(out[k] for k in ("k_codes", "k_meta", "k_resid", "k_sparse",
                                              "v_codes", "v_meta", "seq_len"))
    return out
