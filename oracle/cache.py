"""Reference KV cache: append with residual flush, packed layout, dequantized
tensors and float64 decode attention. Test infrastructure only (see
oracle/__init__).

State per sequence b (identical for every KV head): L = tokens held.
  * Values are quantized per token on append ([P2-gran]; [P1-kivi]).
  * Per-token keys are quantized on append the same way.
  * Per-channel keys ([P1-kivi]: keys per channel, with a small full-precision
    residual for the most recent tokens). Reading: keys enter an fp16 residual
    window of R slots; when it holds R keys, all R are quantized as R/32
    groups of 32 consecutive tokens per channel and the window empties. So
    Q = L - (L mod R) keys are quantized and L mod R are fp16. A bulk append
    of n keys reaches the same state as n single appends (pinned by a test).
  * Dense-and-sparse keys ([P1-kivi], KVQuant): each key vector being quantized
    first gives up its k largest-|x| entries (quant.split_sparse); residual
    keys are never split.

  * fp8 E4M3 keys and values (oracle/fp8.py, [P3-fmt]): one code per element
    with one fp32 scale per cache for keys and one for values; no groups, so
    no metadata arrays. fp8 keys are on the token axis.
  * Symmetric 32-element blocks ("sym32"; [P2-int] "Symmetric vs asymmetric",
    [P3-fmt]'s q8_0 / q4_0 blocks of 32 elements sharing a scale): each token
    vector is cut into 4 blocks of 32 consecutive channels, each quantized
    symmetrically (quant.quantize_sym_groups) with one fp16 scale. Keys on the
    token axis.

Logical arrays (host numpy): codes q as int8 per element (fp8: the uint8
codes), scales and zeros as fp16 per group, residual keys as fp16, sparse
entries as (channel, fp16). ``pack()`` turns them into the byte layout that
include/kvq.h documents.
"""
import numpy as np

from . import fp8, quant, rope

F16 = np.float16
BLOCK = 32  # tokens per per-channel key group and per value code block


class Config:
    """Same fields as the C struct kvq_config."""

    def __init__(self, d_head=128, n_kv_heads=1, n_q_heads=1, k_bits=8, v_bits=8,
                 k_axis="token", k_group_tokens=0, k_residual_tokens=0,
                 k_sparse_per_vector=0, k_format="int", v_format="int",
                 k_scale=1.0, v_scale=1.0, k_rope=0, rope_theta=10000.0):
        self.d_head = d_head
        self.n_kv_heads = n_kv_heads
        self.n_q_heads = n_q_heads
        self.k_bits = k_bits
        self.v_bits = v_bits
        self.k_axis = k_axis
        self.k_group_tokens = k_group_tokens
        self.k_residual_tokens = k_residual_tokens
        self.k_sparse_per_vector = k_sparse_per_vector
        self.k_format = k_format          # "int" (affine codes), "fp8" (E4M3) or
                                          # "sym32" (symmetric 32-channel blocks)
        self.v_format = v_format
        self.k_scale = k_scale            # fp8 only: the per-cache fp32 scales
        self.v_scale = v_scale
        self.k_rope = k_rope              # 1: keys cached before the rotary embedding,
        self.rope_theta = rope_theta      # which attention applies (oracle/rope.py)

    @property
    def per_channel(self):
        return self.k_axis == "channel"

    @property
    def k_fp8(self):
        return self.k_format == "fp8"

    @property
    def v_fp8(self):
        return self.v_format == "fp8"

    @property
    def k_sym(self):
        return self.k_format == "sym32"

    @property
    def v_sym(self):
        return self.v_format == "sym32"


class RefCache:
    def __init__(self, cfg, batch, max_tokens):
        assert max_tokens % BLOCK == 0
        if cfg.per_channel:
            assert cfg.k_group_tokens == BLOCK
            assert cfg.k_residual_tokens > 0 and cfg.k_residual_tokens % BLOCK == 0
            assert not cfg.k_fp8 and not cfg.k_sym, "fp8 and block keys are on the token axis"
        for f, bits in ((cfg.k_format, cfg.k_bits), (cfg.v_format, cfg.v_bits)):
            assert f in ("int", "fp8", "sym32") and (f != "fp8" or bits == 8)
        self.cfg = cfg
        self.B, self.T = batch, max_tokens
        H, D = cfg.n_kv_heads, cfg.d_head
        self.H, self.D = H, D
        self.length = np.zeros(batch, np.int64)
        self.kq = np.zeros((batch, H, max_tokens, D), np.uint8 if cfg.k_fp8 else np.int8)
        if cfg.per_channel:
            nb = max_tokens // BLOCK
            self.ks = np.zeros((batch, H, nb, D), F16)
            self.kz = np.zeros((batch, H, nb, D), F16)
            self.kres = np.zeros((batch, H, cfg.k_residual_tokens, D), F16)
        elif cfg.k_sym:
            self.ks = np.zeros((batch, H, max_tokens, D // SYM_BLOCK), F16)
            self.kz = None
            self.kres = None
        else:
            self.ks = np.zeros((batch, H, max_tokens), F16)
            self.kz = np.zeros((batch, H, max_tokens), F16)
            self.kres = None
        ksp = cfg.k_sparse_per_vector
        self.sp_col = np.zeros((batch, H, max_tokens, ksp), np.int64)
        self.sp_val = np.zeros((batch, H, max_tokens, ksp), F16)
        self.vq = np.zeros((batch, H, max_tokens, D), np.uint8 if cfg.v_fp8 else np.int8)
        if cfg.v_sym:
            self.vs = np.zeros((batch, H, max_tokens, D // SYM_BLOCK), F16)
            self.vz = None
        else:
            self.vs = np.zeros((batch, H, max_tokens), F16)
            self.vz = np.zeros((batch, H, max_tokens), F16)

    # ------------------------------------------------------------------ state
    def n_quantized(self, b):
        """Keys held as codes: all of them (token axis) or L - L mod R."""
        L = int(self.length[b])
        if not self.cfg.per_channel:
            return L
        return L - L % self.cfg.k_residual_tokens

    def append(self, k_new, v_new, n_new):
        """k_new, v_new: fp16 [N, H, D] packed back to back by sequence;
        n_new[b] rows belong to sequence b."""
        cfg = self.cfg
        k_new = np.asarray(k_new, F16)
        v_new = np.asarray(v_new, F16)
        off = 0
        for b in range(self.B):
            n = int(n_new[b])
            kb = k_new[off:off + n].transpose(1, 0, 2)   # [H, n, D]
            vb = v_new[off:off + n].transpose(1, 0, 2)
            off += n
            L = int(self.length[b])
            if L + n > self.T:
                raise ValueError("capacity")
            if n == 0:
                continue
            # values: one group per (head, token) over the D channels; fp8:
            # one code per element
            if cfg.v_fp8:
                self.vq[b, :, L:L + n] = fp8.quantize(vb, cfg.v_scale)
            elif cfg.v_sym:
                self.vq[b, :, L:L + n], self.vs[b, :, L:L + n] = _sym_blocks(vb, cfg.v_bits)
            else:
                q, s, z = quant.quantize_groups(vb, cfg.v_bits)
                self.vq[b, :, L:L + n] = q
                self.vs[b, :, L:L + n] = s
                self.vz[b, :, L:L + n] = z
            if cfg.k_fp8:
                self.kq[b, :, L:L + n] = fp8.quantize(kb, cfg.k_scale)
            elif cfg.k_sym:
                self.kq[b, :, L:L + n], self.ks[b, :, L:L + n] = _sym_blocks(kb, cfg.k_bits)
            elif not cfg.per_channel:
                q, s, z = quant.quantize_groups(kb, cfg.k_bits)
                self.kq[b, :, L:L + n] = q
                self.ks[b, :, L:L + n] = s
                self.kz[b, :, L:L + n] = z
            else:
                self._append_channel_keys(b, L, kb)
            self.length[b] = L + n

    def _append_channel_keys(self, b, L, kb):
        R = self.cfg.k_residual_tokens
        n = kb.shape[1]
        Q = L - L % R
        L2 = L + n
        Q2 = L2 - L2 % R
        if Q2 == Q:                       # window not full: keys wait in fp16
            self.kres[b, :, L - Q:L - Q + n] = kb
            return
        # the window fills: old residual keys, then new keys, up to token Q2
        window = np.concatenate([self.kres[b, :, :L - Q], kb[:, :Q2 - L]], axis=1)
        W = Q2 - Q
        ksp = self.cfg.k_sparse_per_vector
        if ksp:
            dense, cols, vals = quant.split_sparse(window, ksp)
            self.sp_col[b, :, Q:Q2] = cols
            self.sp_val[b, :, Q:Q2] = vals
            window = dense
        # groups: (head, 32-token block, channel), 32 tokens each
        g = window.reshape(self.H, W // BLOCK, BLOCK, self.D).transpose(0, 1, 3, 2)
        q, s, z = quant.quantize_groups(g, self.cfg.k_bits)   # q [H, nb, D, 32]
        self.kq[b, :, Q:Q2] = q.transpose(0, 1, 3, 2).reshape(self.H, W, self.D)
        self.ks[b, :, Q // BLOCK:Q2 // BLOCK] = s
        self.kz[b, :, Q // BLOCK:Q2 // BLOCK] = z
        self.kres[b, :, :L2 - Q2] = kb[:, Q2 - L:]

    # ------------------------------------------------------- dequantized views
    def k_hat(self, b, h, dtype=np.float64):
        """Dequantized keys of (sequence b, KV head h), [L, D]: codes through
        x_hat = s*(q - z), plus the sparse entries added back, then the fp16
        residual keys verbatim."""
        L, Q = int(self.length[b]), self.n_quantized(b)
        if self.cfg.k_fp8:
            return _fp8_hat(self.kq[b, h, :L], self.cfg.k_scale, dtype)
        if self.cfg.k_sym:
            return _sym_hat(self.kq[b, h, :L], self.ks[b, h, :L], dtype)
        deq = quant.dequantize_f64 if dtype == np.float64 else quant.dequantize
        if self.cfg.per_channel:
            blk = np.arange(Q) // BLOCK
            kh = deq(self.kq[b, h, :Q], self.ks[b, h, blk], self.kz[b, h, blk])
            if self.cfg.k_sparse_per_vector:
                rows = np.arange(Q)[:, None]
                np.add.at(kh, (rows, self.sp_col[b, h, :Q]),
                          self.sp_val[b, h, :Q].astype(kh.dtype))
            res = self.kres[b, h, :L - Q].astype(kh.dtype)
            return np.concatenate([kh, res], axis=0)
        return deq(self.kq[b, h, :L], self.ks[b, h, :L, None], self.kz[b, h, :L, None])

    def v_hat(self, b, h, dtype=np.float64):
        L = int(self.length[b])
        if self.cfg.v_fp8:
            return _fp8_hat(self.vq[b, h, :L], self.cfg.v_scale, dtype)
        if self.cfg.v_sym:
            return _sym_hat(self.vq[b, h, :L], self.vs[b, h, :L], dtype)
        deq = quant.dequantize_f64 if dtype == np.float64 else quant.dequantize
        return deq(self.vq[b, h, :L], self.vs[b, h, :L, None], self.vz[b, h, :L, None])

    def dequantize_f16(self):
        """What kvq_dequantize writes: fp16 [B, T, H, D], RNE of the exact fp32
        reconstruction; slots past the sequence end are +0."""
        k = np.zeros((self.B, self.T, self.H, self.D), F16)
        v = np.zeros_like(k)
        for b in range(self.B):
            L = int(self.length[b])
            for h in range(self.H):
                k[b, :L, h] = self.k_hat(b, h, np.float32).astype(F16)
                v[b, :L, h] = self.v_hat(b, h, np.float32).astype(F16)
        return k, v

    # ----------------------------------------------------------- attention
    def attention(self, q16, softmax_scale, pairs=None):
        """Decode attention in float64 ([P2-dec]; the plain definition
        out = softmax(scale * q . K_hat) V_hat over every held token; with
        k_rope, K_hat rotated by each key's position first, the query taken as
        already rotated).

        q16: fp16 [B, Hq, D]. Returns float64 [B, Hq, D]. Query head h reads
        KV head h // (Hq/H). pairs: optional iterable of (b, kv_head) to
        compute (the rest stays 0). A sequence with no tokens gives 0.
        """
        Hq = q16.shape[1]
        grp = Hq // self.H
        out = np.zeros(q16.shape, np.float64)
        scale = float(np.float32(softmax_scale))
        todo = pairs if pairs is not None else [(b, h) for b in range(self.B) for h in range(self.H)]
        for b, h in todo:
            if self.length[b] == 0:
                continue
            K = self.k_hat(b, h)
            if self.cfg.k_rope:           # pre-RoPE keys: rotate by position after dequantization
                K = rope.rope(K, np.arange(K.shape[0]), self.cfg.rope_theta)
            V = self.v_hat(b, h)
            for hq in range(h * grp, (h + 1) * grp):
                qv = q16[b, hq].astype(np.float64)
                sc = scale * (K @ qv)
                p = np.exp(sc - sc.max())
                out[b, hq] = (p @ V) / p.sum()
        return out

    # ------------------------------------------------------------- packing
    def pack(self):
        """Byte arrays in the layout of include/kvq.h (the library's own format;
        not fixed by the pages)."""
        cfg = self.cfg
        B, H, T, D = self.B, self.H, self.T, self.D
        # stored code = q - q_min for integer codes, the code itself for fp8
        kqmin = 0 if cfg.k_fp8 else quant.qrange(cfg.k_bits)[0]
        vqmin = 0 if cfg.v_fp8 else quant.qrange(cfg.v_bits)[0]
        # stored unsigned codes; token slots without a code stay 0
        ku = np.zeros((B, H, T, D), np.uint8)
        vu = np.zeros((B, H, T, D), np.uint8)
        kmeta_len = []
        for b in range(B):
            Q, L = self.n_quantized(b), int(self.length[b])
            ku[b, :, :Q] = (self.kq[b, :, :Q].astype(np.int16) - kqmin).astype(np.uint8)
            vu[b, :, :L] = (self.vq[b, :, :L].astype(np.int16) - vqmin).astype(np.uint8)
            kmeta_len.append(Q)
        out = {}
        out["k_codes"] = pack_fields(ku, cfg.k_bits)                       # [B,H,T,D*kb/8]
        vblk = vu.reshape(B, H, T // BLOCK, BLOCK, D).transpose(0, 1, 2, 4, 3)
        out["v_codes"] = pack_fields(vblk, cfg.v_bits)                     # [B,H,T/32,D,4*vb]
        if cfg.v_sym:
            out["v_meta"] = quant.f16_bits(self.vs)                        # [B,H,T,4] scales
        elif not cfg.v_fp8:
            out["v_meta"] = meta_words(self.vs, self.vz)
        if cfg.per_channel:
            out["k_meta"] = meta_words(self.ks, self.kz)                   # [B,H,T/32,D]
            out["k_resid"] = quant.f16_bits(self.kres)
            if cfg.k_sparse_per_vector:
                assert cfg.k_sparse_per_vector == 2
                sp = np.zeros((B, H, T, 2), np.uint32)
                vb = quant.f16_bits(self.sp_val).astype(np.uint32)
                cb = self.sp_col.astype(np.uint32)
                sp[..., 0] = vb[..., 0] | (vb[..., 1] << 16)
                sp[..., 1] = cb[..., 0] | (cb[..., 1] << 16)
                for b in range(B):
                    sp[b, :, kmeta_len[b]:] = 0
                out["k_sparse"] = sp
        elif cfg.k_sym:
            out["k_meta"] = quant.f16_bits(self.ks)                        # [B,H,T,4] scales
        elif not cfg.k_fp8:
            out["k_meta"] = meta_words(self.ks, self.kz)                   # [B,H,T]
        return out


SYM_BLOCK = 32  # channels per symmetric block


def _sym_blocks(x16, bits):
    """x16 fp16 [H, n, D] -> (codes int8 [H, n, D], scales fp16 [H, n, D/32]):
    each token vector cut into blocks of 32 consecutive channels."""
    H, n, D = x16.shape
    q, s = quant.quantize_sym_groups(x16.reshape(H, n, D // SYM_BLOCK, SYM_BLOCK), bits)
    return q.reshape(H, n, D), s


def _sym_hat(q, s16, dtype):
    """scale of each element's block * code, [L, D]; exact in float64 and in
    float32."""
    L, D = q.shape
    s = np.repeat(np.asarray(s16, F16).astype(dtype), SYM_BLOCK, axis=-1)
    return s * np.asarray(q).astype(dtype)


def _fp8_hat(codes, scale, dtype):
    """scale * value(code): exact in float64; in float32 the product rounded
    once (the value kvq_dequantize rounds to fp16)."""
    if dtype == np.float64:
        return fp8.dequantize_f64(codes, scale)
    return np.float32(scale) * fp8.e4m3_value(codes).astype(np.float32)


def pack_fields(u, bits):
    """Pack unsigned b-bit fields along the last axis, little-endian within
    each byte: element i goes to bits [(i*b) mod 8, +b) of byte (i*b)//8."""
    u = np.asarray(u, np.uint8)
    per = 8 // bits
    n = u.shape[-1]
    assert n % per == 0
    f = u.reshape(u.shape[:-1] + (n // per, per)).astype(np.uint32)
    byte = np.zeros(f.shape[:-1], np.uint32)
    for i in range(per):
        byte |= (f[..., i] & ((1 << bits) - 1)) << (i * bits)
    return byte.astype(np.uint8)


def unpack_fields(packed, bits):
    """Inverse of pack_fields."""
    p = np.asarray(packed, np.uint8).astype(np.uint32)
    per = 8 // bits
    parts = [(p >> (i * bits)) & ((1 << bits) - 1) for i in range(per)]
    return np.stack(parts, axis=-1).reshape(p.shape[:-1] + (p.shape[-1] * per,)).astype(np.uint8)


def meta_words(s16, z16):
    """uint32 word per group: fp16 scale bits | fp16 zero bits << 16."""
    return (quant.f16_bits(s16).astype(np.uint32)
            | (quant.f16_bits(z16).astype(np.uint32) << 16))


# ------------------------------------------------------- split-K merge
def softmax_partial(sc, V):
    """Softmax state of one token range (float64): m = the range's largest
    score, l = sum exp(s - m), o = sum exp(s - m) * V_t. An empty range has
    m = -inf, l = 0, o = 0. This is the state a split of the sequence hands to
    the merge; the merge step is not on the pages (it is how a decode kernel
    that splits a long sequence over several workgroups finishes), so it is
    pinned only by its closed form: merging the partials of any split of the
    tokens gives exactly the unsplit softmax result."""
    sc = np.asarray(sc, np.float64)
    V = np.asarray(V, np.float64)
    if sc.size == 0:
        return -np.inf, 0.0, np.zeros(V.shape[-1], np.float64)
    m = float(sc.max())
    p = np.exp(sc - m)
    return m, float(p.sum()), p @ V


def merge_partials(parts):
    """Log-sum-exp merge of split partials: M = max m_i,
    l = sum exp(m_i - M) l_i, o = sum exp(m_i - M) o_i, output o / l
    (0 when every range is empty)."""
    ms = [m for m, _, _ in parts]
    M = max(ms)
    if M == -np.inf:
        return np.zeros_like(parts[0][2])
    l = sum(np.exp(m - M) * li for m, li, _ in parts if m != -np.inf)
    o = sum(np.exp(m - M) * oi for m, _, oi in parts if m != -np.inf)
    return o / l
