"""Low-bit KV-cache quantization and fused-dequant decode attention for MI355X.

The work runs in hand-written HIP kernels (gfx950) behind the C ABI declared in
include/kvq.h; this module is a thin binding with the same entry names
(argument marshalling only). PyTorch supplies device memory and streams.
Importing the package loads nothing; the native library is loaded on first use
and its absence is an error (there is no CPU fallback).
"""
import ctypes

from . import _native as N

__all__ = ["Config", "KVCache", "kvq_cache_sizes", "kvq_workspace_bytes", "kvq_append",
           "kvq_decode_attention", "kvq_decode_attention_noalloc", "kvq_dequantize", "KVQError"]

KVQError = N.KVQError


_FORMATS = {"int": N.KVQ_FORMAT_INT, "fp8": N.KVQ_FORMAT_FP8, "sym32": N.KVQ_FORMAT_SYM32}


class Config:
    """Mirror of kvq_config. k_axis is "token" or "channel"; k_format and
    v_format are "int" (affine codes), "fp8" (E4M3 with the per-cache scales
    k_scale, v_scale) or "sym32" (symmetric 32-channel blocks)."""

    def __init__(self, n_kv_heads, n_q_heads, k_bits, v_bits, k_axis="token",
                 k_group_tokens=0, k_residual_tokens=0, k_sparse_per_vector=0, d_head=128,
                 k_format="int", v_format=None, k_scale=1.0, v_scale=1.0, k_rope=0,
                 rope_theta=10000.0):
        self.d_head = d_head
        self.n_kv_heads = n_kv_heads
        self.n_q_heads = n_q_heads
        self.k_bits = k_bits
        self.v_bits = v_bits
        self.k_axis = k_axis
        self.k_group_tokens = k_group_tokens
        self.k_residual_tokens = k_residual_tokens
        self.k_sparse_per_vector = k_sparse_per_vector
        self.k_format = k_format
        self.v_format = k_format if v_format is None else v_format
        for f in (self.k_format, self.v_format):
            if f not in _FORMATS:
                raise ValueError(f"format {f!r}: expected one of {sorted(_FORMATS)}")
        self.k_scale = k_scale
        self.v_scale = v_scale
        self.k_rope = k_rope          # 1: keys cached before the rotary embedding
        self.rope_theta = rope_theta

    @classmethod
    def from_spec(cls, s):
        return cls(s.n_kv_heads, s.n_q_heads, s.k_bits, s.v_bits, s.k_axis, s.k_group,
                   s.k_residual, s.k_sparse, s.d_head, s.fmt, s.fmt, s.k_scale, s.v_scale,
                   s.k_rope, s.rope_theta)

    def c(self):
        return N.kvq_config(self.d_head, self.n_kv_heads, self.n_q_heads, self.k_bits,
                            self.v_bits,
                            N.KVQ_AXIS_CHANNEL if self.k_axis == "channel" else N.KVQ_AXIS_TOKEN,
                            self.k_group_tokens, self.k_residual_tokens, self.d_head,
                            self.k_sparse_per_vector, _FORMATS[self.k_format],
                            _FORMATS[self.v_format], self.k_scale, self.v_scale, self.k_rope,
                            self.rope_theta)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _check(t, name, dtype, shape=None, device=None):
    """Raise ValueError unless t is a contiguous device tensor of the given
    dtype (and shape and device); the kernels read exactly that many elements
    through the raw pointer."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, the cache is on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def kvq_cache_sizes(cfg, batch, max_tokens):
    out = N.kvq_sizes()
    c = cfg.c()
    N.check(N.lib().kvq_cache_sizes(ctypes.byref(c), batch, max_tokens, ctypes.byref(out)),
            "kvq_cache_sizes")
    return {f: getattr(out, f) for f, _ in N.kvq_sizes._fields_}


def kvq_workspace_bytes(cfg, batch, max_tokens):
    c = cfg.c()
    return int(N.lib().kvq_workspace_bytes(ctypes.byref(c), batch, max_tokens))


class KVCache:
    """One layer's packed cache in caller-owned (torch) device memory, laid out
    as include/kvq.h documents. Buffers start zero-filled."""

    def __init__(self, cfg, batch, max_tokens, device="cuda"):
        import torch
        self.cfg, self.batch, self.max_tokens = cfg, batch, max_tokens
        sz = kvq_cache_sizes(cfg, batch, max_tokens)
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        self.sizes = sz

        def buf(n):
            return torch.zeros(max(int(n), 1), dtype=torch.uint8, device=device) if n else None

        self.k_codes = buf(sz["k_codes"])
        self.k_meta = buf(sz["k_meta"])
        self.k_resid = buf(sz["k_resid"])
        self.k_sparse = buf(sz["k_sparse"])
        self.v_codes = buf(sz["v_codes"])
        self.v_meta = buf(sz["v_meta"])
        self.seq_len = torch.zeros(batch, dtype=torch.int32, device=device)
        self.len_host = (ctypes.c_int32 * batch)()
        self._c = N.kvq_cache(
            batch, max_tokens, _ptr(self.k_codes), _ptr(self.k_meta), _ptr(self.k_resid),
            _ptr(self.k_sparse), _ptr(self.v_codes), _ptr(self.v_meta),
            ctypes.cast(ctypes.c_void_p(self.seq_len.data_ptr()), ctypes.POINTER(ctypes.c_int32)),
            ctypes.cast(self.len_host, ctypes.POINTER(ctypes.c_int32)))
        self._cfg = cfg.c()
        self._n_prev, self._n_arr = None, None   # last host counts passed to kvq_append

    def lengths(self):
        return list(self.len_host)

    _ARRAYS = ("k_codes", "k_meta", "k_resid", "k_sparse", "v_codes", "v_meta", "seq_len")

    def copy_from(self, other):
        """Copy the whole state of another cache of the same shape (device
        buffers and host lengths)."""
        for name in self._ARRAYS:
            a, b = getattr(self, name), getattr(other, name)
            if a is not None:
                a.copy_(b)
        for i in range(self.batch):
            self.len_host[i] = other.len_host[i]

    def state(self):
        """Checkpoint: host copies of every device buffer and the lengths (a
        dict of numpy arrays). Synchronizes with the device."""
        import numpy as np
        out = {name: getattr(self, name).cpu().numpy() for name in self._ARRAYS
               if getattr(self, name) is not None}
        out["len_host"] = np.array(list(self.len_host), np.int32)
        return out

    def load_state(self, st):
        """Resume from state(): every buffer and the lengths are overwritten
        (same configuration and shape required)."""
        import torch
        for name in self._ARRAYS:
            a = getattr(self, name)
            if a is None:
                continue
            src = st[name]
            if tuple(src.shape) != tuple(a.shape) or str(src.dtype) != str(a.dtype).replace("torch.", ""):
                raise ValueError(f"{name}: checkpoint {src.dtype}{tuple(src.shape)} does not fit "
                                 f"{a.dtype}{tuple(a.shape)}")
            a.copy_(torch.from_numpy(src))
        if len(st["len_host"]) != self.batch:
            raise ValueError("len_host: wrong batch")
        for i in range(self.batch):
            self.len_host[i] = int(st["len_host"][i])


def kvq_append(cache, k_new, v_new, cu_new, n_new, stream=None):
    """k_new, v_new: fp16 device tensors [N, H, D], N = sum(n_new), the new
    tokens of all sequences back to back; cu_new: int32 device tensor [B+1]
    of their prefix offsets (None: built here from n_new); n_new: host
    sequence of B ints."""
    import torch
    n_list = n_new if type(n_new) is list else [int(x) for x in n_new]
    if len(n_list) != cache.batch:
        raise ValueError(f"n_new: {len(n_list)} counts for a batch of {cache.batch}")
    if cache.batch and min(n_list) < 0:
        raise ValueError("n_new: negative count")
    cfg, dev = cache.cfg, cache.device
    rows = (sum(n_list), cfg.n_kv_heads, cfg.d_head)
    _check(k_new, "k_new", torch.float16, rows, dev)
    _check(v_new, "v_new", torch.float16, rows, dev)
    if cu_new is None:
        cu = [0]
        for x in n_list:
            cu.append(cu[-1] + x)
        cu_new = torch.tensor(cu, dtype=torch.int32, device=dev)
    _check(cu_new, "cu_new", torch.int32, (cache.batch + 1,), dev)
    # the host counts as a C array, kept while they repeat (every decode step)
    if n_list != cache._n_prev:
        cache._n_arr = (ctypes.c_int32 * cache.batch)(*n_list)
        cache._n_prev = list(n_list)
    N.check(N.lib().kvq_append(ctypes.byref(cache._cfg), ctypes.byref(cache._c), _ptr(k_new), _ptr(v_new),
                               _ptr(cu_new), cache._n_arr, _stream(stream)), "kvq_append")


def kvq_decode_attention(cache, q, out, softmax_scale, ws, stream=None):
    """q: fp16 [B, Hq, D]; out: fp32 [B, Hq, D]; ws: contiguous device
    buffer of at least kvq_workspace_bytes bytes (any dtype)."""
    import torch
    cfg, dev = cache.cfg, cache.device
    _check(q, "q", torch.float16, (cache.batch, cfg.n_q_heads, cfg.d_head), dev)
    _check(out, "out", torch.float32, (cache.batch, cfg.n_q_heads, cfg.d_head), dev)
    _check(ws, "ws", ws.dtype if isinstance(ws, torch.Tensor) else None, None, dev)
    N.check(N.lib().kvq_decode_attention(ctypes.byref(cache._cfg), ctypes.byref(cache._c),
                                         _ptr(q), _ptr(out), ctypes.c_float(softmax_scale),
                                         _ptr(ws), ctypes.c_size_t(ws.numel() * ws.element_size()),
                                         _stream(stream)), "kvq_decode_attention")


def kvq_decode_attention_noalloc(cache, q, out, softmax_scale, stream=None):
    """kvq_decode_attention with the library's own device scratch instead of
    a caller workspace (no allocation in the call). q: fp16 [B, Hq, D];
    out: fp32 [B, Hq, D]."""
    import torch
    cfg, dev = cache.cfg, cache.device
    _check(q, "q", torch.float16, (cache.batch, cfg.n_q_heads, cfg.d_head), dev)
    _check(out, "out", torch.float32, (cache.batch, cfg.n_q_heads, cfg.d_head), dev)
    N.check(N.lib().kvq_decode_attention_noalloc(ctypes.byref(cache._cfg), ctypes.byref(cache._c),
                                                 _ptr(q), _ptr(out), ctypes.c_float(softmax_scale),
                                                 _stream(stream)), "kvq_decode_attention_noalloc")


def kvq_dequantize(cache, k_out, v_out, stream=None):
    """k_out, v_out: fp16 device tensors [B, T, H, D]."""
    import torch
    cfg, dev = cache.cfg, cache.device
    shape = (cache.batch, cache.max_tokens, cfg.n_kv_heads, cfg.d_head)
    _check(k_out, "k_out", torch.float16, shape, dev)
    _check(v_out, "v_out", torch.float16, shape, dev)
    N.check(N.lib().kvq_dequantize(ctypes.byref(cache._cfg), ctypes.byref(cache._c), _ptr(k_out),
                                   _ptr(v_out), _stream(stream)), "kvq_dequantize")
