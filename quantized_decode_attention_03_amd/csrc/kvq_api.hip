// C-ABI entry points of the kvq library: argument validation on the host,
// then kernel launches on the caller's stream. No allocation, no
// synchronization (except under KVQ_DEBUG=1, which also prints HIP errors),
// no state kept between calls beyond per-device constants read once (compute
// units, resident attention workgroups per compute unit).
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <cmath>

#include "kvq.h"
#include "kvq_internal.h"

using namespace kvq;

namespace {

bool debug_sync() {
  static const int on = [] {
    const char* e = getenv("KVQ_DEBUG");
    return (e && e[0] == '1') ? 1 : 0;
  }();
  return on != 0;
}

kvq_status hip_failed(hipError_t e, const char* where) {
  if (debug_sync()) fprintf(stderr, "kvq: %s: %s\n", where, hipGetErrorString(e));
  return KVQ_EHIP;
}

kvq_status after_launch(hipError_t e, hipStream_t st) {
  if (e != hipSuccess) return hip_failed(e, "launch");
  if (debug_sync()) {
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return hip_failed(e, "stream synchronize");
    if ((e = hipGetLastError()) != hipSuccess) return hip_failed(e, "after synchronize");
  }
  return KVQ_OK;
}

bool bits_ok(int b) { return b == 2 || b == 4 || b == 8; }

// Compute units of the current device (read once per device; 256 if the
// query fails).
int compute_units() {
  static std::atomic<int> cache[64];  // 0 = not read yet; threads may race to fill it
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Attention work plan from the host's lengths (the appends keep them equal
// to the device's): U = 32-token tiles of quantized keys of all (sequence,
// KV head) pairs, and the workgroup count, as many as the chip holds at once,
// each taking U / n contiguous tiles, but never fewer than kMinUnitsPerWg
// (which bounds the partial results per pair by the workspace size).
// KVQ_SPLIT_TOKENS=n (read on every call) sets the tiles per workgroup to
// n/32 instead, for checks that vary the work split on one input. The merge
// kernel runs when a pair spans several workgroups or a sequence is empty
// (its output is written as 0 there).
int64_t wg_of_unit_host(int64_t u, int64_t U, int64_t nwg) { return ((u + 1) * nwg + U - 1) / U - 1; }

void plan_attention(const kvq_config* cfg, const kvq_cache* cache, int64_t slots, AttnPlan* p) {
  const int64_t H = cfg->n_kv_heads;
  const bool chan = cfg->k_axis == KVQ_AXIS_CHANNEL;
  // units of one (sequence, KV head): its quantized 32-token tiles, or one
  // unit for residual keys alone
  auto units = [&](int b) -> int64_t {
    const int64_t L = cache->len_host[b];
    const int64_t Q = chan ? L - L % cfg->k_residual_tokens : L;
    return Q > 0 ? (Q + kBlock - 1) / kBlock : (L > 0 ? 1 : 0);
  };
  int64_t U = 0;
  bool need = false;
  for (int b = 0; b < cache->batch; ++b) {
    U += H * units(b);
    need = need || cache->len_host[b] == 0;
  }
  int64_t per = kMinUnitsPerWg;
  if (const char* e = getenv("KVQ_SPLIT_TOKENS")) {
    const long v = strtol(e, nullptr, 10);
    if (v > 0) per = std::max<int64_t>((v + kBlock - 1) / kBlock, kMinUnitsPerWg);
  }
  int64_t nwg = 0;
  if (U > 0) nwg = per > kMinUnitsPerWg ? std::max<int64_t>(1, U / per)
                                         : std::min<int64_t>(std::max<int64_t>(1, slots), std::max<int64_t>(1, U / per));
  nwg = std::min<int64_t>(nwg, kMaxWgs);
  p->units = U;
  p->n_wg = (int)nwg;
  int64_t most = 1;  // the most workgroups one pair spans (the merge kernel's batch size follows it)
  if (nwg > 1) {
    int64_t base = 0;
    for (int b = 0; b < cache->batch; ++b) {
      const int64_t nt = units(b);
      for (int64_t h = 0; h < H && nt > 0; ++h) {
        const int64_t s0 = base + h * nt;
        most = std::max(most, wg_of_unit_host(s0 + nt - 1, U, nwg) - wg_of_unit_host(s0, U, nwg) + 1);
      }
      base += H * nt;
    }
  }
  p->need_combine = (need || most > 1) ? 1 : 0;
  p->max_pieces = (int)most;
}

kvq_status check_config(const kvq_config* cfg) {
  if (!cfg) return KVQ_EINVAL;
  if (cfg->n_kv_heads < 1 || cfg->n_q_heads < 1) return KVQ_EINVAL;
  if (cfg->n_q_heads % cfg->n_kv_heads != 0) return KVQ_EINVAL;
  const int g = cfg->n_q_heads / cfg->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return KVQ_EUNSUPPORTED;
  if (cfg->d_head != kD) return KVQ_EUNSUPPORTED;
  if (cfg->v_group_channels != cfg->d_head) return KVQ_EUNSUPPORTED;
  if (!bits_ok(cfg->k_bits) || !bits_ok(cfg->v_bits)) return KVQ_EUNSUPPORTED;
  const int fmt = cfg->k_format;
  if (fmt != KVQ_FORMAT_INT && fmt != KVQ_FORMAT_FP8 && fmt != KVQ_FORMAT_SYM32) return KVQ_EINVAL;
  if (cfg->v_format != fmt) return KVQ_EUNSUPPORTED;  // one format for keys and values
  if (fmt != KVQ_FORMAT_INT && cfg->k_axis != KVQ_AXIS_TOKEN) return KVQ_EUNSUPPORTED;
  if (fmt == KVQ_FORMAT_FP8) {
    if (cfg->k_bits != 8 || cfg->v_bits != 8) return KVQ_EINVAL;
    for (float sc : {cfg->k_scale, cfg->v_scale})
      if (!(sc > 0.0f) || !std::isfinite(sc)) return KVQ_EINVAL;
  }
  if (cfg->k_rope != 0 && cfg->k_rope != 1) return KVQ_EINVAL;
  if (cfg->k_rope) {
    if (!(cfg->rope_theta > 1.0f) || !std::isfinite(cfg->rope_theta)) return KVQ_EINVAL;
    if (cfg->k_axis != KVQ_AXIS_CHANNEL || fmt != KVQ_FORMAT_INT || cfg->k_sparse_per_vector != 0)
      return KVQ_EUNSUPPORTED;
  }
  if (cfg->k_axis == KVQ_AXIS_TOKEN) {
    if (cfg->k_group_tokens != 0 || cfg->k_residual_tokens != 0) return KVQ_EINVAL;
    if (cfg->k_sparse_per_vector != 0) return KVQ_EUNSUPPORTED;
  } else if (cfg->k_axis == KVQ_AXIS_CHANNEL) {
    if (cfg->k_group_tokens != kBlock) return KVQ_EUNSUPPORTED;
    if (cfg->k_residual_tokens <= 0 || cfg->k_residual_tokens % kBlock != 0) return KVQ_EINVAL;
    if (cfg->k_sparse_per_vector != 0 && cfg->k_sparse_per_vector != 2) return KVQ_EUNSUPPORTED;
  } else {
    return KVQ_EINVAL;
  }
  return KVQ_OK;
}

// Shape of a cache for a valid cfg. Beyond 2^44 (sequence, KV head, token)
// slots (4 PB of fp16 keys) the byte counts would leave 64-bit range.
kvq_status check_shape(const kvq_config* cfg, int32_t batch, int64_t max_tokens) {
  if (batch < 1 || max_tokens < kBlock || max_tokens % kBlock != 0) return KVQ_EINVAL;
  if (max_tokens > (1 << 24)) return KVQ_EUNSUPPORTED;
  if ((int64_t)batch * cfg->n_kv_heads > ((int64_t)1 << 44) / max_tokens) return KVQ_EUNSUPPORTED;
  return KVQ_OK;
}

bool aligned(const void* p) { return ((uintptr_t)p & 255u) == 0; }

kvq_status check_cache(const kvq_config* cfg, const kvq_cache* c) {
  if (!c) return KVQ_EINVAL;
  kvq_status s = check_shape(cfg, c->batch, c->max_tokens);
  if (s != KVQ_OK) return s;
  const void* req[] = {c->k_codes, c->v_codes, c->seq_len};
  for (const void* p : req)
    if (!p || !aligned(p)) return KVQ_EINVAL;
  if (cfg->k_format != KVQ_FORMAT_FP8) {  // fp8 caches have no metadata arrays
    for (const void* p : {c->k_meta, c->v_meta})
      if (!p || !aligned(p)) return KVQ_EINVAL;
  }
  if (!c->len_host) return KVQ_EINVAL;
  if (cfg->k_axis == KVQ_AXIS_CHANNEL && (!c->k_resid || !aligned(c->k_resid))) return KVQ_EINVAL;
  if (cfg->k_sparse_per_vector && (!c->k_sparse || !aligned(c->k_sparse))) return KVQ_EINVAL;
  for (int b = 0; b < c->batch; ++b)
    if (c->len_host[b] < 0 || c->len_host[b] > c->max_tokens) return KVQ_EINVAL;
  return KVQ_OK;
}

CacheView view_of(const kvq_config* cfg, const kvq_cache* c) {
  CacheView v;
  v.B = c->batch;
  v.H = cfg->n_kv_heads;
  v.T = c->max_tokens;
  v.kbits = cfg->k_bits;
  v.vbits = cfg->v_bits;
  v.kaxis = cfg->k_axis == KVQ_AXIS_CHANNEL ? 1 : 0;
  v.R = cfg->k_residual_tokens;
  v.sparse = cfg->k_sparse_per_vector;
  v.fmt = cfg->k_format == KVQ_FORMAT_FP8 ? kFmtFp8 : (cfg->k_format == KVQ_FORMAT_SYM32 ? kFmtSym32 : kFmtInt);
  v.kscale = cfg->k_scale;
  v.vscale = cfg->v_scale;
  v.k_codes = (uint8_t*)c->k_codes;
  v.k_meta = (uint32_t*)c->k_meta;
  v.k_resid = (uint16_t*)c->k_resid;
  v.k_sparse = (uint32_t*)c->k_sparse;
  v.v_codes = (uint8_t*)c->v_codes;
  v.v_meta = (uint32_t*)c->v_meta;
  v.seq_len = c->seq_len;
  return v;
}

// Validation, plan and launch shared by the two attention entry points;
// ws_bytes = 0 means ws is the library's own scratch (checked against the
// plan instead of the shape bound).
kvq_status decode_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q, float* out,
                            float softmax_scale, void* ws, size_t ws_bytes, bool own_scratch, void* stream) {
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVQ_OK) return s;
  if (!q || !out || !aligned(q) || !aligned(out)) return KVQ_EINVAL;
  if (!own_scratch) {
    if (!ws || !aligned(ws)) return KVQ_EINVAL;
    if (ws_bytes < kvq_workspace_bytes(cfg, cache->batch, cache->max_tokens)) return KVQ_EWORKSPACE;
  }
  const CacheView v = view_of(cfg, cache);
  // tile indices are 32-bit on the device
  if ((int64_t)cache->batch * cfg->n_kv_heads * (cache->max_tokens / kBlock) > INT32_MAX) return KVQ_EUNSUPPORTED;
  AttnPlan p;
  p.Hq = cfg->n_q_heads;
  p.group = cfg->n_q_heads / cfg->n_kv_heads;
  p.scale = softmax_scale;
  p.rope = cfg->k_rope;
  p.rope_log2_theta = cfg->k_rope ? (double)log2l((long double)cfg->rope_theta) : 0.0;
  plan_attention(cfg, cache, (int64_t)compute_units() * attention_blocks_per_cu(v, p.group, p.rope), &p);
  if (own_scratch) {
    if (workspace_bytes_for(p.n_wg, p.group) > ws_bytes) return KVQ_EWORKSPACE;
    if (!ws) return KVQ_EHIP;
  }
  hipStream_t st = (hipStream_t)stream;
  return after_launch(launch_decode_attention(v, p, (const uint16_t*)q, out, (float*)ws, st), st);
}

// Scratch of the entry point that allocates nothing: the largest workspace an
// attention call can need (kMaxWgs workgroups, two partial slots each, 8 query
// heads per KV head), 17.3 MB, held on every device the library runs on until
// the process ends. Host code uses the device address from
// hipGetSymbolAddress, never the array's name (a host-side stand-in).
constexpr size_t kScratchBytes = (size_t)2 * kMaxWgs * 8 * kPartialFloats * sizeof(float);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` on the current device, looked up once per
// device (threads may race to store the same value); nullptr if the lookup fails.
void* scratch_address() {
  static std::atomic<void*> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = cache[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      if (debug_sync()) fprintf(stderr, "kvq: hipGetSymbolAddress of the attention scratch failed\n");
      return nullptr;
    }
    cache[dev].store(p, std::memory_order_relaxed);
  }
  return p;
}

}  // namespace

extern "C" {

const char* kvq_status_string(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_EUNSUPPORTED: return "unsupported configuration";
    case KVQ_ECAPACITY: return "append exceeds cache capacity";
    case KVQ_EWORKSPACE: return "workspace too small";
    case KVQ_EHIP: return "HIP launch failed";
  }
  return "unknown status";
}

kvq_status kvq_cache_sizes(const kvq_config* cfg, int32_t batch, int64_t max_tokens,
                           kvq_sizes* out) {
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if ((s = check_shape(cfg, batch, max_tokens)) != KVQ_OK) return s;
  if (!out) return KVQ_EINVAL;
  const uint64_t n = (uint64_t)batch * cfg->n_kv_heads, T = (uint64_t)max_tokens, D = kD;
  memset(out, 0, sizeof(*out));
  out->k_codes = n * T * D * cfg->k_bits / 8;
  out->v_codes = n * T * D * cfg->v_bits / 8;
  // metadata per token: one word (affine), 4 fp16 block scales (sym32), none (fp8)
  const uint64_t meta_tok = cfg->k_format == KVQ_FORMAT_FP8 ? 0 : (cfg->k_format == KVQ_FORMAT_SYM32 ? 2 * kSymBlocks : 4);
  out->v_meta = n * T * meta_tok;
  out->seq_len = (uint64_t)batch * 4;
  if (cfg->k_axis == KVQ_AXIS_CHANNEL) {
    out->k_meta = n * (T / kBlock) * D * 4;
    out->k_resid = n * (uint64_t)cfg->k_residual_tokens * D * 2;
    out->k_sparse = cfg->k_sparse_per_vector ? n * T * 8 : 0;
  } else {
    out->k_meta = n * T * meta_tok;
  }
  out->nominal_bytes = n * T * D * (cfg->k_bits + cfg->v_bits) / 8;
  out->total_bytes = out->k_codes + out->k_meta + out->k_resid + out->k_sparse + out->v_codes +
                     out->v_meta + out->seq_len;
  return KVQ_OK;
}

size_t kvq_workspace_bytes(const kvq_config* cfg, int32_t batch, int64_t max_tokens) {
  if (check_config(cfg) != KVQ_OK || check_shape(cfg, batch, max_tokens) != KVQ_OK) return 0;
  return workspace_bytes_for(max_wgs_for(batch, cfg->n_kv_heads, max_tokens), cfg->n_q_heads / cfg->n_kv_heads);
}

kvq_status kvq_append(const kvq_config* cfg, kvq_cache* cache, const void* k_new, const void* v_new,
                      const int32_t* cu_new_dev, const int32_t* n_new_host, void* stream) {
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVQ_OK) return s;
  if (!cu_new_dev || !n_new_host) return KVQ_EINVAL;
  int64_t total = 0;
  int max_tok_blocks = 0, max_flush_blocks = 0;
  bool one_each = true;  // a decode step: one new token for every sequence
  const int R = cfg->k_residual_tokens;
  for (int b = 0; b < cache->batch; ++b) {
    const int n = n_new_host[b];
    if (n < 0) return KVQ_EINVAL;
    one_each = one_each && n == 1;
    const int L = cache->len_host[b];
    if ((int64_t)L + n > cache->max_tokens) return KVQ_ECAPACITY;
    total += n;
    if (n == 0) continue;
    const int L2 = L + n;
    max_tok_blocks = std::max(max_tok_blocks, (L2 - 1) / kBlock - L / kBlock + 1);
    if (cfg->k_axis == KVQ_AXIS_CHANNEL) {
      const int Q = L - L % R, Q2 = L2 - L2 % R;
      max_flush_blocks = std::max(max_flush_blocks, (Q2 - Q) / kBlock);
    }
  }
  if (total == 0) return KVQ_OK;
  if (total > INT32_MAX) return KVQ_EINVAL;
  if (!k_new || !v_new || !aligned(k_new) || !aligned(v_new)) return KVQ_EINVAL;
  const CacheView v = view_of(cfg, cache);
  const AppendInputs in{(const uint16_t*)k_new, (const uint16_t*)v_new, cu_new_dev, (int)total};
  hipStream_t st = (hipStream_t)stream;
  if (max_flush_blocks > 0) {
    if ((s = after_launch(launch_flush_keys(v, in, max_flush_blocks, st), st)) != KVQ_OK) return s;
  }
  if (one_each) {
    if ((s = after_launch(launch_append_decode(v, in, st), st)) != KVQ_OK) return s;
  } else {
    if ((s = after_launch(launch_append_tokens(v, in, max_tok_blocks, st), st)) != KVQ_OK) return s;
    if ((s = after_launch(launch_update_lengths(v, in, st), st)) != KVQ_OK) return s;
  }
  for (int b = 0; b < cache->batch; ++b) cache->len_host[b] += n_new_host[b];
  return KVQ_OK;
}

kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                float* out, float softmax_scale, void* ws, size_t ws_bytes,
                                void* stream) {
  return decode_attention(cfg, cache, q, out, softmax_scale, ws, ws_bytes, false, stream);
}

kvq_status kvq_decode_attention_noalloc(const kvq_config* cfg, const kvq_cache* cache, const void* q,
                                        float* out, float softmax_scale, void* stream) {
  // validate before touching the device, so argument errors need no HIP call
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVQ_OK) return s;
  if (!q || !out || !aligned(q) || !aligned(out)) return KVQ_EINVAL;
  return decode_attention(cfg, cache, q, out, softmax_scale, scratch_address(), kScratchBytes, true, stream);
}

kvq_status kvq_dequantize(const kvq_config* cfg, const kvq_cache* cache, void* k_out, void* v_out,
                          void* stream) {
  kvq_status s = check_config(cfg);
  if (s != KVQ_OK) return s;
  if ((s = check_cache(cfg, cache)) != KVQ_OK) return s;
  if (!k_out || !v_out || !aligned(k_out) || !aligned(v_out)) return KVQ_EINVAL;
  const CacheView v = view_of(cfg, cache);
  hipStream_t st = (hipStream_t)stream;
  return after_launch(launch_dequantize(v, (uint16_t*)k_out, (uint16_t*)v_out, st), st);
}

}  // extern "C"
