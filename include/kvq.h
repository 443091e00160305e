/*
 * kvq.h — C ABI of the low-bit KV-cache library for MI355X (gfx950).
 *
 * What it computes
 *   Asymmetric affine integer codes for a transformer's key/value cache and
 *   single-token decode attention that reads the packed codes and dequantizes
 *   them inside the attention kernel.
 *
 *   - Affine quantizer: q = round(x / scale) + zero_point, x_hat = scale * (q -
 *     zero_point), scale = (x_max - x_min) / (q_max - q_min), zero_point =
 *     q_min - round(x_min / scale); int8 range [-128, 127], int4 [-8, 7].
 *     ("KV Cache Quantization — 8-bit and 4-bit", section "Integer quantization
 *     in one screen".)  int2 uses [-2, 1]: the four levels that "Sub-8-Bit KV
 *     Cache Quantization Is Not a Free Lever for an RDNA4 Agent Swarm" names in
 *     "Why 8 bits hides the problem and 4 bits exposes it".
 *   - Axis split: values per token; keys per token or per channel over groups
 *     of consecutive tokens, with a full-precision residual window of the most
 *     recent keys (KIVI, as described in "Sub-8-Bit KV Cache Quantization ...",
 *     FAQ and "What the low-bit numbers actually cost"; "KV Cache Quantization —
 *     8-bit and 4-bit", "The outlier problem: keys have outlier channels" and
 *     "Why keys and values want different treatment").
 *   - Dense-and-sparse keys: the largest-magnitude entries of each key vector
 *     kept in fp16 outside the dense codes (KVQuant, "Sub-8-Bit KV Cache
 *     Quantization ...", "What the low-bit numbers actually cost").
 *   - Decode attention that streams the packed cache and dequantizes on the
 *     fly ("KV Cache Quantization — 8-bit and 4-bit", "Decode is memory-bound,
 *     so smaller is also faster").
 *   - Two more element formats for token-axis caches ("KV Cache Quantization
 *     Benchmarked: 8-bit Is Nearly Lossless, How Much Does 4-bit Cost?", the
 *     glossary and memory paragraphs: an fp8 cache with a 4-bit exponent and
 *     a 3-bit mantissa, and llama.cpp-style blocks of 32 elements sharing one
 *     scale; "KV Cache Quantization — 8-bit and 4-bit", "Symmetric vs
 *     asymmetric" for the zero point forced to zero):
 *       KVQ_FORMAT_FP8:   one OCP E4M3 byte per element (sign bit 7, exponent
 *                         bits 6..3 with bias 7, mantissa bits 2..0; no
 *                         infinities, S.1111.111 is NaN, largest finite 448)
 *                         and one fp32 scale per cache side:
 *                         code = e4m3(x / scale), x_hat = scale * value(code).
 *                         e4m3() rounds to the nearest magnitude, ties to the
 *                         even code, saturates above 448 and keeps the sign
 *                         (a negative value that rounds to zero is 0x80).
 *       KVQ_FORMAT_SYM32: each token vector cut into 4 blocks of 32
 *                         consecutive channels; per block
 *                         s16 = smallest fp16 >= max|x| / (float)q_max
 *                         (1.0 for an all-zero block), s = (float)s16,
 *                         q_i = clamp(rint(x_i / s), -q_max, q_max),
 *                         stored u_i = q_i - q_min, x_hat_i = s * q_i.
 *     Both formats keep keys on the token axis and apply to keys and values
 *     alike (k_format == v_format).
 *   - Pre-RoPE keys (k_rope = 1): keys are quantized before the rotary
 *     position embedding and attention rotates each dequantized key by its
 *     position, so the rotation does not smear the channel structure the
 *     per-channel scales rely on (KVQuant, as described in "Sub-8-Bit KV
 *     Cache Quantization ...", "What the low-bit numbers actually cost"). The
 *     pages define no embedding; this is the textbook one:
 *       theta_i = rope_theta^(-2 i / D), i = 0 .. D/2 - 1, and key t (0-based
 *       position in its sequence) becomes, for each pair (i, i + D/2),
 *         y_i       = x_i cos(t theta_i) - x_{i+D/2} sin(t theta_i)
 *         y_{i+D/2} = x_{i+D/2} cos(t theta_i) + x_i sin(t theta_i);
 *     the query passed to attention is already rotated by its own position.
 *     Channel-axis affine keys without sparse entries only. kvq_dequantize
 *     returns the keys as cached (before the rotation).
 *
 * Exact arithmetic of one quantization group (x_i are fp16 values widened to
 * fp32; every operation is IEEE fp32 with round-to-nearest-even):
 *   q_min = -2^(b-1), q_max = 2^(b-1) - 1, n_lev = q_max - q_min
 *   x_min, x_max  = min / max of the group
 *   if x_max > x_min:  s32 = (x_max - x_min) / (float)n_lev
 *                      s16 = smallest fp16 >= s32 (round toward +inf)
 *   else (constant):   s16 = |x_min| if x_min != 0, else 1.0
 *   s  = (float)s16
 *   r  = rint(x_min / s)
 *   if |r| > 2048 + q_min (a group far from zero compared with its spread):
 *                      s16 = smallest fp16 >= |x_min| / (float)(2048 + q_min),
 *                      s = (float)s16, r = rint(x_min / s)
 *   z  = (float)q_min - r;  z16 = fp16(z)
 *   (|r| <= 2048 + q_min keeps z and z - q_min = -r exact fp16 integers)
 *   q_i = clamp(rint(x_i / s) + z, q_min, q_max)       (rint: half to even)
 *   stored code u_i = q_i - q_min  (unsigned, b bits)
 *   x_hat_i = s * (q_i - z)   (exact in fp32)
 * Divisions are true IEEE divisions, never multiplication by a reciprocal.
 * Rounding the scale up, and widening it for far-off groups, keeps every
 * element within s/2 of its reconstruction at the stored scale, the bound the
 * "Integer quantization in one screen" section states.
 *
 * Token state of one sequence (per KV head, identical for all heads)
 *   L  = tokens held (device seq_len[b]; host copy len_host[b]).
 *   Per-token keys:   all L tokens are quantized (Q = L).
 *   Per-channel keys: Q = L - (L mod R) tokens are quantized in groups of
 *                     G = 32 tokens aligned at multiples of 32 from token 0;
 *                     the last r = L mod R keys stay fp16 in the residual
 *                     window. Appending keys fills the window; when it holds R
 *                     keys all R are quantized (R/32 groups) and it empties.
 *   Values are always quantized per token on append.
 *
 * ---------------------------------------------------------------------------
 * Memory layout (all arrays dense, little-endian, device memory, caller-owned;
 * T = max_tokens, a multiple of 32; H = n_kv_heads; D = d_head = 128;
 * kb / vb = key / value bits; "meta word" = uint32 (fp16 scale bits) |
 * (fp16 zero bits) << 16):
 *
 *   k_codes  uint8 [B][H][T][D*kb/8]
 *            token-major rows; channel c's code occupies bits
 *            [(c*kb) mod 8, +kb) of byte (c*kb)/8 of its token row.
 *   k_meta   per-token keys:   uint32 meta word [B][H][T]
 *            per-channel keys: uint32 meta word [B][H][T/32][D]
 *            (one word per (32-token group, channel)).
 *   k_resid  per-channel keys only: fp16 [B][H][R][D]; slot j holds token
 *            Q + j (j < r). Unused slots are not read.
 *   k_sparse per-channel keys with k_sparse_per_vector == 2 only:
 *            uint32 [B][H][T][2]: word 0 = fp16 value of entry 0 | fp16 value
 *            of entry 1 << 16; word 1 = channel of entry 0 | channel of entry
 *            1 << 16. A row-regular CSR: every quantized token has exactly two
 *            entries, so the row pointer of token t is implicitly 2*t.
 *            Entries are ordered by ascending channel.
 *   v_codes  uint8 [B][H][T/32][D][4*vb]
 *            per 32-token block, one record of 32 codes per channel; token
 *            tau (0..31 within the block) occupies bits [(tau*vb) mod 8, +vb)
 *            of byte (tau*vb)/8 of the record.
 *   v_meta   uint32 meta word [B][H][T]
 *   seq_len  int32 [B]
 * KVQ_FORMAT_FP8 caches have no k_meta or v_meta (size 0; the pointers may be
 * NULL); their codes are the E4M3 bytes, in the 8-bit layouts above.
 * KVQ_FORMAT_SYM32 caches store k_meta and v_meta as fp16 [B][H][T][4] (the
 * scales of channel blocks 0..31, 32..63, 64..95, 96..127 of each token).
 * Code bits of token slots >= L inside a byte written by the library are 0.
 * Buffers must be zero-filled before the first append of a sequence.
 *
 * Fresh input tensors
 *   k_new, v_new: fp16 [N][H][D], the new tokens of all sequences packed back
 *   to back; sequence b owns rows cu_new[b] .. cu_new[b+1]-1 (cu_new int32
 *   [B+1] on the device, cu_new[0] = 0) and n_new_host[b] = cu_new[b+1] -
 *   cu_new[b] on the host.
 *   q:   fp16 [B][Hq][D];  out: fp32 [B][Hq][D].
 *   Query head h attends with KV head h / (Hq / H) (consecutive grouping).
 *   Base pointers must be 256-byte aligned.
 *
 * Ownership and concurrency
 *   The library never allocates, frees, or synchronizes; every kernel is
 *   enqueued on the caller's stream and returns at once. It keeps no state
 *   between calls. Calls that touch the same cache must be ordered by the
 *   caller (same stream). Asynchronous device faults surface at the caller's
 *   next synchronization.
 *
 * Environment (read by the library; both optional)
 *   KVQ_DEBUG=1         synchronize after every launch and print HIP errors.
 *   KVQ_SPLIT_TOKENS=n  make every workgroup of kvq_decode_attention take n
 *                       tokens' worth of 32-token tiles (at least 8 tiles)
 *                       instead of the built-in plan (as many workgroups as
 *                       the device holds at once); for checks that vary the
 *                       split of the work on one input.
 *
 * Errors
 *   Arguments are validated on the host before anything is launched; an error
 *   status means nothing was enqueued and no host state changed. KVQ_EHIP is
 *   returned when a launch fails (hipGetLastError).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
  KVQ_OK = 0,
  KVQ_EINVAL = 1,        /* a null pointer, a bad size or a bad alignment   */
  KVQ_EUNSUPPORTED = 2,  /* a configuration this build does not implement   */
  KVQ_ECAPACITY = 3,     /* an append would exceed max_tokens               */
  KVQ_EWORKSPACE = 4,    /* workspace smaller than kvq_workspace_bytes      */
  KVQ_EHIP = 5           /* a HIP launch failed                             */
} kvq_status;

enum { KVQ_AXIS_TOKEN = 0, KVQ_AXIS_CHANNEL = 1 };
enum { KVQ_FORMAT_INT = 0, KVQ_FORMAT_FP8 = 1, KVQ_FORMAT_SYM32 = 2 };

/* Quantization configuration, passed by value through a host pointer. */
typedef struct kvq_config {
  int32_t d_head;              /* channels per head; 128 is supported        */
  int32_t n_kv_heads;          /* H >= 1                                     */
  int32_t n_q_heads;           /* Hq, a multiple of H with Hq/H in {1,2,4,8} */
  int32_t k_bits;              /* 8, 4 or 2                                  */
  int32_t v_bits;              /* 8, 4 or 2                                  */
  int32_t k_axis;              /* KVQ_AXIS_TOKEN or KVQ_AXIS_CHANNEL         */
  int32_t k_group_tokens;      /* G: 32 for channel axis, 0 for token axis   */
  int32_t k_residual_tokens;   /* R: a positive multiple of 32 for channel
                                  axis, 0 for token axis                     */
  int32_t v_group_channels;    /* channels per value group; must be d_head   */
  int32_t k_sparse_per_vector; /* 0, or 2 (channel axis only)                */
  int32_t k_format;            /* KVQ_FORMAT_*; 0 (INT) for the affine codes */
  int32_t v_format;            /* equal to k_format                          */
  float k_scale;               /* FP8 only: per-cache key scale, finite > 0  */
  float v_scale;               /* FP8 only: per-cache value scale            */
  int32_t k_rope;              /* 1: keys are cached before the rotary
                                  embedding, which attention applies; 0: keys
                                  are used as cached                         */
  float rope_theta;            /* k_rope only: frequency base (> 1, finite)  */
} kvq_config;

/* Host-side descriptor of one cache; pointers name device memory except
 * len_host. All pointers are owned by the caller. */
typedef struct kvq_cache {
  int32_t batch;        /* B                                                 */
  int32_t max_tokens;   /* T, capacity per sequence, a multiple of 32        */
  void* k_codes;
  void* k_meta;
  void* k_resid;        /* NULL unless k_axis == KVQ_AXIS_CHANNEL            */
  void* k_sparse;       /* NULL unless k_sparse_per_vector > 0               */
  void* v_codes;
  void* v_meta;
  int32_t* seq_len;     /* device int32 [B]                                  */
  int32_t* len_host;    /* host int32 [B], kept equal to seq_len by appends  */
} kvq_cache;

/* Byte sizes of every cache array for (cfg, batch, max_tokens), plus the
 * nominal size 2*H*D*T*bits/8*B from the bytes-per-token formula ("KV Cache
 * Quantization — 8-bit and 4-bit", "The bytes-per-token formula" and "A worked
 * memory example", one layer) and the cache's actual total. */
typedef struct kvq_sizes {
  uint64_t k_codes, k_meta, k_resid, k_sparse, v_codes, v_meta, seq_len;
  uint64_t nominal_bytes;  /* codes only, no scales, per the formula        */
  uint64_t total_bytes;    /* sum of every array above                      */
} kvq_sizes;

/* Fills *out_host. max_tokens must be a positive multiple of 32;
 * KVQ_EINVAL on a bad configuration, size or null pointer, KVQ_EUNSUPPORTED
 * past 2^24 tokens per sequence (the capacity a kvq_cache can describe) or
 * past 2^44 (sequence, KV head, token) slots in all (where byte counts would
 * leave 64-bit range). Pure host function. */
kvq_status kvq_cache_sizes(const kvq_config* cfg, int32_t batch,
                           int64_t max_tokens, kvq_sizes* out_host);

/* Bytes of device workspace kvq_decode_attention needs for this shape:
 * partial results (m, l, o[128] in fp32 for each query head of a KV head),
 * two per attention workgroup, for at most min(2048, batch * n_kv_heads *
 * ceil(max_tokens / 32) / 8) workgroups (at most 17.3 MB). 0 on a bad
 * configuration or size (the rules of kvq_cache_sizes). Pure host function. */
size_t kvq_workspace_bytes(const kvq_config* cfg, int32_t batch,
                           int64_t max_tokens);

/* Quantize-on-append. Appends n_new_host[b] tokens of keys and values to
 * sequence b, quantizing per the group arithmetic above: values per token;
 * keys per token, or into the residual window with a flush of R keys as R/32
 * per-channel groups whenever the window fills. With k_sparse_per_vector == 2
 * each key vector being flushed first gives up its two largest-|x| entries
 * (ties to the lower channel) to k_sparse and has them set to +0 before the
 * group statistics. Updates seq_len on the device and len_host on the host.
 * Errors: KVQ_EINVAL (null pointer, negative count, misaligned base),
 * KVQ_EUNSUPPORTED, KVQ_ECAPACITY (len_host[b] + n_new_host[b] > max_tokens),
 * KVQ_EHIP. */
kvq_status kvq_append(const kvq_config* cfg, kvq_cache* cache,
                      const void* k_new, const void* v_new,
                      const int32_t* cu_new_dev, const int32_t* n_new_host,
                      void* stream /* hipStream_t */);

/* Decode attention for one new query token per sequence:
 *   out[b][h] = sum_t softmax_t(softmax_scale * q[b][h] . K_hat[b][kv][t])
 *               * V_hat[b][kv][t],   kv = h / (Hq / H), t < seq_len[b],
 * where K_hat / V_hat are the dequantized codes (plus sparse entries), and
 * residual keys are the stored fp16 values. A sequence with no tokens gets
 * out = 0. The work (every 32-token tile of every (sequence, KV head)) is
 * cut into equal contiguous ranges, one per workgroup; pairs whose tiles span
 * several ranges are merged by a log-sum-exp in a second kernel. ws is device
 * workspace of at least kvq_workspace_bytes(cfg, cache->batch,
 * cache->max_tokens) bytes for those partial results; its contents need no
 * initial value. Calls that share a workspace must be ordered on one stream.
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED (also when batch * n_kv_heads *
 * max_tokens / 32 exceeds 2^31 - 1, the device's tile index range),
 * KVQ_EWORKSPACE, KVQ_EHIP. */
kvq_status kvq_decode_attention(const kvq_config* cfg, const kvq_cache* cache,
                                const void* q, float* out, float softmax_scale,
                                void* ws, size_t ws_bytes,
                                void* stream /* hipStream_t */);

/* kvq_decode_attention for callers that cannot allocate device memory or
 * bring a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments and result, without ws: the
 * partial results go to a scratch array the library holds in device memory,
 * 17.3 MB on every GPU it runs on (looked up once per device with
 * hipGetSymbolAddress), which bounds the work split to what
 * kvq_workspace_bytes allows. It calls no allocating routine. Every call on
 * one GPU shares that GPU's scratch, which keeps the last call's contents
 * (nothing in it needs an initial value): calls that can overlap on one GPU
 * (different streams, or threads without ordering) race; order them on one
 * stream. Errors: as kvq_decode_attention; KVQ_EWORKSPACE if a call would need
 * more scratch than held (not reachable within the checked shapes), KVQ_EHIP
 * if the scratch address cannot be found. */
kvq_status kvq_decode_attention_noalloc(const kvq_config* cfg, const kvq_cache* cache,
                                        const void* q, float* out, float softmax_scale,
                                        void* stream /* hipStream_t */);

/* Writes the dequantized cache as fp16 [B][T][H][D]: K_hat = fp16(s*(q - z))
 * plus sparse entries for quantized keys, the stored fp16 value for residual
 * keys, V_hat = fp16(s*(q - z)); token slots t >= seq_len[b] are written as
 * +0. The fp16 conversions round to nearest even. This is the separate
 * materializing pass the attention path avoids; it exists for checking and
 * for callers that need plain fp16 tensors.
 * Errors: KVQ_EINVAL, KVQ_EUNSUPPORTED, KVQ_EHIP. */
kvq_status kvq_dequantize(const kvq_config* cfg, const kvq_cache* cache,
                          void* k_out, void* v_out,
                          void* stream /* hipStream_t */);

/* Static text for a status code. */
const char* kvq_status_string(kvq_status s);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
