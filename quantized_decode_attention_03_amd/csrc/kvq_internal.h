// Internal launch interface between the C-ABI glue (kvq_api.hip) and the
// kernel translation units. Host-side only declarations plus the POD argument
// blocks the kernels receive by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kD = 128;      // channels per head
constexpr int kBlock = 32;   // tokens per key group / value code block

// Element formats (keys and values alike): affine integer codes with scale
// and zero point, fp8 E4M3 bytes with one scale per cache side, or symmetric
// codes with one fp16 scale per 32-channel block of a token.
enum : int { kFmtInt = 0, kFmtFp8 = 1, kFmtSym32 = 2 };
// Attention only: affine codes whose channel-axis keys are cached before the
// rotary position embedding, which the kernel applies after dequantization.
constexpr int kFmtRope = 3;
constexpr int kSymBlocks = 4;  // 32-channel blocks per token vector

// Everything a kernel needs to address one layer's cache.
struct CacheView {
  int B, H, T;                 // batch, KV heads, capacity (multiple of 32)
  int kbits, vbits;
  int kaxis;                   // 0 token, 1 channel
  int R;                       // residual slots (channel axis), else 0
  int sparse;                  // entries per key vector in k_sparse (0 or 2)
  int fmt;                     // kFmt*: element format of keys and values
  float kscale, vscale;        // fp8: per-cache scales (x_hat = scale * value)
  uint8_t* k_codes;
  uint32_t* k_meta;
  uint16_t* k_resid;
  uint32_t* k_sparse;
  uint8_t* v_codes;
  uint32_t* v_meta;
  int32_t* seq_len;
};

struct AppendInputs {
  const uint16_t* k_new;       // fp16 [rows][H][D]
  const uint16_t* v_new;
  const int32_t* cu_new;       // [B+1]
  int rows;                    // rows of k_new / v_new (sum of the new counts)
};

// Launchers; each returns the hipError_t of its launch.
hipError_t launch_flush_keys(const CacheView& c, const AppendInputs& in,
                             int max_blocks, hipStream_t st);
hipError_t launch_append_tokens(const CacheView& c, const AppendInputs& in,
                                int max_blocks, hipStream_t st);
hipError_t launch_update_lengths(const CacheView& c, const AppendInputs& in,
                                 hipStream_t st);
// One new token per sequence: append and length update in one launch.
hipError_t launch_append_decode(const CacheView& c, const AppendInputs& in,
                                hipStream_t st);
hipError_t launch_dequantize(const CacheView& c, uint16_t* k_out,
                             uint16_t* v_out, hipStream_t st);

struct AttnPlan {
  int Hq, group;               // query heads, query heads per KV head
  float scale;                 // softmax scale
  int64_t units;               // 32-token tiles of all (sequence, KV head) pairs
  int n_wg;                    // attention workgroups (each takes units / n_wg)
  int need_combine;            // some pair spans several workgroups, or a sequence is empty
  int max_pieces;              // the most workgroups any one pair spans
  int rope;                    // keys cached before the rotary embedding
  double rope_log2_theta;      // log2 of its frequency base
};
hipError_t launch_decode_attention(const CacheView& c, const AttnPlan& p,
                                   const uint16_t* q, float* out, float* ws,
                                   hipStream_t st);
// Workgroups of the attention kernel variant for (c, group, rotary keys)
// resident per compute unit (at least 1).
int attention_blocks_per_cu(const CacheView& c, int group, int rope);

// Workspace: fp32 partial results [2 n_wg][G][kPartialFloats] = m, l, 2 pad,
// o[128]: two slots per attention workgroup (the first and the last segment
// of its range, the only ones that can be pieces of a shared pair), each with
// the G query heads of its KV head. Every workgroup takes at least
// kMinUnitsPerWg tiles, and there are at most kMaxWgs of them.
constexpr int kPartialFloats = 4 + kD;
constexpr int kMinUnitsPerWg = 8;
constexpr int kMaxWgs = 2048;
// Upper bound on the workgroups of an attention call for (batch, KV heads,
// capacity): every (sequence, KV head) has at most ceil(T / 32) units.
inline int64_t max_wgs_for(int64_t batch, int64_t n_kv_heads, int64_t max_tokens) {
  const int64_t units = batch * n_kv_heads * ((max_tokens + kBlock - 1) / kBlock);
  const int64_t by_units = units / kMinUnitsPerWg > 1 ? units / kMinUnitsPerWg : 1;
  return by_units < kMaxWgs ? by_units : kMaxWgs;
}
inline size_t workspace_bytes_for(int64_t n_wg, int group) {
  return (size_t)(2 * n_wg) * group * kPartialFloats * sizeof(float);
}

}  // namespace kvq
