// Internal launch interface between the C-ABI glue (kvq_api.hip) and the
// kernel translation units. Host-side only declarations plus the POD argument
// blocks the kernels receive by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kD = 128;      // channels per head
constexpr int kBlock = 32;   // tokens per key group / value code block

// Everything a kernel needs to address one layer's cache.
struct CacheView {
  int B, H, T;                 // batch, KV heads, capacity (multiple of 32)
  int kbits, vbits;
  int kaxis;                   // 0 token, 1 channel
  int R;                       // residual slots (channel axis), else 0
  int sparse;                  // entries per key vector in k_sparse (0 or 2)
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
  int n_split;                 // splits per (sequence, KV head)
  int tokens_per_split;        // multiple of 32
  float scale;                 // softmax scale
};
hipError_t launch_decode_attention(const CacheView& c, const AttnPlan& p,
                                   const uint16_t* q, float* out, float* ws,
                                   hipStream_t st);
// Workgroups of the attention kernel variant for (c, group) resident per
// compute unit (at least 1).
int attention_blocks_per_cu(const CacheView& c, int group);

// Workspace: fp32 partials [B][Hq][n_split][kPartialFloats] = m, l, 2 pad,
// o[128].
constexpr int kPartialFloats = 4 + kD;
constexpr int kMinSplitTokens = 256;
constexpr int kMinSplitTiles = kMinSplitTokens / kBlock;
// Upper bound on splits per (sequence, KV head) for a given capacity.
inline int max_splits_for(int max_tokens) {
  return (max_tokens + kMinSplitTokens - 1) / kMinSplitTokens;
}

}  // namespace kvq
