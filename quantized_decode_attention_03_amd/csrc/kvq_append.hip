// Quantize-on-append kernels (gfx950).
//
// Values, and keys on the token axis, are quantized one token vector (128
// channels) at a time: one wavefront per token, two channels per lane, a
// cross-lane min/max reduction along the channel axis. Keys on the channel
// axis wait in the fp16 residual window; a window that fills is quantized as
// groups of one channel over 32 consecutive tokens (a min/max along the token
// axis), after the dense-and-sparse split when it is enabled. (KIVI's axis
// split and residual, KVQuant's per-vector outlier isolation: "Sub-8-Bit KV
// Cache Quantization Is Not a Free Lever for an RDNA4 Agent Swarm", "What the
// low-bit numbers actually cost"; the per-token/per-channel choice: "KV Cache
// Quantization — 8-bit and 4-bit", "Why keys and values want different
// treatment".)
#include "kvq_device.h"

namespace kvq {

namespace {

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fminf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// Per-channel key flush: one workgroup per (32-token block of the window,
// KV head, sequence). The window is tokens [Q, Q2) with Q = L - L mod R and
// Q2 = L2 - L2 mod R; tokens below L come from the residual, the rest from
// the new keys.
__global__ __launch_bounds__(256) void flush_keys_kernel(CacheView c, AppendInputs in) {
  const int b = blockIdx.z, h = blockIdx.y, blk = blockIdx.x;
  const int tid = threadIdx.x;
  const int L = c.seq_len[b];
  const int row0 = in.cu_new[b];
  const int n = in.cu_new[b + 1] - row0;
  const int R = c.R;
  const int Q = L - L % R, L2 = L + n, Q2 = L2 - L2 % R;
  const int t0 = Q + blk * kBlock;
  if (t0 + kBlock > Q2) return;
  const size_t bh = (size_t)b * c.H + h;

  __shared__ uint16_t xs[kBlock][kD];
  __shared__ uint8_t codes[kBlock][kD];

  {  // stage the 32 x 128 fp16 block
    const int tau = tid >> 3, c0 = (tid & 7) * 16;
    const int t = t0 + tau;
    const uint16_t* src = (t < L)
        ? c.k_resid + (bh * R + (t - Q)) * kD + c0
        : in.k_new + ((size_t)(row0 + t - L) * c.H + h) * kD + c0;
    const uint4 a = reinterpret_cast<const uint4*>(src)[0];
    const uint4 d = reinterpret_cast<const uint4*>(src)[1];
    uint4* dst = reinterpret_cast<uint4*>(&xs[tau][c0]);
    dst[0] = a;
    dst[1] = d;
  }
  __syncthreads();

  if (c.sparse) {
    // top-2 |x| per key vector, ties to the lower channel; kept in fp16 and
    // zeroed in the dense copy
    const int w = tid >> 6, lane = tid & 63;
    for (int tau = w * 8; tau < w * 8 + 8; ++tau) {
      const uint32_t b0 = xs[tau][2 * lane], b1 = xs[tau][2 * lane + 1];
      const uint32_t k0 = ((b0 & 0x7FFFu) << 8) | (255u - 2 * lane);
      const uint32_t k1 = ((b1 & 0x7FFFu) << 8) | (255u - (2 * lane + 1));
      const uint32_t best = wave_umax(k0 > k1 ? k0 : k1);
      const uint32_t e0 = (k0 == best) ? 0u : k0, e1 = (k1 == best) ? 0u : k1;
      const uint32_t second = wave_umax(e0 > e1 ? e0 : e1);
      const uint32_t ca = 255u - (best & 0xFFu), cb = 255u - (second & 0xFFu);
      const uint32_t lo = ca < cb ? ca : cb, hi = ca < cb ? cb : ca;
      if (lane == 0) {
        const int t = t0 + tau;
        uint32_t* rec = c.k_sparse + (bh * c.T + t) * 2;
        rec[0] = (uint32_t)xs[tau][lo] | ((uint32_t)xs[tau][hi] << 16);
        rec[1] = lo | (hi << 16);
        xs[tau][lo] = 0;
        xs[tau][hi] = 0;
      }
    }
    __syncthreads();
  }

  if (tid < kD) {  // one thread per channel group (32 tokens)
    const int ch = tid;
    float mn = h2f(xs[0][ch]), mx = mn;
    for (int tau = 1; tau < kBlock; ++tau) {
      const float v = h2f(xs[tau][ch]);
      mn = __builtin_fminf(mn, v);
      mx = __builtin_fmaxf(mx, v);
    }
    const GroupQ g = group_params(mn, mx, c.kbits);
    c.k_meta[(bh * (c.T / kBlock) + t0 / kBlock) * kD + ch] = g.meta;
    for (int tau = 0; tau < kBlock; ++tau)
      codes[tau][ch] = (uint8_t)quant_code(h2f(xs[tau][ch]), g, c.kbits);
  }
  __syncthreads();

  // pack token rows along channels
  const int kb = c.kbits, per = 32 / kb, row_words = 4 * kb;
  for (int i = tid; i < kBlock * row_words; i += 256) {
    const int tau = i / row_words, wd = i % row_words;
    uint32_t word = 0;
    for (int j = 0; j < per; ++j) word |= (uint32_t)codes[tau][wd * per + j] << (j * kb);
    uint32_t* row = reinterpret_cast<uint32_t*>(c.k_codes + (bh * c.T + t0 + tau) * (size_t)(16 * kb));
    row[wd] = word;
  }
}

// Token-axis quantization of the new tokens in one 32-token block: values
// always, keys when they are on the token axis; channel-axis keys that stay in
// the window are copied into the residual.
__global__ __launch_bounds__(256) void append_tokens_kernel(CacheView c, AppendInputs in) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int L = c.seq_len[b];
  const int row0 = in.cu_new[b];
  const int n = in.cu_new[b + 1] - row0;
  if (n <= 0) return;
  const int L2 = L + n;
  const int j = L / kBlock + blockIdx.x;
  if (j > (L2 - 1) / kBlock) return;
  const int t0 = j * kBlock;
  const int tlo = max(L - t0, 0), thi = min(L2 - t0, kBlock);
  const size_t bh = (size_t)b * c.H + h;
  const bool ktok = c.kaxis == 0;
  const int Q2 = ktok ? L2 : L2 - L2 % c.R;

  __shared__ uint8_t vcodes[kBlock][kD];
  __shared__ uint8_t kcodes[kBlock][kD];

  for (int tau = tlo + w; tau < thi; tau += 4) {
    const int t = t0 + tau;
    const size_t src = ((size_t)(row0 + t - L) * c.H + h) * kD;
    {
      const uint32_t pr = reinterpret_cast<const uint32_t*>(in.v_new + src)[lane];
      const float f0 = h2f((uint16_t)(pr & 0xFFFFu)), f1 = h2f((uint16_t)(pr >> 16));
      const float mn = wave_min(__builtin_fminf(f0, f1)), mx = wave_max(__builtin_fmaxf(f0, f1));
      const GroupQ g = group_params(mn, mx, c.vbits);
      vcodes[tau][2 * lane] = (uint8_t)quant_code(f0, g, c.vbits);
      vcodes[tau][2 * lane + 1] = (uint8_t)quant_code(f1, g, c.vbits);
      if (lane == 0) c.v_meta[bh * c.T + t] = g.meta;
    }
    const uint32_t pk = reinterpret_cast<const uint32_t*>(in.k_new + src)[lane];
    if (ktok) {
      const float f0 = h2f((uint16_t)(pk & 0xFFFFu)), f1 = h2f((uint16_t)(pk >> 16));
      const float mn = wave_min(__builtin_fminf(f0, f1)), mx = wave_max(__builtin_fmaxf(f0, f1));
      const GroupQ g = group_params(mn, mx, c.kbits);
      kcodes[tau][2 * lane] = (uint8_t)quant_code(f0, g, c.kbits);
      kcodes[tau][2 * lane + 1] = (uint8_t)quant_code(f1, g, c.kbits);
      if (lane == 0) c.k_meta[bh * c.T + t] = g.meta;
    } else if (t >= Q2) {
      reinterpret_cast<uint32_t*>(c.k_resid + (bh * c.R + (t - Q2)) * kD)[lane] = pk;
    }
  }
  __syncthreads();

  {  // value records: per channel, 32 tokens of vb bits; merge with old tokens
    const int vb = c.vbits, per = 32 / vb;
    const uint32_t mask = (1u << vb) - 1u;
    uint32_t* blk = reinterpret_cast<uint32_t*>(
        c.v_codes + (bh * (c.T / kBlock) + j) * (size_t)(kD * 4 * vb));
    for (int i = tid; i < kD * vb; i += 256) {
      const int ch = i / vb, wd = i % vb;
      const int tok0 = wd * per;
      if (tok0 + per <= tlo) continue;  // only old tokens in this word
      uint32_t word = (tok0 < tlo) ? blk[ch * vb + wd] : 0u;
      for (int k = 0; k < per; ++k) {
        const int tau = tok0 + k;
        if (tau < tlo) continue;
        word &= ~(mask << (k * vb));
        if (tau < thi) word |= (uint32_t)vcodes[tau][ch] << (k * vb);
      }
      blk[ch * vb + wd] = word;
    }
  }
  if (ktok) {  // key rows of the new tokens, packed along channels
    const int kb = c.kbits, per = 32 / kb, row_words = 4 * kb;
    const int nt = thi - tlo;
    for (int i = tid; i < nt * row_words; i += 256) {
      const int tau = tlo + i / row_words, wd = i % row_words;
      uint32_t word = 0;
      for (int k = 0; k < per; ++k) word |= (uint32_t)kcodes[tau][wd * per + k] << (k * kb);
      reinterpret_cast<uint32_t*>(c.k_codes + (bh * c.T + t0 + tau) * (size_t)(16 * kb))[wd] = word;
    }
  }
}

__global__ void update_lengths_kernel(int32_t* seq_len, const int32_t* cu_new, int B) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) seq_len[b] += cu_new[b + 1] - cu_new[b];
}

}  // namespace

hipError_t launch_flush_keys(const CacheView& c, const AppendInputs& in, int max_blocks,
                             hipStream_t st) {
  dim3 grid(max_blocks, c.H, c.B);
  hipLaunchKernelGGL(flush_keys_kernel, grid, dim3(256), 0, st, c, in);
  return hipGetLastError();
}

hipError_t launch_append_tokens(const CacheView& c, const AppendInputs& in, int max_blocks,
                                hipStream_t st) {
  dim3 grid(max_blocks, c.H, c.B);
  hipLaunchKernelGGL(append_tokens_kernel, grid, dim3(256), 0, st, c, in);
  return hipGetLastError();
}

hipError_t launch_update_lengths(const CacheView& c, const int32_t* cu_new, hipStream_t st) {
  hipLaunchKernelGGL(update_lengths_kernel, dim3((c.B + 255) / 256), dim3(256), 0, st,
                     c.seq_len, cu_new, c.B);
  return hipGetLastError();
}

}  // namespace kvq
