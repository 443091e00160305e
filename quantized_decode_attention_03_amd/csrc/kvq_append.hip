// Quantize-on-append kernels (gfx950).
//
// Values, and keys on the token axis, are quantized one token vector (128
// channels) at a time: one wavefront per token, two channels per lane, a
// cross-lane min/max reduction along the channel axis (max |x| over 16 lanes
// per 32-channel block for symmetric blocks; none for fp8, whose scale is per
// cache). Keys on the channel
// axis wait in the fp16 residual window; a window that fills is quantized as
// groups of one channel over 32 consecutive tokens (a min/max along the token
// axis), after the dense-and-sparse split when it is enabled. (KIVI's axis
// split and residual, KVQuant's per-vector outlier isolation: "Sub-8-Bit KV
// Cache Quantization Is Not a Free Lever for an RDNA4 Agent Swarm", "What the
// low-bit numbers actually cost"; the per-token/per-channel choice: "KV Cache
// Quantization — 8-bit and 4-bit", "Why keys and values want different
// treatment".)
//
// Counts read from the device (lengths, new-token offsets) are clamped to the
// cache capacity and to the rows of the packed input, so inconsistent
// arguments give wrong contents but never an access outside the buffers.
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

// Stored codes of channels 2 lane and 2 lane + 1 (values f0, f1) of one token
// vector held by a wavefront, in the cache's element format; the token's
// metadata goes to the token's slot `tok` of `meta`:
//   affine codes: one meta word per token (group = the 128 channels);
//   symmetric blocks: 4 fp16 scales per token (group = 32 channels = 16 lanes);
//   fp8: no metadata; code = e4m3(x / scale).
__device__ __forceinline__ uint2 quant_token(float f0, float f1, int fmt, int bits, float scale,
                                             uint32_t* meta, size_t tok, int lane) {
#pragma clang fp contract(off)
  if (fmt == kFmtFp8) return make_uint2(e4m3_code(f0 / scale), e4m3_code(f1 / scale));
  if (fmt == kFmtSym32) {
    float a = __builtin_fmaxf(__builtin_fabsf(f0), __builtin_fabsf(f1));
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off, 64));
    const uint16_t s16 = sym_scale16(a, bits);
    if ((lane & 15) == 0) reinterpret_cast<uint16_t*>(meta)[tok * kSymBlocks + (lane >> 4)] = s16;
    const float sc = h2f(s16), rc = __builtin_amdgcn_rcpf(sc);
    return make_uint2(sym_code(f0, sc, rc, bits), sym_code(f1, sc, rc, bits));
  }
  const float mn = wave_min(__builtin_fminf(f0, f1)), mx = wave_max(__builtin_fmaxf(f0, f1));
  const GroupQ g = group_params(mn, mx, bits);
  if (lane == 0) meta[tok] = g.meta;
  return make_uint2(quant_code(f0, g, bits), quant_code(f1, g, bits));
}

// Stored codes u[0..7] of channels 8 l .. 8 l + 7 (values x) of one token
// vector held by the 16 lanes l = lane mod 16 of a lane group, in the cache's
// element format (the arithmetic of quant_token); the token's metadata goes
// to slot `tok` of `meta` when `write` is set (lanes of a group that holds no
// token compute on a copy and write nothing).
__device__ __forceinline__ void quant_token8(const float (&x)[8], int fmt, int bits, float scale, uint32_t* meta,
                                             size_t tok, int l, bool write, uint32_t (&u)[8]) {
#pragma clang fp contract(off)
  if (fmt == kFmtFp8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = e4m3_code(x[i] / scale);
    return;
  }
  if (fmt == kFmtSym32) {  // a 32-channel block is 4 lanes
    float a = __builtin_fabsf(x[0]);
#pragma unroll
    for (int i = 1; i < 8; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(x[i]));
    a = __builtin_fmaxf(a, __shfl_xor(a, 1, 64));
    a = __builtin_fmaxf(a, __shfl_xor(a, 2, 64));
    const uint16_t s16 = sym_scale16(a, bits);
    if (write && (l & 3) == 0) reinterpret_cast<uint16_t*>(meta)[tok * kSymBlocks + (l >> 2)] = s16;
    const float sc = h2f(s16), rc = __builtin_amdgcn_rcpf(sc);
#pragma unroll
    for (int i = 0; i < 8; ++i) u[i] = sym_code(x[i], sc, rc, bits);
    return;
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    mn = __builtin_fminf(mn, x[i]);
    mx = __builtin_fmaxf(mx, x[i]);
  }
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) {
    mn = __builtin_fminf(mn, __shfl_xor(mn, off, 64));
    mx = __builtin_fmaxf(mx, __shfl_xor(mx, off, 64));
  }
  const GroupQ g = group_params(mn, mx, bits);
  if (write && l == 0) meta[tok] = g.meta;
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = quant_code(x[i], g, bits);
}

__device__ __forceinline__ void widen8(uint4 w, float (&x)[8]) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = h2f((uint16_t)(a[i] & 0xFFFFu));
    x[2 * i + 1] = h2f((uint16_t)(a[i] >> 16));
  }
}

__device__ __forceinline__ uint2 pack8(const uint32_t (&u)[8]) {
  return make_uint2(u[0] | (u[1] << 8) | (u[2] << 16) | (u[3] << 24), u[4] | (u[5] << 8) | (u[6] << 16) | (u[7] << 24));
}

// Sequence b's state before the append: L tokens held, its new tokens are
// rows row0 .. row0 + n - 1 of the packed input. Clamped: 0 <= L <= T,
// 0 <= row0 <= rows, 0 <= n <= min(T - L, rows - row0).
struct SeqNew {
  int L, row0, n;
};
__device__ __forceinline__ SeqNew seq_new(const CacheView& c, const AppendInputs& in, int b) {
  SeqNew s;
  s.L = min(max(c.seq_len[b], 0), c.T);
  s.row0 = min(max(in.cu_new[b], 0), in.rows);
  s.n = min(max(in.cu_new[b + 1] - s.row0, 0), min(in.rows - s.row0, c.T - s.L));
  return s;
}

// Per-channel key flush: one workgroup per (32-token block of the window,
// KV head, sequence). The window is tokens [Q, Q2) with Q = L - L mod R and
// Q2 = L2 - L2 mod R; tokens below L come from the residual, the rest from
// the new keys.
__global__ __launch_bounds__(256) void flush_keys_kernel(CacheView c, AppendInputs in) {
  const int b = blockIdx.z, h = blockIdx.y, blk = blockIdx.x;
  const int tid = threadIdx.x;
  const SeqNew sn = seq_new(c, in, b);
  const int L = sn.L, row0 = sn.row0, R = c.R;
  const int Q = L - L % R, L2 = L + sn.n, Q2 = L2 - L2 % R;
  const int t0 = Q + blk * kBlock;
  if (t0 + kBlock > Q2) return;
  const size_t bh = (size_t)b * c.H + h;

  __shared__ uint16_t xs[kBlock][kD];
  __shared__ uint8_t codes[kBlock][kD];
  __shared__ float part[2][2][kD];  // [min, max][token half][channel]

  {  // stage the 32 x 128 fp16 block: 8 threads per 256-byte token row
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

  // two threads per channel group, 16 tokens each: partial extremes, then
  // the group's scale and zero point (identical in both), then the codes
  const int ch = tid & (kD - 1), half = tid >> 7;
  const int tb = 16 * half;
  float xv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) xv[i] = h2f(xs[tb + i][ch]);
  float mn = xv[0], mx = xv[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    mn = __builtin_fminf(mn, xv[i]);
    mx = __builtin_fmaxf(mx, xv[i]);
  }
  part[0][half][ch] = mn;
  part[1][half][ch] = mx;
  __syncthreads();
  mn = __builtin_fminf(part[0][0][ch], part[0][1][ch]);
  mx = __builtin_fmaxf(part[1][0][ch], part[1][1][ch]);
  const GroupQ g = group_params(mn, mx, c.kbits);
  if (half == 0) c.k_meta[(bh * (c.T / kBlock) + t0 / kBlock) * kD + ch] = g.meta;
#pragma unroll
  for (int i = 0; i < 16; ++i) codes[tb + i][ch] = (uint8_t)quant_code(xv[i], g, c.kbits);
  __syncthreads();

  // pack token rows along channels (consecutive threads, consecutive words)
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
  const SeqNew sn = seq_new(c, in, b);
  const int L = sn.L, row0 = sn.row0, n = sn.n;
  if (n <= 0) return;
  const int L2 = L + n;
  const int j = L / kBlock + blockIdx.x;
  if (j > (L2 - 1) / kBlock) return;
  const int t0 = j * kBlock;
  const int tlo = max(L - t0, 0), thi = min(L2 - t0, kBlock);
  const size_t bh = (size_t)b * c.H + h;
  const bool ktok = c.kaxis == 0;
  const int Q2 = ktok ? L2 : L2 - L2 % c.R;

  __shared__ __attribute__((aligned(16))) uint8_t vcodes[kBlock][kD];
  __shared__ __attribute__((aligned(16))) uint8_t kcodes[kBlock][kD];

  // Four token vectors per wavefront at a time: lane group q (16 lanes, 8
  // channels each) takes token tlo + 16 r + 4 q + w in round r = 0, 1. Every
  // load is issued first, at a clamped token index; groups past the last
  // token compute on a copy and write nothing. (Keys only when they are
  // quantized here, on the token axis; channel-axis keys are read by the
  // flush, or below for the ones left in the window.)
  const int q4 = lane >> 4, l16 = lane & 15;
  uint4 vraw[2], kraw[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int tau = min(tlo + 16 * r + 4 * q4 + w, thi - 1);
    const size_t src = ((size_t)(row0 + t0 + tau - L) * c.H + h) * kD + 8 * l16;
    vraw[r] = *reinterpret_cast<const uint4*>(in.v_new + src);
    kraw[r] = ktok ? *reinterpret_cast<const uint4*>(in.k_new + src) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int tau = tlo + 16 * r + 4 * q4 + w;
    const bool live = tau < thi;
    const int tc = min(tau, thi - 1);
    float x[8];
    uint32_t u[8];
    widen8(vraw[r], x);
    quant_token8(x, c.fmt, c.vbits, c.vscale, c.v_meta, bh * c.T + t0 + tc, l16, live, u);
    if (live) *reinterpret_cast<uint2*>(&vcodes[tau][8 * l16]) = pack8(u);
    if (ktok) {
      widen8(kraw[r], x);
      quant_token8(x, c.fmt, c.kbits, c.kscale, c.k_meta, bh * c.T + t0 + tc, l16, live, u);
      if (live) *reinterpret_cast<uint2*>(&kcodes[tau][8 * l16]) = pack8(u);
    }
  }
  if (!ktok) {  // channel-axis keys that stay in the residual window
    for (int tau = max(tlo, Q2 - t0) + w; tau < thi; tau += 4) {
      const int t = t0 + tau;
      const size_t src = ((size_t)(row0 + t - L) * c.H + h) * kD;
      reinterpret_cast<uint32_t*>(c.k_resid + (bh * c.R + (t - Q2)) * kD)[lane] =
          reinterpret_cast<const uint32_t*>(in.k_new + src)[lane];
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

// Decode-step append: one new token for every sequence. One workgroup per
// sequence takes all its KV heads (a wavefront per head at a time), so it
// alone reads and then advances seq_len[b]: no separate length update. Same
// arithmetic and layout as append_tokens_kernel; the channel-axis flush of a
// window this token fills runs before it (flush_keys_kernel).
__global__ __launch_bounds__(256) void append_decode_kernel(CacheView c, AppendInputs in) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const SeqNew sn = seq_new(c, in, b);
  if (sn.n < 1) return;  // a full sequence keeps its length
  const int t = sn.L, L2 = sn.L + 1;
  const bool ktok = c.kaxis == 0;
  const int Q2 = ktok ? L2 : L2 - L2 % c.R;
  const int j = t / kBlock, tau = t % kBlock;
  const int vb = c.vbits, per = 32 / vb, wd = tau / per, f = tau % per;
  // fields of earlier tokens in a value-record word are kept, later ones are
  // zero (keep = 0 for the first token of a word)
  const uint32_t keep = (1u << (f * vb)) - 1u;
  // This wavefront's heads w, w + 4, ..., two at a time: every load first (the
  // new token's key and value rows and the two value-record words per lane it
  // extends; a clamped head index for the second when there is none), then the
  // quantization and the stores.
  for (int h0 = w; h0 < c.H; h0 += 8) {
    uint32_t pr[2], pk[2], o0[2], o1[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int h = min(h0 + 4 * x, c.H - 1);
      const size_t bh = (size_t)b * c.H + h;
      const size_t src = ((size_t)sn.row0 * c.H + h) * kD;
      pr[x] = reinterpret_cast<const uint32_t*>(in.v_new + src)[lane];
      pk[x] = reinterpret_cast<const uint32_t*>(in.k_new + src)[lane];
      const uint32_t* rec =
          reinterpret_cast<const uint32_t*>(c.v_codes + (bh * (c.T / kBlock) + j) * (size_t)(kD * 4 * vb));
      o0[x] = rec[(2 * lane) * vb + wd];
      o1[x] = rec[(2 * lane + 1) * vb + wd];
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int h = h0 + 4 * x;
      if (h >= c.H) break;
      const size_t bh = (size_t)b * c.H + h;
      {  // value codes of channels 2 lane and 2 lane + 1 into their records
        const uint2 u = quant_token(h2f((uint16_t)(pr[x] & 0xFFFFu)), h2f((uint16_t)(pr[x] >> 16)), c.fmt, c.vbits,
                                    c.vscale, c.v_meta, bh * c.T + t, lane);
        uint32_t* rec = reinterpret_cast<uint32_t*>(c.v_codes + (bh * (c.T / kBlock) + j) * (size_t)(kD * 4 * vb));
        rec[(2 * lane) * vb + wd] = (o0[x] & keep) | (u.x << (f * vb));
        rec[(2 * lane + 1) * vb + wd] = (o1[x] & keep) | (u.y << (f * vb));
      }
      if (ktok) {  // the token's key row, channels packed low bits first
        const uint2 u = quant_token(h2f((uint16_t)(pk[x] & 0xFFFFu)), h2f((uint16_t)(pk[x] >> 16)), c.fmt, c.kbits,
                                    c.kscale, c.k_meta, bh * c.T + t, lane);
        const uint32_t u0 = u.x, u1 = u.y;
        uint8_t* row = c.k_codes + (bh * c.T + t) * (size_t)(16 * c.kbits);
        if (c.kbits == 8) {
          reinterpret_cast<uint16_t*>(row)[lane] = (uint16_t)(u0 | (u1 << 8));
        } else if (c.kbits == 4) {
          row[lane] = (uint8_t)(u0 | (u1 << 4));
        } else {  // byte m holds channels 4m .. 4m+3: lanes 2m and 2m + 1
          const uint32_t v = u0 | (u1 << 2);
          const uint32_t o = (uint32_t)__shfl_xor((int)v, 1, 64);
          if ((lane & 1) == 0) row[lane >> 1] = (uint8_t)(v | (o << 4));
        }
      } else if (t >= Q2) {
        reinterpret_cast<uint32_t*>(c.k_resid + (bh * c.R + (t - Q2)) * kD)[lane] = pk[x];
      }
    }
  }
  __syncthreads();  // every wavefront has read the old length
  if (tid == 0) c.seq_len[b] = L2;
}

// Length update after append_tokens_kernel: one thread per sequence, the same
// clamped count the append kernels used.
__global__ void update_lengths_kernel(CacheView c, AppendInputs in) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < c.B) {
    const SeqNew sn = seq_new(c, in, b);
    c.seq_len[b] = sn.L + sn.n;
  }
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

hipError_t launch_append_decode(const CacheView& c, const AppendInputs& in, hipStream_t st) {
  hipLaunchKernelGGL(append_decode_kernel, dim3(c.B), dim3(256), 0, st, c, in);
  return hipGetLastError();
}

hipError_t launch_update_lengths(const CacheView& c, const AppendInputs& in, hipStream_t st) {
  hipLaunchKernelGGL(update_lengths_kernel, dim3((c.B + 255) / 256), dim3(256), 0, st, c, in);
  return hipGetLastError();
}

}  // namespace kvq
