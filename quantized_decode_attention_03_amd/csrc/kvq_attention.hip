// Fused-dequant decode attention (gfx950).
//
// Decode streams the whole cache once per token and is bound by memory
// bandwidth, so the packed integer codes are read directly and dequantized in
// registers, never materialized ("KV Cache Quantization — 8-bit and 4-bit",
// "Decode is memory-bound, so smaller is also faster"). Keys on the channel
// axis and values on the token axis carry their scales along different axes,
// so the inner loop handles both layouts plus the fp16 residual keys and the
// sparse key entries ("Sub-8-Bit KV Cache Quantization Is Not a Free Lever for
// an RDNA4 Agent Swarm", "The RDNA4 kernel angle").
//
// Work split: grid (split, KV head, sequence); each workgroup reduces a token
// range with an online softmax and writes (m, l, o[128]) per query head; a
// second kernel merges the splits with a log-sum-exp.
#include "kvq_device.h"

namespace kvq {

namespace {

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int KB, int VB, int KAXIS, int G, bool SPARSE>
__global__ __launch_bounds__(256) void attn_valu_kernel(CacheView c, AttnPlan p, const uint16_t* q,
                                                        float* ws) {
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int L = c.seq_len[b];
  const int Q = KAXIS ? L - L % c.R : L;
  const int ts0 = split * p.tokens_per_split;
  const int ts1 = min(ts0 + p.tokens_per_split, L);
  const size_t bh = (size_t)b * c.H + h;

  __shared__ float qs[G][kD];
  __shared__ float pw[4][G][32];
  __shared__ uint32_t vm[4][32];
  __shared__ float red_m[4][G], red_l[4][G];
  __shared__ float red_o[4][G][kD];

  for (int i = tid; i < G * kD; i += 256)
    qs[i / kD][i % kD] = h2f(q[((size_t)b * p.Hq + h * G + i / kD) * kD + i % kD]) * p.scale;
  __syncthreads();

  float m[G], l[G], o[G][2];
#pragma unroll
  for (int i = 0; i < G; ++i) { m[i] = -INFINITY; l[i] = 0.f; o[i][0] = o[i][1] = 0.f; }

  const int tau = lane & 31, half = lane >> 5;
  for (int t0 = ts0 + w * kBlock; t0 < ts1; t0 += 4 * kBlock) {
    const int nv = min(kBlock, ts1 - t0);
    const int t = t0 + tau;
    float dot[G];
#pragma unroll
    for (int i = 0; i < G; ++i) dot[i] = 0.f;
    if (tau < nv) {
      if (t < Q) {
        const uint8_t* row = c.k_codes + (bh * c.T + t) * (16 * KB);
        const uint32_t mt = KAXIS ? 0u : c.k_meta[bh * c.T + t];
        const uint32_t* mc = c.k_meta + (bh * (c.T / kBlock) + t / kBlock) * kD;
        for (int cc = 0; cc < 64; ++cc) {
          const int ch = half * 64 + cc;
          const float kh = dequant(get_field(row, ch, KB), KAXIS ? mc[ch] : mt, KB);
#pragma unroll
          for (int i = 0; i < G; ++i) dot[i] += qs[i][ch] * kh;
        }
        if (SPARSE && half == 0) {
          const uint32_t sv = c.k_sparse[(bh * c.T + t) * 2];
          const uint32_t sc = c.k_sparse[(bh * c.T + t) * 2 + 1];
          const float v0 = h2f((uint16_t)(sv & 0xFFFFu)), v1 = h2f((uint16_t)(sv >> 16));
#pragma unroll
          for (int i = 0; i < G; ++i) dot[i] += qs[i][sc & 0xFFFFu] * v0 + qs[i][sc >> 16] * v1;
        }
      } else {
        const uint16_t* rr = c.k_resid + (bh * c.R + (t - Q)) * kD;
        for (int cc = 0; cc < 64; ++cc) {
          const int ch = half * 64 + cc;
          const float kh = h2f(rr[ch]);
#pragma unroll
          for (int i = 0; i < G; ++i) dot[i] += qs[i][ch] * kh;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < G; ++i) dot[i] += __shfl_xor(dot[i], 32, 64);
    if (half == 0 && tau < nv) vm[w][tau] = c.v_meta[bh * c.T + t];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float sc = (tau < nv) ? dot[i] : -INFINITY;
      float mt = sc;
      for (int off = 16; off >= 1; off >>= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
      const float mn = fmaxf(m[i], mt);
      const float alpha = __expf(m[i] - mn);
      const float pv = (tau < nv) ? __expf(sc - mn) : 0.f;
      float ls = pv;
      for (int off = 16; off >= 1; off >>= 1) ls += __shfl_xor(ls, off, 64);
      l[i] = l[i] * alpha + ls;
      m[i] = mn;
      o[i][0] *= alpha;
      o[i][1] *= alpha;
      if (half == 0) pw[w][i][tau] = pv;
    }
    wave_sync_lds();
    const uint8_t* vblk = c.v_codes + (bh * (c.T / kBlock) + t0 / kBlock) * (size_t)(kD * 4 * VB);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int ch = 2 * lane + k;
      const uint8_t* rec = vblk + ch * 4 * VB;
      for (int tt = 0; tt < nv; ++tt) {
        const float vh = dequant(get_field(rec, tt, VB), vm[w][tt], VB);
#pragma unroll
        for (int i = 0; i < G; ++i) o[i][k] += pw[w][i][tt] * vh;
      }
    }
    wave_sync_lds();
  }

#pragma unroll
  for (int i = 0; i < G; ++i) {
    red_o[w][i][2 * lane] = o[i][0];
    red_o[w][i][2 * lane + 1] = o[i][1];
    if (lane == 0) { red_m[w][i] = m[i]; red_l[w][i] = l[i]; }
  }
  __syncthreads();
  for (int e = tid; e < G * kD; e += 256) {
    const int i = e / kD, ch = e % kD;
    float M = red_m[0][i];
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, red_m[ww][i]);
    float acc = 0.f, lsum = 0.f;
    if (M != -INFINITY) {
      for (int ww = 0; ww < 4; ++ww) {
        const float f = __expf(red_m[ww][i] - M);
        acc += f * red_o[ww][i][ch];
        lsum += f * red_l[ww][i];
      }
    }
    float* part = ws + (((size_t)b * p.Hq + h * G + i) * p.n_split + split) * kPartialFloats;
    if (ch == 0) { part[0] = M; part[1] = lsum; part[2] = 0.f; part[3] = 0.f; }
    part[4 + ch] = acc;
  }
}

// Log-sum-exp merge of the split partials: one workgroup per (sequence,
// query head), one thread per channel.
__global__ __launch_bounds__(128) void combine_kernel(const float* ws, float* out, int n_split) {
  const int bq = blockIdx.x, ch = threadIdx.x;
  const float* part = ws + (size_t)bq * n_split * kPartialFloats;
  float M = -INFINITY;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, part[s * kPartialFloats]);
  float acc = 0.f, lsum = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < n_split; ++s) {
      const float f = __expf(part[s * kPartialFloats] - M);
      acc += f * part[s * kPartialFloats + 4 + ch];
      lsum += f * part[s * kPartialFloats + 1];
    }
  }
  out[(size_t)bq * kD + ch] = (lsum > 0.f) ? acc / lsum : 0.f;
}

template <int KB, int VB, int KAXIS, int G, bool SPARSE>
hipError_t launch_t(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* ws,
                    hipStream_t st) {
  dim3 grid(p.n_split, c.H, c.B);
  hipLaunchKernelGGL((attn_valu_kernel<KB, VB, KAXIS, G, SPARSE>), grid, dim3(256), 0, st, c, p, q,
                     ws);
  return hipGetLastError();
}

template <int KB, int VB, int KAXIS, bool SPARSE>
hipError_t dispatch_g(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* ws,
                      hipStream_t st) {
  switch (p.group) {
    case 1: return launch_t<KB, VB, KAXIS, 1, SPARSE>(c, p, q, ws, st);
    case 2: return launch_t<KB, VB, KAXIS, 2, SPARSE>(c, p, q, ws, st);
    case 4: return launch_t<KB, VB, KAXIS, 4, SPARSE>(c, p, q, ws, st);
    case 8: return launch_t<KB, VB, KAXIS, 8, SPARSE>(c, p, q, ws, st);
  }
  return hipErrorInvalidValue;
}

template <int KB, int VB>
hipError_t dispatch_axis(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* ws,
                         hipStream_t st) {
  if (c.kaxis == 0) return dispatch_g<KB, VB, 0, false>(c, p, q, ws, st);
  if (c.sparse) return dispatch_g<KB, VB, 1, true>(c, p, q, ws, st);
  return dispatch_g<KB, VB, 1, false>(c, p, q, ws, st);
}

template <int KB>
hipError_t dispatch_vb(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* ws,
                       hipStream_t st) {
  switch (c.vbits) {
    case 8: return dispatch_axis<KB, 8>(c, p, q, ws, st);
    case 4: return dispatch_axis<KB, 4>(c, p, q, ws, st);
    case 2: return dispatch_axis<KB, 2>(c, p, q, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_attention(const CacheView& c, const AttnPlan& p, const uint16_t* q,
                                   float* out, float* ws, hipStream_t st) {
  hipError_t e;
  switch (c.kbits) {
    case 8: e = dispatch_vb<8>(c, p, q, ws, st); break;
    case 4: e = dispatch_vb<4>(c, p, q, ws, st); break;
    case 2: e = dispatch_vb<2>(c, p, q, ws, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(c.B * p.Hq), dim3(kD), 0, st, ws, out, p.n_split);
  return hipGetLastError();
}

}  // namespace kvq
