// Dequantize kernel (gfx950): the packed cache back to fp16 tensors.
//
// x_hat = scale * (q - zero_point) ("KV Cache Quantization — 8-bit and 4-bit",
// "Integer quantization in one screen"), exact in fp32 and rounded once to
// fp16; symmetric blocks x_hat = s * q (exact in fp32); fp8 x_hat = scale *
// value(code), the fp32 product rounded to fp16. This materializing pass is what the attention kernel avoids ("Decode
// is memory-bound, so smaller is also faster"); it exists for checking and
// for callers that need plain fp16 tensors.
#include "kvq_device.h"

namespace kvq {

namespace {

// fp32 reconstruction of element ch of token t (code u) for a token-axis cache
// side: meta points at that side's metadata array.
__device__ __forceinline__ float token_elem(const CacheView& c, uint32_t u, const uint32_t* meta, size_t tok,
                                           int ch, int bits, float scale) {
#pragma clang fp contract(off)
  if (c.fmt == kFmtFp8) return scale * e4m3_value(u);
  if (c.fmt == kFmtSym32) {
    const float s = h2f(reinterpret_cast<const uint16_t*>(meta)[tok * kSymBlocks + ch / 32]);
    return s * (float)((int)u + qmin_of(bits));
  }
  return dequant(u, meta[tok], bits);
}

// One workgroup per (32-token block, KV head, sequence); thread -> (token,
// 16 channels).
__global__ __launch_bounds__(256) void dequant_kernel(CacheView c, uint16_t* kout, uint16_t* vout) {
  const int b = blockIdx.z, h = blockIdx.y, j = blockIdx.x;
  const int tid = threadIdx.x;
  const int tau = tid >> 3, c0 = (tid & 7) * 16;
  const int t = j * kBlock + tau;
  const int L = min(max(c.seq_len[b], 0), c.T);  // clamped: never past the capacity
  const int Q = c.kaxis == 0 ? L : L - L % c.R;
  const size_t bh = (size_t)b * c.H + h;
  const size_t o = (((size_t)b * c.T + t) * c.H + h) * kD;
  const uint8_t* krow = c.k_codes + (bh * c.T + t) * (size_t)(16 * c.kbits);
  const uint8_t* vblk = c.v_codes + (bh * (c.T / kBlock) + j) * (size_t)(kD * 4 * c.vbits);
  uint32_t sp_val = 0, sp_col = 0xFFFFFFFFu;
  if (c.sparse && t < Q) {
    sp_val = c.k_sparse[(bh * c.T + t) * 2];
    sp_col = c.k_sparse[(bh * c.T + t) * 2 + 1];
  }
  for (int ch = c0; ch < c0 + 16; ++ch) {
    uint16_t kh = 0, vh = 0;
    if (t < Q) {
      const uint32_t u = get_field(krow, ch, c.kbits);
      float x = c.kaxis == 0 ? token_elem(c, u, c.k_meta, bh * c.T + t, ch, c.kbits, c.kscale)
                             : dequant(u, c.k_meta[(bh * (c.T / kBlock) + j) * kD + ch], c.kbits);
      if ((sp_col & 0xFFFFu) == (uint32_t)ch) x = x + h2f((uint16_t)(sp_val & 0xFFFFu));
      if ((sp_col >> 16) == (uint32_t)ch) x = x + h2f((uint16_t)(sp_val >> 16));
      kh = f2h_rne(x);
    } else if (t < L) {
      kh = c.k_resid[(bh * c.R + (t - Q)) * kD + ch];
    }
    if (t < L) {
      const float x = token_elem(c, get_field(vblk + ch * 4 * c.vbits, tau, c.vbits), c.v_meta, bh * c.T + t,
                                 ch, c.vbits, c.vscale);
      vh = f2h_rne(x);
    }
    kout[o + ch] = kh;
    vout[o + ch] = vh;
  }
}

}  // namespace

hipError_t launch_dequantize(const CacheView& c, uint16_t* k_out, uint16_t* v_out, hipStream_t st) {
  dim3 grid(c.T / kBlock, c.H, c.B);
  hipLaunchKernelGGL(dequant_kernel, grid, dim3(256), 0, st, c, k_out, v_out);
  return hipGetLastError();
}

}  // namespace kvq
