// Fused-dequant decode attention on the matrix cores (gfx950).
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
// Shape of the work. The g query heads that share a KV head turn both products
// into small dense contractions, so they run on v_mfma_f32_16x16x32_f16:
//   S^T[token, col] = sum_c A[token, c] * B[c, col]
//   O[row, c]       = sum_t P[row, t] * V[t, c]
// Codes enter the matrix cores as their own bit patterns: a stored code u
// placed at bit SH of an fp16 (u << SH < 2^10) is the subnormal u * 2^(SH-24),
// which the matrix cores multiply exactly. Unpacking is therefore only shifts
// and masks. SH is 8 for 2-bit codes, 4 for 4-bit and 0 for 8-bit: chains of
// accumulating MFMAs lose accuracy when the operands are very small (measured:
// 2-bit codes at u * 2^-24 gave key-score errors near 2e-3, at u * 2^-16 near
// 5e-6 on the same data), so small codes sit as high in the subnormal range
// as the shift-and-mask extraction allows. The zero points are not subtracted element by element; their
// contribution is a rank-one term that runs on the matrix cores as well:
//   keys, channel axis: x = s_c (u - z'_c); B = q * s_c (scaled query, split
//     into fp16 hi and lo parts in columns h and g + h, ~22 bits); the term
//     sum_c z'_c B[c, col] is the same for every token of a block and seeds
//     the accumulator (an A operand whose rows all hold -z', in the same
//     code-step units as the codes);
//   keys, token axis: x = s_t (u - z'_t); B = raw fp16 query (exact); the
//     term z'_t sum_c q_c seeds the accumulator the same way (row t of the A
//     operand holds -z'_t); s_t multiplies the scores afterwards;
//   values, token axis: x = s_t (u - z'_t); P = p_t * s_t * 2^kv as hi/lo rows
//     h and g + h; the product with a B operand whose columns all hold z'_t
//     is subtracted once at the end.
// The factor 2^kv keeps p * s inside fp16: it is one exponent per wavefront,
// raised lazily (rarely) when a larger value scale shows up, like the softmax
// reference.
//
// Work split: grid (split, KV head, sequence), 4 wavefronts per workgroup,
// each wavefront owns every 4th 32-token tile of the split and keeps its own
// online softmax; the wavefronts merge through LDS. Sequences longer than one
// split leave (m, l, o) partials in the workspace that a second, small kernel
// merges with a log-sum-exp. (Merging in the last-arriving workgroup instead
// needs device-scope fences, whose L2 writeback and invalidation cost far more
// than the extra launch on this chip.)
#include <algorithm>
#include <atomic>

#include "kvq_device.h"

namespace kvq {

namespace {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTwoM24 = 1.f / 16777216.f;     // 2^-24, the smallest fp16 subnormal
#ifndef KVQ_WAVE_LDS_BUDGET
#define KVQ_WAVE_LDS_BUDGET 19968
#endif
constexpr int kWaveBudget = KVQ_WAVE_LDS_BUDGET;  // LDS bytes per wavefront

struct Frag {  // 8 fp16 MFMA operand values as 4 packed pairs
  uint32_t p[4];
};

__device__ __forceinline__ h2v as_h2(uint32_t x) { return __builtin_bit_cast(h2v, x); }
__device__ __forceinline__ uint32_t as_u32(h2v x) { return __builtin_bit_cast(uint32_t, x); }

// fp16 halves of a word, widened (v_cvt or folded into a v_fma_mix_f32)
__device__ __forceinline__ float f16lo(uint32_t w) { return (float)as_h2(w)[0]; }
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)as_h2(w)[1]; }
// x * (fp16 low half of w) as one v_fma_mix_f32 (a -0 product comes out +0)
__device__ __forceinline__ float mul_lo(float x, uint32_t w) { return __builtin_fmaf(x, f16lo(w), 0.f); }

// fp16 pair (a * m + c, b * m + c) of the fp16 halves of w (one v_pk_fma_f16)
__device__ __forceinline__ uint32_t pk_fma16(uint32_t w, _Float16 m, _Float16 c) {
  const h2v mm = {m, m}, cc = {c, c};
  return as_u32(__builtin_elementwise_fma(as_h2(w), mm, cc));
}

__device__ __forceinline__ f4v mfma(const Frag& a, const Frag& b, f4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8v, a),
                                                 __builtin_bit_cast(h8v, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// fp16 pair (RTZ) of two floats.
__device__ __forceinline__ uint32_t pk_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// Bit position of a code inside its fp16 operand (the code's value is
// u * 2^(SH-24)).
template <int BITS>
constexpr int code_shift() { return BITS == 2 ? 8 : (BITS == 4 ? 4 : 0); }

// Two fields of BITS bits, at bit n and n + 16 of w, moved to bit SH of each
// half: the fp16 pair (u0 * 2^(SH-24), u1 * 2^(SH-24)).
template <int BITS>
__device__ __forceinline__ uint32_t field_pair(uint32_t w, int n) {
  constexpr int SH = code_shift<BITS>();
  constexpr uint32_t kMask = (((1u << BITS) - 1u) << SH) * 0x10001u;
  if (n == SH) return w & kMask;
  if (n < SH) return (w << (SH - n)) & kMask;
  return (w >> (n - SH)) & kMask;
}

// 8 codes -> 4 fp16 code pairs, k-slot pairs (2p, 2p+1) taking:
//   BITS 4: word a, nibbles (p, p+4);
//   BITS 2: word a, 2-bit fields (4y + p, 4y + p + 8), y = 0 or 1;
//   BITS 8: bytes (2p, 2p+1) of the 8 bytes a, b.
template <int BITS>
__device__ __forceinline__ Frag codes8(uint32_t a, uint32_t b, int y) {
  Frag f;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int p = 0; p < 4; ++p) f.p[p] = field_pair<4>(a, 4 * p);
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int p = 0; p < 4; ++p) f.p[p] = field_pair<2>(a, 8 * y + 2 * p);
  } else {
    f.p[0] = perm(0u, a, 0x0C010C00u);
    f.p[1] = perm(0u, a, 0x0C030C02u);
    f.p[2] = perm(0u, b, 0x0C010C00u);
    f.p[3] = perm(0u, b, 0x0C030C02u);
  }
  return f;
}

// Channel of k-slot pair p (first or second slot) in chunk j of lane group
// grp, for key codes of BITS bits. Key rows are channel-packed with the low
// bits first; this is the order codes8() produces.
template <int BITS>
__device__ __forceinline__ int key_channel(int grp, int j, int p, int second) {
  if constexpr (BITS == 8) return 32 * grp + 8 * j + 2 * p + second;
  if constexpr (BITS == 4) return 32 * grp + 8 * j + p + 4 * second;
  return 32 * grp + 16 * (j >> 1) + 4 * (j & 1) + p + 8 * second;
}

// Geometry of one 32-token tile as staged in LDS:
//   [key codes 32 x 16*KB][value block 128 x 4*VB][value meta 32 words]
//   [key meta: 128 words (channel axis) or 32 (token axis)][sparse 32 x 2 words]
// Key codes and the value block are contiguous in global memory and move
// with 1 KiB direct-to-LDS loads (64 lanes x 16 bytes); the metadata pieces
// follow with one load per array, each lane group gathering 16-byte chunks
// into consecutive LDS.
template <int KB, int VB, int KAXIS, int G, bool SPARSE>
struct Geom {
  static constexpr int kRowK = 16 * KB;               // key code bytes per token
  static constexpr int kK = 32 * kRowK;               // key codes of a tile
  static constexpr int kV = 512 * VB;                 // value block
  static constexpr int kVm = 128;
  static constexpr int kKm = KAXIS ? 512 : 128;
  static constexpr int kSp = SPARSE ? 256 : 0;
  static constexpr int kMetaLanes = (kVm + kKm + kSp) / 16;
  static constexpr int kBytes = kK + kV + kVm + kKm + kSp;
  static constexpr int kLoads = kK / 1024 + kV / 1024 + (SPARSE ? 3 : 2);  // DMA instructions per tile
  // the key-product B operand and zero-point operand (channel axis only)
  static constexpr int kWaveLds = KAXIS ? (4 * (2 * G + 1) * 4 * 16 + 4 * 4 * 4 * 4) : 0;
  // tile slots per wavefront: as many as fit the per-wavefront LDS budget
  // (kWaveBudget, chosen so that several 4-wavefront workgroups share a CU's
  // 160 KiB), between 2 and 4
  static constexpr int kSlotsFit = (kWaveBudget - kWaveLds) / kBytes;
  static constexpr int kSlots = kSlotsFit < 2 ? 2 : (kSlotsFit > 4 ? 4 : kSlotsFit);
  static_assert(kK % 1024 == 0 && kV % 1024 == 0, "1 KiB load granularity");
  static_assert(kMetaLanes <= 64, "metadata fits one load");
};

// Buffer resource (V#) over `bytes` bytes at `base`: a raw descriptor (stride
// 0) whose loads read zeros, without touching memory, at any offset at or past
// `bytes`. The four words are made wave-uniform (readfirstlane), each as a
// 32-bit value, so they live in SGPRs.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  u32x4 r;
  r.x = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) & 0xFFFFu;  // stride 0
  r.z = (uint32_t)__builtin_amdgcn_readfirstlane((int)bytes);                          // num_records
  r.w = 0x00020000u;  // 32-bit data format, no swizzle, no index
  return r;
}

// 16 bytes per lane from a buffer (byte offset voff) straight into LDS at
// lds_base + 16 * lane (gfx950 buffer_load_dwordx4 ... lds). Issued from
// inline assembly so that the compiler neither waits on it at every LDS read
// nor keeps stale LDS values across it; completion is awaited explicitly with
// wait_vm(). The offset sits entirely in the VGPR operand (no SGPR or
// immediate offset), which is what the range check covers.
__device__ __forceinline__ void dma16(u32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// LDS per wavefront for channel-axis keys: the B operand of the key product
// for the current block (hi rows 0..G-1, lo rows G..2G-1, an all-zero row 2G;
// [grp][row][chunk] fragments) and the zero-point A operand, -z' in code-step units per
// channel ([grp][chunk][pair]).
template <int G>
struct WaveLds {
  Frag qb[4][2 * G + 1][4];
  uint32_t zc[4][4][4];
};

template <int G>
struct MergeLds {
  float o[4][2 * G][kD];
  float m[4][G];
  float l[4][G];
};

// max / sum over lanes l, l^16, l^32, l^48 (the four lane groups of one
// column); used only when the softmax reference moves and once per split
__device__ __forceinline__ float grp_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float grp_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// The softmax reference m of a head moves only when a score exceeds it by
// more than 2^kLazy (log2 units), so most tiles need no cross-lane maximum and
// no rescaling; weights stay <= 2^kLazy.
constexpr float kLazy = 8.f;

// The value-scale factor 2^kv, kv = kKvTop - E, is set from the largest fp16
// biased exponent E among the value scales seen so far, so that s * 2^kv < 2^6
// and the P operand p * s * 2^kv < 2^14 stays inside fp16.
constexpr int kKvTop = 20;

// Token (0..31 within the tile) of A row m in MFMA row block e: row block e
// holds tokens 8*(m/4) + 4e + m%4, so the output lane group g ends up with
// the 8 consecutive tokens 8g..8g+7, the k-slots of its P operand.
__device__ __forceinline__ int a_token(int e, int m) { return 8 * (m >> 2) + 4 * e + (m & 3); }

__device__ __forceinline__ uint16_t umax16(uint16_t a, uint16_t b) { return a > b ? a : b; }

template <int KB, int VB, int KAXIS, int G, bool SPARSE>
__global__ __launch_bounds__(256) void attn_kernel(CacheView c, AttnPlan p, const uint16_t* __restrict__ q,
                                                   float* __restrict__ out, float* __restrict__ ws) {
  using Gm = Geom<KB, VB, KAXIS, G, SPARSE>;
  constexpr int NB = Gm::kSlots;
  constexpr int kQMinK = -(1 << (KB - 1));
  constexpr int kQMinV = -(1 << (VB - 1));
  constexpr bool kPermV = VB != 8;  // k-slot pairs (i, i+4) for 4/2-bit values
  static_assert(2 * G <= 16, "hi/lo rows must fit 16");
  // value of one code step in the key / value operands, and its inverse
  constexpr int kShK = code_shift<KB>(), kShV = code_shift<VB>();
  const float kUnitK = __builtin_bit_cast(float, (uint32_t)(127 - 24 + kShK) << 23);
  const float kInvUnitK = __builtin_bit_cast(float, (uint32_t)(127 + 24 - kShK) << 23);

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c16 = lane & 15, grp = lane >> 4;
  const int L = min(max(c.seq_len[b], 0), c.T);  // clamped: never past the capacity
  const int nsplit_b = (L + p.tokens_per_split - 1) / p.tokens_per_split;
  if (split > 0 && split >= nsplit_b) return;  // beyond this sequence (split 0 always runs)
  const int Q = KAXIS ? L - L % c.R : L;
  const int ts0 = split * p.tokens_per_split;
  const int ts1 = min(ts0 + p.tokens_per_split, L);
  const size_t bh = (size_t)b * c.H + h;
  const int hq = c16 & (G - 1);           // head of this lane's column / row
  const bool live = c16 < 2 * G;          // lanes whose column / row is used

  constexpr int kWaveBytes = NB * Gm::kBytes + Gm::kWaveLds;
  constexpr int kMain = 4 * kWaveBytes;
  constexpr int kMerge = (int)sizeof(MergeLds<G>);
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMain > kMerge ? kMain : kMerge];
  __shared__ float qsh[SPARSE ? G : 1][kD];

  uint8_t* wbase = smem + w * kWaveBytes;             // this wavefront's slots
  WaveLds<G>& wl = *reinterpret_cast<WaveLds<G>*>(wbase + NB * Gm::kBytes);
  const uint32_t wbase_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)wbase;

  // query heads of this KV head, pre-scaled by softmax_scale * log2(e)
  const float qscale = p.scale * kLog2e;
  const uint16_t* qg = q + ((size_t)b * p.Hq + (size_t)h * G) * kD;
  if constexpr (SPARSE) {  // sparse entries add q * x directly to the scaled score
    for (int i = tid; i < G * kD; i += 256) qsh[i / kD][i % kD] = h2f(qg[i]) * (qscale * kUnitK);
    __syncthreads();
  }

  // Channel axis: this lane builds the scaled query of 2 channels, all heads:
  // k-slot pair bp of chunk bj in lane group bg, bq = lane / 4 = 4 bg + bj.
  const int bq = lane >> 2, bp = lane & 3, bg = bq >> 2, bj = bq & 3;
  const int bc0 = key_channel<KB>(bg, bj, bp, 0), bc1 = key_channel<KB>(bg, bj, bp, 1);
  float qv0[G], qv1[G];
  // token axis: the B operand is the raw fp16 query (exact), column n = head n mod G
  Frag qfrag[KAXIS ? 1 : 4];
  // rows of the key-product B operand this lane reads (the zero row when unused)
  const int brow_hi = live ? hq : 2 * G;
  const int brow_lo = live ? G + hq : 2 * G;
  if constexpr (KAXIS) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      qv0[hh] = h2f(qg[hh * kD + bc0]) * qscale;
      qv1[hh] = h2f(qg[hh * kD + bc1]) * qscale;
    }
    if (lane < 16) wl.qb[lane >> 2][2 * G][lane & 3] = Frag{{0u, 0u, 0u, 0u}};
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int pp = 0; pp < 4; ++pp) {
        uint32_t v = 0;
        if (live) {
          const int ch0 = key_channel<KB>(grp, j, pp, 0), ch1 = key_channel<KB>(grp, j, pp, 1);
          v = (uint32_t)qg[hq * kD + ch0] | ((uint32_t)qg[hq * kD + ch1] << 16);
        }
        qfrag[j].p[pp] = v;
      }
    }
  }

  // This wavefront's tiles: k = w, w + 4, ... over [ts0, ts1).
  const int ntiles = (ts1 - ts0 + kBlock - 1) / kBlock;
  const int tq = (Q > ts0) ? min((Q - ts0 + kBlock - 1) / kBlock, ntiles) : 0;  // quantized tiles
  const int nw = (w < tq) ? (tq - w + 3) / 4 : 0;                               // of them, mine

  // Tile loads go through bounded descriptors over this (sequence, KV head)'s
  // slice of each cache array, so an offset outside the slice reads zeros
  // and never touches other memory. Byte offsets of the next tile to issue:
  // key codes and value blocks, the tile's start plus lane * 16 (+ 1 KiB
  // steps); metadata, each lane its 16-byte piece of one of the arrays (value
  // scales, key scales, sparse entries; one load per array). Offsets advance
  // by 4 tiles per issue (the wavefront takes every 4th tile).
  const int tw0 = ts0 + w * kBlock;
  const uint32_t Tu = (uint32_t)c.T;
  const u32x4 rk = make_rsrc(c.k_codes + bh * c.T * (size_t)Gm::kRowK, Tu * Gm::kRowK);
  const u32x4 rv = make_rsrc(c.v_codes + bh * (c.T / kBlock) * (size_t)Gm::kV, (Tu / kBlock) * Gm::kV);
  const u32x4 rvm = make_rsrc(c.v_meta + bh * c.T, Tu * 4);
  const u32x4 rkm = KAXIS ? make_rsrc(c.k_meta + bh * (c.T / kBlock) * kD, (Tu / kBlock) * kD * 4)
                          : make_rsrc(c.k_meta + bh * c.T, Tu * 4);
  const u32x4 rsp = SPARSE ? make_rsrc(c.k_sparse + bh * c.T * 2, Tu * 8) : rvm;
  uint32_t koff = (uint32_t)tw0 * Gm::kRowK + lane * 16;
  uint32_t voff = (uint32_t)(tw0 / kBlock) * Gm::kV + lane * 16;
  // metadata lanes: 0..7 value scales, then key scales, then sparse entries
  const int mkind = lane < 8 ? 0 : (lane < 8 + Gm::kKm / 16 ? 1 : 2);
  uint32_t moff, mstep;
  if (mkind == 0) {
    moff = (uint32_t)tw0 * 4 + lane * 16;
    mstep = 4 * kBlock * 4;
  } else if (mkind == 1) {
    moff = (KAXIS ? (uint32_t)(tw0 / kBlock) * kD * 4 : (uint32_t)tw0 * 4) + (lane - 8) * 16;
    mstep = KAXIS ? 4 * kD * 4 : 4 * kBlock * 4;
  } else {
    moff = (uint32_t)tw0 * 8 + (uint32_t)(lane - 8 - Gm::kKm / 16) * 16;
    mstep = 4 * kBlock * 8;
  }

  // DMA of the next tile of this wavefront into slot `slot`.
  auto issue = [&](int slot) {
    const uint32_t lb = wbase_lds + slot * Gm::kBytes;
#pragma unroll
    for (int x = 0; x < Gm::kK / 1024; ++x) dma16(rk, koff + x * 1024, lb + x * 1024);
#pragma unroll
    for (int x = 0; x < Gm::kV / 1024; ++x) dma16(rv, voff + x * 1024, lb + Gm::kK + x * 1024);
    const uint32_t lbm = lb + Gm::kK + Gm::kV;
    if (mkind == 0) dma16(rvm, moff, lbm);
    if (mkind == 1) dma16(rkm, moff, lbm);
    if constexpr (SPARSE) {
      if (mkind == 2 && lane < Gm::kMetaLanes) dma16(rsp, moff, lbm);
    }
    koff += 4 * Gm::kK;
    voff += 4 * Gm::kV;
    moff += mstep;
  };

  float m_ref = -INFINITY, l_run = 0.f;
  int vE = 0;                       // exponent the value-scale factor is set for
  f4v acc[8], accz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f4v{0.f, 0.f, 0.f, 0.f};
  const float rowlo = (c16 >= G && c16 < 2 * G) ? 1.f : 0.f;  // lo rows of P
  // zero-point operands: (z - qmin) in code-step units, from the fp16 z
  constexpr _Float16 kZk = (_Float16)((float)(1 << kShK) * kTwoM24);
  constexpr _Float16 kZkOfs = (_Float16)(kQMinK * (float)(1 << kShK) * kTwoM24);
  constexpr _Float16 kZv = (_Float16)((float)(1 << kShV) * kTwoM24);
  constexpr _Float16 kZvOfs = (_Float16)(-kQMinV * (float)(1 << kShV) * kTwoM24);

  // ---- scores of one tile -> online softmax -> P.V ---------------------------
  // sc[4e + r] is the scaled score (score = sc * cs + const) of token
  // 8grp + 4e + r; vm[i] the value meta of token 8grp + i; vcl/vch[j] the
  // lane's value codes of channel chunk j.
  auto softmax_pv = [&](float (&sc)[8], float cs, const uint32_t (&vm)[8], const uint32_t (&vcl)[8],
                        const uint32_t (&vch)[8], int t0) {
    const int nvalid = ts1 - t0;
    if (nvalid < kBlock) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (8 * grp + i >= nvalid) sc[i] = -INFINITY;
    }
    const float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])),
                           fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    if (__builtin_amdgcn_ballot_w64(live && __builtin_fmaf(mx, cs, -m_ref) > kLazy)) {
      const float m_new = fmaxf(m_ref, grp_max(mx * cs));
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, (4 * grp + r) & (G - 1), 64);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j][r] *= ar[r];
        accz[r] *= ar[r];
      }
      l_run *= alpha;
      m_ref = m_new;
    }
    // value-scale exponent: raise it when a scale of this tile reaches 2^6 * 2^-kv
    const uint16_t smax =
        umax16(umax16(umax16((uint16_t)vm[0], (uint16_t)vm[1]), umax16((uint16_t)vm[2], (uint16_t)vm[3])),
               umax16(umax16((uint16_t)vm[4], (uint16_t)vm[5]), umax16((uint16_t)vm[6], (uint16_t)vm[7])));
    if (__builtin_amdgcn_ballot_w64(smax >= (uint16_t)((vE + 1) << 10))) {
      uint32_t sm = smax;
      sm = max(sm, (uint32_t)__shfl_xor((int)sm, 16, 64));
      sm = max(sm, (uint32_t)__shfl_xor((int)sm, 32, 64));
      const int e_new = max(vE, (int)__builtin_amdgcn_readfirstlane(sm >> 10));
      const float f = __builtin_bit_cast(float, (uint32_t)(127 + vE - e_new) << 23);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j][r] *= f;
        accz[r] *= f;
      }
      l_run *= f;
      vE = e_new;
    }
    const float kvm = (float)(kKvTop - vE) - m_ref;
    // P = p * s * 2^kv; lo rows keep p * s * 2^kv - fp16(p * s * 2^kv)
    float a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], cs, kvm));
      l_run += x;
      a[i] = mul_lo(x, vm[i]);
    }
    Frag pf, bz;
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int i0 = kPermV ? pp : 2 * pp;
      const int i1 = kPermV ? pp + 4 : 2 * pp + 1;
      const uint32_t hi = pk_rtz(a[i0], a[i1]);
      pf.p[pp] = pk_rtz(__builtin_fmaf(f16lo(hi), -rowlo, a[i0]), __builtin_fmaf(f16hi(hi), -rowlo, a[i1]));
      // (z'_i0, z'_i1) in code-step units, z' = z - qmin
      bz.p[pp] = pk_fma16(perm(vm[i1], vm[i0], 0x07060302u), kZv, kZvOfs);
    }
    accz = mfma(pf, bz, accz);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = mfma(pf, codes8<VB>(vcl[j], vch[j], 1), acc[j]);
  };

  // the B operand of the key product for a block: scaled query (hi/lo) with
  // the per-channel scales in the low halves of km0, km1; with_zero also
  // writes the zero-point operand -(z - qmin) (code-step units) from their high halves
  auto build_qb = [&](uint32_t km0, uint32_t km1, bool with_zero) {
    wave_lds_fence();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float v0 = mul_lo(qv0[hh], km0), v1 = mul_lo(qv1[hh], km1);
      const uint32_t hi = pk_rtz(v0, v1);
      wl.qb[bg][hh][bj].p[bp] = hi;
      wl.qb[bg][G + hh][bj].p[bp] = pk_rtz(__builtin_fmaf(f16lo(hi), -1.f, v0), __builtin_fmaf(f16hi(hi), -1.f, v1));
    }
    if (with_zero) wl.zc[bg][bj][bp] = pk_fma16(perm(km1, km0, 0x07060302u), -kZk, kZkOfs);
    wave_lds_fence();
  };

  // ---- quantized tiles through the LDS pipeline -----------------------------
  if (nw > 0) {
#pragma unroll
    for (int i = 0; i < NB - 1; ++i)
      if (i < nw) issue(i);
    for (int i = 0; i < nw; ++i) {
      const int slot = i % NB;
      if (i + NB - 1 < nw) issue((i + NB - 1) % NB);
      // tile i has landed once at most (tiles issued after it) x loads remain
      switch (min(NB - 1, nw - 1 - i)) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<Gm::kLoads>(); break;
        case 2: wait_vm<(NB > 2 ? 2 : 1) * Gm::kLoads>(); break;
        default: wait_vm<(NB > 3 ? 3 : 1) * Gm::kLoads>(); break;
      }
      const uint8_t* sb = wbase + slot * Gm::kBytes;
      const uint8_t* kbuf = sb;
      const uint8_t* vbuf = sb + Gm::kK;
      const uint32_t* vmeta = reinterpret_cast<const uint32_t*>(sb + Gm::kK + Gm::kV);
      const uint32_t* kmeta = vmeta + 32;
      const uint32_t* spr = kmeta + Gm::kKm / 4;
      const int t0 = ts0 + (w + 4 * i) * kBlock;

      uint32_t vm[8];
      {
        const uint4 a = reinterpret_cast<const uint4*>(vmeta + 8 * grp)[0];
        const uint4 bb = reinterpret_cast<const uint4*>(vmeta + 8 * grp)[1];
        vm[0] = a.x; vm[1] = a.y; vm[2] = a.z; vm[3] = a.w;
        vm[4] = bb.x; vm[5] = bb.y; vm[6] = bb.z; vm[7] = bb.w;
      }
      // key codes of the lane's two A rows: bytes [grp*4KB, +4KB) of each row
      uint32_t kc[2][KB];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint8_t* row = kbuf + a_token(e, c16) * Gm::kRowK + grp * 4 * KB;
#pragma unroll
        for (int x = 0; x < KB; x += 2) {
          const uint2 y = reinterpret_cast<const uint2*>(row)[x / 2];
          kc[e][x] = y.x;
          kc[e][x + 1] = y.y;
        }
      }
      auto key_frag = [&](int e, int j) -> Frag {
        if constexpr (KB == 4) return codes8<4>(kc[e][j], 0u, 0);
        else if constexpr (KB == 8) return codes8<8>(kc[e][2 * j], kc[e][2 * j + 1], 0);
        else return codes8<2>(kc[e][j >> 1], 0u, j & 1);
      };
      float sc[8];
      float cs;
      if constexpr (KAXIS) {
        build_qb(kmeta[bc0], kmeta[bc1], true);
        // zero-point term, the same for every token of the block
        f4v cz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const Frag az = *reinterpret_cast<const Frag*>(wl.zc[grp][j]);
          cz = mfma(az, wl.qb[grp][brow_hi][j], cz);
          cz = mfma(az, wl.qb[grp][brow_lo][j], cz);
        }
        f4v s[2] = {cz, cz};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const Frag qh = wl.qb[grp][brow_hi][j];
          const Frag ql = wl.qb[grp][brow_lo][j];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const Frag kf = key_frag(e, j);
            s[e] = mfma(kf, qh, s[e]);
            s[e] = mfma(kf, ql, s[e]);
          }
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[4 * e + r] = s[e][r];
        cs = kInvUnitK;
      } else {
        uint32_t km[8];
        {
          const uint4 a = reinterpret_cast<const uint4*>(kmeta + 8 * grp)[0];
          const uint4 bb = reinterpret_cast<const uint4*>(kmeta + 8 * grp)[1];
          km[0] = a.x; km[1] = a.y; km[2] = a.z; km[3] = a.w;
          km[4] = bb.x; km[5] = bb.y; km[6] = bb.z; km[7] = bb.w;
        }
        f4v s[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          // zero-point term of the row's token: -(z - qmin) * sum_c q_c
          const uint32_t ka = kmeta[a_token(e, c16)];
          const uint32_t az1 = pk_fma16(perm(ka, ka, 0x07060706u), -kZk, kZkOfs);
          const Frag az = {{az1, az1, az1, az1}};
          s[e] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j) s[e] = mfma(az, qfrag[j], s[e]);
#pragma unroll
          for (int j = 0; j < 4; ++j) s[e] = mfma(key_frag(e, j), qfrag[j], s[e]);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[4 * e + r] = mul_lo(s[e][r], km[4 * e + r]);
        cs = kInvUnitK * qscale;
      }
      if constexpr (SPARSE) {
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) {
          const uint2 rec = reinterpret_cast<const uint2*>(spr)[8 * grp + i2];
          sc[i2] += qsh[hq][rec.y & 0xFFFFu] * f16lo(rec.x) + qsh[hq][rec.y >> 16] * f16hi(rec.x);
        }
      }
      // value codes: channel 16j + c16, tokens 8grp .. 8grp+7 of the block
      uint32_t vcl[8], vch[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint8_t* rec = vbuf + (16 * j + c16) * 4 * VB;
        if constexpr (VB == 4) {
          vcl[j] = reinterpret_cast<const uint32_t*>(rec)[grp];
          vch[j] = 0u;
        } else if constexpr (VB == 8) {
          const uint2 x = reinterpret_cast<const uint2*>(rec)[grp];
          vcl[j] = x.x;
          vch[j] = x.y;
        } else {
          // 8 two-bit fields -> byte 1 (tokens 0..3) and byte 3 (tokens 4..7)
          vcl[j] = perm(0u, reinterpret_cast<const uint16_t*>(rec)[grp], 0x010C000Cu);
          vch[j] = 0u;
        }
      }
      softmax_pv(sc, cs, vm, vcl, vch, t0);
    }
  }

  // ---- residual (fp16) key tiles: channel axis only ------------------------
  if constexpr (KAXIS) {
    for (int k = tq + ((w - tq) % 4 + 4) % 4; k < ntiles; k += 4) {
      const int t0 = ts0 + k * kBlock;
      uint32_t vm[8], vcl[8], vch[8];
      {
        const uint8_t* vblk = c.v_codes + (bh * (c.T / kBlock) + t0 / kBlock) * (size_t)Gm::kV;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint8_t* rec = vblk + (16 * j + c16) * 4 * VB;
          if constexpr (VB == 4) { vcl[j] = reinterpret_cast<const uint32_t*>(rec)[grp]; vch[j] = 0u; }
          else if constexpr (VB == 8) {
            const uint2 x = reinterpret_cast<const uint2*>(rec)[grp];
            vcl[j] = x.x; vch[j] = x.y;
          } else {
            vcl[j] = perm(0u, reinterpret_cast<const uint16_t*>(rec)[grp], 0x010C000Cu);
            vch[j] = 0u;
          }
        }
        const uint4* vmg = reinterpret_cast<const uint4*>(c.v_meta + bh * c.T + t0 + 8 * grp);
        const uint4 a = vmg[0], bb = vmg[1];
        vm[0] = a.x; vm[1] = a.y; vm[2] = a.z; vm[3] = a.w;
        vm[4] = bb.x; vm[5] = bb.y; vm[6] = bb.z; vm[7] = bb.w;
      }
      // B operand: query scaled by the softmax factor only (scale 1.0), hi/lo
      build_qb(0x3C00u, 0x3C00u, false);
      f4v s[2] = {f4v{0.f, 0.f, 0.f, 0.f}, f4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int tt = t0 + a_token(e, c16);
        const bool ok = tt < ts1;
        // the lane group's 32 fp16 keys, channels 32grp .. 32grp+31
        const uint4* kr = reinterpret_cast<const uint4*>(c.k_resid + (bh * c.R + (ok ? tt - Q : 0)) * kD + 32 * grp);
        uint32_t rw[16];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          uint4 v = kr[x];
          if (!ok) v = make_uint4(0u, 0u, 0u, 0u);
          rw[4 * x] = v.x; rw[4 * x + 1] = v.y; rw[4 * x + 2] = v.z; rw[4 * x + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // k-slot pair pp of chunk j: the keys of the channels the codes use
          Frag kf;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const int c0 = key_channel<KB>(0, j, pp, 0), c1 = key_channel<KB>(0, j, pp, 1);
            const uint32_t sel = ((c0 & 1) ? 0x0302u : 0x0100u) | ((c1 & 1) ? 0x07060000u : 0x05040000u);
            kf.p[pp] = perm(rw[c1 >> 1], rw[c0 >> 1], sel);
          }
          s[e] = mfma(kf, wl.qb[grp][brow_hi][j], s[e]);
          s[e] = mfma(kf, wl.qb[grp][brow_lo][j], s[e]);
        }
      }
      float sc[8];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[4 * e + r] = s[e][r] * kUnitK;
      softmax_pv(sc, kInvUnitK, vm, vcl, vch, t0);
    }
  }

  // ---- merge the wavefronts of the workgroup --------------------------------
  // o = (acc - accz) / (value code step) * 2^-kv, l = l_run * 2^-kv
  const float ofac = __builtin_bit_cast(float, (uint32_t)(127 + 24 - kShV - kKvTop + vE) << 23);
  const float lfac = __builtin_bit_cast(float, (uint32_t)(127 - kKvTop + vE) << 23);
  const float lsum = grp_sum(l_run) * lfac;
  __syncthreads();  // every wavefront is done with its slots
  MergeLds<G>& mg = *reinterpret_cast<MergeLds<G>*>(smem);
  if (grp == 0 && c16 < G) {
    mg.m[w][c16] = m_ref;
    mg.l[w][c16] = lsum;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * grp + r;
      if (row < 2 * G) mg.o[w][row][16 * j + c16] = (acc[j][r] - accz[r]) * ofac;
    }
  __syncthreads();
  const bool single = nsplit_b <= 1;
  for (int e = tid; e < G * kD; e += 256) {
    const int hh = e / kD, ch = e % kD;
    float M = mg.m[0][hh];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) M = fmaxf(M, mg.m[ww][hh]);
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float f = __builtin_amdgcn_exp2f(mg.m[ww][hh] - M);
        o += f * (mg.o[ww][hh][ch] + mg.o[ww][G + hh][ch]);
        l += f * mg.l[ww][hh];
      }
    }
    const size_t qh = (size_t)b * p.Hq + (size_t)h * G + hh;
    if (single) {
      out[qh * kD + ch] = (l > 0.f) ? o / l : 0.f;
    } else {
      float* part = ws + (qh * p.n_split + split) * kPartialFloats;
      if (ch == 0) { part[0] = M; part[1] = l; }
      part[4 + ch] = o;
    }
  }
}

// Log-sum-exp merge of the split partials of sequences that were split: one
// workgroup per (sequence, query head), one thread per channel.
__global__ __launch_bounds__(128) void combine_kernel(CacheView c, AttnPlan p, const float* __restrict__ ws,
                                                      float* __restrict__ out) {
  const int bq = blockIdx.x, ch = threadIdx.x;
  const int b = bq / p.Hq;
  const int L = min(max(c.seq_len[b], 0), c.T);  // clamped: never past the capacity
  const int ns = (L + p.tokens_per_split - 1) / p.tokens_per_split;
  if (ns <= 1) return;  // written directly by the attention kernel
  const float* part = ws + (size_t)bq * p.n_split * kPartialFloats;
  float M = -INFINITY;
  for (int s2 = 0; s2 < ns; ++s2) M = fmaxf(M, part[s2 * kPartialFloats]);
  float o = 0.f, l = 0.f;
  if (M != -INFINITY) {
    for (int s2 = 0; s2 < ns; ++s2) {
      const float f = __builtin_amdgcn_exp2f(part[s2 * kPartialFloats] - M);
      o += f * part[s2 * kPartialFloats + 4 + ch];
      l += f * part[s2 * kPartialFloats + 1];
    }
  }
  out[(size_t)bq * kD + ch] = (l > 0.f) ? o / l : 0.f;
}

// Launch of one kernel variant, or (occ != nullptr) its resident workgroups
// per compute unit.
template <int KB, int VB, int KAXIS, int G, bool SPARSE>
hipError_t launch_t(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                    hipStream_t st, int* occ) {
  if (occ) {
    const void* fn = reinterpret_cast<const void*>(attn_kernel<KB, VB, KAXIS, G, SPARSE>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, attn_kernel<KB, VB, KAXIS, G, SPARSE>, 256, 0) ==
            hipSuccess && *occ > 0)
      return hipSuccess;
    (void)hipGetLastError();  // the query is optional: do not leave its error behind
    // estimate from the kernel's resources: one wavefront per SIMD per
    // workgroup, 512 VGPRs per SIMD lane, 160 KiB of LDS per compute unit
    hipFuncAttributes a;
    if (hipFuncGetAttributes(&a, fn) != hipSuccess) {
      (void)hipGetLastError();
      *occ = 1;
      return hipSuccess;
    }
    const int vgprs = a.numRegs > 0 ? (a.numRegs + 7) / 8 * 8 : 512;
    const int by_vgpr = 512 / vgprs;
    const int by_lds = a.sharedSizeBytes > 0 ? (int)((160 * 1024) / a.sharedSizeBytes) : 8;
    *occ = std::max(1, std::min(std::min(by_vgpr, by_lds), 8));
    return hipSuccess;
  }
  dim3 grid(p.n_split, c.H, c.B);
  hipLaunchKernelGGL((attn_kernel<KB, VB, KAXIS, G, SPARSE>), grid, dim3(256), 0, st, c, p, q, out, ws);
  return hipGetLastError();
}

template <int KB, int VB, int KAXIS, bool SPARSE>
hipError_t dispatch_g(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                      hipStream_t st, int* occ) {
  switch (p.group) {
    case 1: return launch_t<KB, VB, KAXIS, 1, SPARSE>(c, p, q, out, ws, st, occ);
    case 2: return launch_t<KB, VB, KAXIS, 2, SPARSE>(c, p, q, out, ws, st, occ);
    case 4: return launch_t<KB, VB, KAXIS, 4, SPARSE>(c, p, q, out, ws, st, occ);
    case 8: return launch_t<KB, VB, KAXIS, 8, SPARSE>(c, p, q, out, ws, st, occ);
  }
  return hipErrorInvalidValue;
}

template <int KB, int VB>
hipError_t dispatch_axis(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                         hipStream_t st, int* occ) {
  if (c.kaxis == 0) return dispatch_g<KB, VB, 0, false>(c, p, q, out, ws, st, occ);
  if (c.sparse) return dispatch_g<KB, VB, 1, true>(c, p, q, out, ws, st, occ);
  return dispatch_g<KB, VB, 1, false>(c, p, q, out, ws, st, occ);
}

template <int KB>
hipError_t dispatch_vb(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                       hipStream_t st, int* occ) {
  switch (c.vbits) {
    case 8: return dispatch_axis<KB, 8>(c, p, q, out, ws, st, occ);
    case 4: return dispatch_axis<KB, 4>(c, p, q, out, ws, st, occ);
    case 2: return dispatch_axis<KB, 2>(c, p, q, out, ws, st, occ);
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                    hipStream_t st, int* occ) {
  switch (c.kbits) {
    case 8: return dispatch_vb<8>(c, p, q, out, ws, st, occ);
    case 4: return dispatch_vb<4>(c, p, q, out, ws, st, occ);
    case 2: return dispatch_vb<2>(c, p, q, out, ws, st, occ);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_attention(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out,
                                   float* ws, hipStream_t st) {
  const hipError_t e = dispatch(c, p, q, out, ws, st, nullptr);
  if (e != hipSuccess || p.n_split <= 1) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(c.B * p.Hq), dim3(kD), 0, st, c, p, ws, out);
  return hipGetLastError();
}

int attention_blocks_per_cu(const CacheView& c, int group) {
  // cached per device and kernel variant (0 = not queried yet; threads may
  // race to fill an entry with the same value)
  static std::atomic<int> cache[16][3][3][2][2][4];
  const auto bi = [](int b) { return b == 2 ? 0 : (b == 4 ? 1 : 2); };
  const int gi = group == 1 ? 0 : (group == 2 ? 1 : (group == 4 ? 2 : 3));
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = -1;
  std::atomic<int>* slot =
      dev >= 0 ? &cache[dev][bi(c.kbits)][bi(c.vbits)][c.kaxis ? 1 : 0][c.sparse ? 1 : 0][gi] : nullptr;
  if (slot) {
    const int known = slot->load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  AttnPlan p{};
  p.group = group;
  int occ = 0;
  if (dispatch(c, p, nullptr, nullptr, nullptr, nullptr, &occ) != hipSuccess || occ < 1) occ = 1;
  if (slot) slot->store(occ, std::memory_order_relaxed);
  return occ;
}

}  // namespace kvq
