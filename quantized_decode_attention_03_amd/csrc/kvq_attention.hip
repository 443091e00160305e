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
//       A = dequantization-ready key codes (u - z') in fp16 (exact integers),
//       B = query columns; for per-channel keys the per-channel scale is
//           folded into the query (q * s_c), split into an fp16 hi and lo
//           part placed in columns h and g + h, so the product keeps ~22 bits.
//   O[row, c] = sum_t P[row, t] * V[t, c]
//       P = p_t * s_t (value scale folded into the softmax weight), again as
//           hi/lo rows h and g + h; V = value codes (u - z') in fp16.
// Codes become fp16 by OR-ing them into the mantissa of a power of two
// ("magic" exponent) and subtracting that power plus the zero-point in one
// packed fp16 operation. For values the magic exponent also absorbs the
// wavefront's largest value-scale exponent, which keeps p * s within fp16.
//
// Work split: grid (split, KV head, sequence), 4 wavefronts per workgroup,
// each wavefront owns every 4th 32-token tile of the split and keeps its own
// online softmax; the wavefronts merge through LDS. Sequences longer than one
// split leave (m, l, o) partials in the workspace that a second, small kernel
// merges with a log-sum-exp. (Merging in the last-arriving workgroup instead
// needs device-scope fences, whose L2 writeback and invalidation cost far more
// than the extra launch on this chip.)
#include "kvq_device.h"

namespace kvq {

namespace {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kMagic1024 = 0x64006400u;  // fp16 pair (1024, 1024)
#ifndef KVQ_WAVE_LDS_BUDGET
#define KVQ_WAVE_LDS_BUDGET 19968
#endif
constexpr int kWaveBudget = KVQ_WAVE_LDS_BUDGET;  // LDS bytes per wavefront

struct Frag {  // 8 fp16 MFMA operand values as 4 packed pairs
  uint32_t p[4];
};

__device__ __forceinline__ h2v as_h2(uint32_t x) { return __builtin_bit_cast(h2v, x); }
__device__ __forceinline__ uint32_t as_u32(h2v x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ uint32_t hsub2(uint32_t a, uint32_t b) {
  return as_u32(as_h2(a) - as_h2(b));
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
// a with the 13 low mantissa bits cleared: the fp16-RTZ value of a (normal range).
__device__ __forceinline__ float trunc16(float a) {
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) & 0xFFFFE000u);
}

// A 32-bit constant held in a VGPR (opaque to the compiler), so that
// (x & mask) | magic can issue as one v_and_or_b32 (gfx9 VOP3 takes no
// literal operands).
__device__ __forceinline__ uint32_t vconst(uint32_t x) {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(x));
  return r;
}

// 8 codes of BITS bits -> 4 fp16 pairs (magic|code) - sub[p].
// BITS 4: lo holds 8 nibbles; pair p = (nibble p, nibble p+4).
// BITS 2: lo holds 8 two-bit fields in its byte lane `half`*2, *2+1; pair p =
//         (field p, field p+4).
// BITS 8: lo, hi hold 8 bytes; pair p = (byte 2p, byte 2p+1).
// mask: 0x000F000F (BITS 4) or 0x00030003 (BITS 2), in a VGPR.
// magic_b: for BITS 8, the magic's high byte replicated in all four bytes.
template <int BITS>
__device__ __forceinline__ Frag unpack8(uint32_t lo, uint32_t hi, int half, uint32_t mask,
                                        uint32_t magic, uint32_t magic_b, const uint32_t* sub) {
  Frag f;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int p = 0; p < 4; ++p) f.p[p] = hsub2(((lo >> (4 * p)) & mask) | magic, sub[p]);
  } else if constexpr (BITS == 2) {
    const uint32_t sp = half ? perm(0u, lo, 0x0C030C02u) : perm(0u, lo, 0x0C010C00u);
#pragma unroll
    for (int p = 0; p < 4; ++p) f.p[p] = hsub2(((sp >> (2 * p)) & mask) | magic, sub[p]);
  } else {
    f.p[0] = hsub2(perm(magic_b, lo, 0x04010400u), sub[0]);
    f.p[1] = hsub2(perm(magic_b, lo, 0x04030402u), sub[1]);
    f.p[2] = hsub2(perm(magic_b, hi, 0x04010400u), sub[2]);
    f.p[3] = hsub2(perm(magic_b, hi, 0x04030402u), sub[3]);
  }
  return f;
}

// Geometry of one 32-token tile as staged in LDS:
//   [key codes 32 x 16*KB][value block 128 x 4*VB][value meta 32 words]
//   [key meta: 128 words (channel axis) or 32 (token axis)][sparse 32 x 2 words]
// Key codes and the value block are contiguous in global memory and move
// with 1 KiB direct-to-LDS loads (64 lanes x 16 bytes); the metadata pieces
// move together in one more load whose lanes gather 16-byte chunks.
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
  static constexpr int kLoads = kK / 1024 + kV / 1024 + 1;   // DMA instructions per tile
  // the key-product B operand and subtrahends (channel axis only)
  static constexpr int kWaveLds = KAXIS ? (4 * (2 * G + 1) * 4 * 16 + 4 * 4 * 4 * 4) : 0;
  // tile slots per wavefront: as many as fit the per-wavefront LDS budget
  // (kWaveBudget, chosen so that several 4-wavefront workgroups share a CU's
  // 160 KiB), between 2 and 4
  static constexpr int kSlotsFit = (kWaveBudget - kWaveLds) / kBytes;
  static constexpr int kSlots = kSlotsFit < 2 ? 2 : (kSlotsFit > 4 ? 4 : kSlotsFit);
  static_assert(kK % 1024 == 0 && kV % 1024 == 0, "1 KiB load granularity");
  static_assert(kMetaLanes <= 64, "metadata fits one load");
};

// 16 bytes per lane from global memory straight into LDS at lds_base + 16*lane
// (gfx950 global_load_lds_dwordx4). Issued from inline assembly so that the
// compiler neither waits on it at every LDS read nor keeps stale LDS values
// across it; completion is awaited explicitly with wait_vm().
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds_base)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// LDS per wavefront for channel-axis keys: the B operand of the key product
// for the current block (hi rows 0..G-1, lo rows G..2G-1, an all-zero row 2G;
// [grp][row][chunk] fragments) and the per-channel subtrahends of the A
// operand ([grp][chunk][pair]).
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

// Token (0..31 within the tile) of A row m in MFMA row block e: row block e
// holds tokens 8*(m/4) + 4e + m%4, so the output lane group g ends up with
// the 8 consecutive tokens 8g..8g+7, the k-slots of its P operand.
__device__ __forceinline__ int a_token(int e, int m) { return 8 * (m >> 2) + 4 * e + (m & 3); }

template <int KB, int VB, int KAXIS, int G, bool SPARSE>
__global__ __launch_bounds__(256) void attn_kernel(CacheView c, AttnPlan p, const uint16_t* __restrict__ q,
                                                   float* __restrict__ out, float* __restrict__ ws) {
  using Gm = Geom<KB, VB, KAXIS, G, SPARSE>;
  constexpr int NB = Gm::kSlots;
  constexpr int kQMinK = -(1 << (KB - 1));
  constexpr int kQMinV = -(1 << (VB - 1));
  constexpr bool kPermK = KB != 8;  // k-slot pairs (i, i+4) for 4/2-bit keys
  constexpr bool kPermV = VB != 8;
  static_assert(2 * G <= 16, "hi/lo rows must fit 16");

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c16 = lane & 15, grp = lane >> 4;
  const int L = c.seq_len[b];
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
  if constexpr (SPARSE) {
    for (int i = tid; i < G * kD; i += 256) qsh[i / kD][i % kD] = h2f(qg[i]) * qscale;
    __syncthreads();
  }

  // channel axis: this lane builds the scaled query of 2 channels, all heads
  // (slot pair p of octet q: channels (p, p+4) for 4/2-bit keys, (2p, 2p+1) for 8-bit)
  int bc0 = 0, bc1 = 0;
  {
    const int oq = lane >> 2, op = lane & 3;
    bc0 = kPermK ? 8 * oq + op : 8 * oq + 2 * op;
    bc1 = kPermK ? bc0 + 4 : bc0 + 1;
  }
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
          const int base = 32 * grp + 8 * j;
          const int ch0 = kPermK ? base + pp : base + 2 * pp;
          const int ch1 = kPermK ? ch0 + 4 : ch0 + 1;
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

  // DMA of quantized tile i of this wavefront into slot `slot`.
  auto issue = [&](int i, int slot) {
    const int t0 = ts0 + (w + 4 * i) * kBlock;
    const uint32_t lb = wbase_lds + slot * Gm::kBytes;
    const uint8_t* kg = c.k_codes + (bh * c.T + t0) * (size_t)Gm::kRowK + lane * 16;
#pragma unroll
    for (int x = 0; x < Gm::kK / 1024; ++x) dma16(kg + x * 1024, lb + x * 1024);
    const uint8_t* vg = c.v_codes + (bh * (c.T / kBlock) + t0 / kBlock) * (size_t)Gm::kV + lane * 16;
#pragma unroll
    for (int x = 0; x < Gm::kV / 1024; ++x) dma16(vg + x * 1024, lb + Gm::kK + x * 1024);
    if (lane < Gm::kMetaLanes) {
      const uint8_t* mg;
      if (lane < 8) {
        mg = reinterpret_cast<const uint8_t*>(c.v_meta + bh * c.T + t0) + lane * 16;
      } else if (lane < 8 + Gm::kKm / 16) {
        const uint32_t* km = KAXIS ? c.k_meta + (bh * (c.T / kBlock) + t0 / kBlock) * kD
                                   : c.k_meta + bh * c.T + t0;
        mg = reinterpret_cast<const uint8_t*>(km) + (lane - 8) * 16;
      } else {
        mg = reinterpret_cast<const uint8_t*>(c.k_sparse + (bh * c.T + t0) * 2) +
             (lane - 8 - Gm::kKm / 16) * 16;
      }
      dma16(mg, lb + Gm::kK + Gm::kV);
    }
  };

  const h2v vofs2 = {(_Float16)(1024 - kQMinV), (_Float16)(1024 - kQMinV)};
  const h2v kofs2 = {(_Float16)(1024 - kQMinK), (_Float16)(1024 - kQMinK)};
  const uint32_t kmask = vconst(KB == 2 ? 0x00030003u : 0x000F000Fu);
  const uint32_t vmask = vconst(VB == 2 ? 0x00030003u : 0x000F000Fu);
  const uint32_t kmagic = vconst(kMagic1024);

  // row factors of the P operand: hi rows (c16 < G) keep p*s, lo rows take the
  // residual p*s - rtz16(p*s), rows >= 2G are zero
  const float rowkeep = live ? 1.f : 0.f;
  const float rowlo = (c16 >= G && live) ? 1.f : 0.f;

  float m_ref = -INFINITY, l_run = 0.f;
  f4v acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f4v{0.f, 0.f, 0.f, 0.f};

  // ---- scores of one tile -> online softmax -> P.V ---------------------------
  // sc[4e + r] is the score of token 8grp + 4e + r (log2 units); vm[i] the value
  // meta of token 8grp + i; vcode(j) gives the lane's value codes of chunk j.
  auto softmax_pv = [&](float (&sc)[8], const uint32_t (&vm)[8], const uint32_t (&vcl)[8],
                        const uint32_t (&vch)[8], int t0) {
    const int nvalid = ts1 - t0;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (8 * grp + 4 * (i >> 2) + (i & 3) >= nvalid) sc[i] = -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    if (__builtin_amdgcn_ballot_w64(live && mx > m_ref + kLazy)) {
      const float m_new = fmaxf(m_ref, grp_max(mx));
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, (4 * grp + r) & (G - 1), 64);
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] *= ar[r];
      l_run *= alpha;
      m_ref = m_new;
    }
    // Magic exponent vx of this lane group's value operand: the largest of its
    // 8 value scales is brought to [1, 2) in P = p * s * 2^-vx, and the value
    // codes carry the 2^vx back (B = (u - z') * 2^vx), so the product is
    // unchanged; k-slots of one lane group meet only each other in the MFMA.
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = h2f((uint16_t)(vm[i] & 0xFFFFu));
    const float smax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                             fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    const int ex = (smax > 0.f) ? (int)((__builtin_bit_cast(uint32_t, smax) >> 23) & 0xFF) - 127 : 0;
    const int vx = min(max(ex, -24), 5);
    const uint32_t vmagic1 = (uint32_t)(25 + vx) << 10;
    const uint32_t vmagic = vmagic1 * 0x10001u;
    const uint32_t vmagic_b = (vmagic1 >> 8) * 0x01010101u;
    const float vpow = __builtin_ldexpf(rowkeep, -vx);
    const uint32_t p2 = (vx >= -14) ? (uint32_t)(vx + 15) << 10 : 1u << (vx + 24);  // fp16 2^vx
    const h2v vpow2 = as_h2(p2 * 0x10001u);
    float pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pr = __builtin_amdgcn_exp2f(sc[i] - m_ref);
      l_run += pr;
      const float x = pr * (sv[i] * vpow);
      pv[i] = x - rowlo * trunc16(x);
    }
    Frag pf;
    uint32_t vsub[4];
#pragma unroll
    for (int pp = 0; pp < 4; ++pp) {
      const int i0 = kPermV ? pp : 2 * pp;
      const int i1 = kPermV ? pp + 4 : 2 * pp + 1;
      pf.p[pp] = pk_rtz(pv[i0], pv[i1]);
      const uint32_t zz = perm(vm[i1], vm[i0], 0x07060302u);  // (z_i0, z_i1)
      vsub[pp] = as_u32((as_h2(zz) + vofs2) * vpow2);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const Frag vf = unpack8<VB>(vcl[j], vch[j], 0, vmask, vmagic, vmagic_b, vsub);
      acc[j] = mfma(pf, vf, acc[j]);
    }
  };

  // the B operand of the key product for a block: scaled query (hi/lo) with
  // per-channel scales s0, s1 of this lane's two build channels
  auto build_qb = [&](float s0, float s1, uint32_t km0, uint32_t km1, bool with_zero) {
    const int bq = lane >> 2, bp = lane & 3, bg = bq >> 2, bj = bq & 3;
    wave_lds_fence();
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float v0 = qv0[hh] * s0, v1 = qv1[hh] * s1;
      wl.qb[bg][hh][bj].p[bp] = pk_rtz(v0, v1);
      wl.qb[bg][G + hh][bj].p[bp] = pk_rtz(v0 - trunc16(v0), v1 - trunc16(v1));
    }
    if (with_zero) wl.zc[bg][bj][bp] = as_u32(as_h2(perm(km1, km0, 0x07060302u)) + kofs2);
    wave_lds_fence();
  };

  // ---- quantized tiles through the LDS pipeline -----------------------------
  if (nw > 0) {
#pragma unroll
    for (int i = 0; i < NB - 1; ++i)
      if (i < nw) issue(i, i);
    for (int i = 0; i < nw; ++i) {
      const int slot = i % NB;
      if (i + NB - 1 < nw) issue(i + NB - 1, (i + NB - 1) % NB);
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
      float sc[8];
      f4v s[2] = {f4v{0.f, 0.f, 0.f, 0.f}, f4v{0.f, 0.f, 0.f, 0.f}};
      if constexpr (KAXIS) {
        const uint32_t km0 = kmeta[bc0], km1 = kmeta[bc1];
        build_qb(h2f((uint16_t)(km0 & 0xFFFFu)), h2f((uint16_t)(km1 & 0xFFFFu)), km0, km1, true);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const Frag qh = wl.qb[grp][brow_hi][j];
          const Frag ql = wl.qb[grp][brow_lo][j];
          uint32_t zsub[4];
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) zsub[pp] = wl.zc[grp][j][pp];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            Frag kf;
            if constexpr (KB == 4) kf = unpack8<4>(kc[e][j], 0u, 0, kmask, kmagic, 0u, zsub);
            else if constexpr (KB == 8) kf = unpack8<8>(kc[e][2 * j], kc[e][2 * j + 1], 0, kmask, kmagic, 0x64646464u, zsub);
            else kf = unpack8<2>(kc[e][j >> 1], 0u, j & 1, kmask, kmagic, 0u, zsub);
            s[e] = mfma(kf, qh, s[e]);
            s[e] = mfma(kf, ql, s[e]);
          }
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[4 * e + r] = s[e][r];
      } else {
        uint32_t km[8];
        {
          const uint4 a = reinterpret_cast<const uint4*>(kmeta + 8 * grp)[0];
          const uint4 bb = reinterpret_cast<const uint4*>(kmeta + 8 * grp)[1];
          km[0] = a.x; km[1] = a.y; km[2] = a.z; km[3] = a.w;
          km[4] = bb.x; km[5] = bb.y; km[6] = bb.z; km[7] = bb.w;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const uint32_t ka = kmeta[a_token(e, c16)];
          const uint32_t zt = (ka >> 16) | (ka & 0xFFFF0000u);  // (z, z)
          const uint32_t zs = as_u32(as_h2(zt) + kofs2);
          const uint32_t zsub[4] = {zs, zs, zs, zs};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            Frag kf;
            if constexpr (KB == 4) kf = unpack8<4>(kc[e][j], 0u, 0, kmask, kmagic, 0u, zsub);
            else if constexpr (KB == 8) kf = unpack8<8>(kc[e][2 * j], kc[e][2 * j + 1], 0, kmask, kmagic, 0x64646464u, zsub);
            else kf = unpack8<2>(kc[e][j >> 1], 0u, j & 1, kmask, kmagic, 0u, zsub);
            s[e] = mfma(kf, qfrag[j], s[e]);
          }
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sc[4 * e + r] = s[e][r] * (h2f((uint16_t)(km[4 * e + r] & 0xFFFFu)) * qscale);
      }
      if constexpr (SPARSE) {
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) {
          const uint2 rec = reinterpret_cast<const uint2*>(spr)[8 * grp + i2];
          sc[i2] += qsh[hq][rec.y & 0xFFFFu] * h2f((uint16_t)(rec.x & 0xFFFFu)) +
                    qsh[hq][rec.y >> 16] * h2f((uint16_t)(rec.x >> 16));
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
          vcl[j] = reinterpret_cast<const uint16_t*>(rec)[grp];
          vch[j] = 0u;
        }
      }
      softmax_pv(sc, vm, vcl, vch, t0);
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
          } else { vcl[j] = reinterpret_cast<const uint16_t*>(rec)[grp]; vch[j] = 0u; }
        }
        const uint4* vmg = reinterpret_cast<const uint4*>(c.v_meta + bh * c.T + t0 + 8 * grp);
        const uint4 a = vmg[0], bb = vmg[1];
        vm[0] = a.x; vm[1] = a.y; vm[2] = a.z; vm[3] = a.w;
        vm[4] = bb.x; vm[5] = bb.y; vm[6] = bb.z; vm[7] = bb.w;
      }
      // B operand: query scaled by the softmax factor only, hi/lo
      build_qb(1.f, 1.f, 0u, 0u, false);
      f4v s[2] = {f4v{0.f, 0.f, 0.f, 0.f}, f4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int tt = t0 + a_token(e, c16);
        const bool ok = tt < ts1;
        const uint16_t* kr = c.k_resid + (bh * c.R + (ok ? tt - Q : 0)) * kD + 32 * grp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint4 x = reinterpret_cast<const uint4*>(kr + 8 * j)[0];
          if (!ok) x = make_uint4(0, 0, 0, 0);
          Frag kf;
          if (kPermK) {  // pairs (channel p, p+4)
            kf.p[0] = perm(x.z, x.x, 0x05040100u);
            kf.p[1] = perm(x.z, x.x, 0x07060302u);
            kf.p[2] = perm(x.w, x.y, 0x05040100u);
            kf.p[3] = perm(x.w, x.y, 0x07060302u);
          } else {
            kf.p[0] = x.x; kf.p[1] = x.y; kf.p[2] = x.z; kf.p[3] = x.w;
          }
          s[e] = mfma(kf, wl.qb[grp][brow_hi][j], s[e]);
          s[e] = mfma(kf, wl.qb[grp][brow_lo][j], s[e]);
        }
      }
      float sc[8];
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[4 * e + r] = s[e][r];
      softmax_pv(sc, vm, vcl, vch, t0);
    }
  }

  // ---- merge the wavefronts of the workgroup --------------------------------
  const float lsum = grp_sum(l_run);
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
      if (row < 2 * G) mg.o[w][row][16 * j + c16] = acc[j][r];
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
  const int L = c.seq_len[b];
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

template <int KB, int VB, int KAXIS, int G, bool SPARSE>
hipError_t launch_t(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                    hipStream_t st) {
  dim3 grid(p.n_split, c.H, c.B);
  hipLaunchKernelGGL((attn_kernel<KB, VB, KAXIS, G, SPARSE>), grid, dim3(256), 0, st, c, p, q, out, ws);
  return hipGetLastError();
}

template <int KB, int VB, int KAXIS, bool SPARSE>
hipError_t dispatch_g(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                      hipStream_t st) {
  switch (p.group) {
    case 1: return launch_t<KB, VB, KAXIS, 1, SPARSE>(c, p, q, out, ws, st);
    case 2: return launch_t<KB, VB, KAXIS, 2, SPARSE>(c, p, q, out, ws, st);
    case 4: return launch_t<KB, VB, KAXIS, 4, SPARSE>(c, p, q, out, ws, st);
    case 8: return launch_t<KB, VB, KAXIS, 8, SPARSE>(c, p, q, out, ws, st);
  }
  return hipErrorInvalidValue;
}

template <int KB, int VB>
hipError_t dispatch_axis(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                         hipStream_t st) {
  if (c.kaxis == 0) return dispatch_g<KB, VB, 0, false>(c, p, q, out, ws, st);
  if (c.sparse) return dispatch_g<KB, VB, 1, true>(c, p, q, out, ws, st);
  return dispatch_g<KB, VB, 1, false>(c, p, q, out, ws, st);
}

template <int KB>
hipError_t dispatch_vb(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                       hipStream_t st) {
  switch (c.vbits) {
    case 8: return dispatch_axis<KB, 8>(c, p, q, out, ws, st);
    case 4: return dispatch_axis<KB, 4>(c, p, q, out, ws, st);
    case 2: return dispatch_axis<KB, 2>(c, p, q, out, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_attention(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out,
                                   float* ws, hipStream_t st) {
  hipError_t e;
  switch (c.kbits) {
    case 8: e = dispatch_vb<8>(c, p, q, out, ws, st); break;
    case 4: e = dispatch_vb<4>(c, p, q, out, ws, st); break;
    case 2: e = dispatch_vb<2>(c, p, q, out, ws, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || p.n_split <= 1) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(c.B * p.Hq), dim3(kD), 0, st, c, p, ws, out);
  return hipGetLastError();
}

}  // namespace kvq
