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
// masked at bit sh of an fp16 half (sh + bits <= 10) is the subnormal
// u * 2^(sh-24), which the matrix cores multiply exactly. Chains of
// accumulating MFMAs have an absolute error floor, so the key products must
// not be small (measured: 2-bit codes at u * 2^-24 gave key-score errors near
// 2e-3, at u * 2^-16 near 5e-6); every key product is kept at the magnitude
// it has with all codes at bit SH, the variant's code unit 2^(SH-24): SH is 8
// for 2-bit, 4 for 4-bit and 0 for 8-bit codes.
//   Channel-axis keys: each pair stays where a single mask reaches it (plus
//     one shift per word for the fields above bit 10), and the factor
//     2^(SH - sh) is folded into the scaled query of its channel, which has
//     the fp16 range to spare.
//   Token-axis keys: their query operand is the raw fp16 query, which cannot
//     absorb a factor without rounding, so every pair is moved to bit SH.
//   Values: each pair also stays where a single mask reaches it, and its
//     softmax weights carry the factor 2^-sh (taken into the exponent), so
//     every product is P * u * 2^-24. Factors at most 1 keep P inside fp16,
//     and the value product is far less sensitive to the floor (measured:
//     error / sum of P near 2e-5 with codes at u * 2^-24).
//
// Zero points are not subtracted element by element:
//   keys, channel axis: x = s_c (u - z'_c); B = q * s_c (scaled query, split
//     into fp16 hi and lo parts); the term sum_c z'_c B[c, col] is the same
//     for every token of a block and seeds the accumulator (an A operand whose
//     rows all hold -z');
//   keys, token axis: x = s_t (u - z'_t); B = raw fp16 query (exact); the
//     term z'_t * sum_c q_c is one FMA per score; s_t multiplies the score;
//   values, token axis: x = s_t (u - z'_t); P = p_t * s_t * 2^kv (times the
//     pair factor) as hi/lo rows h and g + h; the product with a B operand
//     whose columns all hold z'_t (at the pair's bit) is subtracted once at
//     the end.
// The two other element formats keep keys on the token axis:
//   fp8 E4M3: bytes become fp16 operands exactly (a hardware conversion; every
//     E4M3 value is an fp16 value); the per-cache key scale multiplies the
//     score, the value scale the output; no zero points, and P = p;
//   symmetric 32-channel blocks: x = s_t,j (u + q_min) for block j of token
//     t. Keys: each block gets its own MFMA (the lane groups' k-slots all in
//     block j), seeded with q_min * (sum of the block's query channels), and
//     the token's block scales combine the four products; values: one P
//     operand per block (p_t * s_t,j * 2^kv) for its two 16-channel chunks, and
//     the constant zero point -q_min through one more MFMA per block.
// The hi and lo parts of the scaled query sit in different columns of one B
// operand (column n: head n mod g, hi part when n / g is even), so one MFMA
// covers both; one DPP add across lanes n and n - g of a 16-lane row sums
// them, and every lane then holds the full score of its column's head.
// The factor 2^kv keeps p * s inside fp16: it is one exponent per wavefront,
// raised lazily (rarely) when a larger value scale shows up, like the softmax
// reference.
//
// Work split: a fixed grid of workgroups (as many as the chip holds at once),
// each taking an equal, contiguous range of the 32-token tiles of all
// (sequence, KV head) pairs, so ragged lengths leave no workgroup idle and
// each pays its start-up latency once. Within a range, a workgroup walks the
// (sequence, KV head) segments it covers; its 4 wavefronts take every 4th tile
// of a segment, keep their own online softmax and merge through LDS. A segment
// that is a whole (sequence, KV head) writes the output; the others leave
// (m, l, o) partials in the workspace that a second, small kernel merges with
// a log-sum-exp. (Merging in the last-arriving workgroup instead needs
// device-scope fences, whose L2 writeback and invalidation cost far more than
// the extra launch on this chip.)
#include <algorithm>
#include <type_traits>
#include <atomic>

#include "kvq_device.h"

namespace kvq {

namespace {

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef _Float16 h8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
// LDS bytes per wavefront for tile slots plus the wavefront's operand area:
// 2 or 3 slots of the 4- and 2-bit tiles (a tile in flight while another is
// computed), about 47 KiB per 4-wavefront workgroup. Measured on the three
// KIVI workloads against budgets of 16 and 20 KiB (more slots, fewer
// workgroups per compute unit): this one was as fast or faster on each.
#ifndef KVQ_WAVE_LDS_BUDGET
#define KVQ_WAVE_LDS_BUDGET 12000
#endif
constexpr int kWaveBudget = KVQ_WAVE_LDS_BUDGET;

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
__device__ __forceinline__ uint32_t pk_fma16(uint32_t w, h2v m, h2v c) {
  return as_u32(__builtin_elementwise_fma(as_h2(w), m, c));
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

// Maximum of the 8 scores of a lane. The NaN-propagating maximum becomes
// v_maximum3_f32 with no canonicalizing maximum in front of each operand (which
// fmaxf takes for operands the compiler cannot prove canonical). Compiler
// built-ins, not inline assembly: scores can come straight from the matrix
// cores, and only compiler-emitted reads get the wait states that requires.
__device__ __forceinline__ float max8(const float (&v)[8]) {
  const auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
  return mx(mx(mx(v[0], v[1]), mx(v[2], v[3])), mx(mx(v[4], v[5]), mx(v[6], v[7])));
}

// -1 that the compiler cannot fold: x * -1 + y then stays one v_fma_mix_f32
// with an fp16 operand instead of a conversion and a subtraction.
__device__ __forceinline__ float opaque_neg1() {
  float r = -1.f;
  asm("" : "+s"(r));
  return r;
}

// fp16 pair (RTZ) of two floats.
__device__ __forceinline__ uint32_t pk_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// 2^e as an exact float (compile-time)
__host__ __device__ constexpr float pow2f(int e) {
  float r = 1.f;
  for (int i = 0; i < e; ++i) r *= 2.f;
  for (int i = 0; i < -e; ++i) r *= 0.5f;
  return r;
}
__device__ __forceinline__ h2v h2_splat(uint16_t bits) {
  const _Float16 x = __builtin_bit_cast(_Float16, bits);
  return h2v{x, x};
}

// ---- code operands -----------------------------------------------------------

// Code unit of the key and value operands: 2^(SH-24).
template <int BITS> constexpr int unit_shift() { return BITS == 2 ? 8 : (BITS == 4 ? 4 : 0); }

// Channel of k-slot pair p (first or second slot) in chunk j of lane group
// grp, for key codes of BITS bits. Key rows are channel-packed with the low
// bits first.
template <int BITS>
__device__ __forceinline__ int key_channel(int grp, int j, int p, int second) {
  if constexpr (BITS == 8) return 32 * grp + 8 * j + 2 * p + second;
  if constexpr (BITS == 4) return 32 * grp + 8 * j + p + 4 * second;
  return 32 * grp + 16 * (j >> 1) + 4 * (j & 1) + p + 8 * second;
}

// Bit position sh of the codes of key k-slot pair p in chunk j. U (uniform):
// every pair at the unit shift.
template <int KB, bool U>
__host__ __device__ constexpr int key_sh(int j, int p) {
  if (KB == 8) return 0;
  if (U) return unit_shift<KB>();
  if (KB == 4) return (p & 1) ? 4 : 0;
  return ((j & 1) && p == 0) ? 8 : 2 * p + 2;
}

// Two fields of BITS bits, at bit n and n + 16 of w, moved to bit SH of each
// half.
template <int BITS>
__device__ __forceinline__ uint32_t field_pair(uint32_t w, int n) {
  constexpr int SH = unit_shift<BITS>();
  constexpr uint32_t kMask = (((1u << BITS) - 1u) << SH) * 0x10001u;
  if (n == SH) return w & kMask;
  if (n < SH) return (w << (SH - n)) & kMask;
  return (w >> (n - SH)) & kMask;
}

// Key operand of chunk j from the lane's code words of one token row (the
// lane group's 32 channels): KB words for 4/2-bit codes, 2 per chunk for 8-bit.
//   4-bit: word j, nibbles (p, p+4) -> pair p; per-pair positions: nibbles
//          0/1 and 4/5 masked in place (sh 0, 4), nibbles 2/3 and 6/7 after
//          one shift by 8.
//   2-bit: word j/2; fields (n, n+16), n = 8 (j odd) + 2p; per-pair
//          positions: j even, all four after one shift left by 2 (sh 2p + 2);
//          j odd, field 8 in place (sh 8), fields 10..14 after one shift
//          right by 6 (sh 2p + 2).
//   8-bit: bytes (2p, 2p+1) of the chunk's two words (sh 0).
template <int KB, bool U>
__device__ __forceinline__ Frag key_frag(const uint32_t* kc, int j) {
  Frag f;
  if constexpr (KB == 8) {
    const uint32_t a = kc[2 * j], b = kc[2 * j + 1];
    f.p[0] = perm(0u, a, 0x0C010C00u);
    f.p[1] = perm(0u, a, 0x0C030C02u);
    f.p[2] = perm(0u, b, 0x0C010C00u);
    f.p[3] = perm(0u, b, 0x0C030C02u);
  } else if constexpr (U) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
      f.p[p] = KB == 4 ? field_pair<4>(kc[j], 4 * p) : field_pair<2>(kc[j >> 1], 8 * (j & 1) + 2 * p);
  } else if constexpr (KB == 4) {
    const uint32_t w = kc[j], t = w >> 8;
    f.p[0] = w & 0x000F000Fu;
    f.p[1] = w & 0x00F000F0u;
    f.p[2] = t & 0x000F000Fu;
    f.p[3] = t & 0x00F000F0u;
  } else {
    const uint32_t w = kc[j >> 1];
    if ((j & 1) == 0) {
      const uint32_t t = w << 2;
#pragma unroll
      for (int p = 0; p < 4; ++p) f.p[p] = t & (0x00030003u << (2 * p + 2));
    } else {
      const uint32_t t = w >> 6;
      f.p[0] = w & 0x03000300u;
#pragma unroll
      for (int p = 1; p < 4; ++p) f.p[p] = t & (0x00030003u << (2 * p + 2));
    }
  }
  return f;
}

// Value operand: 8 tokens of one channel. k-slot pair p holds tokens (p,
// p+4) for 4/2-bit values, (2p, 2p+1) for 8-bit ones, each pair where one mask
// reaches it: codes at bit val_sh<VB>(p) of each half, the subnormal
// u * 2^(val_sh - 24). The P operand of pair p carries the factor 2^-val_sh
// (folded into its softmax weights), so every product is P * u * 2^-24.
//   4-bit: the record word (nibble i = token i); nibbles (p, p+4) masked in
//          place for p = 0, 1 (bits 0 and 4), after one shift by 8 for p = 2, 3;
//   2-bit: the 16-bit record spread to bytes 0 and 2 (tokens 0..3, 4..7),
//          fields (2p, 16 + 2p) masked in place;
//   8-bit: bytes of two words.
template <int VB>
__host__ __device__ constexpr int val_sh(int p) {
  return VB == 2 ? 2 * p : (VB == 4 ? 4 * (p & 1) : 0);
}
template <int VB>
__device__ __forceinline__ Frag val_frag(uint32_t a, uint32_t b) {
  Frag f;
  if constexpr (VB == 8) {
    f.p[0] = perm(0u, a, 0x0C010C00u);
    f.p[1] = perm(0u, a, 0x0C030C02u);
    f.p[2] = perm(0u, b, 0x0C010C00u);
    f.p[3] = perm(0u, b, 0x0C030C02u);
  } else if constexpr (VB == 4) {
    const uint32_t t = a >> 8;
    f.p[0] = a & 0x000F000Fu;
    f.p[1] = a & 0x00F000F0u;
    f.p[2] = t & 0x000F000Fu;
    f.p[3] = t & 0x00F000F0u;
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) f.p[p] = a & (0x00030003u << (2 * p));
  }
  return f;
}
// The lane's value record words of one channel, as val_frag takes them.
// 2-bit records are 16 bits, half of the aligned word at rec + 4 (grp / 2):
// sel2 spreads the lane's half to bytes 0 and 2 (0x0C010C00 for even lane
// groups, 0x0C030C02 for odd ones).
template <int VB>
__device__ __forceinline__ void val_words(const uint8_t* rec, int grp, uint32_t sel2, uint32_t& lo, uint32_t& hi) {
  if constexpr (VB == 4) {
    lo = reinterpret_cast<const uint32_t*>(rec)[grp];
    hi = 0u;
  } else if constexpr (VB == 8) {
    const uint2 x = reinterpret_cast<const uint2*>(rec)[grp];
    lo = x.x;
    hi = x.y;
  } else {
    lo = perm(0u, reinterpret_cast<const uint32_t*>(rec)[grp >> 1], sel2);
    hi = 0u;
  }
}

// fp8 E4M3 bytes to an fp16 operand: bytes (0, 1) and (2, 3) of a, then of b,
// as k-slot pairs 0..3 (the 8-bit layout of key_frag and val_frag). Every
// E4M3 value is an fp16 value, so the conversion (scale 1) is exact.
__device__ __forceinline__ Frag fp8_frag(uint32_t a, uint32_t b) {
  Frag f;
  f.p[0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, false));
  f.p[1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, true));
  f.p[2] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false));
  f.p[3] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true));
  return f;
}

// Key operand of one 32-channel block for symmetric block codes: MFMA j takes
// block j, and lane group g its k-slots, the channels key_channel(j, g, ...)
// (the roles of the lane group and the chunk swapped against the affine
// layout). The lane's words (row bytes [32 j + 8 g, +8) for 8-bit codes,
// [16 j + 4 g, +4) for 4-bit, [8 j + 4 (g / 2), +4) shifted right by 8 (g mod
// 2) for 2-bit) hold exactly those channels.
template <int KB>
__device__ __forceinline__ Frag sym_key_frag(uint32_t w0, uint32_t w1) {
  Frag f;
  if constexpr (KB == 8) {
    f.p[0] = perm(0u, w0, 0x0C010C00u);
    f.p[1] = perm(0u, w0, 0x0C030C02u);
    f.p[2] = perm(0u, w1, 0x0C010C00u);
    f.p[3] = perm(0u, w1, 0x0C030C02u);
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) f.p[p] = field_pair<KB>(w0, KB * p);
  }
  return f;
}

// Rotary-embedding keys: MFMA j of lane group g takes channels [16 g, 16 g +
// 16) (j = 0, 1) and their rotation partners, 64 higher (j = 2, 3), in the
// in-chunk order of the affine layout, so every lane holds both channels of
// each of its pairs and chunk j + 2 pairs up with chunk j element by element.
template <int KB>
__device__ __forceinline__ int rope_channel(int grp, int j, int p, int s) {
  return ((j >> 1) ? 64 : 0) + 16 * grp + key_channel<KB>(0, j & 1, p, s);
}

// cos and sin of the rotation angle t theta_i, from the angle in revolutions
// t phi_i = t theta_i / (2 pi) (phi_i = ph.x + ph.y, two floats): the product
// t * ph.x is split into its rounded value and exact error (t < 2^24 is exact
// in fp32), the whole revolutions are dropped, and what is left, in [-1/2,
// 1/2] to about 2^-25, goes to the hardware sine and cosine, which take
// revolutions.
__device__ __forceinline__ void rope_cs(float t, float2 ph, float& c, float& s) {
#pragma clang fp contract(off)
  const float p = t * ph.x;
  const float e = __builtin_fmaf(t, ph.x, -p);
  const float r = (p - __builtin_rintf(p)) + __builtin_fmaf(t, ph.y, e);
  c = __builtin_amdgcn_cosf(r);
  s = __builtin_amdgcn_sinf(r);
}

// fp16 hi and lo parts of two floats (y - hi is exact): the A operands of two
// products whose sum keeps about 22 bits of y.
__device__ __forceinline__ void split_hilo(float y0, float y1, uint32_t& hi, uint32_t& lo) {
  const float m1 = opaque_neg1();
  hi = pk_rtz(y0, y1);
  lo = pk_rtz(__builtin_fmaf(f16lo(hi), m1, y0), __builtin_fmaf(f16hi(hi), m1, y1));
}

// Geometry of one 32-token tile as staged in LDS:
//   [key codes 32 x 16*KB][value block 128 x 4*VB][value meta, 32 tokens]
//   [key meta: 128 words (channel axis) or 32 tokens (token axis)]
//   [sparse 32 x 2 words]
// Metadata per token: one word (affine codes), 4 fp16 block scales (symmetric
// blocks), none (fp8). Key codes and the value block are contiguous in global
// memory and move with 1 KiB direct-to-LDS loads (64 lanes x 16 bytes); the
// metadata pieces follow with one load per array, each lane group gathering
// 16-byte chunks into consecutive LDS.
template <int KB, int VB, int KAXIS, int G, bool SPARSE, int FMT>
struct Geom {
  static constexpr int kRowK = 16 * KB;               // key code bytes per token
  static constexpr int kK = 32 * kRowK;               // key codes of a tile
  static constexpr int kV = 512 * VB;                 // value block
  static constexpr int kMetaTok = FMT == kFmtFp8 ? 0 : (FMT == kFmtSym32 ? 2 * kSymBlocks : 4);
  static constexpr int kVm = 32 * kMetaTok;
  static constexpr int kKm = KAXIS ? 512 : 32 * kMetaTok;
  static constexpr int kSp = SPARSE ? 256 : 0;
  static constexpr int kMetaLanes = (kVm + kKm + kSp) / 16;
  static constexpr int kMetaLoads = (kVm > 0) + (kKm > 0) + (SPARSE ? 1 : 0);
  static constexpr int kBytes = kK + kV + kVm + kKm + kSp;
  static constexpr int kLoads = kK / 1024 + kV / 1024 + kMetaLoads;  // DMA instructions per tile
  // the key-product B operand and zero-point operand (channel axis only)
  static constexpr int kWaveLds = (KAXIS && FMT != kFmtRope) ? (4 * (2 * G) * 4 * 16 + 4 * 4 * 4 * 4) : 0;
  // tile slots per wavefront: as many as fit the per-wavefront budget, 2 to 6
  static constexpr int kSlotsFit = (kWaveBudget - kWaveLds - (SPARSE ? G * kD : 0)) / kBytes;
  static constexpr int kSlots = kSlotsFit < 2 ? 2 : (kSlotsFit > 6 ? 6 : kSlotsFit);
  static constexpr int kQLoads = G == 8 ? 2 : 1;      // DMA instructions for the query heads
  static_assert(kK % 1024 == 0 && kV % 1024 == 0, "1 KiB load granularity");
  static_assert(kMetaLanes <= 64, "metadata fits one load");
  static_assert((kSlots - 1) * kLoads <= 63, "waits fit the vmcnt field");
  // a residual tile (16 fp16 key rows, the value block and scales) fits the slots
  static_assert(!KAXIS || 4096 + kV + 128 <= kSlots * kBytes, "residual tile fits the slots");
  static_assert(kBytes >= G * kD * 2, "the query heads fit one tile slot");
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
// Wait until at most n * K loads (n <= 5) are outstanding.
template <int K>
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<K>(); break;
    case 2: wait_vm<2 * K>(); break;
    case 3: wait_vm<3 * K>(); break;
    case 4: wait_vm<4 * K>(); break;
    default: wait_vm<5 * K>(); break;
  }
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// LDS per wavefront for channel-axis keys: the B operand of the key product
// for the current block (hi rows 0..G-1, lo rows G..2G-1; [grp][row][chunk]
// fragments) and the zero-point A operand, -z' per channel in the unit of its
// codes ([grp][chunk][pair]).
template <int G>
struct WaveLds {
  Frag qb[4][2 * G][4];
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

// x plus x of lane n - G (mod 16) of the same 16-lane row (DPP row_ror:G):
// lanes n and n -+ G hold the hi and lo parts of the same head's score.
template <int G>
__device__ __forceinline__ float add_ror(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + G, 0xF, 0xF, false);
  return x + __builtin_bit_cast(float, y);
}

// The softmax reference m of a head moves only when a score exceeds it by
// more than 2^kLazy (log2 units), so most tiles need no cross-lane maximum and
// no rescaling; weights stay <= 2^kLazy.
constexpr float kLazy = 8.f;

// Token (0..31 within the tile) of A row m in MFMA row block e: row block e
// holds tokens 8*(m/4) + 4e + m%4, so the output lane group g ends up with
// the 8 consecutive tokens 8g..8g+7, the k-slots of its P operand.
__device__ __forceinline__ int a_token(int e, int m) { return 8 * (m >> 2) + 4 * e + (m & 3); }

__device__ __forceinline__ uint16_t umax16(uint16_t a, uint16_t b) { return a > b ? a : b; }

// Units of work: the 32-token tiles of quantized keys of every (sequence, KV
// head), ordered by sequence, then KV head, then tile; sequence b contributes
// H * ceil(Q_b / 32) units (Q_b = tokens whose keys are codes: all of them on
// the token axis, L_b - L_b mod R on the channel axis), or H units when it
// holds residual keys only. The residual fp16 keys of a (sequence, KV head)
// go with its last unit. Workgroup i of n takes the contiguous units
// [i U / n, (i+1) U / n), so every workgroup gets the same amount of work
// whatever the lengths, and walks the (sequence, KV head) segments its range
// covers.
__device__ __forceinline__ int seq_len_of(const CacheView& c, int b) {
  return min(max(c.seq_len[b], 0), c.T);  // clamped: never past the capacity
}
__device__ __forceinline__ int quant_len(const CacheView& c, int L) { return c.kaxis ? L - L % c.R : L; }
__device__ __forceinline__ int units_of(const CacheView& c, int L) {
  const int Q = quant_len(c, L);
  return Q > 0 ? (Q + kBlock - 1) / kBlock : (L > 0 ? 1 : 0);
}

// Workgroup whose range holds unit u.
__device__ __forceinline__ int wg_of_unit(int u, int64_t U, int nwg) {
  return (int)(((int64_t)(u + 1) * nwg + U - 1) / U) - 1;
}

struct UnitPos {
  int b;     // sequence holding the unit (B if the unit is past the last one)
  int base;  // its first unit
  int len;   // its length (clamped), 0 past the last sequence
};

// The sequence holding unit u: a wavefront-wide scan of the sequences' unit
// counts, 256 sequences (4 per lane) at a time. Every lane returns the same.
// Lengths are loaded at a clamped index, unconditionally, so that the four
// loads of a lane are in flight together.
__device__ UnitPos locate_unit(const CacheView& c, int u) {
  const int lane = threadIdx.x & 63;
  int acc = 0;
  for (int cb = 0; cb < c.B; cb += 256) {
    int n[4], len[4], sum = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) len[r] = seq_len_of(c, min(cb + 4 * lane + r, c.B - 1));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      n[r] = cb + 4 * lane + r < c.B ? c.H * units_of(c, len[r]) : 0;
      sum += n[r];
    }
    int incl = sum;  // inclusive scan over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    const int chunk = __shfl(incl, 63, 64);
    if (u < acc + chunk) {
      const uint64_t over = __builtin_amdgcn_ballot_w64(acc + incl > u);
      const int ll = (int)__builtin_ctzll(over);
      int base = acc + __shfl(incl - sum, ll, 64);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int nr = __shfl(n[r], ll, 64);
        if (u < base + nr) return UnitPos{__builtin_amdgcn_readfirstlane(cb + 4 * ll + r),
                                          __builtin_amdgcn_readfirstlane(base),
                                          __builtin_amdgcn_readfirstlane(__shfl(len[r], ll, 64))};
        base += nr;
      }
    }
    acc += chunk;
  }
  return UnitPos{c.B, __builtin_amdgcn_readfirstlane(acc), 0};
}

// Units of the sequences before b (a wavefront-wide sum; every lane returns it).
__device__ int units_before(const CacheView& c, int b) {
  const int lane = threadIdx.x & 63;
  int sum = 0;
  for (int b0 = 0; b0 < b; b0 += 256) {
    int len[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) len[k] = seq_len_of(c, min(b0 + lane + 64 * k, b - 1));  // in flight together
    int n[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) n[k] = b0 + lane + 64 * k < b ? units_of(c, len[k]) : 0;
    sum += c.H * (n[0] + n[1] + n[2] + n[3]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  return __builtin_amdgcn_readfirstlane(sum);
}

template <int KB, int VB, int KAXIS, int G, bool SPARSE, int FMT>
__global__ __launch_bounds__(256) void attn_kernel(CacheView c, AttnPlan p, const uint16_t* __restrict__ q,
                                                   float* __restrict__ out, float* __restrict__ ws) {
  using Gm = Geom<KB, VB, KAXIS, G, SPARSE, FMT>;
  constexpr bool kFp8 = FMT == kFmtFp8, kSym = FMT == kFmtSym32, kRope = FMT == kFmtRope;
  static_assert(FMT == kFmtInt || kRope || (KAXIS == 0 && !SPARSE), "fp8 and block formats are token-axis only");
  static_assert(!kRope || (KAXIS == 1 && !SPARSE), "rotary keys: channel axis, no sparse entries");
  static_assert(!kFp8 || (KB == 8 && VB == 8), "fp8 codes are bytes");
  constexpr int NB = Gm::kSlots;
  constexpr int kQMinK = -(1 << (KB - 1));
  constexpr int kQMinV = -(1 << (VB - 1));
  constexpr bool kPermV = VB != 8;  // k-slot pairs (i, i+4) for 4/2-bit values
  static_assert(2 * G <= 16, "hi/lo rows must fit 16");
  // unit of one code step in the key / value operands, and its inverse
  constexpr int kShK = unit_shift<KB>();
  constexpr float kUnitK = pow2f(kShK - 24), kInvUnitK = pow2f(24 - kShK);
  // The value-scale factor 2^kv, kv = kKvTop - E, is set from the largest fp16
  // biased exponent E among the value scales seen so far, so that s * 2^kv <
  // 2^6 and the P operand p * s * 2^kv < 2^14 stays inside fp16.
  constexpr int kKvTop = 20;
  // symmetric blocks: x = s (u + q_min), so the zero point in code steps is
  // -q_min for every token: a constant B operand (pair p at bit val_sh(p),
  // like the codes it goes with)
  const Frag bsym = {{(uint32_t)(-kQMinV << val_sh<VB>(0)) * 0x10001u, (uint32_t)(-kQMinV << val_sh<VB>(1)) * 0x10001u,
                      (uint32_t)(-kQMinV << val_sh<VB>(2)) * 0x10001u, (uint32_t)(-kQMinV << val_sh<VB>(3)) * 0x10001u}};
  // value blocks feeding one P.V product (one per 32-channel block for
  // symmetric blocks, whose scales differ per block)
  constexpr int kPB = kSym ? kSymBlocks : 1;
  constexpr int kVmW = kSym ? 16 : 8;  // value meta words of the lane's 8 tokens

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, c16 = lane & 15, grp = lane >> 4;
  const int hq = c16 % G;                         // head of this lane's column / row
  const bool lo_col = ((c16 / G) & 1) != 0;       // column / row holds the lo part
  const int brow = lo_col ? G + hq : hq;          // B-operand row this lane reads
  const float rowlo = lo_col ? 1.f : 0.f;         // lo rows of P
  const float qscale = p.scale * kLog2e;          // scores in log2 units
  const uint32_t vsel2 = (grp & 1) ? 0x0C030C02u : 0x0C010C00u;  // 2-bit value records: this lane's half

  constexpr int kWaveBytes = NB * Gm::kBytes + Gm::kWaveLds;
  constexpr int kMain = 4 * kWaveBytes;
  constexpr int kMerge = (int)sizeof(MergeLds<G>);
  __shared__ __attribute__((aligned(16))) uint8_t smem[kMain > kMerge ? kMain : kMerge];
  // query heads pre-scaled for the sparse entries (written identically by every wavefront)
  // (rows padded by one word: the heads' copies of a channel fall in different banks)
  __shared__ float qsh[SPARSE ? G : 1][SPARSE ? kD + 1 : 1];
  // rotary keys: revolutions per token of frequency i, theta_i / (2 pi) with
  // theta_i = base^(-i / 64), as two floats (computed in double)
  __shared__ float2 rphi[kRope ? 64 : 1];
  if constexpr (kRope) {
    if (tid < 64) {
      const double ph = exp2(-(double)tid / 64.0 * p.rope_log2_theta) * 0.15915494309189533577;
      const float hi = (float)ph;
      rphi[tid] = make_float2(hi, (float)(ph - (double)hi));
    }
    __syncthreads();
  }

  uint8_t* wbase = smem + w * kWaveBytes;             // this wavefront's slots
  WaveLds<G>& wl = *reinterpret_cast<WaveLds<G>*>(wbase + NB * Gm::kBytes);
  const uint32_t wbase_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)wbase;
  // the query heads land in the last slot, which no tile load touches before
  // the pipeline loop starts
  const uint32_t q_lds = wbase_lds + (NB - 1) * Gm::kBytes;
  const uint16_t* qlds = reinterpret_cast<const uint16_t*>(wbase + (NB - 1) * Gm::kBytes);

  // Channel axis: this lane builds the scaled query of 2 channels, all heads:
  // k-slot pair bp of chunk bj in lane group bg, bq = lane / 4 = 4 bg + bj.
  // The pair's codes sit at bit bsh, so its query carries 2^(kShK - bsh).
  const int bq = lane >> 2, bp = lane & 3, bg = bq >> 2, bj = bq & 3;
  const int bc0 = key_channel<KB>(bg, bj, bp, 0), bc1 = key_channel<KB>(bg, bj, bp, 1);
  const int bsh = KB == 8 ? 0 : (KB == 4 ? ((bp & 1) ? 4 : 0) : (((bj & 1) && bp == 0) ? 8 : 2 * bp + 2));
  // zero-point operand constants of the pair: -2^(bsh-24) and q_min * 2^(bsh-24)
  const h2v zmul = h2_splat((uint16_t)(0x8000u | (1u << bsh)));
  const h2v zofs = h2_splat((uint16_t)(0x8000u | (1u << (bsh + KB - 1))));
  // residual keys are plain fp16: their "scale" 2^(bsh - kShK) cancels the factor
  const uint32_t kres = (uint32_t)(15 + bsh - kShK) << 10;
  // metadata lanes of the tile loads: value scales, then key scales, then sparse entries
  const int mkind = lane < Gm::kVm / 16 ? 0 : (lane < (Gm::kVm + Gm::kKm) / 16 ? 1 : 2);

  // this workgroup's units
  const int nwg = gridDim.x, iwg = blockIdx.x;
  const int64_t U = p.units;
  const int u1 = (int)(((int64_t)iwg + 1) * U / nwg);
  int u = (int)((int64_t)iwg * U / nwg);
  const UnitPos pos = locate_unit(c, u);
  int b = pos.b, base = pos.base, L = pos.len;
  bool first_seg = true;
  while (u < u1 && b < c.B) {
    // ---- the segment: tiles [k0, k1) of (sequence b, KV head h) -------------
    const int Q = quant_len(c, L);
    const int nt = units_of(c, L);  // > 0: sequences without units are skipped
    const int rel = u - base;
    const int h = rel / nt, k0 = rel - h * nt;
    const int k1 = min(nt, k0 + (u1 - u));
    // a segment that is the whole (sequence, KV head) writes the output;
    // otherwise a partial result into the workgroup's slot for its first
    // segment (2 iwg) or for its last one (2 iwg + 1): only those two can be
    // pieces of a pair that other workgroups share
    const bool whole = k0 == 0 && k1 == nt;
    const int slot = 2 * iwg + (first_seg ? 0 : 1);
    const size_t bh = (size_t)b * c.H + h;
    const int ts0 = min(k0 * kBlock, Q), ts1 = min(k1 * kBlock, Q);
    // This wavefront's quantized tiles: k = w, w + 4, ... over [ts0, ts1).
    const int ntiles = (ts1 - ts0 + kBlock - 1) / kBlock;
    // (wave-uniform: made scalar so that the loop's waits and issues branch on SGPRs)
    const int nw = __builtin_amdgcn_readfirstlane((w < ntiles) ? (ntiles - w + 3) / 4 : 0);
    // residual fp16 keys [Q, L): with the pair's last unit
    const int nres = (k1 == nt) ? (L - Q + kBlock - 1) / kBlock : 0;

    // Tile loads go through bounded descriptors over this (sequence, KV
    // head)'s slice of each cache array, so an offset outside the slice reads
    // zeros and never touches other memory. Byte offsets of the next tile to
    // issue: key codes and value blocks, the tile's start plus lane * 16 (+ 1
    // KiB steps); metadata, each lane its 16-byte piece of one of the arrays
    // (value scales, key scales, sparse entries; one load per array). Offsets
    // advance by 4 tiles per issue (the wavefront takes every 4th tile).
    const int tw0 = ts0 + w * kBlock;
    const uint32_t Tu = (uint32_t)c.T;
    const u32x4 rk = make_rsrc(c.k_codes + bh * c.T * (size_t)Gm::kRowK, Tu * Gm::kRowK);
    const u32x4 rv = make_rsrc(c.v_codes + bh * (c.T / kBlock) * (size_t)Gm::kV, (Tu / kBlock) * Gm::kV);
    constexpr int kMt = Gm::kMetaTok;
    const u32x4 rvm = make_rsrc(reinterpret_cast<const uint8_t*>(c.v_meta) + bh * c.T * kMt, Tu * kMt);
    const u32x4 rkm = KAXIS ? make_rsrc(c.k_meta + bh * (c.T / kBlock) * kD, (Tu / kBlock) * kD * 4)
                            : make_rsrc(reinterpret_cast<const uint8_t*>(c.k_meta) + bh * c.T * kMt, Tu * kMt);
    const u32x4 rsp = SPARSE ? make_rsrc(c.k_sparse + bh * c.T * 2, Tu * 8) : rvm;
    const u32x4 rq = make_rsrc(q + ((size_t)b * p.Hq + (size_t)h * G) * kD, G * kD * 2);
    uint32_t koff = (uint32_t)tw0 * Gm::kRowK + lane * 16;
    uint32_t voff = (uint32_t)(tw0 / kBlock) * Gm::kV + lane * 16;
    uint32_t moff, mstep;
    if (mkind == 0) {
      moff = (uint32_t)tw0 * kMt + lane * 16;
      mstep = 4 * kBlock * kMt;
    } else if (mkind == 1) {
      moff = (KAXIS ? (uint32_t)(tw0 / kBlock) * kD * 4 : (uint32_t)tw0 * kMt) + (lane - Gm::kVm / 16) * 16;
      mstep = KAXIS ? 4 * kD * 4 : 4 * kBlock * kMt;
    } else {
      moff = (uint32_t)tw0 * 8 + (uint32_t)(lane - (Gm::kVm + Gm::kKm) / 16) * 16;
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
      if constexpr (Gm::kVm > 0) {
        if (mkind == 0) dma16(rvm, moff, lbm);
      }
      if constexpr (Gm::kKm > 0) {
        if (mkind == 1) dma16(rkm, moff, lbm);
      }
      if constexpr (SPARSE) {
        if (mkind == 2 && lane < Gm::kMetaLanes) dma16(rsp, moff, lbm);
      }
      koff += 4 * Gm::kK;
      voff += 4 * Gm::kV;
      moff += mstep;
    };

    // the query heads, then the first tiles
#pragma unroll
    for (int x = 0; x < Gm::kQLoads; ++x) dma16(rq, x * 1024 + lane * 16, q_lds + x * 1024);
    const int npro = min(NB - 1, nw);
#pragma unroll
    for (int i = 0; i < NB - 1; ++i)
      if (i < npro) issue(i);
    // the query has landed once at most the tile loads issued after it remain
    wait_vm_n<Gm::kLoads>(npro);
    if constexpr (SPARSE) {  // sparse entries add q * x directly to the scaled score
      for (int i = lane; i < G * kD; i += 64) qsh[i / kD][i % kD] = h2f(qlds[i]) * (qscale * kUnitK);
    }
    float qv0[KAXIS ? G : 1], qv1[KAXIS ? G : 1];
    // token axis: the B operand is the raw fp16 query of head n mod G (exact);
    // qsum_u = unit * sum_c q_c for the zero-point term (symmetric blocks: the
    // sum over each block's channels, qsum_b[j])
    Frag qfrag[(KAXIS && !kRope) ? 1 : 4];
    float qsum_u = 0.f, qsum_b[kSym ? kSymBlocks : 1];
    if constexpr (KAXIS && !kRope) {
      const float qs = qscale * (float)(1 << (kShK - bsh));
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        qv0[hh] = h2f(qlds[hh * kD + bc0]) * qs;
        qv1[hh] = h2f(qlds[hh * kD + bc1]) * qs;
      }
    } else {
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float sj = 0.f;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          // symmetric blocks: MFMA j covers channel block j (lane group and
          // chunk roles swapped)
          // (rotary keys: a chunk and its partner chunk hold each pair's channels)
          const int ch0 = kRope ? rope_channel<KB>(grp, j, pp, 0)
                                : (kSym ? key_channel<KB>(j, grp, pp, 0) : key_channel<KB>(grp, j, pp, 0));
          const int ch1 = kRope ? rope_channel<KB>(grp, j, pp, 1)
                                : (kSym ? key_channel<KB>(j, grp, pp, 1) : key_channel<KB>(grp, j, pp, 1));
          const uint32_t a0 = qlds[hq * kD + ch0], a1 = qlds[hq * kD + ch1];
          qfrag[j].p[pp] = a0 | (a1 << 16);
          sj += h2f((uint16_t)a0) + h2f((uint16_t)a1);
        }
        if constexpr (kSym) qsum_b[j] = grp_sum(sj) * kUnitK;
        sum += sj;
      }
      qsum_u = grp_sum(sum) * kUnitK;
    }
    wait_lgkm0();  // the query is in registers before its slot is reused
    wave_lds_fence();

    float m_ref = -INFINITY, l_run = 0.f;
    int vE = 0;                       // exponent the value-scale factor is set for
    f4v acc[8], accz[kPB];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int z = 0; z < kPB; ++z) accz[z] = f4v{0.f, 0.f, 0.f, 0.f};

    // ---- scores of one tile -> online softmax -> P.V ---------------------------
    // sc[4e + r] is the scaled score (log2 units = sc * cs) of token
    // 8grp + 4e + r; vm the value meta of tokens 8grp .. 8grp + 7 (affine: one
    // word each; symmetric blocks: words 2i, 2i + 1 of token i, the scales of
    // blocks 0, 1 and 2, 3; fp8: none); vcl/vch[j] the lane's value code
    // words of channel chunk j.
    auto softmax_pv = [&](float (&sc)[8], float cs, const uint32_t (&vm)[kVmW], const uint32_t (&vcl)[8],
                          const uint32_t (&vch)[8], int t0, int tend) {
      const int nvalid = __builtin_amdgcn_readfirstlane(tend - t0);
      if (__builtin_expect(nvalid < kBlock, 0)) {  // a partial tile (rare): a branch, not 16 selects per tile
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (8 * grp + i >= nvalid) sc[i] = -INFINITY;
      }
      const float mx = max8(sc);
      if (__builtin_amdgcn_ballot_w64(__builtin_fmaf(mx, cs, -m_ref) > kLazy)) {
        const float m_new = fmaxf(m_ref, grp_max(mx * cs));
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, (4 * grp + r) % G, 64);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j][r] *= ar[r];
#pragma unroll
          for (int z = 0; z < kPB; ++z) accz[z][r] *= ar[r];
        }
        l_run *= alpha;
        m_ref = m_new;
      }
      if constexpr (!kFp8) {
        // value-scale exponent: raise it when a scale of this tile reaches 2^6 * 2^-kv
        uint16_t smax;
        if constexpr (kSym) {  // both halves of every word are scales
          uint16_t m0 = 0, m1 = 0;
#pragma unroll
          for (int i = 0; i < kVmW; ++i) {
            m0 = umax16(m0, (uint16_t)vm[i]);
            m1 = umax16(m1, (uint16_t)(vm[i] >> 16));
          }
          smax = umax16(m0, m1);
        } else {
          smax = umax16(umax16(umax16((uint16_t)vm[0], (uint16_t)vm[1]), umax16((uint16_t)vm[2], (uint16_t)vm[3])),
                        umax16(umax16((uint16_t)vm[4], (uint16_t)vm[5]), umax16((uint16_t)vm[6], (uint16_t)vm[7])));
        }
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
#pragma unroll
            for (int z = 0; z < kPB; ++z) accz[z][r] *= f;
          }
          l_run *= f;
          vE = e_new;
        }
      }
      // fp8: P = p (at most 2^kLazy); otherwise P = p * s * 2^kv; both times
      // 2^-val_sh of the token's k-slot pair (the position of its value codes),
      // taken into the exponent; l_run sums the weights p without it
      const float kvm = (kFp8 ? 0.f : (float)(kKvTop - vE)) - m_ref;
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int sh = val_sh<VB>(kPermV ? (i & 3) : (i >> 1));
        x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], cs, kvm - (float)sh));
        l_run = __builtin_fmaf(x[i], __builtin_ldexpf(1.f, sh), l_run);
      }
      // the P operand from the 8 weights a[] of the lane's tokens; lo rows keep
      // P - fp16(P)
      auto p_frag = [&](const float (&a)[8]) {
        Frag pf;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int i0 = kPermV ? pp : 2 * pp;
          const int i1 = kPermV ? pp + 4 : 2 * pp + 1;
          const uint32_t hi = pk_rtz(a[i0], a[i1]);
          pf.p[pp] = pk_rtz(__builtin_fmaf(f16lo(hi), -rowlo, a[i0]), __builtin_fmaf(f16hi(hi), -rowlo, a[i1]));
        }
        return pf;
      };
      if constexpr (kFp8) {
        const Frag pf = p_frag(x);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mfma(pf, fp8_frag(vcl[j], vch[j]), acc[j]);
      } else if constexpr (kSym) {
        // channel chunk j (channels 16 j .. 16 j + 15) lies in block j / 2
#pragma unroll
        for (int bk = 0; bk < kSymBlocks; ++bk) {
          float a[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t w2 = vm[2 * i + (bk >> 1)];
            a[i] = __builtin_fmaf(x[i], (bk & 1) ? f16hi(w2) : f16lo(w2), 0.f);
          }
          const Frag pf = p_frag(a);
          accz[bk] = mfma(pf, bsym, accz[bk]);
          acc[2 * bk] = mfma(pf, val_frag<VB>(vcl[2 * bk], vch[2 * bk]), acc[2 * bk]);
          acc[2 * bk + 1] = mfma(pf, val_frag<VB>(vcl[2 * bk + 1], vch[2 * bk + 1]), acc[2 * bk + 1]);
        }
      } else {
        float a[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = mul_lo(x[i], vm[i]);
        const Frag pf = p_frag(a);
        Frag bz;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int i0 = kPermV ? pp : 2 * pp;
          const int i1 = kPermV ? pp + 4 : 2 * pp + 1;
          // (z'_i0, z'_i1) in code steps at the pair's bit, z' = z - qmin
          const int sh = val_sh<VB>(pp);
          const _Float16 zs = (_Float16)__builtin_ldexpf(1.f, sh - 24), zo = (_Float16)__builtin_ldexpf((float)-kQMinV, sh - 24);
          bz.p[pp] = pk_fma16(perm(vm[i1], vm[i0], 0x07060302u), h2v{zs, zs}, h2v{zo, zo});
        }
        accz[0] = mfma(pf, bz, accz[0]);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = mfma(pf, val_frag<VB>(vcl[j], vch[j]), acc[j]);
      }
    };

    // the B operand of the key product for a block: scaled query (hi/lo) with
    // the per-channel scales in the low halves of km0, km1; with_zero also
    // writes the zero-point operand -(z - qmin) from their high halves
    auto build_qb = [&](uint32_t km0, uint32_t km1, bool with_zero) {
      const float m1 = opaque_neg1();
      wave_lds_fence();
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float v0 = mul_lo(qv0[hh], km0), v1 = mul_lo(qv1[hh], km1);
        const uint32_t hi = pk_rtz(v0, v1);
        wl.qb[bg][hh][bj].p[bp] = hi;
        wl.qb[bg][G + hh][bj].p[bp] = pk_rtz(__builtin_fmaf(f16lo(hi), m1, v0), __builtin_fmaf(f16hi(hi), m1, v1));
      }
      if (with_zero) wl.zc[bg][bj][bp] = pk_fma16(perm(km1, km0, 0x07060302u), zmul, zofs);
      wave_lds_fence();
    };

    // ---- quantized tiles through the LDS pipeline -----------------------------
    // Tile i sits in slot i mod NB.
    auto tile = [&](const int i, const int slot) {
      if (i + NB - 1 < nw) issue((slot + NB - 1) % NB);
      // tile i has landed once at most (tiles issued after it) x loads remain
      wait_vm_n<Gm::kLoads>(min(NB - 1, nw - 1 - i));
      const uint8_t* sb = wbase + slot * Gm::kBytes;
      const uint8_t* kbuf = sb;
      const uint8_t* vbuf = sb + Gm::kK;
      const uint32_t* vmeta = reinterpret_cast<const uint32_t*>(sb + Gm::kK + Gm::kV);
      const uint32_t* kmeta = vmeta + Gm::kVm / 4;
      const uint32_t* spr = kmeta + Gm::kKm / 4;
      const int t0 = ts0 + (w + 4 * i) * kBlock;

      // metadata words of the lane's tokens 8grp .. 8grp + 7 (kVmW per array)
      uint32_t vm[kVmW];
      if constexpr (!kFp8) {
#pragma unroll
        for (int x = 0; x < kVmW / 4; ++x) {
          const uint4 a = reinterpret_cast<const uint4*>(vmeta + kVmW * grp)[x];
          vm[4 * x] = a.x; vm[4 * x + 1] = a.y; vm[4 * x + 2] = a.z; vm[4 * x + 3] = a.w;
        }
      }
      // sparse key entries of the lane's tokens 8grp .. 8grp + 7 and the
      // scaled query at their channels, read before the key product (whose
      // LDS fences would otherwise hold these reads back until after it)
      float spq[SPARSE ? 16 : 1];
      uint32_t spv[SPARSE ? 8 : 1];
      if constexpr (SPARSE) {
        uint32_t spc[8];
#pragma unroll
        for (int i2 = 0; i2 < 8; i2 += 2) {
          const uint4 r2 = reinterpret_cast<const uint4*>(spr)[(8 * grp + i2) / 2];
          spv[i2] = r2.x; spc[i2] = r2.y; spv[i2 + 1] = r2.z; spc[i2 + 1] = r2.w;
        }
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) {
          spq[2 * i2] = qsh[hq][spc[i2] & 0xFFFFu];
          spq[2 * i2 + 1] = qsh[hq][spc[i2] >> 16];
        }
      }
      // key codes of the lane's two A rows: bytes [grp*4KB, +4KB) of each row
      // (symmetric blocks: kc[e][j] / kc[e][2j, 2j+1] the words sym_key_frag
      // takes for block j)
      uint32_t kc[2][kSym ? (KB == 8 ? 8 : 4) : KB];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint8_t* rowb = kbuf + a_token(e, c16) * Gm::kRowK;
        if constexpr (kRope) {
          // channels [16 grp, +16) (2 KB bytes at 2 KB grp) and their partners
          // 64 higher (8 KB bytes on): KB / 2 words each
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const uint8_t* src = rowb + hf * 8 * KB + 2 * KB * grp;
            if constexpr (KB == 8) {
              const uint4 y = reinterpret_cast<const uint4*>(src)[0];
              kc[e][4 * hf] = y.x; kc[e][4 * hf + 1] = y.y; kc[e][4 * hf + 2] = y.z; kc[e][4 * hf + 3] = y.w;
            } else if constexpr (KB == 4) {
              const uint2 y = reinterpret_cast<const uint2*>(src)[0];
              kc[e][2 * hf] = y.x; kc[e][2 * hf + 1] = y.y;
            } else {
              kc[e][hf] = reinterpret_cast<const uint32_t*>(src)[0];
            }
          }
        } else if constexpr (kSym) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if constexpr (KB == 8) {
              const uint2 y = reinterpret_cast<const uint2*>(rowb + 32 * j + 8 * grp)[0];
              kc[e][2 * j] = y.x;
              kc[e][2 * j + 1] = y.y;
            } else if constexpr (KB == 4) {
              kc[e][j] = reinterpret_cast<const uint32_t*>(rowb + 16 * j + 4 * grp)[0];
            } else {
              kc[e][j] = reinterpret_cast<const uint32_t*>(rowb + 8 * j + 4 * (grp >> 1))[0] >> (8 * (grp & 1));
            }
          }
        } else {
          const uint8_t* row = rowb + grp * 4 * KB;
#pragma unroll
          for (int x = 0; x < KB; x += 2) {
            const uint2 y = reinterpret_cast<const uint2*>(row)[x / 2];
            kc[e][x] = y.x;
            kc[e][x + 1] = y.y;
          }
        }
      }
      float sc[8];
      float cs;
      if constexpr (kRope) {
        // keys dequantized exactly, x = s (u - z) + s q_min, rotated by their
        // positions and split into fp16 hi and lo parts: two products each
        // with the raw query; chunk jj and its partner chunk jj + 2
        f4v s[2] = {f4v{0.f, 0.f, 0.f, 0.f}, f4v{0.f, 0.f, 0.f, 0.f}};
        const float tq[2] = {(float)(t0 + a_token(0, c16)), (float)(t0 + a_token(1, c16))};
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          Frag fa[2], fb[2], ah[2], al[2], bh[2], bl[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            fa[e] = key_frag<KB, true>(kc[e], jj);
            fb[e] = key_frag<KB, true>(kc[e], jj + 2);
          }
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            float ya[2][2], yb[2][2];  // [row block][half]
#pragma unroll
            for (int hs = 0; hs < 2; ++hs) {
              const int cc = 16 * grp + key_channel<KB>(0, jj, pp, hs);  // frequency index
              const uint32_t ma = kmeta[cc], mb = kmeta[cc + 64];
              // x = operand * (s / unit) + s (q_min - z), exact in fp32
              const float sa = f16lo(ma), sb = f16lo(mb);
              const float aa = sa * kInvUnitK, ab = sb * kInvUnitK;
              const float ba = sa * ((float)kQMinK - f16hi(ma)), bb = sb * ((float)kQMinK - f16hi(mb));
              const float2 ph = rphi[cc];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                const float xa = __builtin_fmaf(hs ? f16hi(fa[e].p[pp]) : f16lo(fa[e].p[pp]), aa, ba);
                const float xb = __builtin_fmaf(hs ? f16hi(fb[e].p[pp]) : f16lo(fb[e].p[pp]), ab, bb);
                float cr, sr;
                rope_cs(tq[e], ph, cr, sr);
                ya[e][hs] = __builtin_fmaf(xa, cr, -xb * sr);
                yb[e][hs] = __builtin_fmaf(xb, cr, xa * sr);
              }
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              split_hilo(ya[e][0], ya[e][1], ah[e].p[pp], al[e].p[pp]);
              split_hilo(yb[e][0], yb[e][1], bh[e].p[pp], bl[e].p[pp]);
            }
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            s[e] = mfma(ah[e], qfrag[jj], s[e]);
            s[e] = mfma(al[e], qfrag[jj], s[e]);
            s[e] = mfma(bh[e], qfrag[jj + 2], s[e]);
            s[e] = mfma(bl[e], qfrag[jj + 2], s[e]);
          }
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[4 * e + r] = s[e][r];
        cs = qscale;
      } else if constexpr (KAXIS) {
        build_qb(kmeta[bc0], kmeta[bc1], true);
        // zero-point term, the same for every token of the block
        f4v cz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) cz = mfma(*reinterpret_cast<const Frag*>(wl.zc[grp][j]), wl.qb[grp][brow][j], cz);
        f4v s[2] = {cz, cz};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const Frag qf = wl.qb[grp][brow][j];
#pragma unroll
          for (int e = 0; e < 2; ++e) s[e] = mfma(key_frag<KB, false>(kc[e], j), qf, s[e]);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[4 * e + r] = add_ror<G>(s[e][r]);
        cs = kInvUnitK;
      } else if constexpr (kFp8) {
        // keys are E4M3 values times the cache's key scale
        f4v s[2] = {f4v{0.f, 0.f, 0.f, 0.f}, f4v{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 2; ++e) s[e] = mfma(fp8_frag(kc[e][2 * j], kc[e][2 * j + 1]), qfrag[j], s[e]);
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[4 * e + r] = s[e][r];
        cs = qscale * c.kscale;
      } else if constexpr (kSym) {
        // one product per 32-channel block (its scale differs per token),
        // seeded with q_min * sum of the block's query channels; then
        // score = sum_j s_j(t) * block product j
        uint32_t km[16];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const uint4 a = reinterpret_cast<const uint4*>(kmeta + 16 * grp)[x];
          km[4 * x] = a.x; km[4 * x + 1] = a.y; km[4 * x + 2] = a.z; km[4 * x + 3] = a.w;
        }
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2) sc[i2] = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float seed = (float)kQMinK * qsum_b[j];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            Frag kf;
            if constexpr (KB == 8) kf = sym_key_frag<KB>(kc[e][2 * j], kc[e][2 * j + 1]);
            else kf = sym_key_frag<KB>(kc[e][j], 0u);
            const f4v sj = mfma(kf, qfrag[j], f4v{seed, seed, seed, seed});
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const uint32_t kw = km[2 * (4 * e + r) + (j >> 1)];
              sc[4 * e + r] = __builtin_fmaf(sj[r], (j & 1) ? f16hi(kw) : f16lo(kw), sc[4 * e + r]);
            }
          }
        }
        cs = kInvUnitK * qscale;
      } else {
        uint32_t km[8];
        {
          const uint4 a = reinterpret_cast<const uint4*>(kmeta + 8 * grp)[0];
          const uint4 bb = reinterpret_cast<const uint4*>(kmeta + 8 * grp)[1];
          km[0] = a.x; km[1] = a.y; km[2] = a.z; km[3] = a.w;
          km[4] = bb.x; km[5] = bb.y; km[6] = bb.z; km[7] = bb.w;
        }
        const float seed = (float)kQMinK * qsum_u;  // sum_c q_c (u_c + q_min) = sum_c q_c q_c'
        f4v s[2] = {f4v{seed, seed, seed, seed}, f4v{seed, seed, seed, seed}};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 2; ++e) s[e] = mfma(key_frag<KB, true>(kc[e], j), qfrag[j], s[e]);
        // minus z_t * sum_c q_c, then times the token's scale
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t kw = km[4 * e + r];
            sc[4 * e + r] = mul_lo(__builtin_fmaf(f16hi(kw), -qsum_u, s[e][r]), kw);
          }
        cs = kInvUnitK * qscale;
      }
      if constexpr (SPARSE) {
#pragma unroll
        for (int i2 = 0; i2 < 8; ++i2)
          sc[i2] += spq[2 * i2] * f16lo(spv[i2]) + spq[2 * i2 + 1] * f16hi(spv[i2]);
      }
      // value codes: channel 16j + c16, tokens 8grp .. 8grp+7 of the block
      uint32_t vcl[8], vch[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) val_words<VB>(vbuf + (16 * j + c16) * 4 * VB, grp, vsel2, vcl[j], vch[j]);
      softmax_pv(sc, cs, vm, vcl, vch, t0, ts1);
    };
    for (int i = 0; i < nw; ++i) tile(i, i % NB);


    // ---- residual (fp16) key tiles, channel axis only: tile j holds tokens
    // Q + 32 j .. + 31 (< L); this wavefront takes j = w, w + 4, ... They go
    // through the wavefront's LDS slots, free after the pipeline: the value
    // block and value scales as for a code tile, and the fp16 keys 16 tokens
    // (one A-row block, 4 KiB) at a time; each half runs the key product, the
    // softmax and P.V of its 16 tokens (the other half's scores masked).
    if constexpr (KAXIS) {
      const uint32_t lk = wbase_lds, lv = wbase_lds + 4096, lm = lv + Gm::kV;
      const uint8_t* kres_lds = wbase;
      const uint8_t* vres_lds = wbase + 4096;
      const uint32_t* vmres_lds = reinterpret_cast<const uint32_t*>(wbase + 4096 + Gm::kV);
      const u32x4 rr = make_rsrc(c.k_resid + bh * c.R * (size_t)kD, (uint32_t)c.R * kD * 2);
      for (int jr = w; jr < nres; jr += 4) {
        const int t0 = Q + jr * kBlock;
        wait_lgkm0();  // earlier LDS reads of the slots are done
        wave_lds_fence();
#pragma unroll
        for (int x = 0; x < Gm::kV / 1024; ++x)
          dma16(rv, (uint32_t)(t0 / kBlock) * Gm::kV + x * 1024 + lane * 16, lv + x * 1024);
        if (lane < 8) dma16(rvm, (uint32_t)t0 * 4 + lane * 16, lm);
        // B operand: query scaled by the softmax factor only (the pair's 2^lf
        // cancelled), hi/lo; rotary keys use the raw query operand instead
        if constexpr (!kRope) build_qb(kres, kres, false);
#pragma nounroll
        for (int e = 0; e < 2; ++e) {
          // keys of row block e: LDS row m (0..15) = token t0 + a_token(e, m);
          // each load moves 4 rows, lane l a 16-byte piece of row 4x + l/16
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int tt = t0 - Q + a_token(e, 4 * x + (lane >> 4));
            dma16(rr, (uint32_t)tt * (kD * 2) + (lane & 15) * 16, lk + x * 1024);
          }
          wait_vm<0>();
          uint32_t rk[16];
          {
            // the lane's 32 channels of its row (rotary keys: [16 grp, +16)
            // and the partners 64 higher)
            const uint4* kr4 = reinterpret_cast<const uint4*>(kres_lds + c16 * (kD * 2) + (kRope ? 32 : 64) * grp);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const uint4 v = kr4[kRope ? (x & 1) + 8 * (x >> 1) : x];
              rk[4 * x] = v.x; rk[4 * x + 1] = v.y; rk[4 * x + 2] = v.z; rk[4 * x + 3] = v.w;
            }
          }
          f4v s1 = {0.f, 0.f, 0.f, 0.f};
          if constexpr (kRope) {
            // rotate by position, split hi / lo, two products with the raw query
            const float tq = (float)(t0 + a_token(e, c16));
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
              Frag ah, al, bh, bl;
#pragma unroll
              for (int pp = 0; pp < 4; ++pp) {
                float ya[2], yb[2];
#pragma unroll
                for (int hs = 0; hs < 2; ++hs) {
                  const int o = key_channel<KB>(0, jj, pp, hs);  // channel 16 grp + o
                  const float xa = (o & 1) ? f16hi(rk[o >> 1]) : f16lo(rk[o >> 1]);
                  const float xb = (o & 1) ? f16hi(rk[8 + (o >> 1)]) : f16lo(rk[8 + (o >> 1)]);
                  float cr, sr;
                  rope_cs(tq, rphi[16 * grp + o], cr, sr);
                  ya[hs] = __builtin_fmaf(xa, cr, -xb * sr);
                  yb[hs] = __builtin_fmaf(xb, cr, xa * sr);
                }
                split_hilo(ya[0], ya[1], ah.p[pp], al.p[pp]);
                split_hilo(yb[0], yb[1], bh.p[pp], bl.p[pp]);
              }
              s1 = mfma(ah, qfrag[jj], s1);
              s1 = mfma(al, qfrag[jj], s1);
              s1 = mfma(bh, qfrag[jj + 2], s1);
              s1 = mfma(bl, qfrag[jj + 2], s1);
            }
          }
#pragma unroll
          for (int j = 0; j < (kRope ? 0 : 4); ++j) {
            // k-slot pair pp of chunk j: the keys of the channels the codes use
            Frag kf;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              const int c0 = key_channel<KB>(0, j, pp, 0), c1 = key_channel<KB>(0, j, pp, 1);
              const uint32_t sel = ((c0 & 1) ? 0x0302u : 0x0100u) | ((c1 & 1) ? 0x07060000u : 0x05040000u);
              kf.p[pp] = perm(rk[c1 >> 1], rk[c0 >> 1], sel);
            }
            s1 = mfma(kf, wl.qb[grp][brow][j], s1);
          }
          float sc[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {  // tokens 8grp + 4e + r: slots 4e + r
            const float v = kRope ? s1[r] : add_ror<G>(s1[r]);
            sc[r] = (e == 0) ? v : -INFINITY;
            sc[4 + r] = (e == 0) ? -INFINITY : v;
          }
          uint32_t vm[kVmW], vcl[8], vch[8];
          {
            const uint4 a = reinterpret_cast<const uint4*>(vmres_lds + 8 * grp)[0];
            const uint4 bb = reinterpret_cast<const uint4*>(vmres_lds + 8 * grp)[1];
            vm[0] = a.x; vm[1] = a.y; vm[2] = a.z; vm[3] = a.w;
            vm[4] = bb.x; vm[5] = bb.y; vm[6] = bb.z; vm[7] = bb.w;
          }
#pragma unroll
          for (int j = 0; j < 8; ++j) val_words<VB>(vres_lds + (16 * j + c16) * 4 * VB, grp, vsel2, vcl[j], vch[j]);
          softmax_pv(sc, kRope ? qscale : 1.f, vm, vcl, vch, t0, L);
          wait_lgkm0();  // the keys are read before the next half's loads
          wave_lds_fence();
        }
      }
    }

    // ---- merge the wavefronts of the workgroup ------------------------------
    // o = (acc - accz) / (value code unit) * 2^-kv, l = l_run * 2^-kv; fp8:
    // o = acc * (value scale), l = l_run
    const float ofac = kFp8 ? c.vscale : __builtin_bit_cast(float, (uint32_t)(127 + 24 - kKvTop + vE) << 23);
    const float lfac = kFp8 ? 1.f : __builtin_bit_cast(float, (uint32_t)(127 - kKvTop + vE) << 23);
    const float lsum = grp_sum(l_run) * lfac;
    wait_vm<0>();     // no tile load still writing LDS
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
        if (row < 2 * G) mg.o[w][row][16 * j + c16] = (kFp8 ? acc[j][r] : acc[j][r] - accz[kSym ? j / 2 : 0][r]) * ofac;
      }
    __syncthreads();
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
      if (whole) {
        out[qh * kD + ch] = (l > 0.f) ? o / l : 0.f;
      } else {
        float* pt = ws + ((size_t)slot * G + hh) * kPartialFloats;
        if (ch == 0) { pt[0] = M; pt[1] = l; }
        pt[4 + ch] = o;
      }
    }
    __syncthreads();  // the merge area is free again before the next segment's loads

    // ---- next segment -------------------------------------------------------
    first_seg = false;
    u += k1 - k0;
    if (k1 == nt && h == c.H - 1) {  // on to the next sequence with units (L > 0)
      base += c.H * nt;
      for (++b; b < c.B; ++b) {
        L = __builtin_amdgcn_readfirstlane(seq_len_of(c, b));
        if (L > 0) break;
      }
    }
  }
}

// Merge kernel: one workgroup of 256 threads per (sequence, query head)
// whose output the attention kernel did not write: sequences with no tokens
// (output 0) and pairs whose units span several workgroups, whose partial
// results it merges with a log-sum-exp. Thread t takes channel t mod 128 and
// every second partial (t / 128 says which): it loads a batch of C partials'
// (m, l, o[channel]) at once, so one round trip to memory covers a whole
// batch, merges them in registers, and the two halves meet in LDS. C is 4
// when no pair has more than 8 pieces and 32 otherwise (a single long
// sequence over many workgroups): the wide batch's registers would cut the
// workgroups resident per compute unit for every launch.
template <int C>
__global__ __launch_bounds__(256) void combine_kernel(CacheView c, AttnPlan p, const float* __restrict__ ws,
                                                      float* __restrict__ out) {
  __shared__ float other[3][kD];  // the second half's (M, l, o)
  const int bq = blockIdx.x, t = threadIdx.x, ch = t & (kD - 1), half = t >> 7;
  const int b = bq / p.Hq, hkv = (bq % p.Hq) / p.group, hh = bq % p.group;
  // the length and the units before the sequence: loads issued together
  const int L = seq_len_of(c, b);
  const int before = units_before(c, b);
  if (L == 0) {
    if (half == 0) out[(size_t)bq * kD + ch] = 0.f;
    return;
  }
  const int nt = units_of(c, L);
  const int s0 = before + hkv * nt;  // the pair's units [s0, s0 + nt)
  const int first = wg_of_unit(s0, p.units, p.n_wg), last = wg_of_unit(s0 + nt - 1, p.units, p.n_wg);
  const int np = last - first + 1;
  if (np <= 1) return;  // written by the attention kernel
  // the pair is the first segment of every workgroup of it but possibly the
  // first one, where it is the last segment unless it starts the range
  const bool mid_start = s0 != (int)((int64_t)first * p.units / p.n_wg);
  auto rec = [&](int j) -> const float* {
    const int slot = 2 * (first + j) + ((j == 0 && mid_start) ? 1 : 0);
    return ws + ((size_t)slot * p.group + hh) * kPartialFloats;
  };
  float M = -INFINITY, o = 0.f, l = 0.f;
  // merge the partials j = half, half + 2, ... in batches of C
  {
    for (int j0 = half; j0 < np; j0 += 2 * C) {
      float mv[C], lv[C], ov[C];
      // loads of a clamped index, unconditional, so that all of them are in
      // flight together; entries past the last partial are masked afterwards
#pragma unroll
      for (int y = 0; y < C; ++y) {
        const float* pt = rec(min(j0 + 2 * y, np - 1));
        mv[y] = pt[0];
        lv[y] = pt[1];
        ov[y] = pt[4 + ch];
      }
#pragma unroll
      for (int y = 0; y < C; ++y)
        if (j0 + 2 * y >= np) mv[y] = -INFINITY;
      float mb = mv[0];
#pragma unroll
      for (int y = 1; y < C; ++y) mb = fmaxf(mb, mv[y]);
      const float m_new = fmaxf(M, mb);
      if (m_new == -INFINITY) continue;
      const float fo = __builtin_amdgcn_exp2f(M - m_new);
      o *= fo;
      l *= fo;
#pragma unroll
      for (int y = 0; y < C; ++y) {  // an absent or empty partial weighs exp2(-inf) = 0
        const float f = __builtin_amdgcn_exp2f(mv[y] - m_new);
        o = __builtin_fmaf(f, ov[y], o);
        l = __builtin_fmaf(f, lv[y], l);
      }
      M = m_new;
    }
  }
  if (half == 1) {
    other[0][ch] = M;
    other[1][ch] = l;
    other[2][ch] = o;
  }
  __syncthreads();
  if (half == 0) {
    const float M2 = other[0][ch], m_new = fmaxf(M, M2);
    float lt = 0.f, ot = 0.f;
    if (m_new != -INFINITY) {
      const float f1 = __builtin_amdgcn_exp2f(M - m_new), f2 = __builtin_amdgcn_exp2f(M2 - m_new);
      lt = f1 * l + f2 * other[1][ch];
      ot = f1 * o + f2 * other[2][ch];
    }
    out[(size_t)bq * kD + ch] = (lt > 0.f) ? ot / lt : 0.f;
  }
}

// Launch of one kernel variant, or (occ != nullptr) its resident workgroups
// per compute unit.
template <int KB, int VB, int KAXIS, int G, bool SPARSE, int FMT>
hipError_t launch_t(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                    hipStream_t st, int* occ) {
  if (occ) {
    const void* fn = reinterpret_cast<const void*>(attn_kernel<KB, VB, KAXIS, G, SPARSE, FMT>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(occ, attn_kernel<KB, VB, KAXIS, G, SPARSE, FMT>, 256, 0) ==
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
  dim3 grid(p.n_wg);
  hipLaunchKernelGGL((attn_kernel<KB, VB, KAXIS, G, SPARSE, FMT>), grid, dim3(256), 0, st, c, p, q, out, ws);
  return hipGetLastError();
}

template <int KB, int VB, int KAXIS, bool SPARSE, int FMT>
hipError_t dispatch_g(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                      hipStream_t st, int* occ) {
  switch (p.group) {
    case 1: return launch_t<KB, VB, KAXIS, 1, SPARSE, FMT>(c, p, q, out, ws, st, occ);
    case 2: return launch_t<KB, VB, KAXIS, 2, SPARSE, FMT>(c, p, q, out, ws, st, occ);
    case 4: return launch_t<KB, VB, KAXIS, 4, SPARSE, FMT>(c, p, q, out, ws, st, occ);
    case 8: return launch_t<KB, VB, KAXIS, 8, SPARSE, FMT>(c, p, q, out, ws, st, occ);
  }
  return hipErrorInvalidValue;
}

// affine codes: keys on either axis (channel axis with or without sparse
// entries); symmetric blocks: token axis
template <int KB, int VB, int FMT>
hipError_t dispatch_axis(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                         hipStream_t st, int* occ) {
  if constexpr (FMT == kFmtRope) {  // channel axis, no sparse entries
    if (c.kaxis != 1 || c.sparse) return hipErrorInvalidValue;
    return dispatch_g<KB, VB, 1, false, FMT>(c, p, q, out, ws, st, occ);
  } else {
    if (c.kaxis == 0) return dispatch_g<KB, VB, 0, false, FMT>(c, p, q, out, ws, st, occ);
    if constexpr (FMT == kFmtInt) {
      if (c.sparse) return dispatch_g<KB, VB, 1, true, FMT>(c, p, q, out, ws, st, occ);
      return dispatch_g<KB, VB, 1, false, FMT>(c, p, q, out, ws, st, occ);
    }
    return hipErrorInvalidValue;
  }
}

template <int KB, int FMT>
hipError_t dispatch_vb(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                       hipStream_t st, int* occ) {
  switch (c.vbits) {
    case 8: return dispatch_axis<KB, 8, FMT>(c, p, q, out, ws, st, occ);
    case 4: return dispatch_axis<KB, 4, FMT>(c, p, q, out, ws, st, occ);
    case 2: return dispatch_axis<KB, 2, FMT>(c, p, q, out, ws, st, occ);
  }
  return hipErrorInvalidValue;
}

template <int FMT>
hipError_t dispatch_kb(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                       hipStream_t st, int* occ) {
  switch (c.kbits) {
    case 8: return dispatch_vb<8, FMT>(c, p, q, out, ws, st, occ);
    case 4: return dispatch_vb<4, FMT>(c, p, q, out, ws, st, occ);
    case 2: return dispatch_vb<2, FMT>(c, p, q, out, ws, st, occ);
  }
  return hipErrorInvalidValue;
}

hipError_t dispatch(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out, float* ws,
                    hipStream_t st, int* occ) {
  if (c.fmt == kFmtFp8) {  // 8-bit keys and values, token axis
    if (c.kbits != 8 || c.vbits != 8 || c.kaxis != 0) return hipErrorInvalidValue;
    return dispatch_g<8, 8, 0, false, kFmtFp8>(c, p, q, out, ws, st, occ);
  }
  if (c.fmt == kFmtSym32) return dispatch_kb<kFmtSym32>(c, p, q, out, ws, st, occ);
  if (p.rope) return dispatch_kb<kFmtRope>(c, p, q, out, ws, st, occ);
  return dispatch_kb<kFmtInt>(c, p, q, out, ws, st, occ);
}

}  // namespace

hipError_t launch_decode_attention(const CacheView& c, const AttnPlan& p, const uint16_t* q, float* out,
                                   float* ws, hipStream_t st) {
  if (p.n_wg > 0) {
    const hipError_t e = dispatch(c, p, q, out, ws, st, nullptr);
    if (e != hipSuccess) return e;
  }
  if (!p.need_combine) return hipSuccess;
  constexpr int kSmallChunk = 4, kChunk = 32;
  if (p.max_pieces <= 2 * kSmallChunk)
    hipLaunchKernelGGL(combine_kernel<kSmallChunk>, dim3(c.B * p.Hq), dim3(256), 0, st, c, p, ws, out);
  else
    hipLaunchKernelGGL(combine_kernel<kChunk>, dim3(c.B * p.Hq), dim3(256), 0, st, c, p, ws, out);
  return hipGetLastError();
}

int attention_blocks_per_cu(const CacheView& c, int group, int rope) {
  const bool p_rope = rope != 0;
  // cached per device and kernel variant (0 = not queried yet; threads may
  // race to fill an entry with the same value)
  static std::atomic<int> cache[16][3][3][2][2][4][4];
  const auto bi = [](int b) { return b == 2 ? 0 : (b == 4 ? 1 : 2); };
  const int gi = group == 1 ? 0 : (group == 2 ? 1 : (group == 4 ? 2 : 3));
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) dev = -1;
  std::atomic<int>* slot =
      dev >= 0 ? &cache[dev][bi(c.kbits)][bi(c.vbits)][c.kaxis ? 1 : 0][c.sparse ? 1 : 0][gi][p_rope ? 3 : c.fmt % 3] : nullptr;
  if (slot) {
    const int known = slot->load(std::memory_order_relaxed);
    if (known > 0) return known;
  }
  AttnPlan p{};
  p.group = group;
  p.rope = rope;
  int occ = 0;
  if (dispatch(c, p, nullptr, nullptr, nullptr, nullptr, &occ) != hipSuccess || occ < 1) occ = 1;
  if (slot) slot->store(occ, std::memory_order_relaxed);
  return occ;
}

}  // namespace kvq
