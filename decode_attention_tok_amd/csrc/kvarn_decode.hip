// KVarN paged decode attention over packed K4/V2 or K4/V4 tiles (read path) for gfx950.
//
// [GR] "The four-stage pipeline" (groundy.com, "Huawei's KVarN puts KV-cache quantization
// inside vLLM's backend"), stage 4: scales are applied when a tile is read for attention;
// nothing is dequantised to memory. The rotation H of stage 1 is orthonormal and symmetric, so
// q . k = (qH) . (kH); per tile, with q_rot = qH:
//   q~_j   = q_rot_j * c-hat^K_j                   (per-channel key scale into the query)
//   s_t    = sm * (s-hat^K_t * <q~, codeK_t> + z-hat^K_t * sum_j q~_j)
//   acc_j  = sum_t (p_t s-hat^V_t) codeV_tj,  beta = sum_t p_t z-hat^V_t
//   o~_j  += c-hat^V_j * (acc_j + beta)            (value scales into probabilities / output)
// with an online softmax over tiles. A second kernel adds the raw fp16 staging tokens (exact
// fp32 attention with the unrotated query), merges the tile splits by log-sum-exp, rotates
// the packed-tile part back (o~ H) and normalises.
//
// Tile kernel. A workgroup of 4 waves serves one (split, KV head, sequence, head group of <= 8
// query heads); each wave walks every 4th tile of the split with its own softmax state, and
// the 4 states are merged in LDS. Per tile a wave issues 64 MFMAs (v_mfma_f32_16x16x32_f16):
//   scores  D[token][col] = codeK[token][ch] x Q[ch][col]   8 token blocks x 4 channel blocks
//   output  O[row][ch]    = W[row][token] x codeV[token][ch] 4 token blocks x 8 channel blocks
// Key codes enter the MFMA as normal fp16 halves (code - 8) / 64: a nibble at bits 0..3 of a
// half goes under exponent 16 (16 + code / 64), a nibble at bits 4..7 under exponent 1
// (1 + code / 64), so one shift by 8 serves the upper two nibbles of each half, and one packed
// fp16 add (exact) centres each pair; the centring term 8 / 64 * sum_j q~_j is added back in
// fp32. Centred operands keep the products small next to the token-dependent part of the
// score: the matrix core's accumulation error follows the largest products, and uncentred
// 1 + code / 16 reached 2e-3 on outputs of magnitude 250 at 16K tokens, against 5e-4 centred. (The MFMA sums products of subnormal fp16 operands
// with far less precision than products of normal ones, so raw codes are not used as
// subnormals; a variant that left nibbles in the low mantissa bits, 1 + code / 1024 with the
// query scaled to match, was far off as well, so every field sits just below the exponent.) Value codes likewise enter as 1 + code / 4 (the 2-bit
// field shifted to mantissa bits 8..9) or 1 + code / 16 (a 4-bit field at bits 6..9), and
// sum_t p_t s-hat^V_t removes the constant part.
// fp32-accurate operands are split into fp16 hi + lo parts: query column g holds hi(q~_g),
// column 8 + g holds lo(q~_g), and one DPP row rotation by 8 adds the two partial scores;
// the probability operand likewise has rows g (hi) and 8 + g (lo), summed once at the end.
// After the score products the lane of column g keeps tokens 4 s + {0, 1} of each token block
// and the lane of column 8 + g tokens 4 s + {2, 3}, so each probability is computed once; one
// more rotation by 8 hands each lane the hi or lo halves it needs for the output operand.
// The score accumulator lanes of token block pair (2 kb, 2 kb + 1) are exactly the operand
// lanes of output token block kb, so probabilities feed the second product without shuffles.
// The running maximum of a head moves only when a tile's maximum exceeds it by more than
// 2 (log2 units), so most tiles skip the rescale of the output accumulators.
// The counts above are for head dimension 128; the tile, merge and dequantisation kernels are
// templated on the head dimension D (64, 128, 256): D / 32 channel blocks in the score product,
// D / 16 in the output product, D / 64 channels per lane in the rotations.

#include "kvarn_device.hpp"
#include "kvarn_kernels.hpp"

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

namespace kvarn {

namespace {

constexpr int kWaves = 4;
constexpr int kTThreads = 64 * kWaves;
constexpr int kHeadGroup = 8;                 // query heads per tile workgroup
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazy = 2.0f;                 // running-maximum slack (log2 units)

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

template <int kDim = 128>
struct WaveMeta {                  // per-wave, per-tile metadata (fp32, factors folded in)
  // c-hat^K_j * pq | s-hat^K_t * kfac | c-hat^V_j | 32 s-hat^V_t (2 kDim + 256 floats; the
  // rest takes the writes of lanes that hold no metadata chunk)
  float f8[kDim == 256 ? 1024 : 512];
  float h16[2 * kT];               // z-hat^K_t * kzfac | z-hat^V_t
  float alpha[16], beta[16];       // per-row rescale and zero-point term of the last tile
};

template <int kDim = 128>
struct TileSmem {
  float qrot[kHeadGroup][kDim + 4];  // rotated queries (fp32); rows padded so the 8 heads
                                     // read by one instruction start on different banks
  WaveMeta<kDim> wm[kWaves];
  float comb_m[kWaves][kHeadGroup], comb_l[kWaves][kHeadGroup];
  float comb_o[kWaves][kHeadGroup][kDim];
  float red[kWaves];
};

template <int kMask>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (kMask == 1)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  else if constexpr (kMask == 2)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  else if constexpr (kMask == 8)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
  else   // 4: swizzle in bit-mask mode, xor within 32 lanes
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (kMask << 10) | 0x1F));
}

// One butterfly stage across lanes: the lane with the bit clear gets own + partner, the lane
// with it set gets partner - own. Across lane bits 4 and 5 a permlane swap of the value with
// itself gives (lower lane's value, upper lane's value) in every lane.
template <int kMask>
__device__ __forceinline__ float fwht_lane_stage(float v, int lane) {
  const float sgn = (lane & kMask) ? -1.0f : 1.0f;
  if constexpr (kMask == 16 || kMask == 32) {
    const auto r = kMask == 16
        ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false)
        : __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaf(sgn, __uint_as_float(r[1]), __uint_as_float(r[0]));
  } else {
    return fmaf(sgn, v, lane_xor<kMask>(v));
  }
}

// 128-point Walsh-Hadamard transform of a vector held as channels 2 lane, 2 lane + 1.
__device__ __forceinline__ void fwht_wave(float& o0, float& o1, int lane) {
  const float a = o0 + o1, c = o0 - o1;
  o0 = a;
  o1 = c;
  o0 = fwht_lane_stage<1>(o0, lane);   o1 = fwht_lane_stage<1>(o1, lane);
  o0 = fwht_lane_stage<2>(o0, lane);   o1 = fwht_lane_stage<2>(o1, lane);
  o0 = fwht_lane_stage<4>(o0, lane);   o1 = fwht_lane_stage<4>(o1, lane);
  o0 = fwht_lane_stage<8>(o0, lane);   o1 = fwht_lane_stage<8>(o1, lane);
  o0 = fwht_lane_stage<16>(o0, lane);  o1 = fwht_lane_stage<16>(o1, lane);
  o0 = fwht_lane_stage<32>(o0, lane);  o1 = fwht_lane_stage<32>(o1, lane);
}

__device__ __forceinline__ float dpp_ror8(float v) {   // lane (l & ~15) | ((l + 8) & 15)
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t dpp_ror8_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
}

// (x & mask) | c in one v_and_or_b32: mask in a VGPR and c in an SGPR, since a gfx9 VOP3
// instruction cannot carry two literal constants (the compiler otherwise emits and + or).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask_v, uint32_t c_s) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(mask_v), "s"(c_s));
  return r;
}

// a where the mask is all ones, b where it is zero: one v_bfi_b32 on a per-lane all-ones /
// zero word. Written out because the optimiser otherwise rewrites a pair of selects between
// two components of an MFMA result into a read at a runtime index (a chain of three compares
// and three selects per value).
__device__ __forceinline__ uint32_t lane_mask(bool c) { return c ? 0xFFFFFFFFu : 0u; }
__device__ __forceinline__ float pick(uint32_t m, float a, float b) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(__float_as_uint(a)), "v"(__float_as_uint(b)));
  return __uint_as_float(r);
}

__device__ __forceinline__ half8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(half8, u);
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {   // both rounded to nearest
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){a, b}, half2v));
}

// Packed fp16 pair (a - k hi(a), b - k hi(b)) with hi = fp16 rounding and k = -negk in {0, 1}:
// the hi parts themselves (k = 0) or the lo parts (k = 1), each one v_fma_mix (exact product
// and sum, one rounding to fp16). a == hi + lo to about 2^-22 relative while normal.
__device__ __forceinline__ uint32_t hi_or_lo(float a, float b, float negk) {
  const uint32_t h = pack_h2(a, b);
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(negk), "v"(a));
  asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(r) : "v"(h), "v"(negk), "v"(b));
  return r;
}

// Sign bits of channels 2 lane and 2 lane + 1 from the four sign words (bit j % 32 of word
// j / 32 negates channel j), as (bit of 2 lane, bit of 2 lane + 1) in bits 0 and 1.
__device__ __forceinline__ uint32_t lane_sign_bits(uint4 signs, int lane) {
  const uint32_t word = lane < 32 ? (lane < 16 ? signs.x : signs.y)
                                  : (lane < 48 ? signs.z : signs.w);
  return (word >> (2 * (lane & 15))) & 3u;
}

// Both fp16 halves of w plus c (v_pk_add_f16; exact for the centring below).
__device__ __forceinline__ uint32_t add_h2(uint32_t w, half2v c) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, w) + c);
}

// Per-lane constants of the key-code operand (masks in VGPRs, exponent words in SGPRs: a VOP3
// instruction takes one literal at most).
struct KeyConsts {
  uint32_t m_lo, m_hi, e16, e1;
};

__device__ __forceinline__ KeyConsts key_consts() {
  KeyConsts k;
  k.m_lo = 0x000F000Fu;
  k.m_hi = 0x00F000F0u;
  asm volatile("" : "+v"(k.m_lo), "+v"(k.m_hi));
  k.e16 = __builtin_amdgcn_readfirstlane(0x4C004C00u);   // 16.0 in both halves
  k.e1 = __builtin_amdgcn_readfirstlane(0x3C003C00u);    // 1.0 in both halves
  return k;
}

// The eight key codes of one 32-bit word (channels 8 d .. 8 d + 7 of a token; channel 8 d + 2 b
// in the low nibble of byte b) as the operand halves of channels 8 d + {0, 4, 1, 5, 2, 6, 3, 7},
// each (code - 8) / 64 exactly.
__device__ __forceinline__ half8 key_operand(uint32_t w, const KeyConsts& k) {
  const half2v c16 = {(_Float16)-16.125f, (_Float16)-16.125f};   // 16 + 8 / 64
  const half2v c1 = {(_Float16)-1.125f, (_Float16)-1.125f};      // 1 + 8 / 64
  const uint32_t w8 = w >> 8;
  return as_h8(add_h2(and_or(w, k.m_lo, k.e16), c16), add_h2(and_or(w, k.m_hi, k.e1), c1),
               add_h2(and_or(w8, k.m_lo, k.e16), c16), add_h2(and_or(w8, k.m_hi, k.e1), c1));
}

// fp16 lo parts of a pair whose packed hi parts are h.
__device__ __forceinline__ uint32_t lo_of(uint32_t h, float a, float b) {
  uint32_t r;
  const float m1 = -1.0f;
  asm("v_fma_mixlo_f16 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(m1), "v"(a));
  asm("v_fma_mixhi_f16 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(r) : "v"(h), "v"(m1), "v"(b));
  return r;
}

// Code registers of one tile, per lane. Key words: token 16 mb + (lane % 16), channels
// (kDim / 4)(lane / 16) + 8 c .. + 7 in word c. Value words of 32-token block kb: 2-bit codes,
// the kDim / 32 section words (kDim / 32)(16 s + n) .. of the block (lane = 16 s + n); 4-bit
// codes, the four words 4 lane .. of each 256-word quarter hb of the block (word 4 hb + d).
template <int kVBits, int kDim = 128>
struct TileRegs {
  static constexpr int kKW = kDim / 32;                            // key words per token block
  static constexpr int kVW = kVBits == 2 ? kDim / 32 : kDim / 16;  // value words per 32 tokens
  static constexpr int kM8 = kDim == 256 ? 2 : 1;                  // metadata chunks per lane
  uint32_t kw[8][kKW];
  uint32_t vw[4][kVW];
  uint2 m8[kM8];      // 8 FP8 metadata bytes per chunk (see meta_chunk)
  uint2 m16;          // 4 fp16 zero-points
};

// Value codes of channel block nb (channel 16 nb + lane % 16) and token block kb as the B
// operand of the output product: 2-bit codes as 1 + code / 4 (the code's field moved to
// mantissa bits 8..9 under exponent 1), 4-bit codes as 1 + code / 16 (field nb % 4 of the
// words of quarter nb / 4 moved to bits 6..9). Normal and exact. Element pair d holds the
// tokens 16 (d / 2) + 4 s + 2 (d % 2) + {0, 1} of the block.
template <int kVBits, int kDim = 128>
__device__ __forceinline__ half8 value_operand(const uint32_t (&vw)[4][TileRegs<kVBits, kDim>::kVW],
                                               int nb, int kb, uint32_t vmask, uint32_t kmask,
                                               uint32_t one16) {
  uint32_t f[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if constexpr (kVBits == 2 && kDim >= 128) {
      // field nb % 8 (bits 2 (nb % 8) and 16 + 2 (nb % 8)) of word 4 (nb / 8) + d
      const uint32_t w = vw[kb][4 * (nb >> 3) + d];
      const int f8 = nb & 7;
      const uint32_t x = f8 < 4 ? (w << (8 - 2 * f8)) : (w >> (2 * f8 - 8));
      f[d] = and_or(x, vmask, one16);
    } else if constexpr (kVBits == 2) {
      // kDim = 64: word d / 2 holds the pair at bits 2 nb + 8 (d % 2) and 16 above
      const uint32_t w = vw[kb][d >> 1];
      const int bit = 2 * nb + 8 * (d & 1);
      const uint32_t x = bit <= 8 ? (w << (8 - bit)) : (w >> (bit - 8));
      f[d] = and_or(x, vmask, one16);
    } else {
      const uint32_t w = vw[kb][4 * (nb >> 2) + d];
      const int kF = nb & 3;
      const uint32_t x = kF < 2 ? (w << (6 - 4 * kF)) : (w >> (4 * kF - 6));
      f[d] = and_or(x, kmask, one16);
    }
  }
  return as_h8(f[0], f[1], f[2], f[3]);
}

// FP8 metadata chunk ci (8 bytes) of a record, and the factor its values are scaled by. The
// FP8 bytes of a metadata half (c-hat: kDim, s-hat: 128) are contiguous, so chunk ci of the
// table [c-hat^K | s-hat^K | c-hat^V | s-hat^V] is record byte kmeta + 8 ci in the key half
// and vmeta + 8 ci' (ci' = ci - (kDim + 128) / 8) in the value half. Chunks past the table
// (lanes without one) read chunk 0 and write into the unused tail of the table.
template <int kVBits, int kDim>
__device__ __forceinline__ uint32_t meta_chunk_off(int ci) {
  using L = RecordLayout<kVBits, kDim>;
  constexpr int kHalf = (kDim + 128) / 8;
  if (ci >= 2 * kHalf) ci = 0;
  return (uint32_t)(ci < kHalf ? L::kKMetaOff + 8 * ci : L::kVMetaOff + 8 * (ci - kHalf));
}
template <int kDim>
__device__ __forceinline__ float meta_chunk_factor(int ci, float pq, float kfac) {
  return ci < kDim / 8 ? pq : (ci < (kDim + 128) / 8 ? kfac : (ci < (2 * kDim + 128) / 8 ? 1.0f : 32.0f));
}

// Per-lane byte offsets (unsigned, so a load is a scalar tile base plus a 32-bit lane offset):
// key codes of token 16 mb + (lane % 16) at koff + 8 kDim mb (koff4 = koff + 4096 serves
// mb >= 4 at kDim = 128, within the 12-bit immediate); value-code words of token block kb at
// voff + 8 kDim kb (2-bit) or voff + 1024 ((kDim / 64) kb + hb) (4-bit); metadata chunks at
// off8[], zero-points at off16 (lanes 0-31 z-hat^K, 32-63 z-hat^V, 8 bytes each).
template <int kDim>
struct LaneOffsets {
  uint32_t koff, koff4, voff, off8[kDim == 256 ? 2 : 1], off16;
};

template <int kVBits, int kDim = 128>
__device__ __forceinline__ LaneOffsets<kDim> lane_offsets(int lane) {
  using L = RecordLayout<kVBits, kDim>;
  LaneOffsets<kDim> o;
  o.koff = (uint32_t)(lane & 15) * (kDim / 2) + (kDim / 8) * (uint32_t)(lane >> 4);
  o.koff4 = o.koff + 4096u;
  o.voff = L::kVCodes + (kVBits == 2 ? (kDim / 8) : 16) * (uint32_t)lane;
  o.off8[0] = meta_chunk_off<kVBits, kDim>(lane);
  if constexpr (kDim == 256) o.off8[1] = meta_chunk_off<kVBits, kDim>(lane + 64);
  o.off16 = (uint32_t)((lane < 32 ? L::kKMetaOff : L::kVMetaOff) + L::kZ + 8 * (lane & 31));
  return o;
}

// n consecutive words at p (n = 2, 4 or 8; 8- or 16-byte aligned) into w.
template <int kN>
__device__ __forceinline__ void load_words(const uint8_t* __restrict__ p, uint32_t* w) {
  if constexpr (kN == 2) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    w[0] = a.x; w[1] = a.y;
  } else {
#pragma unroll
    for (int i = 0; i < kN; i += 4) {
      const uint4 a = *reinterpret_cast<const uint4*>(p + 4 * i);
      w[i] = a.x; w[i + 1] = a.y; w[i + 2] = a.z; w[i + 3] = a.w;
    }
  }
}

template <int kVBits, int kDim>
__device__ __forceinline__ void load_keys(const uint8_t* __restrict__ rec,
                                          const LaneOffsets<kDim>& o,
                                          TileRegs<kVBits, kDim>& r) {
  constexpr int kKW = TileRegs<kVBits, kDim>::kKW;
  if constexpr (kDim == 128) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) load_words<4>(rec + o.koff + 1024u * mb, r.kw[mb]);
#pragma unroll
    for (int mb = 4; mb < 8; ++mb) load_words<4>(rec + o.koff4 + 1024u * (mb - 4), r.kw[mb]);
  } else {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) load_words<kKW>(rec + o.koff + 8u * kDim * mb, r.kw[mb]);
  }
#pragma unroll
  for (int k = 0; k < TileRegs<kVBits, kDim>::kM8; ++k)
    r.m8[k] = *reinterpret_cast<const uint2*>(rec + o.off8[k]);
  r.m16 = *reinterpret_cast<const uint2*>(rec + o.off16);
}

template <int kVBits, int kDim>
__device__ __forceinline__ void load_values(const uint8_t* __restrict__ rec,
                                            const LaneOffsets<kDim>& o,
                                            TileRegs<kVBits, kDim>& r) {
  if constexpr (kVBits == 2) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      load_words<kDim / 32>(rec + o.voff + 8u * kDim * kb, r.vw[kb]);
  } else {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int hb = 0; hb < kDim / 64; ++hb)
        load_words<4>(rec + o.voff + 1024u * ((kDim / 64) * kb + hb), r.vw[kb] + 4 * hb);
    }
  }
}

// A lane converts its 8 FP8 bytes (one metadata chunk) and stores them, times a factor, at
// f8[0..7]; the FP8 conversion is the hardware E4M3 one (exact for every finite code).
__device__ __forceinline__ void decode_meta8(const uint2 m8, float* __restrict__ f8, float fm) {
  const float2v a = __builtin_amdgcn_cvt_pk_f32_fp8((int)m8.x, false);
  const float2v b = __builtin_amdgcn_cvt_pk_f32_fp8((int)m8.x, true);
  const float2v c = __builtin_amdgcn_cvt_pk_f32_fp8((int)m8.y, false);
  const float2v d = __builtin_amdgcn_cvt_pk_f32_fp8((int)m8.y, true);
  float4* dst = reinterpret_cast<float4*>(f8);
  dst[0] = make_float4(a[0] * fm, a[1] * fm, b[0] * fm, b[1] * fm);
  dst[1] = make_float4(c[0] * fm, c[1] * fm, d[0] * fm, d[1] * fm);
}

// ... and its 4 fp16 zero-points, times fz, at h16[0..3].
__device__ __forceinline__ void decode_meta16(const uint2 m16, float* __restrict__ h16, float fz) {
  const float2v e = __builtin_convertvector(__builtin_bit_cast(half2v, m16.x), float2v);
  const float2v f = __builtin_convertvector(__builtin_bit_cast(half2v, m16.y), float2v);
  *reinterpret_cast<float4*>(h16) = make_float4(e[0] * fz, e[1] * fz, f[0] * fz, f[1] * fz);
}

// Every lane converts its metadata (the same instructions on all lanes) and stores it, times
// per-lane factors, at 8 lane and 4 lane of the wave's tables (head dimension 128).
__device__ __forceinline__ void decode_meta(const uint2 m8, const uint2 m16, int lane,
                                            float* __restrict__ f8, float* __restrict__ h16,
                                            float fm, float fz) {
  decode_meta8(m8, f8 + 8 * lane, fm);
  decode_meta16(m16, h16 + 4 * lane, fz);
}

// Walsh-Hadamard transform (unscaled) of a vector of 64 kPer channels held kPer per lane:
// channel kPer lane + i in v[i]. Butterflies on the channel bits inside a lane first, then on
// the lane bits.
template <int kPer>
__device__ __forceinline__ void fwht_lanes(float (&v)[kPer], int lane) {
#pragma unroll
  for (int h = 1; h < kPer; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    v[i] = fwht_lane_stage<1>(v[i], lane);
    v[i] = fwht_lane_stage<2>(v[i], lane);
    v[i] = fwht_lane_stage<4>(v[i], lane);
    v[i] = fwht_lane_stage<8>(v[i], lane);
    v[i] = fwht_lane_stage<16>(v[i], lane);
    v[i] = fwht_lane_stage<32>(v[i], lane);
  }
}

// Sign bits of channels kPer lane .. + kPer - 1 (bit i = channel kPer lane + i).
template <int kPer>
__device__ __forceinline__ uint32_t lane_sign_bits_d(const SignWords& signs, int lane) {
  const int c0 = kPer * lane;
  return (sign_word(signs, c0 >> 5) >> (c0 & 31)) & ((1u << kPer) - 1u);
}

// This lane's kPer fp16 values at p (kPer = 1, 2 or 4) as floats.
template <int kPer>
__device__ __forceinline__ void load_h(const __half* __restrict__ p, float (&v)[kPer]) {
  if constexpr (kPer == 1) {
    v[0] = __half2float(p[0]);
  } else if constexpr (kPer == 2) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    v[0] = fp16_bits_to_float(w & 0xFFFFu);
    v[1] = fp16_bits_to_float(w >> 16);
  } else {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    v[0] = fp16_bits_to_float(w.x & 0xFFFFu);
    v[1] = fp16_bits_to_float(w.x >> 16);
    v[2] = fp16_bits_to_float(w.y & 0xFFFFu);
    v[3] = fp16_bits_to_float(w.y >> 16);
  }
}

// kCausal: several query tokens per sequence (nq > 1) with the causal mask; a separate
// instantiation so the one-token decode carries no mask code. kVBits: 2 or 4 bits per value
// code; kDim: head dimension 64, 128 or 256 (the record layout of that preset). At kDim = 256
// the score products run channel block by channel block (one query operand live at a time),
// and the tile's codes and 16 output accumulators need more than the 256 registers of two
// waves per SIMD, so that instantiation runs one wave per SIMD.
// Full tiles of a sequence of length len in the paged table (none when the length is invalid:
// negative, or more full tiles than the table holds), and the pairs they form (the last one
// single for an odd count).
__device__ __forceinline__ int full_tiles(int len, int max_blocks) {
  return (len < 0 || (len >> 7) > max_blocks) ? 0 : (len >> 7);
}
__device__ __forceinline__ int tile_pairs(int len, int max_blocks) {
  return (full_tiles(len, max_blocks) + 1) >> 1;
}
// List positions of a sequence: its full tiles (kUnit 1) or tile pairs (kUnit 2).
template <int kUnit>
__device__ __forceinline__ int unit_positions(int len, int max_blocks) {
  return kUnit == 1 ? full_tiles(len, max_blocks) : tile_pairs(len, max_blocks);
}

// The work list's positions per sequence (full tiles or tile pairs, x KV heads), summed over
// lanes: lane l
// holds sequences [l k, l k + k), k = ceil(batch / 64); mine = its positions, excl = those of
// the lanes before it, total = the list length (the same in every lane). The list is shorter
// than 2^31: the paired-tile kernel only serves tables of fewer entries than that.
struct ListScan {
  int mine, excl, total;
  int lo, hi;
};

template <int kUnit>
__device__ __forceinline__ ListScan scan_list(const int32_t* __restrict__ seq_lens, int batch,
                                              int max_blocks, int hkv, int lane) {
  ListScan r;
  const int k = (batch + 63) >> 6;
  r.lo = min(batch, lane * k);
  r.hi = min(batch, r.lo + k);
  int mine = 0;
  for (int i = r.lo; i < r.hi; ++i) mine += unit_positions<kUnit>(seq_lens[i], max_blocks);
  mine *= hkv;
  int incl = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d);
    if (lane >= d) incl += t;
  }
  r.mine = mine;
  r.excl = incl - mine;
  r.total = __builtin_amdgcn_readlane(incl, 63);
  return r;
}

// The sequence holding list position pos (0 <= pos < total) and the positions before it.
template <int kUnit>
__device__ __forceinline__ void locate_position(const ListScan& ls,
                                                const int32_t* __restrict__ seq_lens,
                                                int max_blocks, int hkv, int pos, int lane,
                                                int& seq, int& before) {
  const unsigned long long m = __ballot(ls.excl + ls.mine > pos);
  const int owner = m ? (int)__builtin_ctzll(m) : 63;
  int bef = ls.excl;
  int sq = ls.lo;
  if (lane == owner) {
    for (; sq < ls.hi - 1; ++sq) {
      const int n = unit_positions<kUnit>(seq_lens[sq], max_blocks) * hkv;
      if (pos < bef + n) break;
      bef += n;
    }
  }
  seq = __builtin_amdgcn_readlane(sq, owner);
  before = __builtin_amdgcn_readlane(bef, owner);
}


// Shares of a list schedule over W workers (waves or workgroups): worker w takes list
// positions [w share, (w + 1) share), share = max(min_share, ceil(total / W)).
struct PairSplit {
  int share;
  __device__ __forceinline__ long long start(int w) const { return (long long)w * share; }
  __device__ __forceinline__ int wave_of(int x) const { return x / share; }
};

__device__ __forceinline__ PairSplit pair_split(int total, int waves, int min_share) {
  PairSplit r;
  const long long s = ((long long)total + waves - 1) / waves;
  r.share = (int)(s > min_share ? s : min_share);
  return r;
}


// Issue priority from the wave's progress: 3 in the first quarter of its tiles down to 0 in
// the last. The two waves a SIMD holds start together with equal work; a SIMD favours its older
// wave among equal priorities, which would finish it well before the younger one and leave the
// younger alone (and latency-bound) for the rest of the kernel. Ranking by work left instead
// keeps the pair level, so they finish together.
#ifndef KVARN_PAIR_PRIO
#define KVARN_PAIR_PRIO 1
#endif
constexpr bool kPairPrio = KVARN_PAIR_PRIO != 0;
__device__ __forceinline__ void set_progress_priority(int done, int total) {
  const int quarter = (4 * done) / total;
  if (quarter <= 0) __builtin_amdgcn_s_setprio(3);
  else if (quarter == 1) __builtin_amdgcn_s_setprio(2);
  else if (quarter == 2) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

#ifndef KVARN_TILE_PRIO
#define KVARN_TILE_PRIO 1
#endif
constexpr bool kTilePrio = KVARN_TILE_PRIO != 0;

// Tiles i0 .. i0 + ntile - 1 (ntile >= 0) of KV head g of sequence b (length len; bad: the
// sequence is invalid) for the virtual heads of head group hg, by the workgroup's four waves
// (wave w takes tiles i0 + w + 4 j); one partial per virtual head into slot `slot` of rows of
// nslot slots. done0 / total: the workgroup's progress before this segment, in tiles, for the
// issue priority. end_mark: also mark the next slot as the rows' end (m = +inf).
template <bool kCausal, int kVBits, int kDim>
__device__ __forceinline__ void tile_segment(
    TileSmem<kDim>& sm, const __half* __restrict__ q, int hq, int hkv, int nq,
    const uint8_t* __restrict__ pool, long long num_blocks,
    const int32_t* __restrict__ block_table, int max_blocks, int len, float sm_scale,
    float* __restrict__ partials, const SignWords& signs, int b, int g, int hg, int i0,
    int ntile, bool bad, int slot, int nslot, int done0, int total, bool end_mark) {
  constexpr int kKW = kDim / 32;        // key words per lane and token block = channel blocks
  constexpr int kNB = kDim / 16;        // output channel blocks
  constexpr int kPer = kDim / 64;       // channels per lane in the query rotation
  constexpr int kPF = 2 + kDim;         // floats per partial
  const int group = hq / hkv, vgroup = group * nq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vbase = hg * kHeadGroup;
  const int nh = min(kHeadGroup, vgroup - vbase);             // rows served (1..8)
  auto row_of = [&](int v) -> long long {                     // row in [B][nq][hq]
    return ((long long)b * nq + v / group) * hq + g * group + v % group;
  };
  // this wave's tiles: i0 + wave + 4 j, j < nw. Block ids are scalar loads (the row pointer
  // and j are wave-uniform), each issued one tile before the tile that needs it.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nw = ntile > wave_u ? (ntile - wave_u + kWaves - 1) / kWaves : 0;
  const int32_t* bt_row = block_table + (long long)b * max_blocks + i0 + wave_u;
  constexpr long long kTileBytes = RecordLayout<kVBits, kDim>::kTileBytes;
  const LaneOffsets<kDim> lo = lane_offsets<kVBits, kDim>(lane);
  TileRegs<kVBits, kDim> cur;
  int id_next = nw > 1 ? bt_row[kWaves] : 0;        // tile 1
  if (nw > 0) {
    const long long blk = bt_row[0];
    if (blk < 0 || blk >= num_blocks) {
      bad = true;
    } else {
      const uint8_t* rec = pool + (blk * hkv + g) * (long long)kTileBytes;
      load_keys(rec, lo, cur);
      load_values(rec, lo, cur);
    }
  }

  // ---- rotated queries in LDS: wave w rotates heads 2 w and 2 w + 1 (channels kPer lane ..)
  float qmax = 0.0f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int gg = 2 * wave + k;
    float o[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) o[i] = 0.0f;
    if (gg < nh) {
      load_h<kPer>(q + row_of(vbase + gg) * kDim + kPer * lane, o);
      const uint32_t sb = lane_sign_bits_d<kPer>(signs, lane);   // optional sign flips
#pragma unroll
      for (int i = 0; i < kPer; ++i) o[i] = (sb >> i) & 1u ? -o[i] : o[i];
    }
    fwht_lanes<kPer>(o, lane);
    constexpr float kInvSqrt = kDim == 64 ? 0.125f
                             : (kDim == 128 ? 0.08838834764831845f : 0.0625f);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      o[i] *= kInvSqrt;
      sm.qrot[gg][kPer * lane + i] = o[i];
      qmax = fmaxf(qmax, fabsf(o[i]));
    }
  }
  qmax = wave_max_nonneg(qmax);
  if (lane == 0) sm.red[wave] = qmax;
  __syncthreads();
  qmax = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
  // power-of-two query prescale pq: |q~ * pq| <= qmax * 448 * pq <= 2^14 keeps the hi part
  // finite in fp16
  int qe = 0;
  frexpf(fmaxf(qmax, 1e-30f) * 448.0f, &qe);
  const float pq = ldexpf(1.0f, 14 - qe);
  const float scale2 = sm_scale * kLog2e;
  const float kfac = scale2 * 64.0f / pq;          // undoes the code / 64 encoding and pq
  const float kzfac = scale2 / pq;                 // multiplies pq * sum_j q~_j
  // per-lane metadata factors: pq on c-hat^K, kfac on s-hat^K, 1 on c-hat^V, 32 on s-hat^V
  // (by chunk, meta_chunk_factor); kzfac on z-hat^K, 1 on z-hat^V
  float fm[TileRegs<kVBits, kDim>::kM8];
#pragma unroll
  for (int k = 0; k < TileRegs<kVBits, kDim>::kM8; ++k)
    fm[k] = meta_chunk_factor<kDim>(lane + 64 * k, pq, kfac);
  const float fz = lane < 32 ? kzfac : 1.0f;

  // lane roles: m / s for operand rows and k groups, n for columns
  const int n = lane & 15, s = lane >> 4;
  const int gq = n & 7;                              // head of this column / row
  const bool colv = gq < nh;                         // column carries a real head
  const bool colhi = n < 8;
  const uint32_t hi_m = lane_mask(colhi);
  const float negk = colhi ? 0.0f : -1.0f;           // hi parts on columns 0-7, lo on 8-15
  const int ih = colhi ? 0 : 2;                      // this lane's rows of each score block
  const uint32_t vmask_col = colv ? 0xFFFFFFFFu : 0u;
  // causal limit of this column's query token (position len - nq + i); only tiles that reach
  // past len - nq are masked, and with nq <= 16 every packed tile keeps >= 112 visible tokens
  const int qlim = len - nq + (vbase + gq) / group;
  WaveMeta<kDim>& wm = sm.wm[wave];
  const float* kc = wm.f8;
  const float* ks = wm.f8 + kDim;
  const float* vc = wm.f8 + kDim + kT;
  const float* vs = wm.f8 + 2 * kDim + kT;
  const float* kz = wm.h16;
  const float* vz = wm.h16 + kT;
  // per-lane copies of the code masks (kept in VGPRs) and the wave-uniform exponent word
  uint32_t kmask = 0x03C003C0u, vmask = 0x03000300u;
  asm volatile("" : "+v"(kmask), "+v"(vmask));
  const uint32_t one16 = __builtin_amdgcn_readfirstlane(0x3C003C00u);
  const KeyConsts kcon = key_consts();

  // running state: score-lane view (column n) and output-row view (rows 4 s + i)
  float m_run = -INFINITY, l_run = 0.0f;
  float4v oacc[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) oacc[nb] = (float4v){0.f, 0.f, 0.f, 0.f};

  // Tile pipeline without extra registers: the next tile's key codes (and metadata) are
  // loaded into the key registers once the score products have consumed them, and the next
  // value codes into the value registers once the output products have.
  for (int j = 0; j < nw && !bad; ++j) {
    if constexpr (kTilePrio) set_progress_priority(done0 + kWaves * j, total);
    const uint8_t* nrec = nullptr;
    if (j + 1 < nw) {
      const long long blk = id_next;
      if (j + 2 < nw) id_next = bt_row[kWaves * (j + 2)];
      if (blk >= 0 && blk < num_blocks) nrec = pool + (blk * hkv + g) * (long long)kTileBytes;
      else bad = true;                             // finishes this tile, then stops
    }
#pragma unroll
    for (int k = 0; k < TileRegs<kVBits, kDim>::kM8; ++k)   // wave-local LDS tables
      decode_meta8(cur.m8[k], wm.f8 + 8 * (lane + 64 * k), fm[k]);
    decode_meta16(cur.m16, wm.h16 + 4 * lane, fz);

    // ---- query operand of channel block c: q' = pq * q_rot * c-hat^K, hi (cols 0-7) or lo
    // (8-15); element e is channel (kDim / 4) s + 8 c + {0,4,1,5,2,6,3,7}[e]
    float asum = 0.0f;                            // sum_j q'_j over this lane's channels
    const float4* qr4 = reinterpret_cast<const float4*>(sm.qrot[gq] + (kDim / 4) * s);
    const float4* kc4 = reinterpret_cast<const float4*>(kc + (kDim / 4) * s);
    auto q_operand = [&](int c) -> half8 {
      const float4 qa = qr4[2 * c], qc = qr4[2 * c + 1];
      const float4 ka = kc4[2 * c], kk = kc4[2 * c + 1];
      const float x0 = qa.x * ka.x, x1 = qa.y * ka.y, x2 = qa.z * ka.z, x3 = qa.w * ka.w;
      const float x4 = qc.x * kk.x, x5 = qc.y * kk.y, x6 = qc.z * kk.z, x7 = qc.w * kk.w;
      asum += ((x0 + x1) + (x2 + x3)) + ((x4 + x5) + (x6 + x7));
      return as_h8(hi_or_lo(x0, x4, negk) & vmask_col, hi_or_lo(x1, x5, negk) & vmask_col,
                   hi_or_lo(x2, x6, negk) & vmask_col, hi_or_lo(x3, x7, negk) & vmask_col);
    };

    // ---- scores: 8 token blocks x kDim / 32 channel blocks
    float4v sc[8];
    float asum_c;
    if constexpr (kDim <= 128) {
      half8 qb[kKW];
#pragma unroll
      for (int c = 0; c < kKW; ++c) qb[c] = q_operand(c);
      asum = add_xor32(add_xor16(asum));          // over all kDim channels of column n
      asum_c = 0.125f * asum;                     // the centring term, 8 / 64 * asum
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kKW; ++c)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand(cur.kw[mb][c], kcon), qb[c],
                                                       acc, 0, 0, 0);
        sc[mb] = acc;
      }
    } else {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) sc[mb] = (float4v){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kKW; ++c) {
        const half8 qc = q_operand(c);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
          sc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand(cur.kw[mb][c], kcon), qc,
                                                          sc[mb], 0, 0, 0);
      }
      asum = add_xor32(add_xor16(asum));
      asum_c = 0.125f * asum;
    }
    if (nrec != nullptr) load_keys(nrec, lo, cur);
    // hi + lo partial scores of this lane's two rows, then the log2-domain score per token:
    // D = sum_j (code_j - 8) / 64 q'_j, so pq <q~, code> = 64 (D + 8 / 64 asum)
    float v[8][2];
    float tmax = -INFINITY;
    const int tpos = kT * (i0 + wave_u + kWaves * j);      // position of this tile's token 0
    const bool masked = kCausal && tpos + kT - 1 > len - nq;   // wave-uniform
    const int tlim = qlim - tpos;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const float snd0 = pick(hi_m, sc[mb][2], sc[mb][0]);
      const float snd1 = pick(hi_m, sc[mb][3], sc[mb][1]);
      const float own0 = pick(hi_m, sc[mb][0], sc[mb][2]);
      const float own1 = pick(hi_m, sc[mb][1], sc[mb][3]);
      const float d0 = own0 + dpp_ror8(snd0), d1 = own1 + dpp_ror8(snd1);
      const int t0 = 16 * mb + 4 * s + ih;
      const float2 ks2 = *reinterpret_cast<const float2*>(ks + t0);
      const float2 kz2 = *reinterpret_cast<const float2*>(kz + t0);
      v[mb][0] = fmaf(ks2.x, d0 + asum_c, kz2.x * asum);
      v[mb][1] = fmaf(ks2.y, d1 + asum_c, kz2.y * asum);
      if (masked) {
        v[mb][0] = t0 > tlim ? -INFINITY : v[mb][0];
        v[mb][1] = t0 + 1 > tlim ? -INFINITY : v[mb][1];
      }
      tmax = fmaxf(tmax, fmaxf(v[mb][0], v[mb][1]));
    }
    tmax = fmaxf(tmax, dpp_ror8(tmax));
    tmax = max_xor32(max_xor16(tmax));
    const bool upd = tmax > m_run + kLazy;        // also true on the first tile
    const float mnew = upd ? tmax : m_run;
    const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;
    const bool rescale = __any(upd) && j > 0;     // wave-uniform
    float psum = 0.0f, beta = 0.0f, wsum = 0.0f;
    // probabilities -> operand rows: hi(32 p s-hat^V) on rows 0-7, lo on rows 8-15;
    // element e of token block kb is token 32 kb + 16 (e / 4) + 4 s + e % 4
    half8 wa[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint32_t u[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int mb = 2 * kb + h2, t0 = 16 * mb + 4 * s + ih;
        const float2 vs2 = *reinterpret_cast<const float2*>(vs + t0);
        const float2 vz2 = *reinterpret_cast<const float2*>(vz + t0);
        const float p0 = __builtin_amdgcn_exp2f(v[mb][0] - mnew);
        const float p1 = __builtin_amdgcn_exp2f(v[mb][1] - mnew);
        psum += p0 + p1;
        beta = fmaf(p0, vz2.x, fmaf(p1, vz2.y, beta));
        const float w0 = p0 * vs2.x, w1 = p1 * vs2.y;
        wsum += w0 + w1;
        const uint32_t hh = pack_h2(w0, w1);
        const uint32_t ll = lo_of(hh, w0, w1);
        const uint32_t rcv = dpp_ror8_u(colhi ? ll : hh);
        u[2 * h2] = (colhi ? hh : rcv) & vmask_col;       // rows 0, 1 of block mb
        u[2 * h2 + 1] = (colhi ? rcv : ll) & vmask_col;   // rows 2, 3
      }
      wa[kb] = as_h8(u[0], u[1], u[2], u[3]);
    }
    psum += dpp_ror8(psum);
    beta += dpp_ror8(beta);
    wsum += dpp_ror8(wsum);
    psum = add_xor32(add_xor16(psum));
    beta = add_xor32(add_xor16(beta));
    wsum = add_xor32(add_xor16(wsum));
    // output rows get D / 8 per tile: D = sum_t W_t (1 + code / 4), W = 32 p s-hat^V, so
    // sum_t p s-hat^V code = D / 8 - 4 sum_t p s-hat^V = D / 8 - wsum / 8; with 4-bit codes
    // D = sum_t W_t (1 + code / 16) and the sum is D / 2 - wsum / 2
    constexpr float kVOut = kVBits == 4 ? 0.5f : 0.125f;
    beta = fmaf(-kVOut, wsum, beta);
    l_run = fmaf(alpha, l_run, psum);
    m_run = mnew;
    if (s == 0) {
      wm.alpha[n] = alpha;
      wm.beta[n] = colhi ? beta : 0.0f;           // the zero-point term enters the hi row once
    }

    // ---- output: kDim / 16 channel blocks x 4 token blocks; each channel block's accumulator
    // is folded into o~ as soon as its 4 products are done (rows 4 s + i: beta of their head,
    // c-hat^V of column 16 nb + n); rows are rescaled first when a running maximum moved
    {
      const float4 b4 = *reinterpret_cast<const float4*>(wm.beta + 4 * s);
      const float br[4] = {b4.x, b4.y, b4.z, b4.w};
      if (rescale) {
        const float4 a4 = *reinterpret_cast<const float4*>(wm.alpha + ((4 * s) & 7));
        const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[nb][i] *= ar[i];
        }
      }
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        float4v po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          po = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              wa[kb], value_operand<kVBits, kDim>(cur.vw, nb, kb, vmask, kmask, one16), po,
              0, 0, 0);
        const float cv = vc[16 * nb + n];
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nb][i] = fmaf(cv, fmaf(po[i], kVOut, br[i]), oacc[nb][i]);
      }
    }
    if (nrec != nullptr) load_values(nrec, lo, cur);
  }

  // ---- combine the waves' states in LDS and write one partial per (slot, head)
  // (score lanes s == 0 hold m, l of column n; rows 4 s + i hold o~ hi (s < 2) and lo parts)
  __syncthreads();
  if (s == 0 && colhi) {
    sm.comb_m[wave][n] = m_run;
    sm.comb_l[wave][n] = l_run;
  }
  {
    // add the lo rows (lanes 32..63) into the hi rows (lanes 0..31)
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float both = add_xor32(oacc[nb][i]);
        if (s < 2) sm.comb_o[wave][4 * s + i][16 * nb + n] = both;
      }
    }
  }
  __syncthreads();
  const int wbad = __syncthreads_or(bad ? 1 : 0);
  for (int idx = tid; idx < nh * kDim; idx += kTThreads) {
    const int gg = idx / kDim, jj = idx % kDim;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm.comb_m[w][gg]);
    float ll = 0.0f, oo = 0.0f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(sm.comb_m[w][gg] - mm);
        ll = fmaf(f, sm.comb_l[w][gg], ll);
        oo = fmaf(f, sm.comb_o[w][gg][jj], oo);
      }
    }
    float* p = partials + (row_of(vbase + gg) * nslot + slot) * kPF;
    if (jj == 0) {
      p[0] = wbad ? NAN : mm;
      p[1] = wbad ? NAN : ll;
      if (end_mark) p[kPF] = INFINITY;             // m of the next slot: the row ends here
    }
    p[2 + jj] = oo;
  }
}

// kList: the list schedule (one head group; grid = the resident workgroups); otherwise the
// split grid (splits x KV heads x head groups, sequences).
template <bool kCausal, int kVBits, int kDim, bool kList>
__global__ void __launch_bounds__(kTThreads)
__attribute__((amdgpu_waves_per_eu(kDim == 256 ? 1 : 2, kDim == 256 ? 1 : 2)))
decode_tiles_kernel(const __half* __restrict__ q, int hq, int hkv, int nq,
                    const uint8_t* __restrict__ pool, long long num_blocks,
                    const int32_t* __restrict__ block_table, int max_blocks,
                    const int32_t* __restrict__ seq_lens, int batch, float sm_scale,
                    float* __restrict__ partials, int nslot, SignWords signs, int min_share) {
  __shared__ TileSmem<kDim> sm;
  // query rows: (query token i, head h) pairs of KV head g, virtual head v = i * group + l for
  // head h = g * group + l; a workgroup serves virtual heads vbase .. vbase + nh - 1
  const int group = hq / hkv, vgroup = group * nq;
  const int ngroups = (vgroup + kHeadGroup - 1) / kHeadGroup;
  if constexpr (kList) {
    // the full tiles of every (sequence, KV head, head group of 8) form one list that the
    // workgroups share evenly, as in the paired-tile schedule (with tiles for positions);
    // unit u = g * ngroups + hg
    const int lane = threadIdx.x & 63;
    const int wgs = gridDim.x, w = blockIdx.x;
    const int hu = hkv * ngroups;
    const ListScan ls = scan_list<1>(seq_lens, batch, max_blocks, hu, lane);
    const PairSplit split = pair_split(ls.total, wgs, min_share);
    const long long start64 = split.start(w);
    if (start64 >= ls.total) return;
    const int start = (int)start64;
    const int end = (int)min(split.start(w + 1), (long long)ls.total);
    for (int cur = start; cur < end;) {
      int b, before;
      locate_position<1>(ls, seq_lens, max_blocks, hu, cur, lane, b, before);
      const int len = seq_lens[b];
      const int nt = full_tiles(len, max_blocks);  // > 0: the sequence holds position cur
      const int u = (cur - before) / nt;
      const int t0 = (cur - before) - u * nt;
      const int seg = min(nt - t0, end - cur);
      const int slot = w - split.wave_of(cur - t0);
      if (cur != start) __syncthreads();           // LDS of the last unit read before this one's
      tile_segment<kCausal, kVBits, kDim>(sm, q, hq, hkv, nq, pool, num_blocks, block_table,
                                          max_blocks, len, sm_scale, partials, signs, b,
                                          u / ngroups, u % ngroups, t0, seg, false, slot, nslot,
                                          cur - start, end - start,
                                          t0 + seg == nt && slot + 1 < nslot);
      cur += seg;
    }
    return;
  }
  const int nsplit = gridDim.x;
  int split = blockIdx.x, g = blockIdx.y / ngroups, hg = blockIdx.y % ngroups, b = blockIdx.z;
  if (ngroups > 1) {
    // workgroups that read the same tiles (same split, KV head, sequence; different head
    // groups) take dispatch ids 8 apart, so they run on the same XCD and share its L2
    const int L = blockIdx.x + nsplit * (blockIdx.y + gridDim.y * blockIdx.z);
    const int P = nsplit * hkv * gridDim.z;
    const int full = P & ~7;
    int p;
    if (L < full * ngroups) {
      const int r = L % (8 * ngroups);
      hg = r >> 3;
      p = (L / (8 * ngroups)) * 8 + (r & 7);
    } else {
      const int rem = P - full, r = L - full * ngroups;
      hg = r / rem;
      p = full + r % rem;
    }
    split = p % nsplit;
    g = (p / nsplit) % hkv;
    b = p / (nsplit * hkv);
  }
  const int len = seq_lens[b];
  const bool bad = len < 0 || (len >> 7) > max_blocks;
  const int n_full = bad ? 0 : (len >> 7);
  const int chunk = (n_full + nsplit - 1) / nsplit;
  const int i0 = min(split * chunk, n_full), i1 = min(i0 + chunk, n_full);
  tile_segment<kCausal, kVBits, kDim>(sm, q, hq, hkv, nq, pool, num_blocks, block_table,
                                      max_blocks, len, sm_scale, partials, signs, b, g, hg, i0,
                                      i1 - i0, bad, split, nsplit, 0, i1 - i0, false);
}

// ------------------------------------------------------------------ 16 virtual heads per tile
//
// With more than 8 virtual heads per KV head (D = 128), a workgroup serves 16 of them, one per
// MFMA column, and a query's fp32-accurate operand enters as its fp16 hi and lo parts along the
// K dimension instead of in two columns: two products with the same unpacked key operand
// accumulate into one column, so the codes are unpacked once per 16 virtual heads instead of
// once per 8. The output product works the same way: a lane's probabilities (column n = head
// n, tokens 16 mb + 4 s + i) are exactly the elements of its operand row n, so its hi and lo
// parts feed two products with one unpacked value operand, and no lane exchanges any value.
// Output rows are heads 4 s + i. Registers per lane stay those of the 8-head kernel.

constexpr int kWideGroup = 16;

struct WideSmem {
  float qrot[kWideGroup][kD + 4];    // rotated queries (fp32)
  WaveMeta<kD> wm[kWaves];
  float comb_m[kWaves][kWideGroup], comb_l[kWaves][kWideGroup];
  float comb_o[kWaves][kWideGroup][kD];
  float red[kWaves];
};

// As tile_segment, for the 16 virtual heads vbase = 16 hg .. of KV head g.
template <bool kCausal, int kVBits>
__device__ __forceinline__ void wide_segment(
    WideSmem& sm, const __half* __restrict__ q, int hq, int hkv, int nq,
    const uint8_t* __restrict__ pool, long long num_blocks,
    const int32_t* __restrict__ block_table, int max_blocks, int len, float sm_scale,
    float* __restrict__ partials, const SignWords& signs, int b, int g, int hg, int i0,
    int ntile, bool bad, int slot, int nslot, int done0, int total, bool end_mark) {
  constexpr int kKW = kD / 32, kNB = kD / 16, kPer = kD / 64, kPF = 2 + kD;
  const int group = hq / hkv, vgroup = group * nq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int vbase = hg * kWideGroup;
  const int nh = min(kWideGroup, vgroup - vbase);             // rows served (1..16)
  auto row_of = [&](int v) -> long long {                     // row in [B][nq][hq]
    return ((long long)b * nq + v / group) * hq + g * group + v % group;
  };
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nw = ntile > wave_u ? (ntile - wave_u + kWaves - 1) / kWaves : 0;
  const int32_t* bt_row = block_table + (long long)b * max_blocks + i0 + wave_u;
  constexpr long long kTileBytes = RecordLayout<kVBits, kD>::kTileBytes;
  const LaneOffsets<kD> lo = lane_offsets<kVBits, kD>(lane);
  TileRegs<kVBits, kD> cur;
  int id_next = nw > 1 ? bt_row[kWaves] : 0;        // tile 1
  if (nw > 0) {
    const long long blk = bt_row[0];
    if (blk < 0 || blk >= num_blocks) {
      bad = true;
    } else {
      const uint8_t* rec = pool + (blk * hkv + g) * (long long)kTileBytes;
      load_keys(rec, lo, cur);
      load_values(rec, lo, cur);
    }
  }

  // ---- rotated queries in LDS: wave w rotates heads 4 w .. 4 w + 3 (channels 2 lane, + 1)
  float qmax = 0.0f;
  const uint32_t sb = lane_sign_bits_d<kPer>(signs, lane);       // optional sign flips
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int gg = 4 * wave + k;
    float o[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) o[i] = 0.0f;
    if (gg < nh) {
      load_h<kPer>(q + row_of(vbase + gg) * kD + kPer * lane, o);
#pragma unroll
      for (int i = 0; i < kPer; ++i) o[i] = (sb >> i) & 1u ? -o[i] : o[i];
    }
    fwht_lanes<kPer>(o, lane);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      o[i] *= 0.08838834764831845f;
      sm.qrot[gg][kPer * lane + i] = o[i];
      qmax = fmaxf(qmax, fabsf(o[i]));
    }
  }
  qmax = wave_max_nonneg(qmax);
  if (lane == 0) sm.red[wave] = qmax;
  __syncthreads();
  qmax = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
  int qe = 0;
  frexpf(fmaxf(qmax, 1e-30f) * 448.0f, &qe);
  const float pq = ldexpf(1.0f, 14 - qe);          // |q~ * pq| <= 2^14: hi parts stay finite
  const float scale2 = sm_scale * kLog2e;
  const float kfac = scale2 * 64.0f / pq;
  const float kzfac = scale2 / pq;
  float fm[TileRegs<kVBits, kD>::kM8];
#pragma unroll
  for (int k = 0; k < TileRegs<kVBits, kD>::kM8; ++k)
    fm[k] = meta_chunk_factor<kD>(lane + 64 * k, pq, kfac);
  const float fz = lane < 32 ? kzfac : 1.0f;

  // lane roles: column n = virtual head n (scores, operand rows of the output product); s
  // for token rows 4 s + i of the score blocks and the K groups; output rows 4 s + i = heads
  const int n = lane & 15, s = lane >> 4;
  const uint32_t vmask_col = n < nh ? 0xFFFFFFFFu : 0u;
  const int qlim = len - nq + (vbase + n) / group;
  WaveMeta<kD>& wm = sm.wm[wave];
  const float* kc = wm.f8;
  const float* ks = wm.f8 + kD;
  const float* vc = wm.f8 + kD + kT;
  const float* vs = wm.f8 + 2 * kD + kT;
  const float* kz = wm.h16;
  const float* vz = wm.h16 + kT;
  uint32_t kmask = 0x03C003C0u, vmask = 0x03000300u;
  asm volatile("" : "+v"(kmask), "+v"(vmask));
  const uint32_t one16 = __builtin_amdgcn_readfirstlane(0x3C003C00u);
  const KeyConsts kcon = key_consts();

  float m_run = -INFINITY, l_run = 0.0f;
  float4v oacc[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) oacc[nb] = (float4v){0.f, 0.f, 0.f, 0.f};

  for (int j = 0; j < nw && !bad; ++j) {
    if constexpr (kTilePrio) set_progress_priority(done0 + kWaves * j, total);
    const uint8_t* nrec = nullptr;
    if (j + 1 < nw) {
      const long long blk = id_next;
      if (j + 2 < nw) id_next = bt_row[kWaves * (j + 2)];
      if (blk >= 0 && blk < num_blocks) nrec = pool + (blk * hkv + g) * (long long)kTileBytes;
      else bad = true;                             // finishes this tile, then stops
    }
#pragma unroll
    for (int k = 0; k < TileRegs<kVBits, kD>::kM8; ++k)
      decode_meta8(cur.m8[k], wm.f8 + 8 * (lane + 64 * k), fm[k]);
    decode_meta16(cur.m16, wm.h16 + 4 * lane, fz);

    // ---- query operands of channel block c, hi and lo parts of q' = pq * q_rot * c-hat^K;
    // element e is channel 32 s + 8 c + {0,4,1,5,2,6,3,7}[e]
    float asum = 0.0f;
    const float4* qr4 = reinterpret_cast<const float4*>(sm.qrot[n] + 32 * s);
    const float4* kc4 = reinterpret_cast<const float4*>(kc + 32 * s);
    half8 qh[kKW], ql[kKW];
#pragma unroll
    for (int c = 0; c < kKW; ++c) {
      const float4 qa = qr4[2 * c], qc = qr4[2 * c + 1];
      const float4 ka = kc4[2 * c], kk = kc4[2 * c + 1];
      const float x0 = qa.x * ka.x, x1 = qa.y * ka.y, x2 = qa.z * ka.z, x3 = qa.w * ka.w;
      const float x4 = qc.x * kk.x, x5 = qc.y * kk.y, x6 = qc.z * kk.z, x7 = qc.w * kk.w;
      asum += ((x0 + x1) + (x2 + x3)) + ((x4 + x5) + (x6 + x7));
      const uint32_t h0 = pack_h2(x0, x4), h1 = pack_h2(x1, x5);
      const uint32_t h2 = pack_h2(x2, x6), h3 = pack_h2(x3, x7);
      qh[c] = as_h8(h0 & vmask_col, h1 & vmask_col, h2 & vmask_col, h3 & vmask_col);
      ql[c] = as_h8(lo_of(h0, x0, x4) & vmask_col, lo_of(h1, x1, x5) & vmask_col,
                    lo_of(h2, x2, x6) & vmask_col, lo_of(h3, x3, x7) & vmask_col);
    }
    asum = add_xor32(add_xor16(asum));            // over all 128 channels of column n
    const float asum_c = 0.125f * asum;           // the centring term, 8 / 64 * asum

    // ---- scores: 8 token blocks x 4 channel blocks, hi and lo products per block
    float4v sc[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kKW; ++c) {
        const half8 kop = key_operand(cur.kw[mb][c], kcon);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qh[c], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, ql[c], acc, 0, 0, 0);
      }
      sc[mb] = acc;
    }
    if (nrec != nullptr) load_keys(nrec, lo, cur);
    // log2-domain scores of this lane's tokens 16 mb + 4 s + i
    float tmax = -INFINITY;
    const int tpos = kT * (i0 + wave_u + kWaves * j);
    const bool masked = kCausal && tpos + kT - 1 > len - nq;   // wave-uniform
    const int tlim = qlim - tpos;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int t0 = 16 * mb + 4 * s;
      const float4 ks4 = *reinterpret_cast<const float4*>(ks + t0);
      const float4 kz4 = *reinterpret_cast<const float4*>(kz + t0);
      const float ksv[4] = {ks4.x, ks4.y, ks4.z, ks4.w}, kzv[4] = {kz4.x, kz4.y, kz4.z, kz4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = fmaf(ksv[i], sc[mb][i] + asum_c, kzv[i] * asum);
        if (masked) v = t0 + i > tlim ? -INFINITY : v;
        sc[mb][i] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = max_xor32(max_xor16(tmax));
    const bool upd = tmax > m_run + kLazy;        // also true on the first tile
    const float mnew = upd ? tmax : m_run;
    const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;
    const bool rescale = __any(upd) && j > 0;     // wave-uniform
    float psum = 0.0f, beta = 0.0f, wsum = 0.0f;
    // probabilities -> this lane's operand row n: element e of token block kb is token
    // 32 kb + 16 (e / 4) + 4 s + e % 4, i.e. score block 2 kb + e / 4, element e % 4
    half8 wh[4], wl[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint32_t hh[4], ll[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int mb = 2 * kb + h2, t0 = 16 * mb + 4 * s;
        const float4 vs4 = *reinterpret_cast<const float4*>(vs + t0);
        const float4 vz4 = *reinterpret_cast<const float4*>(vz + t0);
        const float p0 = __builtin_amdgcn_exp2f(sc[mb][0] - mnew);
        const float p1 = __builtin_amdgcn_exp2f(sc[mb][1] - mnew);
        const float p2 = __builtin_amdgcn_exp2f(sc[mb][2] - mnew);
        const float p3 = __builtin_amdgcn_exp2f(sc[mb][3] - mnew);
        psum += (p0 + p1) + (p2 + p3);
        beta = fmaf(p0, vz4.x, fmaf(p1, vz4.y, fmaf(p2, vz4.z, fmaf(p3, vz4.w, beta))));
        const float w0 = p0 * vs4.x, w1 = p1 * vs4.y, w2 = p2 * vs4.z, w3 = p3 * vs4.w;
        wsum += (w0 + w1) + (w2 + w3);
        hh[2 * h2] = pack_h2(w0, w1);
        hh[2 * h2 + 1] = pack_h2(w2, w3);
        ll[2 * h2] = lo_of(hh[2 * h2], w0, w1);
        ll[2 * h2 + 1] = lo_of(hh[2 * h2 + 1], w2, w3);
      }
      wh[kb] = as_h8(hh[0] & vmask_col, hh[1] & vmask_col, hh[2] & vmask_col, hh[3] & vmask_col);
      wl[kb] = as_h8(ll[0] & vmask_col, ll[1] & vmask_col, ll[2] & vmask_col, ll[3] & vmask_col);
    }
    psum = add_xor32(add_xor16(psum));
    beta = add_xor32(add_xor16(beta));
    wsum = add_xor32(add_xor16(wsum));
    constexpr float kVOut = kVBits == 4 ? 0.5f : 0.125f;
    beta = fmaf(-kVOut, wsum, beta);
    l_run = fmaf(alpha, l_run, psum);
    m_run = mnew;
    if (s == 0) {
      wm.alpha[n] = alpha;
      wm.beta[n] = beta;
    }

    // ---- output: 8 channel blocks x 4 token blocks x hi, lo; rows 4 s + i are heads
    {
      const float4 b4 = *reinterpret_cast<const float4*>(wm.beta + 4 * s);
      const float br[4] = {b4.x, b4.y, b4.z, b4.w};
      if (rescale) {
        const float4 a4 = *reinterpret_cast<const float4*>(wm.alpha + 4 * s);
        const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[nb][i] *= ar[i];
        }
      }
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        float4v po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const half8 vop = value_operand<kVBits, kD>(cur.vw, nb, kb, vmask, kmask, one16);
          po = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh[kb], vop, po, 0, 0, 0);
          po = __builtin_amdgcn_mfma_f32_16x16x32_f16(wl[kb], vop, po, 0, 0, 0);
        }
        const float cv = vc[16 * nb + n];
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nb][i] = fmaf(cv, fmaf(po[i], kVOut, br[i]), oacc[nb][i]);
      }
    }
    if (nrec != nullptr) load_values(nrec, lo, cur);
  }

  // ---- combine the waves' states in LDS and write one partial per (slot, head)
  __syncthreads();
  if (s == 0) {
    sm.comb_m[wave][n] = m_run;
    sm.comb_l[wave][n] = l_run;
  }
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.comb_o[wave][4 * s + i][16 * nb + n] = oacc[nb][i];
  }
  __syncthreads();
  const int wbad = __syncthreads_or(bad ? 1 : 0);
  for (int idx = tid; idx < nh * kD; idx += kTThreads) {
    const int gg = idx / kD, jj = idx % kD;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm.comb_m[w][gg]);
    float ll = 0.0f, oo = 0.0f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(sm.comb_m[w][gg] - mm);
        ll = fmaf(f, sm.comb_l[w][gg], ll);
        oo = fmaf(f, sm.comb_o[w][gg][jj], oo);
      }
    }
    float* p = partials + (row_of(vbase + gg) * nslot + slot) * kPF;
    if (jj == 0) {
      p[0] = wbad ? NAN : mm;
      p[1] = wbad ? NAN : ll;
      if (end_mark) p[kPF] = INFINITY;             // m of the next slot: the row ends here
    }
    p[2 + jj] = oo;
  }
}

// kList: the list schedule over (sequence, KV head, head group) units (grid = the resident
// workgroups); otherwise the split grid (splits x KV heads x head groups of 16, sequences).
template <bool kCausal, int kVBits, bool kList>
__global__ void __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_wide_kernel(const __half* __restrict__ q, int hq, int hkv, int nq,
                   const uint8_t* __restrict__ pool, long long num_blocks,
                   const int32_t* __restrict__ block_table, int max_blocks,
                   const int32_t* __restrict__ seq_lens, int batch, float sm_scale,
                   float* __restrict__ partials, int nslot, SignWords signs, int min_share) {
  __shared__ WideSmem sm;
  const int vgroup = hq / hkv * nq;
  const int ngroups = (vgroup + kWideGroup - 1) / kWideGroup;
  if constexpr (kList) {
    // units are (sequence, KV head, head group of 16): the list runs over hkv * ngroups units
    // per sequence, unit u = g * ngroups + hg
    const int lane = threadIdx.x & 63;
    const int wgs = gridDim.x, w = blockIdx.x;
    const int hu = hkv * ngroups;
    const ListScan ls = scan_list<1>(seq_lens, batch, max_blocks, hu, lane);
    const PairSplit split = pair_split(ls.total, wgs, min_share);
    const long long start64 = split.start(w);
    if (start64 >= ls.total) return;
    const int start = (int)start64;
    const int end = (int)min(split.start(w + 1), (long long)ls.total);
    for (int cur = start; cur < end;) {
      int b, before;
      locate_position<1>(ls, seq_lens, max_blocks, hu, cur, lane, b, before);
      const int len = seq_lens[b];
      const int nt = full_tiles(len, max_blocks);  // > 0: the sequence holds position cur
      const int u = (cur - before) / nt;
      const int t0 = (cur - before) - u * nt;
      const int seg = min(nt - t0, end - cur);
      const int slot = w - split.wave_of(cur - t0);
      if (cur != start) __syncthreads();           // LDS of the last unit read before this one's
      wide_segment<kCausal, kVBits>(sm, q, hq, hkv, nq, pool, num_blocks, block_table,
                                    max_blocks, len, sm_scale, partials, signs, b, u / ngroups,
                                    u % ngroups, t0, seg, false, slot, nslot, cur - start,
                                    end - start, t0 + seg == nt && slot + 1 < nslot);
      cur += seg;
    }
    return;
  }
  const int nsplit = gridDim.x;
  int split = blockIdx.x, g = blockIdx.y / ngroups, hg = blockIdx.y % ngroups, b = blockIdx.z;
  if (ngroups > 1) {
    // workgroups that read the same tiles (same split, KV head, sequence; different head
    // groups) take dispatch ids 8 apart, so they run on the same XCD and share its L2
    const int L = blockIdx.x + nsplit * (blockIdx.y + gridDim.y * blockIdx.z);
    const int P = nsplit * hkv * gridDim.z;
    const int full = P & ~7;
    int p;
    if (L < full * ngroups) {
      const int r = L % (8 * ngroups);
      hg = r >> 3;
      p = (L / (8 * ngroups)) * 8 + (r & 7);
    } else {
      const int rem = P - full, r = L - full * ngroups;
      hg = r / rem;
      p = full + r % rem;
    }
    split = p % nsplit;
    g = (p / nsplit) % hkv;
    b = p / (nsplit * hkv);
  }
  const int len = seq_lens[b];
  const bool bad = len < 0 || (len >> 7) > max_blocks;
  const int n_full = bad ? 0 : (len >> 7);
  const int chunk = (n_full + nsplit - 1) / nsplit;
  const int i0 = min(split * chunk, n_full), i1 = min(i0 + chunk, n_full);
  wide_segment<kCausal, kVBits>(sm, q, hq, hkv, nq, pool, num_blocks, block_table, max_blocks,
                                len, sm_scale, partials, signs, b, g, hg, i0, i1 - i0, bad, split,
                                nsplit, 0, i1 - i0, false);
}

// ------------------------------------------------------------------ paired tiles (<= 4 heads)
//
// With at most four virtual heads per KV head (G * nq <= 4) one tile fills only half of the 16
// MFMA columns (a hi and a lo part per head), so a wave takes its tiles two at a time and the
// products carry both: columns (score product) and rows (output product) 0..7 belong to the
// first tile of the pair, 8..15 to the second, and within each half position h holds head h's
// hi part and position 7 - h its lo part (DPP row_half_mirror pairs the two). Each tile's
// operand is zero in the other tile's half, so the two tiles' MFMAs accumulate into one set of
// accumulators and everything between and after them (combining the score parts, the softmax,
// the probability operand, folding the output scales) runs once per pair.
//
// Schedule: the tile pairs of every (sequence, KV head) in order (sequence, KV head, pair) form
// one work list (a unit of n full tiles holds ceil(n / 2) pairs, the last single when n is
// odd), and the grid is as many one-wave workgroups as the device holds at once (W). The waves
// split the list into consecutive equal shares (PairSplit) whatever the mix of lengths; all of
// them run at once, so there is no tail of late waves, and a share never splits a pair. Where a wave's range crosses from one
// (sequence, KV head) to the next it finishes the first, writes its partial (m, l, o~) per
// virtual head, and starts the next; the partial goes to slot w - wave_of(T(u)) of the unit u
// it belongs to (T(u) = the unit's first list position), so a unit fills slots 0 ..
// wave_of(T(u) + m - 1) - wave_of(T(u)) for its m pairs. The wave that finishes a unit marks
// the slot after its own with m = +inf (where the row has one), which is how the merge kernel
// finds the row's end without redoing the schedule. Only a unit's last pair can be single: its
// second tile's products are then skipped and its columns carry no probability.

struct PairSmem {
  float qrot[4][kD + 4];           // rotated queries of the virtual heads (fp32)
  float f8[2][4 * kD];             // per tile: c-hat^K * pq | s-hat^K * kfac | c-hat^V | 32 s-hat^V
  float h16[2][2 * kT];            // per tile: z-hat^K * kzfac | z-hat^V
  float alpha[16], beta[16];       // per column / row of the pair layout
};

__device__ __forceinline__ float dpp_half_mirror(float v) {   // lane (l & ~7) | (7 - (l & 7))
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t dpp_half_mirror_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);
}



// Tiles i0 .. i0 + ntile - 1 (ntile >= 1) of KV head g of sequence b (length len, valid) into
// partial slot `slot` of each virtual head's row (rows of nslot slots); end_mark: also mark
// the next slot as the rows' end (m = +inf).
template <bool kCausal, int kVBits>
__device__ __forceinline__ void pair_segment(
    PairSmem& sm, const __half* __restrict__ q, int hq, int hkv, int nq,
    const uint8_t* __restrict__ pool, long long num_blocks,
    const int32_t* __restrict__ block_table, int max_blocks, int len, float sm_scale,
    float* __restrict__ partials, const SignWords& signs, int b, int g, int i0, int ntile,
    int slot, int nslot, int done0, int wave_tiles, bool end_mark) {
  const int group = hq / hkv, nh = group * nq;                // virtual heads served (1..4)
  const int lane = threadIdx.x;
  auto row_of = [&](int v) -> long long {                     // row in [B][nq][hq]
    return ((long long)b * nq + v / group) * hq + g * group + v % group;
  };
  bool bad = false;
  const int npair = (ntile + 1) >> 1;              // pair p: tiles i0 + 2 p, i0 + 2 p + 1
  const int32_t* bt_row = block_table + (long long)b * max_blocks + i0;
  constexpr long long kTileBytes = RecordLayout<kVBits>::kTileBytes;
  const LaneOffsets<kD> lo = lane_offsets<kVBits, kD>(lane);
  TileRegs<kVBits, kD> cx, cy;
  // block ids are scalar loads issued one pair before the pair that needs them
  int idx_next = 0, idy_next = 0;
  if (npair > 1) {
    idx_next = bt_row[2];
    if (3 < ntile) idy_next = bt_row[3];
  }
  {
    const long long bx = bt_row[0];
    const bool y0 = 1 < ntile;
    const long long by = y0 ? bt_row[1] : 0;
    if (bx < 0 || bx >= num_blocks || (y0 && (by < 0 || by >= num_blocks))) {
      bad = true;
    } else {
      const uint8_t* rx = pool + (bx * hkv + g) * kTileBytes;
      load_keys(rx, lo, cx);
      load_values(rx, lo, cx);
      if (y0) {
        const uint8_t* ry = pool + (by * hkv + g) * kTileBytes;
        load_keys(ry, lo, cy);
        load_values(ry, lo, cy);
      }
    }
  }

  // ---- rotated queries in LDS (channels 2 lane, 2 lane + 1 of each virtual head)
  float qmax = 0.0f;
  const uint32_t sb = lane_sign_bits(signs.lo, lane);           // optional sign flips
  for (int k = 0; k < 4; ++k) {
    float o0 = 0.0f, o1 = 0.0f;
    if (k < nh) {
      uint32_t w = reinterpret_cast<const uint32_t*>(q + row_of(k) * kD)[lane];
      w ^= ((sb & 1u) << 15) | ((sb >> 1) << 31);
      o0 = fp16_bits_to_float(w & 0xFFFFu);
      o1 = fp16_bits_to_float(w >> 16);
      fwht_wave(o0, o1, lane);
      o0 *= 0.08838834764831845f;
      o1 *= 0.08838834764831845f;
    }
    *reinterpret_cast<float2*>(&sm.qrot[k][2 * lane]) = make_float2(o0, o1);
    qmax = fmaxf(qmax, fmaxf(fabsf(o0), fabsf(o1)));
  }
  qmax = wave_max_nonneg(qmax);
  int qe = 0;
  frexpf(fmaxf(qmax, 1e-30f) * 448.0f, &qe);
  const float pq = ldexpf(1.0f, 14 - qe);          // |q~ * pq| <= 2^14: hi parts stay finite
  const float scale2 = sm_scale * kLog2e;
  const float kfac = scale2 * 64.0f / pq;          // undoes the code / 64 encoding and pq
  const float kzfac = scale2 / pq;
  const int mgrp = lane >> 4;
  const float fm = mgrp == 0 ? pq : (mgrp == 1 ? kfac : (mgrp == 2 ? 1.0f : 32.0f));
  const float fz = lane < 32 ? kzfac : 1.0f;

  // lane roles: column / row n of the pair layout, score rows and output k groups s
  const int n = lane & 15, s = lane >> 4;
  const int tsel = n >> 3;                         // first or second tile of the pair
  const int pos = n & 7;
  const bool colhi = pos < 4;
  const uint32_t hi_m = lane_mask(colhi);
  const int hh = colhi ? pos : 7 - pos;            // virtual head of this column / row
  const bool colv = hh < nh;
  const float negk = colhi ? 0.0f : -1.0f;         // hi parts at positions 0-3, lo at 4-7
  const int ih = colhi ? 0 : 2;                    // this lane's rows of each score block
  const uint32_t mask_x = (colv && tsel == 0) ? 0xFFFFFFFFu : 0u;
  const uint32_t mask_y = (colv && tsel == 1) ? 0xFFFFFFFFu : 0u;
  // causal limit of this column's query token (position len - nq + i); with nq <= 16 every
  // packed tile keeps >= 112 visible tokens
  const int qlim = len - nq + hh / group;
  uint32_t vmask = 0x03000300u, kmask = 0x03C003C0u;
  asm volatile("" : "+v"(vmask), "+v"(kmask));
  const uint32_t one16 = __builtin_amdgcn_readfirstlane(0x3C003C00u);
  const KeyConsts kcon = key_consts();

  float m_run = -INFINITY, l_run = 0.0f;
  float4v oacc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) oacc[nb] = (float4v){0.f, 0.f, 0.f, 0.f};

  for (int p = 0; p < npair && !bad; ++p) {
    if constexpr (kPairPrio) set_progress_priority(done0 + 2 * p, wave_tiles);
    const bool has_y = 2 * p + 1 < ntile;          // wave-uniform
    const uint8_t* nrx = nullptr;
    const uint8_t* nry = nullptr;
    if (p + 1 < npair) {
      const bool ny = 2 * p + 3 < ntile;
      const long long bx = idx_next, by = idy_next;
      if (p + 2 < npair) {
        idx_next = bt_row[2 * p + 4];
        idy_next = 2 * p + 5 < ntile ? bt_row[2 * p + 5] : 0;
      }
      if (bx >= 0 && bx < num_blocks && (!ny || (by >= 0 && by < num_blocks))) {
        nrx = pool + (bx * hkv + g) * kTileBytes;
        if (ny) nry = pool + (by * hkv + g) * kTileBytes;
      } else {
        bad = true;                                // finishes this pair, then stops
      }
    }
    decode_meta(cx.m8[0], cx.m16, lane, sm.f8[0], sm.h16[0], fm, fz);
    if (has_y) decode_meta(cy.m8[0], cy.m16, lane, sm.f8[1], sm.h16[1], fm, fz);
    // tables this lane reads: its column's tile (the first tile's when the pair is single; the
    // second tile's columns are then masked), and its output rows' tile
    const int tcol = has_y ? tsel : 0;
    const int trow = has_y ? (s >> 1) : 0;
    const bool col_live = tsel == 0 || has_y;

    // ---- query operands: q' = pq * q_rot * c-hat^K of this column's tile, hi or lo part;
    // element e of channel block c is channel 32 s + 8 c + {0,4,1,5,2,6,3,7}[e]
    half8 qx[4], qy[4];
    float asum = 0.0f;
    {
      const float4* qr4 = reinterpret_cast<const float4*>(sm.qrot[colv ? hh : 0] + 32 * s);
      const float4* kc4 = reinterpret_cast<const float4*>(sm.f8[tcol] + 32 * s);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 qa = qr4[2 * c], qc = qr4[2 * c + 1];
        const float4 ka = kc4[2 * c], kk = kc4[2 * c + 1];
        const float x0 = qa.x * ka.x, x1 = qa.y * ka.y, x2 = qa.z * ka.z, x3 = qa.w * ka.w;
        const float x4 = qc.x * kk.x, x5 = qc.y * kk.y, x6 = qc.z * kk.z, x7 = qc.w * kk.w;
        asum += ((x0 + x1) + (x2 + x3)) + ((x4 + x5) + (x6 + x7));
        const uint32_t h0 = hi_or_lo(x0, x4, negk), h1 = hi_or_lo(x1, x5, negk);
        const uint32_t h2 = hi_or_lo(x2, x6, negk), h3 = hi_or_lo(x3, x7, negk);
        qx[c] = as_h8(h0 & mask_x, h1 & mask_x, h2 & mask_x, h3 & mask_x);
        qy[c] = as_h8(h0 & mask_y, h1 & mask_y, h2 & mask_y, h3 & mask_y);
      }
    }
    asum = add_xor32(add_xor16(asum));             // over all 128 channels of column n
    const float asum_c = 0.125f * asum;            // the centring term, 8 / 64 * asum

    // ---- scores: 8 token blocks x (4 channel blocks of the first tile, 4 of the second)
    float4v sc[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      float4v acc = {0.f, 0.f, 0.f, 0.f};
      const uint32_t* wx = cx.kw[mb];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand(wx[c], kcon), qx[c], acc, 0, 0, 0);
      if (has_y) {
        const uint32_t* wy = cy.kw[mb];
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(key_operand(wy[c], kcon), qy[c], acc, 0, 0, 0);
      }
      sc[mb] = acc;
    }
    if (nrx != nullptr) load_keys(nrx, lo, cx);
    if (nry != nullptr) load_keys(nry, lo, cy);
    // hi + lo partial scores of this lane's two rows, then the log2-domain score per token
    const float* ks = sm.f8[tcol] + kT;
    const float* kz = sm.h16[tcol];
    float v[8][2];
    float tmax = -INFINITY;
    const int tpos = kT * (i0 + 2 * p + tsel);     // position of token 0 of this column's tile
    const bool masked = kCausal && tpos + kT - 1 > len - nq;
    const int tlim = qlim - tpos;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const float snd0 = pick(hi_m, sc[mb][2], sc[mb][0]);
      const float snd1 = pick(hi_m, sc[mb][3], sc[mb][1]);
      const float own0 = pick(hi_m, sc[mb][0], sc[mb][2]);
      const float own1 = pick(hi_m, sc[mb][1], sc[mb][3]);
      const float d0 = own0 + dpp_half_mirror(snd0), d1 = own1 + dpp_half_mirror(snd1);
      const int t0 = 16 * mb + 4 * s + ih;
      const float2 ks2 = *reinterpret_cast<const float2*>(ks + t0);
      const float2 kz2 = *reinterpret_cast<const float2*>(kz + t0);
      v[mb][0] = fmaf(ks2.x, d0 + asum_c, kz2.x * asum);
      v[mb][1] = fmaf(ks2.y, d1 + asum_c, kz2.y * asum);
      if (masked) {
        v[mb][0] = t0 > tlim ? -INFINITY : v[mb][0];
        v[mb][1] = t0 + 1 > tlim ? -INFINITY : v[mb][1];
      }
      if (!col_live) {
        v[mb][0] = -INFINITY;
        v[mb][1] = -INFINITY;
      }
      tmax = fmaxf(tmax, fmaxf(v[mb][0], v[mb][1]));
    }
    tmax = fmaxf(tmax, dpp_half_mirror(tmax));     // hi and lo columns of the head
    tmax = fmaxf(tmax, dpp_ror8(tmax));            // the head's columns of the other tile
    tmax = max_xor32(max_xor16(tmax));             // all score rows
    const bool upd = tmax > m_run + kLazy;         // also true on the first pair
    const float mnew = upd ? tmax : m_run;
    const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;
    const bool rescale = __any(upd) && p > 0;      // wave-uniform
    float psum = 0.0f, beta = 0.0f, wsum = 0.0f;
    // probabilities -> operand rows: row n holds hi(32 p s-hat^V) (positions 0-3) or lo
    // (positions 4-7) of its tile's tokens; element e of token block kb is token
    // 32 kb + 16 (e / 4) + 4 s + e % 4
    const float* vs = sm.f8[tcol] + 3 * kT;
    const float* vz = sm.h16[tcol] + kT;
    half8 wx[4], wy[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint32_t u[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int mb = 2 * kb + h2, t0 = 16 * mb + 4 * s + ih;
        const float2 vs2 = *reinterpret_cast<const float2*>(vs + t0);
        const float2 vz2 = *reinterpret_cast<const float2*>(vz + t0);
        const float p0 = __builtin_amdgcn_exp2f(v[mb][0] - mnew);
        const float p1 = __builtin_amdgcn_exp2f(v[mb][1] - mnew);
        psum += p0 + p1;
        beta = fmaf(p0, vz2.x, fmaf(p1, vz2.y, beta));
        const float w0 = p0 * vs2.x, w1 = p1 * vs2.y;
        wsum += w0 + w1;
        const uint32_t hp = pack_h2(w0, w1);
        const uint32_t lp = lo_of(hp, w0, w1);
        const uint32_t rcv = dpp_half_mirror_u(colhi ? lp : hp);
        u[2 * h2] = colhi ? hp : rcv;              // rows 0, 1 of block mb
        u[2 * h2 + 1] = colhi ? rcv : lp;          // rows 2, 3
      }
      wx[kb] = as_h8(u[0] & mask_x, u[1] & mask_x, u[2] & mask_x, u[3] & mask_x);
      wy[kb] = as_h8(u[0] & mask_y, u[1] & mask_y, u[2] & mask_y, u[3] & mask_y);
    }
    // per tile and head: hi and lo columns, all score rows; psum also over both tiles
    psum += dpp_half_mirror(psum);
    beta += dpp_half_mirror(beta);
    wsum += dpp_half_mirror(wsum);
    psum += dpp_ror8(psum);
    psum = add_xor32(add_xor16(psum));
    beta = add_xor32(add_xor16(beta));
    wsum = add_xor32(add_xor16(wsum));
    constexpr float kVOut = kVBits == 4 ? 0.5f : 0.125f;
    beta = fmaf(-kVOut, wsum, beta);
    l_run = fmaf(alpha, l_run, psum);
    m_run = mnew;
    if (s == 0) {
      sm.alpha[n] = alpha;
      sm.beta[n] = colhi ? beta : 0.0f;            // the zero-point term enters the hi row once
    }

    // ---- output: 8 channel blocks x (4 token blocks of each tile); rows 4 s + i of channel
    // 16 nb + n; each block's accumulator is folded with the c-hat^V of its rows' tile
    {
      const float4 b4 = *reinterpret_cast<const float4*>(sm.beta + 4 * s);
      const float br[4] = {b4.x, b4.y, b4.z, b4.w};
      if (rescale) {
        const float4 a4 = *reinterpret_cast<const float4*>(sm.alpha + 4 * s);
        const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
        for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[nb][i] *= ar[i];
        }
      }
      const float* vc = sm.f8[trow] + 2 * kT;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        float4v po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          po = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              wx[kb], value_operand<kVBits>(cx.vw, nb, kb, vmask, kmask, one16), po, 0, 0, 0);
        if (has_y) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            po = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                wy[kb], value_operand<kVBits>(cy.vw, nb, kb, vmask, kmask, one16), po, 0, 0, 0);
        }
        const float cv = vc[16 * nb + n];
#pragma unroll
        for (int i = 0; i < 4; ++i) oacc[nb][i] = fmaf(cv, fmaf(po[i], kVOut, br[i]), oacc[nb][i]);
      }
    }
    if (nrx != nullptr) load_values(nrx, lo, cx);
    if (nry != nullptr) load_values(nry, lo, cy);
  }

  // ---- partial per virtual head: rows h (first tile, hi), 7 - h (first, lo), 8 + h and
  // 15 - h (second tile) sit in lane groups s = 0, 1, 2, 3 at register h, 3 - h, h, 3 - h
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = add_xor32(oacc[nb][i]);     // + the other tile's row
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = (s & 1) ? x[3 - i] : x[i];   // lo rows in head order
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float both = add_xor16(y[i]);                           // + the lo part
      if (s == 0 && i < nh)
        partials[(row_of(i) * nslot + slot) * kPartialFloats + 2 + 16 * nb + n] = both;
    }
  }
  if (s == 0 && colhi && tsel == 0 && colv) {
    float* pp = partials + (row_of(hh) * nslot + slot) * kPartialFloats;
    pp[0] = bad ? NAN : m_run;
    pp[1] = bad ? NAN : l_run;
    if (end_mark) pp[kPartialFloats] = INFINITY;   // m of the next slot: the row ends here
  }
}


template <bool kCausal, int kVBits>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_pairs_kernel(const __half* __restrict__ q, int hq, int hkv, int nq,
                    const uint8_t* __restrict__ pool, long long num_blocks,
                    const int32_t* __restrict__ block_table, int max_blocks,
                    const int32_t* __restrict__ seq_lens, int batch, float sm_scale,
                    float* __restrict__ partials, int nslot, SignWords signs, int min_share) {
  __shared__ PairSmem sm;
  const int lane = threadIdx.x;
  const int waves = gridDim.x, w = blockIdx.x;
  const ListScan ls = scan_list<2>(seq_lens, batch, max_blocks, hkv, lane);
  const PairSplit split = pair_split(ls.total, waves, min_share);
  const long long start64 = split.start(w);
  if (start64 >= ls.total) return;                 // more waves than list positions
  const int start = (int)start64;
  const int end = (int)min(split.start(w + 1), (long long)ls.total);
  // one segment per call: the first outside any loop (most waves have no other), the rest in
  // a loop
  auto segment = [&](int cur) -> int {
    int b, before;                                 // the unit holding position cur
    locate_position<2>(ls, seq_lens, max_blocks, hkv, cur, lane, b, before);
    const int len = seq_lens[b];
    const int nt = full_tiles(len, max_blocks);
    const int np = (nt + 1) >> 1;                  // > 0: the sequence holds position cur
    const int g = (cur - before) / np;
    const int p0 = (cur - before) - g * np;        // first pair of the segment in its unit
    const int seg = min(np - p0, end - cur);       // pairs
    const int slot = w - split.wave_of(cur - p0);  // cur - p0 = T(u)
    pair_segment<kCausal, kVBits>(sm, q, hq, hkv, nq, pool, num_blocks, block_table, max_blocks,
                                  len, sm_scale, partials, signs, b, g, 2 * p0,
                                  min(2 * seg, nt - 2 * p0), slot, nslot, 2 * (cur - start),
                                  2 * (end - start), p0 + seg == np && slot + 1 < nslot);
    return cur + seg;
  };
  int cur = segment(start);
  while (cur < end) {
    __syncthreads();                               // LDS of the last unit read before this one's
    cur = segment(cur);
  }
}


// grid (nq * hq, batch), one wave per (sequence, query token, query head): the staging tokens
// the query token sees (exact fp32
// attention with the unrotated query), the log-sum-exp merge of the tile splits, o~ H + o_raw,
// / l (the fp16-cache path's partials are not rotated: o + o_raw, / l). Lane l owns output
// channels kPer l .. kPer l + kPer - 1 (kPer = head dimension / 64); the inverse rotation is a
// butterfly on the channel bits inside a lane in registers and on the lane bits across lanes
// l ^ 1 .. l ^ 32. Every global load
// that does not depend on another is issued first; split weights and staging probabilities
// are broadcast from the lane that computed them.
constexpr int kMThreads = 64;
constexpr int kMaxSplits = 64;
#ifndef KVARN_PAIR_MIN_TILES_PER_CU
#define KVARN_PAIR_MIN_TILES_PER_CU 64
#endif
constexpr int kPairMinTilesPerCU = KVARN_PAIR_MIN_TILES_PER_CU;
#ifndef KVARN_PAIR_ROUNDS
#define KVARN_PAIR_ROUNDS 1
#endif
constexpr int kPairRounds = KVARN_PAIR_ROUNDS;   // paired-tile waves per resident wave slot
#ifndef KVARN_TILE_LIST_MAX_PER_CU
#define KVARN_TILE_LIST_MAX_PER_CU 2
#endif
// four-wave workgroups per compute unit on the tile list at most (D = 64 fits 3, and the
// shorter workers lose more to their start-up than the extra occupancy gains)
constexpr int kTileListMaxPerCU = KVARN_TILE_LIST_MAX_PER_CU;
#ifndef KVARN_WIDE_HEADS
#define KVARN_WIDE_HEADS 1
#endif
constexpr bool kWideHeads = KVARN_WIDE_HEADS != 0;   // 16-head kernel for > 8 virtual heads
#ifndef KVARN_MERGE_PRELOAD
#define KVARN_MERGE_PRELOAD 8
#endif
// splits whose o~ is loaded before the weights exist (and the chunk of the rest)
constexpr int kMergePreload = KVARN_MERGE_PRELOAD;
constexpr int kStageChunk = 32;           // staging value rows loaded per round

// <q, k> over kDim channels: k is one fp16 staging row, q the fp32 query in LDS.
template <int kDim>
__device__ __forceinline__ float staging_dot(const __half* __restrict__ krow, const float* qs) {
  const uint4* k4 = reinterpret_cast<const uint4*>(krow);
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int k = 0; k < kDim / 8; ++k) {
    float kv[8];
    unpack_h8(k4[k], kv);
    const float4 qa = *reinterpret_cast<const float4*>(qs + 8 * k);
    const float4 qc = *reinterpret_cast<const float4*>(qs + 8 * k + 4);
    acc0 = fmaf(qa.x, kv[0], fmaf(qa.y, kv[1], fmaf(qa.z, kv[2], fmaf(qa.w, kv[3], acc0))));
    acc1 = fmaf(qc.x, kv[4], fmaf(qc.y, kv[5], fmaf(qc.z, kv[6], fmaf(qc.w, kv[7], acc1))));
  }
  return acc0 + acc1;
}

// kPer consecutive floats at p (kPer = 1, 2 or 4) into v. p is 8-byte aligned for kPer >= 2
// (a partial holds 2 + D floats, so at D = 256 its rows are not 16-byte aligned): pairs.
template <int kPer>
__device__ __forceinline__ void load_f(const float* __restrict__ p, float (&v)[kPer]) {
  if constexpr (kPer == 1) {
    v[0] = p[0];
  } else {
#pragma unroll
    for (int i = 0; i < kPer; i += 2) {
      const float2 a = *reinterpret_cast<const float2*>(p + i);
      v[i] = a.x; v[i + 1] = a.y;
    }
  }
}

// This lane's kPer fp16 bit patterns at p, kept packed (one 16-bit pattern per element).
template <int kPer>
struct HalfBits {
  uint32_t w[(kPer + 1) / 2];
  __device__ __forceinline__ void load(const __half* __restrict__ p) {
    if constexpr (kPer == 1) w[0] = *reinterpret_cast<const uint16_t*>(p);
    else if constexpr (kPer == 2) w[0] = *reinterpret_cast<const uint32_t*>(p);
    else {
      const uint2 a = *reinterpret_cast<const uint2*>(p);
      w[0] = a.x; w[1] = a.y;
    }
  }
  __device__ __forceinline__ float at(int i) const {
    return fp16_bits_to_float((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
  }
};

template <bool kRotated, bool kCausal, int kDim>
__global__ void __launch_bounds__(kMThreads)
decode_merge_kernel(const __half* __restrict__ q, int hq, int hkv, int nq, int max_blocks,
                    const int32_t* __restrict__ seq_lens, const __half* __restrict__ staging_k,
                    const __half* __restrict__ staging_v, float sm_scale,
                    const float* __restrict__ partials, int nsplit, float* __restrict__ out,
                    SignWords signs, int list) {
  constexpr int kPer = kDim / 64;      // output channels per lane: kPer lane .. + kPer - 1
  constexpr int kPF = 2 + kDim;        // floats per partial
  __shared__ float qs[kDim];
  // The group query heads of one (sequence, query token, KV head) read the same staging tile:
  // they take dispatch ids 8 apart, so the round-robin dispatch runs them on one XCD and the
  // second and later reads of the tile come from that XCD's L2.
  const int group = hq / hkv;
  int qi, h, b;
  {
    const int L = blockIdx.x + gridDim.x * blockIdx.y;
    const int P = gridDim.y * nq * hkv;                  // (sequence, query token, KV head)
    const int full = P & ~7;
    int p, k;
    if (L < full * group) {
      const int r = L % (8 * group);
      k = r >> 3;
      p = (L / (8 * group)) * 8 + (r & 7);
    } else {
      const int rem = P - full, r = L - full * group;
      k = r / rem;
      p = full + r % rem;
    }
    h = (p % hkv) * group + k;
    qi = (p / hkv) % nq;
    b = p / (hkv * nq);
  }
  const int lane = threadIdx.x;
  const int g = h / group;
  const long long row = ((long long)b * nq + qi) * hq + h;              // row in [B][nq][hq]
  const float* pp = partials + row * nsplit * kPF;
  // independent loads: this lane's split (m, l), the first splits' o~ values, the query values
  const float msp = lane < nsplit ? pp[lane * kPF] : -INFINITY;
  const float lsp = lane < nsplit ? pp[lane * kPF + 1] : 0.0f;
  const float* col = pp + 2 + kPer * lane;
  float ov[kMergePreload][kPer];
#pragma unroll
  for (int sp = 0; sp < kMergePreload; ++sp) {
    if (sp < nsplit) {
      load_f<kPer>(col + sp * kPF, ov[sp]);
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) ov[sp][i] = 0.0f;
    }
  }
  HalfBits<kPer> qw;
  qw.load(q + row * kDim + kPer * lane);
  const int len = seq_lens[b];
  const bool bad = len < 0 || (len >> 7) > max_blocks;
  // slots holding a partial: all nsplit after a split grid; after a list schedule, none for a
  // sequence without full tiles, else those before the first slot whose m is +inf (written by
  // the worker that finished the row's last tile; none when the row fills every slot)
  int nuse = nsplit;
  if (list) {
    const unsigned long long ends = __ballot(lane < nsplit && msp == INFINITY);
    nuse = (bad || (len >> 7) == 0) ? 0 : (ends ? (int)__builtin_ctzll(ends) : nsplit);
  }
  // staging tokens this query token sees: positions up to len - nq + qi
  const int n_stage = bad ? 0 : max(0, (len & (kT - 1)) - (kCausal ? nq - 1 - qi : 0));
  const float scale2 = sm_scale * kLog2e;
  const __half* sk = staging_k + ((long long)b * hkv + g) * kT * kDim;
  const __half* sv = staging_v + ((long long)b * hkv + g) * kT * kDim;
  // this lane's staging key row (token lane) is loaded before the length is known when it
  // fits in registers (kDim <= 128): the row is always inside the staging tile, and used only
  // if the token is live
  constexpr int kPre = kDim <= 128 ? kDim / 8 : 1;
  uint4 krow[kPre];
  if constexpr (kDim <= 128) {
    const uint4* k4 = reinterpret_cast<const uint4*>(sk + lane * kDim);
#pragma unroll
    for (int i = 0; i < kPre; ++i) krow[i] = k4[i];
  }
  HalfBits<kPer> vpre0, vpre1;
  vpre0.load(sv + kPer * lane);
  vpre1.load(sv + kDim + kPer * lane);
#pragma unroll
  for (int i = 0; i < kPer; ++i) qs[kPer * lane + i] = qw.at(i);
  __syncthreads();
  // staging scores of tokens lane and lane + 64
  float s0 = -INFINITY, s1 = -INFINITY;
  if (lane < n_stage) {
    if constexpr (kDim <= 128) {
      float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
      for (int k = 0; k < kPre; ++k) {
        float kv[8];
        unpack_h8(krow[k], kv);
        const float4 qa = *reinterpret_cast<const float4*>(qs + 8 * k);
        const float4 qc = *reinterpret_cast<const float4*>(qs + 8 * k + 4);
        acc0 = fmaf(qa.x, kv[0], fmaf(qa.y, kv[1], fmaf(qa.z, kv[2], fmaf(qa.w, kv[3], acc0))));
        acc1 = fmaf(qc.x, kv[4], fmaf(qc.y, kv[5], fmaf(qc.z, kv[6], fmaf(qc.w, kv[7], acc1))));
      }
      s0 = (acc0 + acc1) * scale2;
    } else {
      s0 = staging_dot<kDim>(sk + lane * kDim, qs) * scale2;
    }
  }
  if (lane + 64 < n_stage) s1 = staging_dot<kDim>(sk + (lane + 64) * kDim, qs) * scale2;
  const float m_use = lane < nuse ? msp : -INFINITY;
  const float l_use = lane < nuse ? lsp : 0.0f;
  const bool invalid = bad || __any(m_use != m_use);
  const float mm = wave_max(fmaxf(m_use, fmaxf(s0, s1)));
  float ls = 0.0f, wsp = 0.0f, p0 = 0.0f, p1 = 0.0f;
  if (mm != -INFINITY) {
    wsp = lane < nuse ? exp2f(m_use - mm) : 0.0f;
    p0 = exp2f(s0 - mm);
    p1 = exp2f(s1 - mm);
    ls = fmaf(wsp, l_use, p0 + p1);
  }
  ls = wave_sum(ls);
  // merged rotated output o~ of this lane's channels
  float o[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) o[i] = 0.0f;
  if (mm != -INFINITY && !invalid) {
#pragma unroll
    for (int sp = 0; sp < kMergePreload; ++sp) {
      if (sp < nuse) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsp), sp));
#pragma unroll
        for (int i = 0; i < kPer; ++i) o[i] = fmaf(w, ov[sp][i], o[i]);
      }
    }
    // the remaining splits kMergePreload at a time, every load of a chunk issued before its
    // values are used
    for (int sp0 = kMergePreload; sp0 < nuse; sp0 += kMergePreload) {
      float v[kMergePreload][kPer];
#pragma unroll
      for (int k = 0; k < kMergePreload; ++k) {
        if (sp0 + k < nuse) {
          load_f<kPer>(col + (sp0 + k) * kPF, v[k]);
        } else {
#pragma unroll
          for (int i = 0; i < kPer; ++i) v[k][i] = 0.0f;
        }
      }
#pragma unroll
      for (int k = 0; k < kMergePreload; ++k) {
        if (sp0 + k < nuse) {
          const float w =
              __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsp), sp0 + k));
#pragma unroll
          for (int i = 0; i < kPer; ++i) o[i] = fmaf(w, v[k][i], o[i]);
        }
      }
    }
  }
  if constexpr (kRotated) {
    fwht_lanes<kPer>(o, lane);
    const uint32_t sb = lane_sign_bits_d<kPer>(signs, lane);     // optional sign flips
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      o[i] = __uint_as_float(__float_as_uint(o[i]) ^ (((sb >> i) & 1u) << 31));
  }
  // H / sqrt(kDim) or none
  constexpr float kBack = !kRotated ? 1.0f
                        : (kDim == 64 ? 0.125f : (kDim == 128 ? 0.08838834764831845f : 0.0625f));
  // raw staging output
  float r[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) r[i] = 0.0f;
  const __half* vcol = sv + kPer * lane;
  // kStageChunk staging rows per round of loads (rows past n_stage are loaded, always inside the
  // staging tile, but never used: they may hold anything)
  for (int t0 = 0; t0 < n_stage; t0 += kStageChunk) {
    HalfBits<kPer> w[kStageChunk];
#pragma unroll
    for (int i = 0; i < kStageChunk; ++i) {
      if (t0 + i == 0) w[i] = vpre0;
      else if (t0 + i == 1) w[i] = vpre1;
      else w[i].load(vcol + (t0 + i) * kDim);
    }
#pragma unroll
    for (int i = 0; i < kStageChunk; ++i) {
      const int t = t0 + i;
      if (t < n_stage) {
        const int src = __float_as_int(t < 64 ? p0 : p1);
        const float pt = __int_as_float(__builtin_amdgcn_readlane(src, t & 63));
#pragma unroll
        for (int e = 0; e < kPer; ++e) r[e] = fmaf(pt, w[i].at(e), r[e]);
      }
    }
  }
  float res[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    res[i] = 0.0f;
    if (invalid) res[i] = NAN;
    else if (ls > 0.0f) res[i] = fmaf(o[i], kBack, r[i]) / ls;
  }
  float* dst = out + row * kDim + kPer * lane;
  if constexpr (kPer == 1) {
    dst[0] = res[0];
  } else if constexpr (kPer == 2) {
    *reinterpret_cast<float2*>(dst) = make_float2(res[0], res[1]);
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(res[0], res[1], res[2], res[3]);
  }
}


// ------------------------------------------------------------------ dequantisation to memory
//
// Stage 4 of [GR] "The four-stage pipeline" written out instead of folded into attention:
// x_tj = sum_i c-hat_i (s-hat_t code_ti + z-hat_t) H_ij / sqrt(D), the record's tile back in
// the original channel space (for inspection, export and error measurement). grid: n_tiles *
// hkv * 2 workgroups (tile, head, K|V) of 4 waves; wave w rebuilds tokens w, w + 4, ..., lane l
// channels kPer l .. kPer l + kPer - 1 (kPer = D / 64), with the same butterfly as the query
// rotation.

template <int kVBits, int kDim>
__global__ void __launch_bounds__(256)
dequantize_tiles_kernel(const uint8_t* __restrict__ pool, long long num_blocks,
                        const int32_t* __restrict__ src_blocks, int n_tiles, int hkv,
                        float* __restrict__ k_out, float* __restrict__ v_out, SignWords signs) {
  constexpr int kPer = kDim / 64;
  const int id = blockIdx.x;
  const int is_v = id & 1, head = (id >> 1) % hkv, tile = (id >> 1) / hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (tile >= n_tiles) return;
  float* out = (is_v ? v_out : k_out) + ((long long)tile * kT * hkv + head) * kDim + kPer * lane;
  const long long row_stride = (long long)hkv * kDim;
  const long long blk = src_blocks[tile];
  if (blk < 0 || blk >= num_blocks) {
    for (int t = wave; t < kT; t += 4) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) out[t * row_stride + i] = NAN;
    }
    return;
  }
  using L = RecordLayout<kVBits, kDim>;
  const uint8_t* rec = pool + (blk * hkv + head) * (long long)L::kTileBytes;
  const uint8_t* meta = rec + (is_v ? L::kVMetaOff : L::kKMetaOff);
  float c[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    c[i] = __builtin_amdgcn_cvt_f32_fp8((int)meta[L::kC + kPer * lane + i], 0);
  const uint32_t sb = lane_sign_bits_d<kPer>(signs, lane);     // optional sign flips
  constexpr float kInvSqrt = kDim == 64 ? 0.125f : (kDim == 128 ? 0.08838834764831845f : 0.0625f);
  constexpr uint32_t kVMax = (1u << kVBits) - 1u;
  for (int t = wave; t < kT; t += 4) {
    const float sh = __builtin_amdgcn_cvt_f32_fp8((int)meta[L::kS + t], 0);
    const float zh = fp16_bits_to_float(*reinterpret_cast<const uint16_t*>(meta + L::kZ + 2 * t));
    float y[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int ch = kPer * lane + i;
      uint32_t code;
      if (!is_v) {
        const uint32_t byte = rec[L::kKCodes + (kDim / 2) * t + (ch >> 1)];
        code = (ch & 1) ? (byte >> 4) : (byte & 15u);
      } else {
        uint32_t off;
        int shift;
        value_code_pos<kVBits, kDim>(t, ch, off, shift);
        code = (rec[L::kVCodes + off] >> shift) & kVMax;
      }
      y[i] = c[i] * fmaf(sh, (float)code, zh);
    }
    fwht_lanes<kPer>(y, lane);
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      out[t * row_stride + i] =
          __uint_as_float(__float_as_uint(y[i] * kInvSqrt) ^ (((sb >> i) & 1u) << 31));
  }
}

// ------------------------------------------------------------------ fp16 cache (comparison path)
//
// The unquantised paged cache the packed cache is compared with. Record of one (block, KV
// head): 65,536 bytes. Keys at byte 0: token-major [t][ch] fp16. Values at byte 32,768:
// channel-major [ch][position] fp16, where position 32 kb + 8 s + e of each row holds token
// 32 kb + 16 (e / 4) + 4 s + e % 4: one 16-byte load then gives a lane exactly the eight tokens
// its score accumulator rows hold (as in the packed value section), so the output product
// needs no shuffles. Same decode structure as the packed tiles, with the query fp16 as given
// (exact, so no hi/lo split: columns g and 8 + g both carry head g and each keeps two of its
// four score rows) and the outputs accumulated in the MFMA accumulators (no per-tile scale).

constexpr long long kFp16Rec = 65536;
constexpr uint32_t kFp16VOff = 32768;
constexpr float kFp16W = 32.0f;               // probability operand prescale (lo parts normal)

__device__ __forceinline__ int fp16_v_token(int p) {
  return 32 * (p >> 5) + 16 * ((p & 7) >> 2) + 4 * ((p >> 3) & 3) + (p & 3);
}

// grid: n_tiles * Hkv workgroups of 256 threads; id = tile * Hkv + head
__global__ void __launch_bounds__(256)
fp16_write_tiles_kernel(const __half* __restrict__ k, const __half* __restrict__ v,
                        long long token_stride, int n_tiles, int hkv,
                        const int32_t* __restrict__ dst_blocks, uint8_t* __restrict__ pool,
                        long long num_blocks) {
  __shared__ uint16_t vt[kT][kD + 8];
  const int id = blockIdx.x;
  const int head = id % hkv, tile = id / hkv;
  const int tid = threadIdx.x;
  if (tile >= n_tiles) return;
  const long long blk = dst_blocks[tile];
  if (blk < 0 || blk >= num_blocks) return;
  uint8_t* rec = pool + (blk * hkv + head) * kFp16Rec;
  const __half* ks = k + (long long)tile * kT * token_stride + head * kD;
  const __half* vs = v + (long long)tile * kT * token_stride + head * kD;
  for (int r = tid; r < kT * 16; r += 256) {
    const int t = r >> 4, c = r & 15;
    *reinterpret_cast<uint4*>(rec + t * 256 + c * 16) =
        *reinterpret_cast<const uint4*>(ks + (long long)t * token_stride + 8 * c);
    *reinterpret_cast<uint4*>(&vt[t][8 * c]) =
        *reinterpret_cast<const uint4*>(vs + (long long)t * token_stride + 8 * c);
  }
  __syncthreads();
  for (int r = tid; r < kD * 16; r += 256) {
    const int ch = r >> 4, pc = r & 15;
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int p0 = 8 * pc + 2 * d;
      w[d] = (uint32_t)vt[fp16_v_token(p0)][ch] | ((uint32_t)vt[fp16_v_token(p0 + 1)][ch] << 16);
    }
    *reinterpret_cast<uint4*>(rec + kFp16VOff + ch * 256 + pc * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

struct alignas(16) Fp16Smem {
  float alpha[kWaves][16];
  float comb_m[kWaves][kHeadGroup], comb_l[kWaves][kHeadGroup];
  float comb_o[kWaves][kHeadGroup][kD];
};

// Chunk i of a tile into buf: i < 8 -> keys of token block i (token 16 i + lane % 16, channels
// 32 c + 8 (lane / 16) .. + 7, c = 0..3); i >= 8 -> values of channel block i - 8 (channel
// 16 (i - 8) + lane % 16, positions 32 kb + 8 (lane / 16) .. + 7, kb = 0..3).
__device__ __forceinline__ void fp16_chunk(const uint8_t* __restrict__ rec, int i, uint32_t off,
                                           uint4 (&buf)[4]) {
  const uint8_t* base = rec + (i < 8 ? 0u : kFp16VOff) + 4096u * (uint32_t)(i & 7);
#pragma unroll
  for (int c = 0; c < 4; ++c) buf[c] = *reinterpret_cast<const uint4*>(base + off + 64u * c);
}

__global__ void __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_fp16_tiles_kernel(const __half* __restrict__ q, int hq, int hkv,
                         const uint8_t* __restrict__ pool, long long num_blocks,
                         const int32_t* __restrict__ block_table, int max_blocks,
                         const int32_t* __restrict__ seq_lens, float sm_scale,
                         float* __restrict__ partials) {
  __shared__ Fp16Smem sm;
  const int split = blockIdx.x, nsplit = gridDim.x;
  const int ngroups = (hq / hkv + kHeadGroup - 1) / kHeadGroup;
  const int g = blockIdx.y / ngroups, hg = blockIdx.y % ngroups;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int group = hq / hkv;
  const int h0 = g * group + hg * kHeadGroup;
  const int nh = min(kHeadGroup, group - hg * kHeadGroup);
  const int len = seq_lens[b];
  bool bad = len < 0 || (len >> 7) > max_blocks;
  const int n_full = bad ? 0 : (len >> 7);
  const int chunk = (n_full + nsplit - 1) / nsplit;
  const int i0 = min(split * chunk, n_full), i1 = min(i0 + chunk, n_full);
  // this wave's tiles: i0 + wave + 4 j, j < nw; block ids are scalar loads, one tile ahead
  const int ntile = i1 - i0;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int nw = ntile > wave_u ? (ntile - wave_u + kWaves - 1) / kWaves : 0;
  const int32_t* bt_row = block_table + (long long)b * max_blocks + i0 + wave_u;
  int id_next = nw > 1 ? bt_row[kWaves] : 0;        // tile 1
  const int n = lane & 15, s = lane >> 4;
  const int gq = n & 7;
  const bool colv = gq < nh;
  const bool colhi = n < 8;
  const uint32_t off = (uint32_t)(lane & 15) * 256u + 16u * (uint32_t)s;
  const uint32_t vmask_col = colv ? 0xFFFFFFFFu : 0u;
  // query operand: columns g and 8 + g carry head g as given, channel 32 c + 8 s + e
  half8 qb[4];
  {
    const __half* qh = q + ((long long)b * hq + h0 + (colv ? gq : 0)) * kD;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 w = *reinterpret_cast<const uint4*>(qh + 32 * c + 8 * s);
      w.x &= vmask_col; w.y &= vmask_col; w.z &= vmask_col; w.w &= vmask_col;
      qb[c] = __builtin_bit_cast(half8, w);
    }
  }
  const float scale2 = sm_scale * kLog2e;
  const int ih = colhi ? 0 : 2;
  float m_run = -INFINITY, l_run = 0.0f;
  float4v oacc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) oacc[nb] = (float4v){0.f, 0.f, 0.f, 0.f};

  // ring of four chunk buffers; chunk i of every tile lives in buf[i % 4] (16 chunks a tile),
  // loaded three chunks ahead, across tile boundaries
  uint4 buf[4][4];
  const uint8_t* rec = nullptr;
  if (nw > 0) {
    const long long blk = bt_row[0];
    if (blk < 0 || blk >= num_blocks) bad = true;
    else rec = pool + (blk * hkv + g) * kFp16Rec;
  }
  if (rec != nullptr) {
    fp16_chunk(rec, 0, off, buf[0]);
    fp16_chunk(rec, 1, off, buf[1]);
    fp16_chunk(rec, 2, off, buf[2]);
  }
  for (int j = 0; j < nw && !bad; ++j) {
    const uint8_t* nrec = nullptr;
    if (j + 1 < nw) {
      const long long blk = id_next;
      if (j + 2 < nw) id_next = bt_row[kWaves * (j + 2)];
      if (blk >= 0 && blk < num_blocks) nrec = pool + (blk * hkv + g) * kFp16Rec;
      else bad = true;
    }
    float4v sc[8];
    half8 wa[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < 8) {
        float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, buf[i & 3][c]),
                                                       qb[c], acc, 0, 0, 0);
        sc[i] = acc;
      } else {
        const int nb = i - 8;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[kb],
                                                            __builtin_bit_cast(half8, buf[i & 3][kb]),
                                                            oacc[nb], 0, 0, 0);
      }
      {
        const int ni = i + 3;
        if (ni < 16) fp16_chunk(rec, ni, off, buf[ni & 3]);
        else if (nrec != nullptr) fp16_chunk(nrec, ni - 16, off, buf[ni & 3]);
      }
      if (i == 7) {
        // scores of this lane's two rows of each block (both column lanes hold all four)
        float v[8][2];
        float tmax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          v[mb][0] = (colhi ? sc[mb][0] : sc[mb][2]) * scale2;
          v[mb][1] = (colhi ? sc[mb][1] : sc[mb][3]) * scale2;
          tmax = fmaxf(tmax, fmaxf(v[mb][0], v[mb][1]));
        }
        tmax = fmaxf(tmax, dpp_ror8(tmax));
        tmax = max_xor32(max_xor16(tmax));
        const bool upd = tmax > m_run + kLazy;
        const float mnew = upd ? tmax : m_run;
        const float alpha = upd ? __builtin_amdgcn_exp2f(m_run - mnew) : 1.0f;
        const bool rescale = __any(upd) && j > 0;
        float psum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          uint32_t u[4];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int mb = 2 * kb + h2;
            const float p0 = __builtin_amdgcn_exp2f(v[mb][0] - mnew);
            const float p1 = __builtin_amdgcn_exp2f(v[mb][1] - mnew);
            psum += p0 + p1;
            const float w0 = p0 * kFp16W, w1 = p1 * kFp16W;
            const uint32_t hh = pack_h2(w0, w1);
            const uint32_t ll = lo_of(hh, w0, w1);
            const uint32_t rcv = dpp_ror8_u(colhi ? ll : hh);
            u[2 * h2] = (colhi ? hh : rcv) & vmask_col;
            u[2 * h2 + 1] = (colhi ? rcv : ll) & vmask_col;
          }
          wa[kb] = as_h8(u[0], u[1], u[2], u[3]);
        }
        psum += dpp_ror8(psum);
        psum = add_xor32(add_xor16(psum));
        l_run = fmaf(alpha, l_run, psum);
        m_run = mnew;
        if (s == 0) sm.alpha[wave][n] = alpha;
        if (rescale) {
          const float4 a4 = *reinterpret_cast<const float4*>(&sm.alpha[wave][(4 * s) & 7]);
          const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) oacc[nb][r] *= ar[r];
          }
        }
      }
    }
    rec = nrec;
  }

  // ---- combine the waves' states (outputs carry the factor kFp16W)
  __syncthreads();
  if (s == 0 && colhi) {
    sm.comb_m[wave][n] = m_run;
    sm.comb_l[wave][n] = l_run;
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float both = add_xor32(oacc[nb][r]);
      if (s < 2) sm.comb_o[wave][4 * s + r][16 * nb + n] = both * (1.0f / kFp16W);
    }
  }
  __syncthreads();
  const int wbad = __syncthreads_or(bad ? 1 : 0);
  for (int idx = tid; idx < nh * kD; idx += kTThreads) {
    const int gg = idx >> 7, jj = idx & (kD - 1);
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm.comb_m[w][gg]);
    float ll = 0.0f, oo = 0.0f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(sm.comb_m[w][gg] - mm);
        ll = fmaf(f, sm.comb_l[w][gg], ll);
        oo = fmaf(f, sm.comb_o[w][gg][jj], oo);
      }
    }
    float* pp = partials + (((long long)b * hq + h0 + gg) * nsplit + split) * kPartialFloats;
    if (jj == 0) {
      pp[0] = wbad ? NAN : mm;
      pp[1] = wbad ? NAN : ll;
    }
    pp[2 + jj] = oo;
  }
}

}  // namespace

namespace {

SignWords sign_words(const uint32_t* signs) {
  SignWords s;
  s.lo = make_uint4(signs[0], signs[1], signs[2], signs[3]);
  s.hi = make_uint4(signs[4], signs[5], signs[6], signs[7]);
  return s;
}

template <int kDim>
void launch_dequantize_t(const uint8_t* pool, long long num_blocks, const int32_t* src_blocks,
                         int n_tiles, int hkv, float* k_out, float* v_out, SignWords sg,
                         int v_bits, hipStream_t stream) {
  const long long groups = 2LL * hkv * n_tiles;
  auto kern = v_bits == 4 ? dequantize_tiles_kernel<4, kDim> : dequantize_tiles_kernel<2, kDim>;
  hipLaunchKernelGGL(kern, dim3((unsigned)groups), dim3(256), 0, stream, pool, num_blocks,
                     src_blocks, n_tiles, hkv, k_out, v_out, sg);
}

}  // namespace

hipError_t launch_dequantize_tiles(const uint8_t* pool, long long num_blocks,
                                   const int32_t* src_blocks, int n_tiles, int hkv, float* k_out,
                                   float* v_out, const uint32_t* signs, int v_bits, int head_dim,
                                   hipStream_t stream) {
  const SignWords sg = sign_words(signs);
  if (head_dim == 64)
    launch_dequantize_t<64>(pool, num_blocks, src_blocks, n_tiles, hkv, k_out, v_out, sg, v_bits, stream);
  else if (head_dim == 256)
    launch_dequantize_t<256>(pool, num_blocks, src_blocks, n_tiles, hkv, k_out, v_out, sg, v_bits, stream);
  else
    launch_dequantize_t<128>(pool, num_blocks, src_blocks, n_tiles, hkv, k_out, v_out, sg, v_bits, stream);
  return hipGetLastError();
}

// Compute units of the current device, read once per device and cached. A host without a
// usable device (argument checks only; nothing is launched there) plans for 256, the MI355X count.
int device_compute_units() {
  constexpr int kDefaultCUs = 256, kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();                    // leave no error behind for a later launch
    return kDefaultCUs;
  }
  const int cached = cache[dev].load(std::memory_order_relaxed);
  if (cached > 0) return cached;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = kDefaultCUs;
  }
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// The paired-tile kernel serves at most four virtual heads per KV head with 2-bit values at
// head dimension 128, and only when the table holds enough tiles for about four one-wave chunks per SIMD slot: with fewer
// tiles than that, one tile per wave of four-wave workgroups fills the device better.
bool pairs_mode(int virtual_heads, int v_bits, int head_dim, int batch, int hkv,
                int max_blocks) {
  const long long tiles = (long long)batch * hkv * max_blocks;
  return virtual_heads <= 4 && v_bits == 2 && head_dim == 128 &&
         tiles >= kPairMinTilesPerCU * device_compute_units() && tiles < (1LL << 31);
}

// Smallest share (in tile pairs) of the paired-tile schedule for a table of max_blocks
// entries: a unit of m <= ceil(max_blocks / 2) pairs at positions [T, T + m) meets waves
// floor(T / share) .. floor((T + m - 1) / share), at most floor((m - 1) / share) + 2 <=
// kMaxSplits partial slots.
int pairs_min_share(int max_blocks) {
  return ((max_blocks + 1) / 2 - 1) / (kMaxSplits - 2) + 1;
}

// Workgroups of `kernel` (block threads) the current device holds at once: its occupancy per
// compute unit (read once per device and kernel, and cached; at most max_per_cu) times the
// compute units. A host without a usable device plans for `fallback` per compute unit.
int resident_workgroups(const void* kernel, int threads, int fallback, int max_per_cu) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0, per_cu = fallback;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
  } else {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find({dev, kernel});
    if (it != cache.end()) {
      per_cu = it->second;
    } else {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess ||
          n <= 0) {
        (void)hipGetLastError();
        n = fallback;
      }
      cache[{dev, kernel}] = n;
      per_cu = n;
    }
  }
  return (per_cu < max_per_cu ? per_cu : max_per_cu) * device_compute_units();
}

// Smallest share (in tiles, at least one per wave) of the tile kernel's list schedule: a unit
// of n <= max_blocks tiles spans at most floor((max_blocks - 1) / share) + 2 <= kMaxSplits
// partial slots.
int tiles_min_share(int max_blocks) {
  const int m = (max_blocks - 1) / (kMaxSplits - 2) + 1;
  return m > kWaves ? m : kWaves;
}

// Which kernel and schedule a packed decode of these sizes runs: the paired-tile kernel (list
// schedule over tile pairs); at head dimension 128 with more than 8 virtual heads per KV head
// the 16-head kernel (list schedule over tiles for at most 16 on a large table, else a grid of
// splits x head groups of 16); else the tile kernel with one head group on a large table (list
// schedule over tiles) or over a grid of splits (several head groups of 8, or a table of fewer
// than kPairMinTilesPerCU entries per compute unit, where the list schedule's longer start-up
// is not repaid).
DecodeKind decode_kind(int batch, int hkv, int max_blocks, int virtual_heads, int v_bits,
                       int head_dim) {
  if (pairs_mode(virtual_heads, v_bits, head_dim, batch, hkv, max_blocks))
    return DecodeKind::kPairList;
  const long long tiles = (long long)batch * hkv * max_blocks;
  const bool large = tiles >= kPairMinTilesPerCU * device_compute_units() && tiles < (1LL << 31);
  if (head_dim == 128 && virtual_heads > kHeadGroup && kWideHeads) {
    // the list runs over (sequence, KV head, head group of 16) units
    const long long groups = (virtual_heads + kWideGroup - 1) / kWideGroup;
    return large && tiles * groups < (1LL << 31) ? DecodeKind::kWideList : DecodeKind::kWideGrid;
  }
  // the list runs over (sequence, KV head, head group of 8) units
  const long long groups = (virtual_heads + kHeadGroup - 1) / kHeadGroup;
  if (large && tiles * groups < (1LL << 31)) return DecodeKind::kTileList;
  return DecodeKind::kTileGrid;
}

int decode_slots(int batch, int hkv, int max_blocks, int virtual_heads, int v_bits,
                 int head_dim) {
  switch (decode_kind(batch, hkv, max_blocks, virtual_heads, v_bits, head_dim)) {
    case DecodeKind::kPairList:
      return ((max_blocks + 1) / 2 - 1) / pairs_min_share(max_blocks) + 2;
    case DecodeKind::kTileList:
    case DecodeKind::kWideList:
      return (max_blocks - 1) / tiles_min_share(max_blocks) + 2;
    default:
      return decode_splits(batch, hkv, max_blocks);
  }
}

int decode_splits(int batch, int hkv, int max_blocks) {
  const long long pairs = (long long)batch * hkv > 0 ? (long long)batch * hkv : 1;
  // two workgroups per compute unit (2 waves per SIMD)
  const long long target = 2LL * device_compute_units();
  long long s = (target + pairs - 1) / pairs;
  // at least two tiles per wave where the table allows it, so a wave's next tile is already
  // loading while it works on the current one; one tile per wave when two per wave would
  // leave the grid short of two workgroups per compute unit
  const long long per_wave = (max_blocks + kWaves - 1) / kWaves;
  const long long cap2 = per_wave / 2 > 0 ? per_wave / 2 : 1;
  const long long cap1 = per_wave > 0 ? per_wave : 1;
  s = pairs * (s < cap2 ? s : cap2) >= target ? (s < cap2 ? s : cap2) : (s < cap1 ? s : cap1);
  // and at most 32 full tiles per split for the longest table the batch may hold (the last
  // entry covers the staging tile): in a ragged batch the longest sequences would otherwise
  // set the kernel's time while the short ones' workgroups sit finished
  const long long need = (max_blocks - 1 + 31) / 32;
  if (s < need) s = need;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

namespace {

template <int kDim>
hipError_t launch_decode_t(const __half* q, int hq, int hkv, int nq, const uint8_t* pool,
                           long long num_blocks, const int32_t* block_table, int max_blocks,
                           const int32_t* seq_lens, const __half* staging_k,
                           const __half* staging_v, float sm_scale, float* out, float* partials,
                           int slots, int batch, SignWords sg, int v_bits, hipStream_t stream) {
  const int vh = hq / hkv * nq;
  const DecodeKind kind = decode_kind(batch, hkv, max_blocks, vh, v_bits, kDim);
  int workers = 0, min_share = 0;
  if (kDim == 128 && (kind == DecodeKind::kWideList || kind == DecodeKind::kWideGrid)) {
    if (kind == DecodeKind::kWideList) {
      auto kern = nq == 1 ? (v_bits == 4 ? decode_wide_kernel<false, 4, true>
                                         : decode_wide_kernel<false, 2, true>)
                          : (v_bits == 4 ? decode_wide_kernel<true, 4, true>
                                         : decode_wide_kernel<true, 2, true>);
      workers = resident_workgroups(reinterpret_cast<const void*>(kern), kTThreads, 2,
                                    kTileListMaxPerCU);
      min_share = tiles_min_share(max_blocks);
      hipLaunchKernelGGL(kern, dim3(workers), dim3(kTThreads), 0, stream, q, hq, hkv, nq, pool,
                         num_blocks, block_table, max_blocks, seq_lens, batch, sm_scale,
                         partials, slots, sg, min_share);
    } else {
      auto kern = nq == 1 ? (v_bits == 4 ? decode_wide_kernel<false, 4, false>
                                         : decode_wide_kernel<false, 2, false>)
                          : (v_bits == 4 ? decode_wide_kernel<true, 4, false>
                                         : decode_wide_kernel<true, 2, false>);
      const int ngroups = (vh + kWideGroup - 1) / kWideGroup;
      hipLaunchKernelGGL(kern, dim3(slots, hkv * ngroups, batch), dim3(kTThreads), 0, stream, q,
                         hq, hkv, nq, pool, num_blocks, block_table, max_blocks, seq_lens, batch,
                         sm_scale, partials, slots, sg, 0);
    }
  } else if (kDim == 128 && kind == DecodeKind::kPairList) {
    auto kern = nq == 1 ? decode_pairs_kernel<false, 2> : decode_pairs_kernel<true, 2>;
    workers = kPairRounds * resident_workgroups(reinterpret_cast<const void*>(kern), 64, 8, 64);
    min_share = pairs_min_share(max_blocks);
    hipLaunchKernelGGL(kern, dim3(workers), dim3(64), 0, stream, q, hq, hkv, nq, pool,
                       num_blocks, block_table, max_blocks, seq_lens, batch, sm_scale, partials,
                       slots, sg, min_share);
  } else {
    if (kind == DecodeKind::kTileList) {
      auto kern = nq == 1 ? (v_bits == 4 ? decode_tiles_kernel<false, 4, kDim, true>
                                         : decode_tiles_kernel<false, 2, kDim, true>)
                          : (v_bits == 4 ? decode_tiles_kernel<true, 4, kDim, true>
                                         : decode_tiles_kernel<true, 2, kDim, true>);
      workers = resident_workgroups(reinterpret_cast<const void*>(kern), kTThreads,
                                    kDim == 256 ? 1 : 2, kTileListMaxPerCU);
      min_share = tiles_min_share(max_blocks);
      hipLaunchKernelGGL(kern, dim3(workers), dim3(kTThreads), 0, stream, q, hq, hkv, nq, pool,
                         num_blocks, block_table, max_blocks, seq_lens, batch, sm_scale,
                         partials, slots, sg, min_share);
    } else {
      auto kern = nq == 1 ? (v_bits == 4 ? decode_tiles_kernel<false, 4, kDim, false>
                                         : decode_tiles_kernel<false, 2, kDim, false>)
                          : (v_bits == 4 ? decode_tiles_kernel<true, 4, kDim, false>
                                         : decode_tiles_kernel<true, 2, kDim, false>);
      const int ngroups = (vh + kHeadGroup - 1) / kHeadGroup;
      hipLaunchKernelGGL(kern, dim3(slots, hkv * ngroups, batch), dim3(kTThreads), 0, stream, q,
                         hq, hkv, nq, pool, num_blocks, block_table, max_blocks, seq_lens, batch,
                         sm_scale, partials, slots, sg, 0);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto merge = nq == 1 ? decode_merge_kernel<true, false, kDim> : decode_merge_kernel<true, true, kDim>;
  hipLaunchKernelGGL(merge, dim3(hq * nq, batch), dim3(kMThreads), 0, stream, q, hq, hkv, nq,
                     max_blocks, seq_lens, staging_k, staging_v, sm_scale, partials, slots, out,
                     sg, (kind == DecodeKind::kPairList || kind == DecodeKind::kTileList ||
                          kind == DecodeKind::kWideList) ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const __half* q, int hq, int hkv, int nq, const uint8_t* pool,
                         long long num_blocks, const int32_t* block_table, int max_blocks,
                         const int32_t* seq_lens, const __half* staging_k,
                         const __half* staging_v, float sm_scale, float* out, float* partials,
                         int slots, int batch, const uint32_t* signs, int v_bits, int head_dim,
                         hipStream_t stream) {
  const SignWords sg = sign_words(signs);
#define KVARN_D(DIM)                                                                         \
  launch_decode_t<DIM>(q, hq, hkv, nq, pool, num_blocks, block_table, max_blocks, seq_lens,   \
                       staging_k, staging_v, sm_scale, out, partials, slots, batch, sg,        \
                       v_bits, stream)
  if (head_dim == 64) return KVARN_D(64);
  if (head_dim == 256) return KVARN_D(256);
  return KVARN_D(128);
#undef KVARN_D
}

hipError_t launch_fp16_write_tiles(const __half* k, const __half* v, long long token_stride,
                                   int n_tiles, int hkv, const int32_t* dst_blocks,
                                   uint8_t* pool, long long num_blocks, hipStream_t stream) {
  const long long groups = (long long)hkv * n_tiles;
  hipLaunchKernelGGL(fp16_write_tiles_kernel, dim3((unsigned)groups), dim3(256), 0, stream, k, v,
                     token_stride, n_tiles, hkv, dst_blocks, pool, num_blocks);
  return hipGetLastError();
}

hipError_t launch_decode_fp16(const __half* q, int hq, int hkv, const uint8_t* pool,
                              long long num_blocks, const int32_t* block_table, int max_blocks,
                              const int32_t* seq_lens, const __half* staging_k,
                              const __half* staging_v, float sm_scale, float* out,
                              float* partials, int splits, int batch, hipStream_t stream) {
  const int ngroups = (hq / hkv + kHeadGroup - 1) / kHeadGroup;
  hipLaunchKernelGGL(decode_fp16_tiles_kernel, dim3(splits, hkv * ngroups, batch),
                     dim3(kTThreads), 0, stream, q, hq, hkv, pool, num_blocks, block_table,
                     max_blocks, seq_lens, sm_scale, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  SignWords none;
  none.lo = make_uint4(0, 0, 0, 0);
  none.hi = none.lo;
  hipLaunchKernelGGL((decode_merge_kernel<false, false, kD>), dim3(hq, batch), dim3(kMThreads), 0,
                     stream, q, hq, hkv, 1, max_blocks, seq_lens, staging_k, staging_v, sm_scale,
                     partials, splits, out, none, 0);
  return hipGetLastError();
}

}  // namespace kvarn
