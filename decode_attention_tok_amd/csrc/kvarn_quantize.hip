// KVarN tile quantiser (write path) for gfx950.
//
// One workgroup of 4 D threads quantises one 128-token x D-channel tile of one KV head (D, the
// head dimension, is 128 in the preset; 64 and 256 are built the same way, described after the
// D = 128 layout below),
// keys or values, through the write-path stages of [GR] "The four-stage pipeline" (groundy.com,
// "Huawei's KVarN puts KV-cache quantization inside vLLM's backend"):
//   1. Hadamard rotation along channels: a 128-point fast Walsh-Hadamard transform.
//   2. Sinkhorn-like normalisation: a fixed number of rounds, each setting every column's
//      scale to the standard deviation over tokens of the row-scaled tile, then every row's
//      scale to the standard deviation over channels of the column-scaled tile (centred,
//      population). The log-space scales are kept as their exponentials' reciprocals; each
//      standard deviation is floored at 2^-16 x (largest |rotated value|) x (largest
//      multiplier applied). The column scales are divided by their geometric mean (the
//      log-space gauge) and rounded to FP8 E4M3 (nearest, ties to even).
//   3. Asymmetric round-to-nearest per token on y = rotated / c-hat: zero-point = FP16 round
//      down of the token minimum, scale = FP8 round up of (max - zero-point) / (2^bits - 1),
//      code = clamp(rne((y - zero-point) / scale), 0, 2^bits - 1).
//
// Work layout. Layout A gives thread (t, q0, q1) the 32 channels c = e + 8 q0 + 16 m + 64 q1
// (e = 0..7, m = 0..3) of token t, held as x[8 m + e]: channel bits 0-2 and 4-5 live in
// registers and bits 3 and 6 across four lanes. At D = 128, t = 16 wave + lane % 16 and
// (q0, q1) = lane bits 4, 5: the transform runs on the matrix cores (rotate_mfma below), whose
// 16 x 16 output blocks put one token per lane column and four channel rows per lane group.
// Layout A does the row statistics and the codes; a thread's eight values of one m are exactly
// one word of key nibbles, its four values of one e are one byte of 2-bit value codes or one
// 16-bit half-word of 4-bit value codes.
// Layout B gives lane (j, th) = (16 wave + lane % 16, lane / 16) the 32 tokens th, th + 4, ...,
// th + 124 of channel j: the column statistics. The rotated tile goes through LDS once (layout
// A writes it, layout B reads its 32 values into registers), so both layouts stay in registers
// for the whole normalisation; a column's sums merge over its four lanes with permlane swaps,
// and a round needs two barriers (after the columns, after the rows: the multipliers one layout
// computes for the other pass through LDS). At D = 128 the 16-byte
// chunks of each LDS row are XOR-swizzled by (row / 2) % 4 and the staged key and 2-bit value
// codes use 17-word rows, so the 16 tokens of a wave, which write the same channels, do not
// share banks.
//
// The 1/sqrt(D) scale of the transform is folded into the rounding stage's per-channel factor
// (the normalisation is scale-free up to the gauge, and the floor is relative to the tile's
// largest value).
//
// Variances use shifted one-pass sums. A column's sums are shifted by its token 0 in all four of
// its lanes, so they merge by plain addition; so are a row's at D = 128 (by its channel 0). At
// D = 64 and 256 a row's threads shift by their own first value and merge with Chan et al.'s
// pairwise update.
//
// Other head dimensions. A token has D / 32 threads (t = tid / (D / 32), lane bits
// 0 .. log2(D / 32) - 1 = q0, q1, q2): channel c = e + 8 q0 + 16 m + 64 q1 + 128 q2 with q2 at
// D = 256 only, no q1 at D = 64. The transform is a butterfly network: five stages in registers,
// then the cross-lane stages as DPP-sourced fused multiply-adds x + s * partner with s = -1 on
// the lane holding the upper index, which leaves that lane's values negated (one factor
// (-1)^(q0 + q1) per thread, applied once by the row statistics and the rounding stage; column
// variances do not see it); the stage on channel bit 7 (D = 256) crosses lanes through
// ds_swizzle and computes the upper lane's difference exactly (partner - own). Layout B keeps 16
// channels per wave (D / 16 waves). A row's statistics merge over D / 32 threads; the gauge and
// the per-channel rounding factor use 1 / D and 1 / sqrt(D). Key codes are staged token-major
// as at D = 128; a thread's value codes form whole bytes (2-bit) or half-words (4-bit) of the
// section, written into an LDS copy of it at the positions of value_code_pos() and then stored.

#include "kvarn_device.hpp"
#include "kvarn_kernels.hpp"

namespace kvarn {

namespace {

// Sizes of the quantiser for head dimension kDim.
template <int kDim>
struct QGeom {
  static constexpr int kThreads = 4 * kDim;                 // 4 kDim / 128 x 128 tokens
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kTPT = kDim / 32;                    // threads per token (layout A)
  // LDS row stride of the rotated tile: the row plus the cpos padding, rounded so that the
  // four token rows th = 0..3 read by one layout-B instruction start 16 banks apart — except at
  // D = 64, where the unrounded 68 keeps the workgroup under 40 KB of LDS, so four fit on a
  // compute unit instead of three (the layout-B reads happen once per tile, so their bank
  // conflicts cost less than the lost occupancy)
  static constexpr int kXs = kDim == 64 ? 68 : (kDim == 128 ? 144 : 272);
  static constexpr int kCp = kDim + 4 * (kDim / 64);        // padded per-channel array length
  static constexpr float kInvSqrt = kDim == 64 ? 0.125f
                                  : (kDim == 128 ? 0.08838834764831845f : 0.0625f);
};

// Position of channel c in an LDS row or per-channel array: each 64-channel block sits 4 floats
// further on, so the quad lanes holding channel bit 6 = 0 and 1 use different banks.
__device__ __forceinline__ int cpos(int c) { return c + ((c >> 6) << 2); }

template <int kDim>
struct QuantSmem {
  using G = QGeom<kDim>;
  alignas(16) float xt[kT][G::kXs];   // rotated tile, layout A -> B; reused to stage the codes
  float u[4][kT / 4];    // per-token multipliers 1 / r_t, token t at [t % 4][t / 4]
  float cs[kDim];        // per-channel standard deviations (unrounded c before the gauge)
  float vinv[G::kCp];    // per-channel multipliers 1 / c_j (at cpos)
  float rq[G::kCp];      // per-channel rounding factor (1 / sqrt(D)) / c-hat_j (at cpos)
  uint32_t meta[96];     // staged FP8 s-hat (32 words) and FP16 z-hat (64 words)
  uint32_t chat[kDim / 4];   // staged FP8 c-hat
  float red[3 * G::kWaves];  // per-wave maxima: |rotated|, column multipliers, row multipliers
  alignas(16) uint32_t sgn[kDim / 2];   // sign-flip masks of channel pairs (2 i, 2 i + 1)
};

constexpr int kDppXor1 = 0xB1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2, 3, 0, 1]

template <int kCtrl>
__device__ __forceinline__ float quad_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, false));
}

// a[i] += s * (a[i] of lane ^ 1), i = 0..7, each one v_fmac_f32 with a DPP-read first source.
// The leading s_nop gives the two wait states a DPP read of a VGPR needs after a VALU write.
__device__ __forceinline__ void fmac_xor1(float* a, float s) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
        "+v"(a[7])
      : "v"(s));
}

// The same across lane ^ 2.
__device__ __forceinline__ void fmac_xor2(float* a, float s) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
      : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
        "+v"(a[7])
      : "v"(s));
}

// Maximum of two non-negative finite floats as an integer maximum of their bit patterns (the
// order is the same): one v_max_u32, where fmaxf would first quiet possible signalling NaNs
// coming out of a lane exchange.
__device__ __forceinline__ float max_nn(float a, float b) {
  return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
}

// Maximum over the 16 lanes of each DPP row (quad pairs, then row rotations by 4 and 8) of a
// non-negative value: integer maxima with the partner read through DPP in the same
// instruction (s_nop 1: the two wait states a DPP read needs after a VALU write).
__device__ __forceinline__ float row16_max(float x) {
  uint32_t v = __float_as_uint(x);
  asm volatile(
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_ror:4 row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %0, %0, %0 row_ror:8 row_mask:0xf bank_mask:0xf"
      : "+v"(v));
  return __uint_as_float(v);
}

// (a of the partner lane) + b and (a of the partner lane) - b for the quad partner selected by
// kCtrl (0xB1: lane ^ 1, 0x4E: lane ^ 2), each one DPP-sourced VALU instruction.
template <int kCtrl>
__device__ __forceinline__ float dpp_add(float a, float b) {
  float r;
  if constexpr (kCtrl == 0xB1)
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %1, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
                 : "=v"(r) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_add_f32_dpp %0, %1, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
                 : "=v"(r) : "v"(a), "v"(b));
  return r;
}
template <int kCtrl>
__device__ __forceinline__ float dpp_sub(float a, float b) {
  float r;
  if constexpr (kCtrl == 0xB1)
    asm volatile("s_nop 1\n\tv_sub_f32_dpp %0, %1, %2 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
                 : "=v"(r) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_sub_f32_dpp %0, %1, %2 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
                 : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Maximum over lane bits 4 and 5 of a non-negative value (permlane swaps).
__device__ __forceinline__ float max_xor48_nn(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nn(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Chan's merge of two equal-count partials (shifted mean m, centred sum of squares q) held by
// lanes l and l ^ kBits (16 or 32): a permlane swap of a value with itself gives the lower and
// the upper lane's value on both lanes, so both get the same bits. nab = n_a n_b / (n_a + n_b).
template <int kBits>
__device__ __forceinline__ void merge_pair(float& m, float& q, float nab) {
  const auto mm = kBits == 16
      ? __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false)
      : __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  const auto qq = kBits == 16
      ? __builtin_amdgcn_permlane16_swap(__float_as_uint(q), __float_as_uint(q), false, false)
      : __builtin_amdgcn_permlane32_swap(__float_as_uint(q), __float_as_uint(q), false, false);
  const float m0 = __uint_as_float(mm[0]), m1 = __uint_as_float(mm[1]);
  const float d = m0 - m1;
  q = fmaf(nab * d, d, __uint_as_float(qq[0]) + __uint_as_float(qq[1]));
  m = 0.5f * (m0 + m1);
}

// Code = rne(clamp(v, 0, qmax)) written into byte `sel` of `acc`: the conversion rounds to
// nearest even and clamps below at 0. The upper clamp (kClamp) is needed only when the
// token's scale saturated at the FP8 maximum: otherwise s-hat >= (max - z-hat) / qmax, so
// v <= qmax up to a few fp32 ulps and rounds to at most qmax.
template <bool kClamp>
__device__ __forceinline__ uint32_t put_code(float v, float qmax, uint32_t sel, uint32_t acc) {
  return __builtin_amdgcn_cvt_pk_u8_f32(kClamp ? fminf(v, qmax) : v, sel, acc);
}

// This thread's codes (token t, its 32 channels) into the LDS staging area (see the callers).
// q2 is used at kDim = 256 only, q1 at kDim >= 128 only.
template <bool kClamp, int kVBits, int kDim>
__device__ __forceinline__ void stage_codes(const float* x, float ca, float cb, float qmax,
                                            int is_v, int t, int q0, int q1, int q2,
                                            uint32_t* stage) {
  if (!is_v) {
    // key codes: token-major nibbles; group m of this thread is word q0 + 2 m + 8 q1 + 16 q2
    // of the token's kDim / 8 words (channel 8 k + e at nibble e of word k)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        lo = put_code<kClamp>(fmaf(x[8 * m + e], ca, cb), qmax, e >> 1, lo);
        hi = put_code<kClamp>(fmaf(x[8 * m + e + 1], ca, cb), qmax, e >> 1, hi);
      }
      // at kDim = 128 token rows are 17 words apart, so the 16 tokens of a wave (lanes 0..15)
      // writing the same word fall in 16 different banks
      stage[t * (kDim == 128 ? 17 : kDim / 8) + q0 + 2 * m + 8 * q1 + 16 * q2] = lo | (hi << 4);
    }
  } else if constexpr (kDim != 128) {
    // value codes of the other head dimensions. The four codes of channels
    // 16 (m + 4 q1 + 8 q2) + n, m = 0..3 (this thread's x[8 m + e], n = 8 q0 + e) share one byte
    // of the section (2-bit codes, at bits 2 m) or one half-word (4-bit codes, at bits 4 m),
    // byte-aligned at the position of the m = 0 channel: each is written whole into an LDS
    // copy of the section, which the writes cover exactly once
    uint8_t* sb = reinterpret_cast<uint8_t*>(stage);
    const int c0 = 16 * (4 * q1 + 8 * q2) + 8 * q0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t packed = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        packed |= put_code<kClamp>(fmaf(x[8 * m + e], ca, cb), qmax, 0, 0) << (kVBits * m);
      uint32_t byte_off;
      int shift;
      value_code_pos<kVBits, kDim>(t, c0 + e, byte_off, shift);   // shift is 0 here
      if constexpr (kVBits == 2)
        sb[byte_off] = (uint8_t)packed;
      else
        *reinterpret_cast<uint16_t*>(sb + byte_off) = (uint16_t)packed;
    }
  } else if constexpr (kVBits == 4) {
    // 4-bit value codes. Channel 16 nb + n with nb = m + 4 q1, n = 8 q0 + e: half-word i % 2 of
    // section word 512 kb + 256 q1 + 4 (16 s + n) + 2 h + i / 2 holds the codes of
    // nb % 4 = m = 0..3 at bits 4 m (t = 32 kb + 16 h + 4 s + i). The section is staged in
    // 16-byte chunks (chunk = word / 4 = 128 kb + 64 q1 + 16 s + 8 q0 + e) with the chunk's low
    // three bits XORed with s + 4 (q1 ^ q0), so one instruction's 64 half-word writes spread
    // over the banks; the store undoes the swizzle.
    uint16_t* sh = reinterpret_cast<uint16_t*>(stage);
    const int kb = t >> 5, h = (t >> 4) & 1, s4 = (t >> 2) & 3, i = t & 3;
    const int sw = s4 + 4 * (q1 ^ q0);
    const int c0 = 128 * kb + 64 * q1 + 16 * s4 + 8 * q0;
    const int lo = 2 * (2 * h + (i >> 1)) + (i & 1);        // half-word within the chunk
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t ev = 0, od = 0;                    // fields m = 0, 2 and m = 1, 3 in bytes 0, 1
      ev = put_code<kClamp>(fmaf(x[e], ca, cb), qmax, 0, ev);
      ev = put_code<kClamp>(fmaf(x[16 + e], ca, cb), qmax, 1, ev);
      od = put_code<kClamp>(fmaf(x[8 + e], ca, cb), qmax, 0, od);
      od = put_code<kClamp>(fmaf(x[24 + e], ca, cb), qmax, 1, od);
      sh[8 * (c0 + (e ^ sw)) + lo] = (uint16_t)(ev | (od << 4));
    }
  } else {
    // value codes. Byte e of this thread holds the codes of channel n = 8 q0 + e, hf = q1,
    // nb' = m at bits 2 m; it is staged at byte 2 (t % 2) + hf of LDS word 17 (t / 2) + n, which
    // makes every LDS word one word of the section (rows of 17 words: the 16 tokens of a wave
    // writing the same n fall in different banks).
    uint8_t* sb = reinterpret_cast<uint8_t*>(stage);
#pragma unroll
    for (int eh = 0; eh < 8; eh += 4) {
      uint32_t d = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t p = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p = put_code<kClamp>(fmaf(x[8 * m + eh + e], ca, cb), qmax, e, p);
        d |= p << (2 * m);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
        sb[((t >> 1) * 17 + 8 * q0 + eh + e) * 4 + (t & 1) * 2 + q1] = (uint8_t)(d >> (8 * e));
    }
  }
}

template <int kVBits, int kDim>
__device__ __forceinline__ void store_record_zero_tile(uint8_t* rec, int is_v, int tid) {
  // All-zero rotated tile: c-hat = 1 (E4M3 0x38), s-hat = 0, z-hat = +0, every code 0.
  using L = RecordLayout<kVBits, kDim>;
  const int code_off = is_v ? L::kVCodes : L::kKCodes;
  const int code_bytes = is_v ? L::kVCodeBytes : 64 * kDim;
  const int meta = is_v ? L::kVMetaOff : L::kKMetaOff;
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < code_bytes / 16; i += QGeom<kDim>::kThreads)
    reinterpret_cast<uint4*>(rec + code_off)[i] = z;
  if (tid < kDim / 4) reinterpret_cast<uint32_t*>(rec + meta + L::kC)[tid] = 0x38383838u;
  if (tid < 32) reinterpret_cast<uint32_t*>(rec + meta + L::kS)[tid] = 0u;
  if (tid < 64) reinterpret_cast<uint32_t*>(rec + meta + L::kZ)[tid] = 0u;
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

// Minimum / maximum of the pair of lanes l, l ^ 16 (or l ^ 32) of a finite value, every lane
// getting the result. One v_min_f32 / v_max_f32 on the swapped pair: fminf would first quiet
// possible signalling NaNs coming out of the lane exchange, which finite values never are.
__device__ __forceinline__ float fmin_raw(float a, float b) {
  float r;
  asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float fmax_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float min_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmin_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float min_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmin_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor16_raw(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32_raw(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(half8, make_uint4(a, b, c, d));
}

// The 128-point transform of a wave's 16 tokens on the matrix cores (head dimension 128).
// Lane l = 16 (2 q1 + q0) + n holds token n's fp16 channels 16 m + 8 q0 + 64 q1 + j (j = 0..7)
// in w[m]; on return x[8 m' + e] is rotated channel e + 8 q0 + 16 m' + 64 q1 of the same token,
// exactly the butterfly layout but with lane bits 4, 5 in place of 0, 1 and no sign folding.
// The Sylvester matrix factorises over channel bits: H[o][c] = prod_b (-1)^(o_b c_b). Channel
// bits 0-3 and 6 are contracted inside v_mfma_f32_16x16x32_f16 (B operand = w[m]: k = 8 (l >> 4)
// + j is channel bits 0-2 = j, 3 = q0, 6 = q1; output row rho = 4 (l >> 4) + r of block mb is
// channel bits 0-1 = r, 2 = mb, 3 = bit 2 of rho, 6 = bit 3 of rho), and channel bits 4-5 (the
// group m) by accumulating four products whose ±1 operand is negated where popcount(m & m')
// is odd. Every product is an exact fp16 times +-1, summed in fp32.
__device__ __forceinline__ void rotate_mfma(const uint4 (&w)[4], int lane, float* x) {
  const int rho = lane & 15, g0 = (lane >> 4) & 1, g1 = lane >> 5;
  constexpr uint32_t kNeg = 0x80008000u;                     // both halves' sign bits
  // A fragment (row rho, halves j of k-group (g0, g1)): sign over bits 0-1 from (rho & 3, j & 3),
  // bit 3 from (bit 2 of rho, g0), bit 6 from (bit 3 of rho, g1); bit 2 (j >= 4) from mb
  const uint32_t all = ((((rho >> 2) & g0) ^ ((rho >> 3) & g1)) & 1) ? kNeg : 0u;
  const uint32_t d0 = 0x3C003C00u ^ all ^ ((rho & 1) ? 0x80000000u : 0u);   // j = 0, 1
  const uint32_t d1 = d0 ^ ((rho & 2) ? kNeg : 0u);                          // j = 2, 3
  const half8 ap[2] = {as_half8(d0, d1, d0, d1), as_half8(d0, d1, d0 ^ kNeg, d1 ^ kNeg)};
  const half8 an[2] = {as_half8(d0 ^ kNeg, d1 ^ kNeg, d0 ^ kNeg, d1 ^ kNeg),
                       as_half8(d0 ^ kNeg, d1 ^ kNeg, d0, d1)};
  half8 b[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) b[m] = __builtin_bit_cast(half8, w[m]);
#pragma unroll
  for (int mp = 0; mp < 4; ++mp) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16((__builtin_popcount(m & mp) & 1) ? an[mb]
                                                                                    : ap[mb],
                                                     b[m], acc, 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[8 * mp + 4 * mb + r] = acc[r];
    }
  }
}

// ds_swizzle across lane bit 2 (bit-mask mode: and 0x1F, xor 4, within 32 lanes).
__device__ __forceinline__ float swz_xor4(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (4 << 10) | 0x1F));
}

// Quantise one tile. `src` points at token 0, channel 0 of this KV head; token t starts at
// src + t * token_stride. If `row127` is not null it replaces token 127 (the append path
// passes the new token there). Writes the key or value half of the record at `rec` (value
// codes of kVBits bits, head dimension kDim).
template <int kVBits, int kDim>
__device__ __forceinline__ void quantize_tile(const __half* __restrict__ src,
                                              long long token_stride,
                                              const __half* __restrict__ row127, int is_v,
                                              int iters, SignWords signs,
                                              uint8_t* __restrict__ rec, QuantSmem<kDim>& sm) {
  using G = QGeom<kDim>;
  using L = RecordLayout<kVBits, kDim>;
  constexpr int kXs = G::kXs, kQW = G::kWaves, kTPT = G::kTPT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // layout A: at D = 128 token t = 16 wave + lane % 16 with q0, q1 = lane bits 4, 5 (the
  // matrix-core transform's output); otherwise t = tid / kTPT with q0, q1, q2 = tid bits 0, 1, 2
  constexpr bool kMfma = kDim == 128;
  const int t = kMfma ? 16 * wave + (lane & 15) : tid / kTPT;
  const int q0 = kMfma ? (lane >> 4) & 1 : tid & 1;
  const int q1 = kDim >= 128 ? (kMfma ? lane >> 5 : (tid >> 1) & 1) : 0;
  const int q2 = kDim == 256 ? (tid >> 2) & 1 : 0;
  const bool lead = kMfma ? lane < 16 : (tid & (kTPT - 1)) == 0;   // one thread per token
  const int jj = 16 * wave + (lane & 15), th = lane >> 4;     // layout B
  const int cbase = 8 * q0 + 64 * q1 + 128 * q2;                // channel of x[0]
  const int pbase = cpos(cbase);                                // its LDS position
  const bool flip = !kMfma && (q0 ^ q1) != 0;                  // values carry a factor -1

  // ---- load (layout A) and rotate
  float x[32];
  {
    const __half* row = (row127 != nullptr && t == kT - 1) ? row127
                                                           : src + (long long)t * token_stride;
    const uint4* r4 = reinterpret_cast<const uint4*>(row + cbase);
    uint4 w[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) w[m] = r4[2 * m];                // channels cbase + 16 m ..
    uint32_t any = 0;
#pragma unroll
    for (int i = 0; i < kDim / 32; ++i) any |= sign_word(signs, i);
    if (any != 0u) {                                            // optional sign flips
      if (tid < kDim / 2) {
        const uint32_t word = sign_word(signs, tid >> 4);
        const uint32_t b2 = (word >> (2 * (tid & 15))) & 3u;
        sm.sgn[tid] = ((b2 & 1u) << 15) | ((b2 >> 1) << 31);
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint4 sg = *reinterpret_cast<const uint4*>(&sm.sgn[(cbase >> 1) + 8 * m]);
        w[m].x ^= sg.x; w[m].y ^= sg.y; w[m].z ^= sg.z; w[m].w ^= sg.w;
      }
    }
    if constexpr (kMfma) {
      rotate_mfma(w, lane, x);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) unpack_h8(w[m], x + 8 * m);
    }
  }
  if constexpr (!kMfma) {                      // butterflies: in registers, then across lanes
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if ((i & h) == 0) {
          const float a = x[i], b = x[i + h];
          x[i] = a + b;
          x[i + h] = a - b;
        }
      }
    }
    const float s1 = q0 ? -1.0f : 1.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) fmac_xor1(x + 8 * g, s1);      // channel bit 3
    if constexpr (kDim == 256) {
      const float s2 = q1 ? -1.0f : 1.0f;
#pragma unroll
      for (int g = 0; g < 4; ++g) fmac_xor2(x + 8 * g, s2);    // channel bit 6
      const float s4 = q2 ? -1.0f : 1.0f;                       // channel bit 7, exact
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = fmaf(s4, x[i], swz_xor4(x[i]));
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = wave_max_nonneg(amax);
  if (lane == 0) sm.red[wave] = amax;
  // ---- transpose A -> B through LDS
  {
    float4* row4 = reinterpret_cast<float4*>(&sm.xt[t][0]);   // rows are 16-byte aligned
    // at D = 128 the 16-byte chunks of row t are XOR-swizzled by (t >> 1) & 3: the 16 tokens
    // of a wave write the same channels, and the swizzle spreads them over the banks
    // (the XOR touches position bits 2-3 only, so it commutes with adding 16 m)
    const int sw = kMfma ? 4 * ((t >> 1) & 3) : 0;
    const int p0 = (pbase ^ sw) >> 2, p1 = ((pbase + 4) ^ sw) >> 2;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
      for (int h = 0; h < 8; h += 4)
        row4[(h ? p1 : p0) + 4 * m] =
            make_float4(x[8 * m + h], x[8 * m + h + 1], x[8 * m + h + 2], x[8 * m + h + 3]);
    }
  }
  if (tid < kT) sm.u[tid & 3][tid >> 2] = 1.0f;
  __syncthreads();
  float big = sm.red[0];
#pragma unroll
  for (int w = 1; w < kQW; ++w) big = max_nn(big, sm.red[w]);
  if (big == 0.0f) {                              // uniform across the workgroup
    store_record_zero_tile<kVBits, kDim>(rec, is_v, tid);
    return;
  }
  // layout B in registers for the whole normalisation: xb[i] = column jj, token th + 4 i (row
  // th + 4 i carries the swizzle th / 2 for even i and 2 + th / 2 for odd i)
  float xb[32];
  {
    const float* xce = &sm.xt[th][cpos(jj) ^ (kMfma ? 4 * (th >> 1) : 0)];
    const float* xco = &sm.xt[th][cpos(jj) ^ (kMfma ? 4 * (2 + (th >> 1)) : 0)];
#pragma unroll
    for (int i = 0; i < 32; ++i) xb[i] = ((i & 1) ? xco : xce)[4 * i * kXs];
  }
  // shifts of the variance sums, the same in every lane of a column or row so that the lanes'
  // sums just add: the column's token 0 and (at D = 128) the token's channel 0
  const float xc0 = sm.xt[0][cpos(jj)];
  const float xr0 = kMfma ? sm.xt[t][4 * ((t >> 1) & 3)] : 0.0f;

  // ---- alternating normalisation
  const float floor_unit = big * 1.52587890625e-05f;   // 2^-16 * max |rotated|
  constexpr float kInvD = 1.0f / kDim;
  float umax = 1.0f;
  for (int it = 0; it < iters; ++it) {
    // column step (layout B): std over tokens of xt_tj * u_t, from sums shifted by the
    // column's token 0, added over the four lanes of the column (lane bits 4, 5)
    {
      float s1, s2;
      if (it == 0) {
        const float k0 = xc0;
        s1 = xb[0] - k0;
        s2 = s1 * s1;
#pragma unroll
        for (int i = 1; i < 32; ++i) {
          const float y = xb[i] - k0;
          s1 += y;
          s2 = fmaf(y, y, s2);
        }
      } else {
        const float* uu = sm.u[th];
        const float k0 = xc0 * sm.u[0][0];        // token 0's multiplier is u[0][0]
        s1 = fmaf(xb[0], uu[0], -k0);
        s2 = s1 * s1;
#pragma unroll
        for (int i = 1; i < 32; ++i) {
          const float y = fmaf(xb[i], uu[i], -k0);
          s1 += y;
          s2 = fmaf(y, y, s2);
        }
      }
      s1 = add_xor32(add_xor16(s1));
      s2 = add_xor32(add_xor16(s2));
      const float qh = fmaxf(fmaf(-s1 * 0.0078125f, s1, s2), 0.0f);   // centred, 128 tokens
      const float sd = fmaxf(__builtin_amdgcn_sqrtf(qh * 0.0078125f), floor_unit * umax);
      if (th == 0) sm.cs[jj] = sd;
      if (it < iters - 1) {                       // the last row step does not change c
        const float vi = __builtin_amdgcn_rcpf(sd);
        if (th == 0) sm.vinv[cpos(jj)] = vi;
        const float vm = row16_max(vi);           // the wave's 16 channels are one DPP row
        if (lane == 0) sm.red[kQW + wave] = vm;
      }
    }
    __syncthreads();
    if (it == iters - 1) break;
    float vmax = sm.red[kQW];
#pragma unroll
    for (int w = 1; w < kQW; ++w) vmax = max_nn(vmax, sm.red[kQW + w]);
    // row step (layout A): std over channels of xt_tj * v_j
    {
      const float* vv = sm.vinv + pbase;
      float qh;
      if constexpr (kMfma) {
        // sums shifted by the token's channel 0 (v of channel 0 at vinv[0]), added over the
        // token's four lanes (lane bits 4, 5)
        const float k0 = xr0 * sm.vinv[0];
        float s1 = fmaf(x[0], vv[0], -k0);
        float s2 = s1 * s1;
#pragma unroll
        for (int i = 1; i < 32; ++i) {
          const float y = fmaf(x[i], vv[16 * (i >> 3) + (i & 7)], -k0);
          s1 += y;
          s2 = fmaf(y, y, s2);
        }
        s1 = add_xor32(add_xor16(s1));
        s2 = add_xor32(add_xor16(s2));
        qh = fmaxf(fmaf(-s1 * kInvD, s1, s2), 0.0f);
      } else {
        // per-thread shift (its first term, left out of the sums: its shifted value is the
        // rounding residual of its product), merged with Chan's update over the token's
        // threads, whose values may carry the butterflies' factor -1
        const float k0 = x[0] * vv[0];
        float s1 = fmaf(x[1], vv[1], -k0);
        float s2 = s1 * s1;
#pragma unroll
        for (int i = 2; i < 32; ++i) {
          const float y = fmaf(x[i], vv[16 * (i >> 3) + (i & 7)], -k0);
          s1 += y;
          s2 = fmaf(y, y, s2);
        }
        float mh = fmaf(s1, 0.03125f, k0);
        if (flip) mh = -mh;
        qh = fmaxf(fmaf(-s1 * 0.03125f, s1, s2), 0.0f);
        {
          const float d = dpp_sub<kDppXor1>(mh, mh);   // partner - own (only d^2 is used)
          const float qs = dpp_add<kDppXor1>(qh, qh);
          mh = 0.5f * dpp_add<kDppXor1>(mh, mh);
          qh = fmaf(16.0f * d, d, qs);
        }
        if constexpr (kDim == 256) {
          const float d = dpp_sub<kDppXor2>(mh, mh);
          const float qs = dpp_add<kDppXor2>(qh, qh);
          mh = 0.5f * dpp_add<kDppXor2>(mh, mh);
          qh = fmaf(32.0f * d, d, qs);
          const float d4 = swz_xor4(mh) - mh;      // and across lane bit 2 (128 channels each)
          qh = fmaf(64.0f * d4, d4, qh + swz_xor4(qh));
        }
      }
      const float sd = fmaxf(__builtin_amdgcn_sqrtf(qh * kInvD), floor_unit * vmax);
      const float uinv = __builtin_amdgcn_rcpf(sd);
      if (lead) sm.u[t & 3][t >> 2] = uinv;
      // the wave's largest multiplier: at D = 128 each 16-lane row holds all 16 of its tokens
      const float um = kMfma ? row16_max(uinv) : max_xor48_nn(row16_max(uinv));
      if (lane == 0) sm.red[2 * kQW + wave] = um;
    }
    __syncthreads();
    umax = sm.red[2 * kQW];
#pragma unroll
    for (int w = 1; w < kQW; ++w) umax = max_nn(umax, sm.red[2 * kQW + w]);
  }

  // ---- gauge (geometric mean of c = 1) and FP8 rounding of c, by wave 0 (lane: channels
  // lane + 64 k)
  const int meta = is_v ? L::kVMetaOff : L::kKMetaOff;
  if (wave == 0) {
    float cl[kDim / 64];
    float lsum = 0.0f;
#pragma unroll
    for (int k = 0; k < kDim / 64; ++k) {
      cl[k] = sm.cs[lane + 64 * k];
      lsum += log2f(cl[k]);
    }
    lsum = wave_sum(lsum);
    const float g = exp2f(-lsum * kInvD);
#pragma unroll
    for (int k = 0; k < kDim / 64; ++k) {
      const uint32_t e = e4m3_rne(fminf(fmaxf(cl[k] * g, 0.001953125f), 448.0f));
      sm.rq[cpos(lane + 64 * k)] = G::kInvSqrt / e4m3_to_float(e);
      reinterpret_cast<uint8_t*>(sm.chat)[lane + 64 * k] = (uint8_t)e;
    }
  }
  __syncthreads();   // also: every read of sm.xt is done, so it may hold the packed codes
  if (tid < kDim / 4) reinterpret_cast<uint32_t*>(rec + meta + L::kC)[tid] = sm.chat[tid];
  uint32_t* stage = reinterpret_cast<uint32_t*>(&sm.xt[0][0]);

  // ---- asymmetric RTN per token (layout A); p = (+-) y, sign `flip`
  const float qmax = is_v ? (float)((1 << kVBits) - 1) : 15.0f;
  float pmin = 3.0e38f, pmax = -3.0e38f;
  {
    const float* rr = sm.rq + pbase;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      x[i] *= rr[16 * (i >> 3) + (i & 7)];
      pmin = fminf(pmin, x[i]);
      pmax = fmaxf(pmax, x[i]);
    }
  }
  float mn = flip ? -pmax : pmin, mx = flip ? -pmin : pmax;
  if constexpr (kMfma) {
    mn = min_xor32(min_xor16(mn));
    mx = max_xor32_raw(max_xor16_raw(mx));
  } else {
    mn = fminf(mn, quad_swap<kDppXor1>(mn));
    mx = fmaxf(mx, quad_swap<kDppXor1>(mx));
  }
  if constexpr (kDim == 256) {
    mn = fminf(mn, quad_swap<kDppXor2>(mn));
    mx = fmaxf(mx, quad_swap<kDppXor2>(mx));
  }
  if constexpr (kDim == 256) {
    mn = fminf(mn, swz_xor4(mn));
    mx = fmaxf(mx, swz_xor4(mx));
  }
  const uint32_t zbits = fp16_rd(fmaxf(mn, -65504.0f));
  const float zf = fp16_bits_to_float(zbits);
  const uint32_t scode = e4m3_ru((mx - zf) / qmax);
  const float sf = e4m3_to_float(scode);
  const float inv_s = sf > 0.0f ? 1.0f / sf : 0.0f;
  const float ca = flip ? -inv_s : inv_s;          // (y - z) / s = p * ca + cb
  const float cb = -zf * inv_s;
  if (lead) {
    reinterpret_cast<uint8_t*>(sm.meta)[t] = (uint8_t)scode;
    reinterpret_cast<uint16_t*>(sm.meta + 32)[t] = (uint16_t)zbits;
  }

  if (scode == 0x7Eu)                                   // s-hat = 448
    stage_codes<true, kVBits, kDim>(x, ca, cb, qmax, is_v, t, q0, q1, q2, stage);
  else
    stage_codes<false, kVBits, kDim>(x, ca, cb, qmax, is_v, t, q0, q1, q2, stage);
  if (!is_v) {                                         // staged as the section: 64 kDim bytes
    __syncthreads();
    uint4 c;
    if constexpr (kDim == 128) {                       // token rows of 17 words
      const uint32_t* r = stage + 17 * (tid >> 2) + 4 * (tid & 3);
      c = make_uint4(r[0], r[1], r[2], r[3]);
    } else {
      c = reinterpret_cast<const uint4*>(stage)[tid];
    }
    reinterpret_cast<uint4*>(rec + L::kKCodes)[tid] = c;
  } else if constexpr (kDim != 128) {
    __syncthreads();
    if (tid < L::kVCodeBytes / 16)
      reinterpret_cast<uint4*>(rec + L::kVCodes)[tid] = reinterpret_cast<const uint4*>(stage)[tid];
  } else if constexpr (kVBits == 4) {                  // chunk tid sits at tid ^ (s + 4 (q1 ^ q0))
    __syncthreads();
    const int sw = ((tid >> 4) & 3) + 4 * (((tid >> 6) ^ (tid >> 3)) & 1);
    reinterpret_cast<uint4*>(rec + kVCodesOff)[tid] =
        reinterpret_cast<const uint4*>(stage)[tid ^ sw];
  } else {
    __syncthreads();
    if (tid < 256) {
      uint32_t out[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int w = 4 * tid + d;                 // word index in the section
        const int kb = w >> 8, s = (w >> 6) & 3, n = (w >> 2) & 15, h = d >> 1, i2 = d & 1;
        out[d] = stage[(16 * kb + 8 * h + 2 * s + i2) * 17 + n];
      }
      reinterpret_cast<uint4*>(rec + kVCodesOff)[tid] = make_uint4(out[0], out[1], out[2], out[3]);
    }
  }
  if (tid < 32) reinterpret_cast<uint32_t*>(rec + meta + L::kS)[tid] = sm.meta[tid];
  else if (tid < 96) reinterpret_cast<uint32_t*>(rec + meta + L::kZ)[tid - 32] = sm.meta[tid];
}

// grid: 2 * num_kv_heads * n_tiles workgroups; id = (tile * Hkv + head) * 2 + kv
template <int kVBits, int kDim>
__global__ void __launch_bounds__(4 * kDim) __attribute__((amdgpu_waves_per_eu(4, 4)))
quantize_tiles_kernel(const __half* __restrict__ k, const __half* __restrict__ v,
                      long long token_stride, int n_tiles, int hkv,
                      const int32_t* __restrict__ dst_blocks, uint8_t* __restrict__ pool,
                      long long num_blocks, int iters, SignWords signs) {
  __shared__ QuantSmem<kDim> sm;
  const int id = blockIdx.x;
  const int is_v = id & 1;
  const int head = (id >> 1) % hkv;
  const int tile = (id >> 1) / hkv;
  if (tile >= n_tiles) return;
  const long long blk = dst_blocks[tile];
  if (blk < 0 || blk >= num_blocks) return;
  const __half* src = (is_v ? v : k) + (long long)tile * kT * token_stride + head * kDim;
  uint8_t* rec = pool + (blk * hkv + head) * (long long)RecordLayout<kVBits, kDim>::kTileBytes;
  quantize_tile<kVBits, kDim>(src, token_stride, nullptr, is_v, iters, signs, rec, sm);
}

// grid: 2 * num_kv_heads * batch workgroups; id = (b * Hkv + head) * 2 + kv
template <int kVBits, int kDim>
__global__ void __launch_bounds__(4 * kDim) __attribute__((amdgpu_waves_per_eu(4, 4)))
append_token_kernel(const __half* __restrict__ k_new, const __half* __restrict__ v_new,
                    const int32_t* __restrict__ positions,
                    const int32_t* __restrict__ block_table, int max_blocks,
                    __half* __restrict__ staging_k, __half* __restrict__ staging_v,
                    uint8_t* __restrict__ pool, long long num_blocks, int hkv, int iters,
                    SignWords signs) {
  __shared__ QuantSmem<kDim> sm;
  const int id = blockIdx.x;
  const int is_v = id & 1;
  const int head = (id >> 1) % hkv;
  const int b = (id >> 1) / hkv;
  const int pos = positions[b];
  if (pos < 0) return;
  const int slot = pos & (kT - 1);
  const __half* src_tok = (is_v ? v_new : k_new) + ((long long)b * hkv + head) * kDim;
  __half* stg = (is_v ? staging_v : staging_k) + ((long long)b * hkv + head) * kT * kDim;
  if (threadIdx.x < kDim / 8) {
    reinterpret_cast<uint4*>(stg + slot * kDim)[threadIdx.x] =
        reinterpret_cast<const uint4*>(src_tok)[threadIdx.x];
  }
  if (slot != kT - 1) return;
  const int bi = pos >> 7;
  if (bi >= max_blocks) return;
  const long long blk = block_table[(long long)b * max_blocks + bi];
  if (blk < 0 || blk >= num_blocks) return;
  uint8_t* rec = pool + (blk * hkv + head) * (long long)RecordLayout<kVBits, kDim>::kTileBytes;
  // token 127 comes from the new token itself, so no read-after-write through global memory
  quantize_tile<kVBits, kDim>(stg, kDim, src_tok, is_v, iters, signs, rec, sm);
}

SignWords sign_words(const uint32_t* signs) {
  SignWords s;
  s.lo = make_uint4(signs[0], signs[1], signs[2], signs[3]);
  s.hi = make_uint4(signs[4], signs[5], signs[6], signs[7]);
  return s;
}

template <int kVBits, int kDim>
void launch_quantize_t(const __half* k, const __half* v, long long token_stride, int n_tiles,
                       int hkv, const int32_t* dst_blocks, uint8_t* pool, long long num_blocks,
                       int iters, SignWords sg, hipStream_t stream) {
  const long long groups = 2LL * hkv * n_tiles;
  hipLaunchKernelGGL((quantize_tiles_kernel<kVBits, kDim>), dim3((unsigned)groups),
                     dim3(4 * kDim), 0, stream, k, v, token_stride, n_tiles, hkv, dst_blocks,
                     pool, num_blocks, iters, sg);
}

template <int kVBits, int kDim>
void launch_append_t(const __half* k_new, const __half* v_new, const int32_t* positions,
                     const int32_t* block_table, int max_blocks, __half* staging_k,
                     __half* staging_v, uint8_t* pool, long long num_blocks, int hkv, int batch,
                     int iters, SignWords sg, hipStream_t stream) {
  const long long groups = 2LL * hkv * batch;
  hipLaunchKernelGGL((append_token_kernel<kVBits, kDim>), dim3((unsigned)groups),
                     dim3(4 * kDim), 0, stream, k_new, v_new, positions, block_table,
                     max_blocks, staging_k, staging_v, pool, num_blocks, hkv, iters, sg);
}

}  // namespace

hipError_t launch_quantize_tiles(const __half* k, const __half* v, long long token_stride,
                                 int n_tiles, int hkv, const int32_t* dst_blocks,
                                 uint8_t* pool, long long num_blocks, int iters,
                                 const uint32_t* signs, int v_bits, int head_dim,
                                 hipStream_t stream) {
  const SignWords sg = sign_words(signs);
#define KVARN_Q(VB, DIM)                                                                    \
  launch_quantize_t<VB, DIM>(k, v, token_stride, n_tiles, hkv, dst_blocks, pool, num_blocks, \
                             iters, sg, stream)
  if (head_dim == 64) {
    if (v_bits == 4) KVARN_Q(4, 64); else KVARN_Q(2, 64);
  } else if (head_dim == 256) {
    if (v_bits == 4) KVARN_Q(4, 256); else KVARN_Q(2, 256);
  } else {
    if (v_bits == 4) KVARN_Q(4, 128); else KVARN_Q(2, 128);
  }
#undef KVARN_Q
  return hipGetLastError();
}

hipError_t launch_append_token(const __half* k_new, const __half* v_new,
                               const int32_t* positions, const int32_t* block_table,
                               int max_blocks, __half* staging_k, __half* staging_v,
                               uint8_t* pool, long long num_blocks, int hkv, int batch,
                               int iters, const uint32_t* signs, int v_bits, int head_dim,
                               hipStream_t stream) {
  const SignWords sg = sign_words(signs);
#define KVARN_A(VB, DIM)                                                                      \
  launch_append_t<VB, DIM>(k_new, v_new, positions, block_table, max_blocks, staging_k,       \
                           staging_v, pool, num_blocks, hkv, batch, iters, sg, stream)
  if (head_dim == 64) {
    if (v_bits == 4) KVARN_A(4, 64); else KVARN_A(2, 64);
  } else if (head_dim == 256) {
    if (v_bits == 4) KVARN_A(4, 256); else KVARN_A(2, 256);
  } else {
    if (v_bits == 4) KVARN_A(4, 128); else KVARN_A(2, 128);
  }
#undef KVARN_A
  return hipGetLastError();
}

}  // namespace kvarn
