// Device-side helpers shared by the libkvarn kernels (gfx950, wave64).
//
// FP8 and FP16 conversions are written from the format definitions: OCP FP8 E4M3 (exponent
// bias 7, three mantissa bits, largest finite 448, subnormals in steps of 2^-9) and IEEE
// binary16 (bias 15, ten mantissa bits, subnormals in steps of 2^-24). Only non-negative FP8
// values occur in the codec (scales), so the FP8 helpers handle the sign-less half.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace kvarn {

constexpr int kT = 128;              // tokens per tile
constexpr int kD = 128;              // head dimension of the preset
constexpr int kKCodesOff = 0;        // key codes: 8,192 bytes (head dimension 128)
constexpr int kVCodesOff = 8192;     // value codes: 2,048 bytes per value bit (head dimension 128)
constexpr int kCRel = 0, kSRel = 128, kZRel = 256;   // c-hat, s-hat, z-hat in a metadata half

// Record of one (block, KV head) for value codes of kVBits bits and head dimension kDim:
// 64 kDim bytes of key codes, 16 kDim kVBits of value codes, then kDim + 384 bytes of key
// metadata and as many of value metadata (c-hat: kDim bytes, s-hat: 128, z-hat: 256).
// kDim = 128, kVBits = 2 is the preset kvarn_k4v2_g128 (13,312 bytes); kVBits = 4 the preset
// kvarn_k4v4_g128 (17,408 bytes); head dimensions 64 and 256 scale the same sections.
template <int kVBits, int kDim = 128>
struct RecordLayout {
  static_assert(kVBits == 2 || kVBits == 4, "value codes are 2 or 4 bits");
  static_assert(kDim == 64 || kDim == 128 || kDim == 256, "head dimension 64, 128 or 256");
  static constexpr int kKCodes = 0;
  static constexpr int kVCodes = 64 * kDim;
  static constexpr int kVCodeBytes = 16 * kDim * kVBits;
  static constexpr int kMetaHalf = kDim + 384;
  static constexpr int kKMetaOff = kVCodes + kVCodeBytes;
  static constexpr int kVMetaOff = kKMetaOff + kMetaHalf;
  static constexpr int kTileBytes = kKMetaOff + 2 * kMetaHalf;
  static constexpr int kC = 0, kS = kDim, kZ = kDim + 128;   // inside a metadata half
};

// Optional per-channel sign flips before the rotation: channel j is negated when bit j % 32 of
// word j / 32 is set (words 0-3 in lo, 4-7 in hi; a head dimension d uses the first d / 32).
struct SignWords {
  uint4 lo, hi;
};

__device__ __forceinline__ uint32_t sign_word(const SignWords& s, int i) {
  const uint4 q = i < 4 ? s.lo : s.hi;
  const int k = i & 3;
  return k == 0 ? q.x : (k == 1 ? q.y : (k == 2 ? q.z : q.w));
}

// Byte offset (in the value-code section) and bit shift of the value code of token t, channel
// j. With nb = j / 16, n = j % 16, kb = t / 32, h = (t / 16) % 2, s = (t / 4) % 4, i = t % 4 and
// e = 2 h + i / 2, in 32-bit words:
//   2-bit, kDim >= 128: word 2 kDim kb + (kDim / 32)(16 s + n) + 4 (nb / 8) + e,
//                       bit 2 (nb % 8) + 16 (i % 2)
//   2-bit, kDim = 64:   word 128 kb + 2 (16 s + n) + e / 2, bit 2 nb + 8 (e % 2) + 16 (i % 2)
//   4-bit:              word 4 kDim kb + 256 (nb / 4) + 4 (16 s + n) + e,
//                       bit 4 (nb % 4) + 16 (i % 2)
// A lane (n, s) of a value product thus finds the codes of its eight tokens of block kb in
// kDim / 32 (2-bit) or kDim / 16 (4-bit) consecutive words.
template <int kVBits, int kDim>
__device__ __forceinline__ void value_code_pos(int t, int j, uint32_t& byte_off, int& shift) {
  const int nb = j >> 4, n = j & 15, kb = t >> 5, h = (t >> 4) & 1, s = (t >> 2) & 3, i = t & 3;
  const int e = 2 * h + (i >> 1);
  int word, bit;
  if constexpr (kVBits == 2 && kDim >= 128) {
    word = 2 * kDim * kb + (kDim / 32) * (16 * s + n) + 4 * (nb >> 3) + e;
    bit = 2 * (nb & 7) + 16 * (i & 1);
  } else if constexpr (kVBits == 2) {
    word = 128 * kb + 2 * (16 * s + n) + (e >> 1);
    bit = 2 * nb + 8 * (e & 1) + 16 * (i & 1);
  } else {
    word = 4 * kDim * kb + 256 * (nb >> 2) + 4 * (16 * s + n) + e;
    bit = 4 * (nb & 3) + 16 * (i & 1);
  }
  byte_off = 4u * (uint32_t)word + (uint32_t)(bit >> 3);
  shift = bit & 7;
}

// ------------------------------------------------------------------ FP8 E4M3 (non-negative)

// Decode a non-negative E4M3 code (sign bit clear, not NaN) to float, exactly.
__device__ __forceinline__ float e4m3_to_float(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// Nearest E4M3 code to v, ties to the even code; v must lie in [2^-9, 448].
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t b = __float_as_uint(v);
  if (b < 0x3C800000u) {                       // v < 2^-6: subnormal grid of 2^-9
    return (uint32_t)rintf(v * 512.0f);        // 1..8 (8 encodes 2^-6)
  }
  uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
  r &= 0xFFF00000u;
  return ((((r >> 23) & 0xFFu) - 120u) << 3) | ((r >> 20) & 7u);
}

// Smallest E4M3 value >= v, as a code; v >= 0. Values above 448 saturate to 448.
__device__ __forceinline__ uint32_t e4m3_ru(float v) {
  if (!(v > 0.0f)) return 0u;
  if (v >= 448.0f) return 0x7Eu;
  const uint32_t b = __float_as_uint(v);
  if (b < 0x3C800000u) return (uint32_t)ceilf(v * 512.0f);
  uint32_t r = (b + 0xFFFFFu) & 0xFFF00000u;
  return ((((r >> 23) & 0xFFu) - 120u) << 3) | ((r >> 20) & 7u);
}

// ------------------------------------------------------------------ FP16 directed rounding

// Largest binary16 <= a for a >= +0 (sign bit clear; saturates at 65504), as bits.
__device__ __forceinline__ uint32_t fp16_rz_pos(float a) {
  if (a >= 65504.0f) return 0x7BFFu;
  const uint32_t b = __float_as_uint(a);
  if (b < 0x38800000u) return (uint32_t)floorf(a * 16777216.0f);  // a < 2^-14: step 2^-24
  return ((((b >> 23) & 0xFFu) - 112u) << 10) | ((b >> 13) & 0x3FFu);
}

// Smallest binary16 >= a for 0 < a <= 65504, as bits.
__device__ __forceinline__ uint32_t fp16_ru_pos(float a) {
  const uint32_t b = __float_as_uint(a);
  if (b < 0x38800000u) return (uint32_t)ceilf(a * 16777216.0f);
  const uint32_t r = b + 0x1FFFu;
  return ((((r >> 23) & 0xFFu) - 112u) << 10) | ((r >> 13) & 0x3FFu);
}

// Largest binary16 <= v for v >= -65504 (callers clamp first), as bits. Both zeros give +0.
__device__ __forceinline__ uint32_t fp16_rd(float v) {
  if (!(v < 0.0f)) return fp16_rz_pos(fabsf(v));
  return 0x8000u | fp16_ru_pos(-v);
}

__device__ __forceinline__ float fp16_bits_to_float(uint32_t h) {
  return __half2float(__ushort_as_half((unsigned short)h));
}

// ------------------------------------------------------------------ wave reductions (wave64)

// Pair reductions across lane bit 4 or 5 with v_permlane16_swap / v_permlane32_swap (VALU,
// no LDS): swapping a value with itself leaves (own, partner) in the two results.
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kCtrl, 0xF, 0xF, false));
}

// Sum over the wave, the same value in every lane: lane pairs 1 and 2 (quad_perm), 8 then 4
// (row rotations, each pairing values that are already equal in pairs), 16 and 32 (swaps).
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x128>(x);
  x += dpp_f<0x124>(x);
  return add_xor32(add_xor16(x));
}

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x128>(x));
  x = fmaxf(x, dpp_f<0x124>(x));
  return max_xor32(max_xor16(x));
}

// Largest value over the wave of a non-negative float (its bit pattern orders like an int):
// DPP maxima within each row of 16 lanes, then the four rows through scalar registers.
__device__ __forceinline__ float wave_max_nonneg(float x) {
  int v = __float_as_int(x);
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x124, 0xF, 0xF, false));  // row_ror:4
  v = max(v, __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false));  // row_ror:8
  const int r = max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
                    max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
  return __int_as_float(r);
}

// Unpack 8 fp16 values held in a uint4.
__device__ __forceinline__ void unpack_h8(const uint4 w, float* out) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = fp16_bits_to_float(u[i] & 0xFFFFu);
    out[2 * i + 1] = fp16_bits_to_float(u[i] >> 16);
  }
}

}  // namespace kvarn
