// KVarN tile quantiser (write path) for gfx950.
//
// One workgroup of 256 threads quantises one 128-token x 128-channel tile of one KV head,
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
// Work layout. Layout A gives thread (t, hf) = (tid / 2, tid % 2) the 64 channels
// 64 hf .. 64 hf + 63 of token t: the transform (six butterfly stages in registers and one
// across the lane pair, a DPP-sourced fused multiply-add), the row statistics and the codes.
// Layout B gives thread (j, th) = (tid % 128, tid / 128) the 64 tokens 64 th .. 64 th + 63 of
// channel j: the column statistics, read from a copy of the rotated tile kept in LDS for the
// whole normalisation (registers hold only the layout-A copy).
//
// Sign folding. The cross-lane butterfly computes x + s * partner with s = -1 on the odd lane
// of each pair, which leaves channels 64..127 negated. Column variances do not see a sign; the
// row step and the rounding stage multiply by per-channel factors anyway, so the stored factor
// for channels 64..127 carries the sign. The 1/sqrt(128) scale of the transform is folded the
// same way into the rounding stage's per-channel factor (the normalisation is scale-free up to
// the gauge, and the floor is relative to the tile's largest value).
//
// Variances use shifted one-pass sums (shift = the thread's first value), merged between the
// two threads sharing a row or column with Chan et al.'s pairwise update.

#include "kvarn_device.hpp"
#include "kvarn_kernels.hpp"

namespace kvarn {

namespace {

constexpr int kQThreads = 256;
constexpr int kXtStride = kD + 1;
constexpr float kInvSqrtD = 0.08838834764831845f;   // 2^-3.5

struct QuantSmem {
  float xt[kT][kXtStride];   // rotated tile, layout A -> B; reused for packed value codes
  float u[kT];               // per-token multipliers 1 / r_t
  float cs[kD];              // per-channel standard deviations (unrounded c before the gauge)
  float vsg[kD];             // per-channel multipliers 1 / c_j, negated for channels 64..127
  float rq[kD];              // per-channel rounding factor 2^-3.5 / c-hat_j (signed likewise)
  float colm[2][kD];         // per-half column shifted means
  float colq[2][kD];         // per-half column centred sums of squares
  uint32_t meta[96];         // staged FP8 s-hat (32 words) and FP16 z-hat (64 words)
  uint32_t chat[32];         // staged FP8 c-hat
  float red[16];
};

// value of lane (lane ^ 1) via DPP quad_perm [1, 0, 3, 2]
__device__ __forceinline__ float pair_swap(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

__device__ __forceinline__ void store_record_zero_tile(uint8_t* rec, int is_v, int tid) {
  // All-zero rotated tile: c-hat = 1 (E4M3 0x38), s-hat = 0, z-hat = +0, every code 0.
  const int code_off = is_v ? kVCodesOff : kKCodesOff;
  const int code_bytes = is_v ? 4096 : 8192;
  const int meta = is_v ? kVMetaOff : kKMetaOff;
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int i = tid; i < code_bytes / 16; i += kQThreads)
    reinterpret_cast<uint4*>(rec + code_off)[i] = z;
  if (tid < 32) reinterpret_cast<uint32_t*>(rec + meta + kCRel)[tid] = 0x38383838u;
  if (tid < 32) reinterpret_cast<uint32_t*>(rec + meta + kSRel)[tid] = 0u;
  if (tid < 64) reinterpret_cast<uint32_t*>(rec + meta + kZRel)[tid] = 0u;
}

// Quantise one tile. `src` points at token 0, channel 0 of this KV head; token t starts at
// src + t * token_stride. If `row127` is not null it replaces token 127 (the append path
// passes the new token there). Writes the key or value half of the record at `rec`.
__device__ __forceinline__ void quantize_tile(const __half* __restrict__ src, long long token_stride,
                              const __half* __restrict__ row127, int is_v, int iters,
                              uint8_t* __restrict__ rec, QuantSmem& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t = tid >> 1, hf = tid & 1;          // layout A
  const int jj = tid & (kD - 1), th = tid >> 7;  // layout B

  // ---- load (layout A) and rotate
  float x[64];
  {
    const __half* row = (row127 != nullptr && t == kT - 1) ? row127
                                                           : src + (long long)t * token_stride;
    const uint4* r4 = reinterpret_cast<const uint4*>(row + hf * 64);
    uint4 w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = r4[k];
#pragma unroll
    for (int k = 0; k < 8; ++k) unpack_h8(w[k], x + 8 * k);
  }
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  const float sgn = hf ? -1.0f : 1.0f;
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    x[i] = fmaf(sgn, pair_swap(x[i]), x[i]);     // channel 64..127 values come out negated
    amax = fmaxf(amax, fabsf(x[i]));
  }
  amax = wave_max(amax);
  if (lane == 0) sm.red[wave] = amax;
  // ---- transpose A -> B through LDS
#pragma unroll
  for (int i = 0; i < 64; i += 4)
    *reinterpret_cast<float4*>(&sm.xt[t][hf * 64 + i]) = make_float4(x[i], x[i + 1], x[i + 2],
                                                                      x[i + 3]);
  if (tid < kT) sm.u[tid] = 1.0f;
  __syncthreads();
  const float big = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
  if (big == 0.0f) {                              // uniform across the workgroup
    store_record_zero_tile(rec, is_v, tid);
    return;
  }
  const float* xcol = &sm.xt[th * 64][jj];       // column jj, tokens 64 th .., stride 129

  // ---- alternating normalisation
  const float floor_unit = big * 1.52587890625e-05f;   // 2^-16 * max |rotated|
  float umax = 1.0f;
  for (int it = 0; it < iters; ++it) {
    // column step (layout B): std over tokens of xt_tj * u_t
    {
      float s1 = 0.0f, s2 = 0.0f, k0;
      if (it == 0) {
        k0 = xcol[0];
#pragma unroll 16
        for (int i = 0; i < 64; ++i) {
          const float y = xcol[i * kXtStride] - k0;
          s1 += y;
          s2 = fmaf(y, y, s2);
        }
      } else {
        const float* uu = sm.u + th * 64;
        k0 = xcol[0] * uu[0];
#pragma unroll 16
        for (int i = 0; i < 64; ++i) {
          const float y = fmaf(xcol[i * kXtStride], uu[i], -k0);
          s1 += y;
          s2 = fmaf(y, y, s2);
        }
      }
      sm.colm[th][jj] = fmaf(s1, 0.015625f, k0);
      sm.colq[th][jj] = fmaxf(fmaf(-s1 * 0.015625f, s1, s2), 0.0f);
    }
    __syncthreads();
    if (th == 0) {
      const float d = sm.colm[0][jj] - sm.colm[1][jj];
      const float m2 = sm.colq[0][jj] + sm.colq[1][jj] + 32.0f * d * d;
      const float sd = fmaxf(sqrtf(m2 * 0.0078125f), floor_unit * umax);
      sm.cs[jj] = sd;
      const float vinv = 1.0f / sd;
      sm.vsg[jj] = jj >= 64 ? -vinv : vinv;
      const float vm = wave_max(vinv);
      if (lane == 0) sm.red[4 + wave] = vm;       // waves 0 and 1
    }
    __syncthreads();
    if (it == iters - 1) break;                   // the last row step does not change c
    const float vmax = fmaxf(sm.red[4], sm.red[5]);
    // row step (layout A): std over channels of xt_tj * v_j (signs restored by vsg)
    {
      const float* vv = sm.vsg + hf * 64;
      const float k0 = x[0] * vv[0];
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const float y = fmaf(x[i], vv[i], -k0);
        s1 += y;
        s2 = fmaf(y, y, s2);
      }
      const float mh = fmaf(s1, 0.015625f, k0);
      const float qh = fmaxf(fmaf(-s1 * 0.015625f, s1, s2), 0.0f);
      const float mo = pair_swap(mh), qo = pair_swap(qh);
      const float d = mh - mo;
      const float m2 = qh + qo + 32.0f * d * d;
      const float sd = fmaxf(sqrtf(m2 * 0.0078125f), floor_unit * vmax);
      const float uinv = 1.0f / sd;
      if (hf == 0) sm.u[t] = uinv;
      const float um = wave_max(uinv);
      if (lane == 0) sm.red[8 + wave] = um;
    }
    __syncthreads();
    umax = fmaxf(fmaxf(sm.red[8], sm.red[9]), fmaxf(sm.red[10], sm.red[11]));
  }

  // ---- gauge (geometric mean of c = 1) and FP8 rounding of c, by wave 0
  const int meta = is_v ? kVMetaOff : kKMetaOff;
  if (wave == 0) {
    const float c0 = sm.cs[lane], c1 = sm.cs[lane + 64];
    const float lsum = wave_sum(log2f(c0) + log2f(c1));
    const float g = exp2f(-lsum * 0.0078125f);
    const uint32_t q0 = e4m3_rne(fminf(fmaxf(c0 * g, 0.001953125f), 448.0f));
    const uint32_t q1 = e4m3_rne(fminf(fmaxf(c1 * g, 0.001953125f), 448.0f));
    sm.rq[lane] = kInvSqrtD / e4m3_to_float(q0);
    sm.rq[lane + 64] = -kInvSqrtD / e4m3_to_float(q1);
    reinterpret_cast<uint8_t*>(sm.chat)[lane] = (uint8_t)q0;
    reinterpret_cast<uint8_t*>(sm.chat)[lane + 64] = (uint8_t)q1;
  }
  __syncthreads();
  if (tid < 32) reinterpret_cast<uint32_t*>(rec + meta + kCRel)[tid] = sm.chat[tid];

  // ---- asymmetric RTN per token (layout A); x[] is overwritten by y, then by the codes
  const float qmax = is_v ? 3.0f : 15.0f;
  float mn = 3.0e38f, mx = -3.0e38f;
  {
    const float* rq = sm.rq + hf * 64;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      x[i] *= rq[i];
      mn = fminf(mn, x[i]);
      mx = fmaxf(mx, x[i]);
    }
  }
  mn = fminf(mn, pair_swap(mn));
  mx = fmaxf(mx, pair_swap(mx));
  const uint32_t zbits = fp16_rd(fmaxf(mn, -65504.0f));
  const float zf = fp16_bits_to_float(zbits);
  const uint32_t scode = e4m3_ru((mx - zf) / qmax);
  const float sf = e4m3_to_float(scode);
  const float inv_s = sf > 0.0f ? 1.0f / sf : 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) x[i] = fminf(fmaxf(rintf((x[i] - zf) * inv_s), 0.0f), qmax);
  if (hf == 0) {
    reinterpret_cast<uint8_t*>(sm.meta)[t] = (uint8_t)scode;
    reinterpret_cast<uint16_t*>(sm.meta + 32)[t] = (uint16_t)zbits;
  }

  if (!is_v) {
    // key codes: token-major nibbles; this thread's 64 channels are 32 contiguous bytes
    uint32_t w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      uint32_t acc = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) acc |= (uint32_t)x[8 * k + q] << (4 * q);
      w[k] = acc;
    }
    uint4* dst = reinterpret_cast<uint4*>(rec + kKCodesOff + t * 64 + hf * 32);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    __syncthreads();
  } else {
    // value codes. Byte (t, n, hf) holds the codes of channels 64 hf + 16 nb' + n, nb' = 0..3,
    // at bits 2 nb'; the 16-bit pair (t, n) is then the token-t half of a section word.
    __syncthreads();                               // everyone is done reading sm.xt
    uint8_t* vb = reinterpret_cast<uint8_t*>(&sm.xt[0][0]);   // [128][16][2] bytes
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const uint32_t b = (uint32_t)x[n] | ((uint32_t)x[16 + n] << 2) |
                         ((uint32_t)x[32 + n] << 4) | ((uint32_t)x[48 + n] << 6);
      vb[t * 32 + 2 * n + hf] = (uint8_t)b;
    }
    __syncthreads();
    const uint16_t* vh = reinterpret_cast<const uint16_t*>(vb);
    uint32_t out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int w = 4 * tid + e;                   // word index in the section
      const int kb = w >> 8, ln = (w >> 2) & 63, d = w & 3;
      const int s = ln >> 4, n = ln & 15;
      const int tb = 32 * kb + 16 * (d >> 1) + 4 * s + ((d & 1) << 1);
      out[e] = (uint32_t)vh[tb * 16 + n] | ((uint32_t)vh[(tb + 1) * 16 + n] << 16);
    }
    reinterpret_cast<uint4*>(rec + kVCodesOff)[tid] = make_uint4(out[0], out[1], out[2], out[3]);
  }
  if (tid < 32) reinterpret_cast<uint32_t*>(rec + meta + kSRel)[tid] = sm.meta[tid];
  else if (tid < 96) reinterpret_cast<uint32_t*>(rec + meta + kZRel)[tid - 32] = sm.meta[tid];
}

// grid: 2 * num_kv_heads * n_tiles workgroups; id = (tile * Hkv + head) * 2 + kv
__global__ void __launch_bounds__(kQThreads)
quantize_tiles_kernel(const __half* __restrict__ k, const __half* __restrict__ v,
                      long long token_stride, int n_tiles, int hkv,
                      const int32_t* __restrict__ dst_blocks, uint8_t* __restrict__ pool,
                      long long num_blocks, int iters) {
  __shared__ QuantSmem sm;
  const int id = blockIdx.x;
  const int is_v = id & 1;
  const int head = (id >> 1) % hkv;
  const int tile = (id >> 1) / hkv;
  if (tile >= n_tiles) return;
  const long long blk = dst_blocks[tile];
  if (blk < 0 || blk >= num_blocks) return;
  const __half* src = (is_v ? v : k) + (long long)tile * kT * token_stride + head * kD;
  uint8_t* rec = pool + (blk * hkv + head) * (long long)kTileBytes;
  quantize_tile(src, token_stride, nullptr, is_v, iters, rec, sm);
}

// grid: 2 * num_kv_heads * batch workgroups; id = (b * Hkv + head) * 2 + kv
__global__ void __launch_bounds__(kQThreads)
append_token_kernel(const __half* __restrict__ k_new, const __half* __restrict__ v_new,
                    const int32_t* __restrict__ positions,
                    const int32_t* __restrict__ block_table, int max_blocks,
                    __half* __restrict__ staging_k, __half* __restrict__ staging_v,
                    uint8_t* __restrict__ pool, long long num_blocks, int hkv, int iters) {
  __shared__ QuantSmem sm;
  const int id = blockIdx.x;
  const int is_v = id & 1;
  const int head = (id >> 1) % hkv;
  const int b = (id >> 1) / hkv;
  const int pos = positions[b];
  if (pos < 0) return;
  const int slot = pos & (kT - 1);
  const __half* src_tok = (is_v ? v_new : k_new) + ((long long)b * hkv + head) * kD;
  __half* stg = (is_v ? staging_v : staging_k) + ((long long)b * hkv + head) * kT * kD;
  if (threadIdx.x < 16) {
    reinterpret_cast<uint4*>(stg + slot * kD)[threadIdx.x] =
        reinterpret_cast<const uint4*>(src_tok)[threadIdx.x];
  }
  if (slot != kT - 1) return;
  const int bi = pos >> 7;
  if (bi >= max_blocks) return;
  const long long blk = block_table[(long long)b * max_blocks + bi];
  if (blk < 0 || blk >= num_blocks) return;
  uint8_t* rec = pool + (blk * hkv + head) * (long long)kTileBytes;
  // token 127 comes from the new token itself, so no read-after-write through global memory
  quantize_tile(stg, kD, src_tok, is_v, iters, rec, sm);
}

}  // namespace

hipError_t launch_quantize_tiles(const __half* k, const __half* v, long long token_stride,
                                 int n_tiles, int hkv, const int32_t* dst_blocks,
                                 uint8_t* pool, long long num_blocks, int iters,
                                 hipStream_t stream) {
  const long long groups = 2LL * hkv * n_tiles;
  hipLaunchKernelGGL(quantize_tiles_kernel, dim3((unsigned)groups), dim3(kQThreads), 0, stream,
                     k, v, token_stride, n_tiles, hkv, dst_blocks, pool, num_blocks, iters);
  return hipGetLastError();
}

hipError_t launch_append_token(const __half* k_new, const __half* v_new,
                               const int32_t* positions, const int32_t* block_table,
                               int max_blocks, __half* staging_k, __half* staging_v,
                               uint8_t* pool, long long num_blocks, int hkv, int batch,
                               int iters, hipStream_t stream) {
  const long long groups = 2LL * hkv * batch;
  hipLaunchKernelGGL(append_token_kernel, dim3((unsigned)groups), dim3(kQThreads), 0, stream,
                     k_new, v_new, positions, block_table, max_blocks, staging_k, staging_v,
                     pool, num_blocks, hkv, iters);
  return hipGetLastError();
}

}  // namespace kvarn
