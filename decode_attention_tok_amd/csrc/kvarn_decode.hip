// KVarN paged decode attention over packed K4/V2 tiles (read path) for gfx950.
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
// Key codes enter the MFMA as normal fp16 halves 1 + code / 16 (the nibble shifted into
// mantissa bits 6..9 under exponent 0x3C00); the constant 1 contributes sum_j q~_j, which the
// score needs anyway and subtracts exactly. (The MFMA sums products of subnormal fp16 operands
// with far less precision than products of normal ones, so raw codes are not used as
// subnormals.) Value codes likewise enter as 1 + code / 4 (the 2-bit field shifted to
// mantissa bits 8..9), and sum_t p_t s-hat^V_t removes the constant part per head.
// fp32-accurate operands are split into fp16 hi + lo parts: query column g holds hi(q~_g),
// column 8 + g holds lo(q~_g), and one DPP row rotation by 8 adds the two partial scores;
// the probability operand likewise has rows g (hi) and 8 + g (lo), summed once at the end.
// The score accumulator lanes of token block pair (2 kb, 2 kb + 1) are exactly the operand
// lanes of output token block kb, so probabilities feed the second product without shuffles.

#include "kvarn_device.hpp"
#include "kvarn_kernels.hpp"

namespace kvarn {

namespace {

constexpr int kWaves = 4;
constexpr int kTThreads = 64 * kWaves;
constexpr int kHeadGroup = 8;                 // query heads per tile workgroup
constexpr float kLog2e = 1.4426950408889634f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

struct WaveMeta {                  // per-wave, per-tile metadata (fp32, factors folded in)
  float kc[kD];                    // c-hat^K_j
  float ks[kT];                    // s-hat^K_t * sm * log2(e) * 16 / pq
  float kz[kT];                    // z-hat^K_t * sm * log2(e)
  float vs[kT];                    // s-hat^V_t * 32 (probability operand prescale)
  float vz[kT];                    // z-hat^V_t
  float vc[kD];                    // c-hat^V_j
  float alpha[16], beta[16];       // per-row rescale and zero-point term of the last tile
};

struct TileSmem {
  float qrot[kHeadGroup][kD];      // rotated queries (fp32)
  WaveMeta wm[kWaves];
  float comb_m[kWaves][kHeadGroup], comb_l[kWaves][kHeadGroup];
  float comb_o[kWaves][kHeadGroup][kD];
  float red[kWaves];
};

__device__ __forceinline__ float dpp_ror8(float v) {   // lane (l & ~15) | ((l + 8) & 15)
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
}

__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  const __fp16 ha = (__fp16)a, hb = (__fp16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// (x & mask) | c in one v_and_or_b32: mask in a VGPR and c in an SGPR, since a gfx9 VOP3
// instruction cannot carry two literal constants (the compiler otherwise emits and + or).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask_v, uint32_t c_s) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(mask_v), "s"(c_s));
  return r;
}

__device__ __forceinline__ half8 as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  uint4 u = make_uint4(a, b, c, d);
  return __builtin_bit_cast(half8, u);
}

typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// fp16 hi / lo parts of a pair (a, b), both rounded to nearest: a == hi + lo to about 2^-22
// relative while normal. Returns the packed hi pair or the packed lo pair.
__device__ __forceinline__ uint32_t split_pair(float a, float b, bool want_hi) {
  const half2v h = __builtin_convertvector((float2v){a, b}, half2v);
  const float2v hb = __builtin_convertvector(h, float2v);
  const half2v l = __builtin_convertvector((float2v){a - hb[0], b - hb[1]}, half2v);
  return want_hi ? __builtin_bit_cast(uint32_t, h) : __builtin_bit_cast(uint32_t, l);
}

struct TileRegs {
  uint4 kw[8];        // key codes: token 16 mb + (lane % 16), channels 32 (lane / 16) .. + 31
  uint4 vw[4];        // value codes: section words 256 kb + 4 lane .. + 3
  uint4 meta;         // 16 bytes of the record's 1 KB metadata at 12288 + 16 lane
};

__device__ __forceinline__ void load_tile(const uint8_t* __restrict__ rec, int lane, TileRegs& r) {
  const int m = lane & 15, s = lane >> 4;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
    r.kw[mb] = *reinterpret_cast<const uint4*>(rec + kKCodesOff + (16 * mb + m) * 64 + 16 * s);
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    r.vw[kb] = *reinterpret_cast<const uint4*>(rec + kVCodesOff + kb * 1024 + lane * 16);
  r.meta = *reinterpret_cast<const uint4*>(rec + kKMetaOff + lane * 16);
}

// Scatter one lane's 16 metadata bytes into the wave's fp32 tables. Lanes 0-7: c-hat^K,
// 8-15: s-hat^K, 16-31: z-hat^K, 32-39: c-hat^V, 40-47: s-hat^V, 48-63: z-hat^V.
// FP8 bytes go through the hardware E4M3 conversion (exact for every finite code).
__device__ __forceinline__ void decode_meta(const uint4 mw, int lane, WaveMeta& wm,
                                            float kfac, float kzfac) {
  const uint32_t w[4] = {mw.x, mw.y, mw.z, mw.w};
  const int grp = lane & 31;
  const bool isv = lane >= 32;
  if (grp < 16) {                         // 16 FP8 values
    const float mul = grp < 8 ? 1.0f : (isv ? 32.0f : kfac);
    float* dst = grp < 8 ? (isv ? wm.vc : wm.kc) : (isv ? wm.vs : wm.ks);
    dst += (grp & 7) * 16;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float2v lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], false);
      const float2v hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], true);
      *reinterpret_cast<float4*>(dst + 4 * d) =
          make_float4(lo[0] * mul, lo[1] * mul, hi[0] * mul, hi[1] * mul);
    }
  } else {                                // 8 fp16 values
    const float mul = isv ? 1.0f : kzfac;
    float* dst = (isv ? wm.vz : wm.kz) + (grp - 16) * 8;
#pragma unroll
    for (int d = 0; d < 4; d += 2) {
      const float2v a = __builtin_convertvector(__builtin_bit_cast(half2v, w[d]), float2v);
      const float2v b = __builtin_convertvector(__builtin_bit_cast(half2v, w[d + 1]), float2v);
      *reinterpret_cast<float4*>(dst + 2 * d) =
          make_float4(a[0] * mul, a[1] * mul, b[0] * mul, b[1] * mul);
    }
  }
}

__global__ void __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_tiles_kernel(const __half* __restrict__ q, int hq, int hkv,
                    const uint8_t* __restrict__ pool, long long num_blocks,
                    const int32_t* __restrict__ block_table, int max_blocks,
                    const int32_t* __restrict__ seq_lens, float sm_scale,
                    float* __restrict__ partials) {
  __shared__ TileSmem sm;
  const int split = blockIdx.x, nsplit = gridDim.x;
  const int ngroups = (hq / hkv + kHeadGroup - 1) / kHeadGroup;
  const int g = blockIdx.y / ngroups, hg = blockIdx.y % ngroups;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int group = hq / hkv;
  const int h0 = g * group + hg * kHeadGroup;                 // first query head served
  const int nh = min(kHeadGroup, group - hg * kHeadGroup);    // heads served (1..8)
  const int len = seq_lens[b];
  bool bad = len < 0 || (len >> 7) > max_blocks;
  const int n_full = bad ? 0 : (len >> 7);
  const int chunk = (n_full + nsplit - 1) / nsplit;
  const int i0 = min(split * chunk, n_full), i1 = min(i0 + chunk, n_full);
  // this wave's tiles: i0 + wave + 4 j, j < nw. Lane j holds the block id of tile j (ids are
  // fetched 64 at a time with one vector load), tile j's id is read back as a scalar.
  const int ntile = i1 - i0;
  const int nw = ntile > wave ? (ntile - wave + kWaves - 1) / kWaves : 0;
  const int32_t* bt_row = block_table + (long long)b * max_blocks + i0 + wave;
  auto fetch_ids = [&](int j0) -> int {
    const int j = j0 + lane;
    return j < nw ? bt_row[kWaves * j] : 0;
  };
  int ids = fetch_ids(0);
  auto block_of = [&](int j) -> long long {
    return (long long)__builtin_amdgcn_readlane(ids, j & 63);
  };
  TileRegs cur;
  if (nw > 0) {
    const long long blk = block_of(0);
    if (blk < 0 || blk >= num_blocks) bad = true;
    else load_tile(pool + (blk * hkv + g) * (long long)kTileBytes, lane, cur);
  }

  // ---- rotated queries in LDS, and a power-of-two prescale for the fp16 query operand
  for (int idx = tid; idx < kHeadGroup * kD; idx += kTThreads) {
    const int gg = idx >> 7, j = idx & (kD - 1);
    sm.qrot[gg][j] = gg < nh ? __half2float(q[((long long)b * hq + h0 + gg) * kD + j]) : 0.0f;
  }
  __syncthreads();
  for (int h = 1; h < kD; h <<= 1) {
    for (int p = tid; p < kHeadGroup * (kD / 2); p += kTThreads) {
      const int gg = p >> 6, pi = p & 63;
      const int i = (pi / h) * 2 * h + (pi % h);
      const float a = sm.qrot[gg][i], c = sm.qrot[gg][i + h];
      sm.qrot[gg][i] = a + c;
      sm.qrot[gg][i + h] = a - c;
    }
    __syncthreads();
  }
  float qmax = 0.0f;
  for (int idx = tid; idx < kHeadGroup * kD; idx += kTThreads) {
    const float v = sm.qrot[idx >> 7][idx & (kD - 1)] * 0.08838834764831845f;
    sm.qrot[idx >> 7][idx & (kD - 1)] = v;
    qmax = fmaxf(qmax, fabsf(v));
  }
  qmax = wave_max(qmax);
  if (lane == 0) sm.red[wave] = qmax;
  __syncthreads();
  qmax = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
  // |q~ * pq| <= qmax * 448 * pq <= 2^14 keeps the hi part finite in fp16
  int qe = 0;
  frexpf(fmaxf(qmax, 1e-30f) * 448.0f, &qe);
  const float pq = ldexpf(1.0f, 14 - qe);
  const float scale2 = sm_scale * kLog2e;
  const float kfac = scale2 * 16.0f / pq;          // undoes the code / 16 encoding and pq
  const float kzfac = scale2 / pq;                 // multiplies pq * sum_j q~_j
  for (int idx = tid; idx < kHeadGroup * kD; idx += kTThreads)
    sm.qrot[idx >> 7][idx & (kD - 1)] *= pq;
  __syncthreads();

  // lane roles: m / s for operand rows and k groups, n for columns
  const int n = lane & 15, s = lane >> 4;
  const int gq = n & 7;                              // head of this column / row
  const bool colv = gq < nh;                         // column carries a real head
  const bool colhi = n < 8;
  WaveMeta& wm = sm.wm[wave];
  // per-lane copies of the code masks (kept in VGPRs) and the wave-uniform exponent word
  uint32_t kmask = 0x03C003C0u, vmask = 0x03000300u;
  asm volatile("" : "+v"(kmask), "+v"(vmask));
  const uint32_t one16 = __builtin_amdgcn_readfirstlane(0x3C003C00u);

  // running state: score-lane view (column n) and output-row view (rows 4 s + i)
  float m_run = -INFINITY, l_run = 0.0f;
  float4v oacc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) oacc[nb] = (float4v){0.f, 0.f, 0.f, 0.f};

  // Tile pipeline without extra registers: the next tile's key codes (and metadata) are
  // loaded into the key registers once the score products have consumed them, and the next
  // value codes into the value registers once the output products have.
  for (int j = 0; j < nw && !bad; ++j) {
    const uint8_t* nrec = nullptr;
    if (j + 1 < nw) {
      if (((j + 1) & 63) == 0) ids = fetch_ids(j + 1);
      const long long blk = block_of(j + 1);
      if (blk >= 0 && blk < num_blocks) nrec = pool + (blk * hkv + g) * (long long)kTileBytes;
      else bad = true;                             // finishes this tile, then stops
    }
    decode_meta(cur.meta, lane, wm, kfac, kzfac);   // wave-local LDS tables (in-order LDS)

    // ---- query operand for this tile: pq q~ = pq q_rot * c-hat^K, hi (cols 0-7) or lo (8-15)
    // element e of channel block c is channel 32 s + 8 c + {0,4,1,5,2,6,3,7}[e]
    half8 qb[4];
    float asum = 0.0f;                            // pq * sum_j q~_j over this lane's channels
    {
      const float4* qr4 = reinterpret_cast<const float4*>(sm.qrot[gq] + 32 * s);
      const float4* kc4 = reinterpret_cast<const float4*>(wm.kc + 32 * s);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 qa = qr4[2 * c], qc = qr4[2 * c + 1];
        const float4 ka = kc4[2 * c], kk = kc4[2 * c + 1];
        const float x0 = qa.x * ka.x, x1 = qa.y * ka.y, x2 = qa.z * ka.z, x3 = qa.w * ka.w;
        const float x4 = qc.x * kk.x, x5 = qc.y * kk.y, x6 = qc.z * kk.z, x7 = qc.w * kk.w;
        asum += ((x0 + x1) + (x2 + x3)) + ((x4 + x5) + (x6 + x7));
        uint32_t u0 = split_pair(x0, x4, colhi), u1 = split_pair(x1, x5, colhi);
        uint32_t u2 = split_pair(x2, x6, colhi), u3 = split_pair(x3, x7, colhi);
        if (!colv) u0 = u1 = u2 = u3 = 0u;
        qb[c] = as_h8(u0, u1, u2, u3);
      }
    }
    asum += __shfl_xor(asum, 16);
    asum += __shfl_xor(asum, 32);                 // over all 128 channels of column n

    // ---- scores: 8 token blocks x 4 channel blocks
    float4v sc[8];
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const uint32_t w4[4] = {cur.kw[mb].x, cur.kw[mb].y, cur.kw[mb].z, cur.kw[mb].w};
      float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // nibble q of the word -> mantissa bits 6..9 of a half under exponent 0x3C00:
        // the half is 1 + code / 16 (normal, exact); slots (q, q + 4) share a word
        const uint32_t w = w4[c];
        const half8 a = as_h8(and_or(w << 6, kmask, one16), and_or(w << 2, kmask, one16),
                              and_or(w >> 2, kmask, one16), and_or(w >> 6, kmask, one16));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[c], acc, 0, 0, 0);
      }
      sc[mb] = acc;
    }
    if (nrec != nullptr) {
      const int m = lane & 15;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
        cur.kw[mb] = *reinterpret_cast<const uint4*>(nrec + kKCodesOff + (16 * mb + m) * 64 + 16 * s);
      cur.meta = *reinterpret_cast<const uint4*>(nrec + kKMetaOff + lane * 16);
    }
    // hi + lo partial scores, then the full log2-domain score per token:
    // D = pq sum_j (1 + code_j / 16) q~_j, so pq <q~, code> = 16 (D - asum)
    float tmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int t0 = 16 * mb + 4 * s;
      const float4 ks4 = *reinterpret_cast<const float4*>(wm.ks + t0);
      const float4 kz4 = *reinterpret_cast<const float4*>(wm.kz + t0);
      const float ksv[4] = {ks4.x, ks4.y, ks4.z, ks4.w};
      const float kzv[4] = {kz4.x, kz4.y, kz4.z, kz4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float d = sc[mb][i] + dpp_ror8(sc[mb][i]);
        const float v = fmaf(ksv[i], d - asum, kzv[i] * asum);
        sc[mb][i] = v;
        tmax = fmaxf(tmax, v);
      }
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);   // 0 on the first tile
    float psum = 0.0f, beta = 0.0f, wsum = 0.0f;
    // probabilities -> operand rows: hi(p s-hat^V 32) on rows 0-7, lo on rows 8-15;
    // element e of token block kb is token 32 kb + 16 (e / 4) + 4 s + e % 4
    half8 wa[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      uint32_t u[4];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int mb = 2 * kb + h2, t0 = 16 * mb + 4 * s;
        const float4 vs4 = *reinterpret_cast<const float4*>(wm.vs + t0);
        const float4 vz4 = *reinterpret_cast<const float4*>(wm.vz + t0);
        const float p0 = __builtin_amdgcn_exp2f(sc[mb][0] - mnew);
        const float p1 = __builtin_amdgcn_exp2f(sc[mb][1] - mnew);
        const float p2 = __builtin_amdgcn_exp2f(sc[mb][2] - mnew);
        const float p3 = __builtin_amdgcn_exp2f(sc[mb][3] - mnew);
        psum += (p0 + p1) + (p2 + p3);
        beta = fmaf(p0, vz4.x, fmaf(p1, vz4.y, fmaf(p2, vz4.z, fmaf(p3, vz4.w, beta))));
        const float w0 = p0 * vs4.x, w1 = p1 * vs4.y, w2 = p2 * vs4.z, w3 = p3 * vs4.w;
        wsum += (w0 + w1) + (w2 + w3);
        u[2 * h2] = split_pair(w0, w1, colhi);
        u[2 * h2 + 1] = split_pair(w2, w3, colhi);
      }
      if (!colv) u[0] = u[1] = u[2] = u[3] = 0u;
      wa[kb] = as_h8(u[0], u[1], u[2], u[3]);
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    beta += __shfl_xor(beta, 16);
    beta += __shfl_xor(beta, 32);
    wsum += __shfl_xor(wsum, 16);
    wsum += __shfl_xor(wsum, 32);
    // output rows get D / 8 per tile: D = sum_t W_t (1 + code / 4), W = 32 p s-hat^V, so
    // sum_t p s-hat^V code = D / 8 - 4 sum_t p s-hat^V = D / 8 - wsum / 8
    beta = fmaf(-0.125f, wsum, beta);
    l_run = fmaf(alpha, l_run, psum);
    m_run = mnew;
    if (s == 0) {
      wm.alpha[n] = alpha;
      wm.beta[n] = colhi ? beta : 0.0f;           // the zero-point term enters the hi row once
    }

    // ---- output: 8 channel blocks x 4 token blocks; each channel block's accumulator is
    // folded into o~ as soon as its 4 products are done (rows 4 s + i: alpha and beta of
    // their head, c-hat^V of column 16 nb + n)
    {
      const float4 a4 = *reinterpret_cast<const float4*>(wm.alpha + ((4 * s) & 7));
      const float4 b4 = *reinterpret_cast<const float4*>(wm.beta + 4 * s);
      const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
      const float br[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        float4v po = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          // field nb (bits 2 nb and 16 + 2 nb) -> mantissa bits 8..9 under exponent 0x3C00:
          // the half is 1 + code / 4 (normal, exact)
          const uint32_t v4[4] = {cur.vw[kb].x, cur.vw[kb].y, cur.vw[kb].z, cur.vw[kb].w};
          uint32_t f[4];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t x = nb < 4 ? (v4[d] << (8 - 2 * nb)) : (v4[d] >> (2 * nb - 8));
            f[d] = and_or(x, vmask, one16);
          }
          po = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa[kb], as_h8(f[0], f[1], f[2], f[3]),
                                                      po, 0, 0, 0);
        }
        const float cv = wm.vc[16 * nb + n];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          oacc[nb][i] = fmaf(ar[i], oacc[nb][i], cv * fmaf(po[i], 0.125f, br[i]));
      }
    }
    if (nrec != nullptr) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        cur.vw[kb] = *reinterpret_cast<const uint4*>(nrec + kVCodesOff + kb * 1024 + lane * 16);
    }
  }

  // ---- combine the waves' states in LDS and write one partial per (split, head)
  // (score lanes s == 0 hold m, l of column n; rows 4 s + i hold o~ hi (s < 2) and lo parts)
  __syncthreads();
  if (s == 0 && colhi) {
    sm.comb_m[wave][n] = m_run;
    sm.comb_l[wave][n] = l_run;
  }
  {
    // add the lo rows (lanes 32..63) into the hi rows (lanes 0..31)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float other = __shfl_xor(oacc[nb][i], 32);
        if (s < 2) sm.comb_o[wave][4 * s + i][16 * nb + n] = oacc[nb][i] + other;
      }
    }
  }
  __syncthreads();
  const int wbad = __syncthreads_or(bad ? 1 : 0);
  for (int idx = tid; idx < nh * kD; idx += kTThreads) {
    const int gg = idx >> 7, j = idx & (kD - 1);
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, sm.comb_m[w][gg]);
    float ll = 0.0f, oo = 0.0f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = exp2f(sm.comb_m[w][gg] - mm);
        ll = fmaf(f, sm.comb_l[w][gg], ll);
        oo = fmaf(f, sm.comb_o[w][gg][j], oo);
      }
    }
    float* p = partials + (((long long)b * hq + h0 + gg) * nsplit + split) * kPartialFloats;
    if (j == 0) {
      p[0] = wbad ? NAN : mm;
      p[1] = wbad ? NAN : ll;
    }
    p[2 + j] = oo;
  }
}

// grid (hq, batch), one wave per (sequence, query head): the staging tokens (exact fp32
// attention with the unrotated query), the log-sum-exp merge of the tile splits, o~ H + o_raw,
// / l. Lane l owns output channels 2 l and 2 l + 1; the inverse rotation is a butterfly on
// channel bit 0 in registers and on bits 1..6 across lanes l ^ 1 .. l ^ 32.
constexpr int kMThreads = 64;
constexpr int kMaxSplits = 64;

struct MergeSmem {
  float q[kD];              // raw query (fp32)
  float p[kT];              // staging probabilities exp2(s_t - m)
  float w[kMaxSplits];      // split weights exp2(m_split - m)
};

template <int kMask>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (kMask == 1)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
  else if constexpr (kMask == 2)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
  else if constexpr (kMask == 8)
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
  else if constexpr (kMask == 32)
    return __shfl_xor(v, 32);
  else   // 4, 16: swizzle in bit-mask mode, xor within 32 lanes
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (kMask << 10) | 0x1F));
}

// One butterfly stage across lanes: the lane with the bit clear gets own + partner, the lane
// with it set gets partner - own.
template <int kMask>
__device__ __forceinline__ float fwht_lane_stage(float v, int lane) {
  return fmaf((lane & kMask) ? -1.0f : 1.0f, v, lane_xor<kMask>(v));
}

// <q, k> over 128 channels: k is one fp16 staging row, q the fp32 query in LDS.
__device__ __forceinline__ float staging_dot(const __half* __restrict__ krow, const float* qs) {
  const uint4* k4 = reinterpret_cast<const uint4*>(krow);
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    float kv[8];
    unpack_h8(k4[k], kv);
    const float4 qa = *reinterpret_cast<const float4*>(qs + 8 * k);
    const float4 qc = *reinterpret_cast<const float4*>(qs + 8 * k + 4);
    acc0 = fmaf(qa.x, kv[0], fmaf(qa.y, kv[1], fmaf(qa.z, kv[2], fmaf(qa.w, kv[3], acc0))));
    acc1 = fmaf(qc.x, kv[4], fmaf(qc.y, kv[5], fmaf(qc.z, kv[6], fmaf(qc.w, kv[7], acc1))));
  }
  return acc0 + acc1;
}

__global__ void __launch_bounds__(kMThreads)
decode_merge_kernel(const __half* __restrict__ q, int hq, int hkv, int max_blocks,
                    const int32_t* __restrict__ seq_lens, const __half* __restrict__ staging_k,
                    const __half* __restrict__ staging_v, float sm_scale,
                    const float* __restrict__ partials, int nsplit, float* __restrict__ out) {
  __shared__ MergeSmem sm;
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int group = hq / hkv, g = h / group;
  const int len = seq_lens[b];
  const bool bad = len < 0 || (len >> 7) > max_blocks;
  const int n_stage = bad ? 0 : (len & (kT - 1));
  const float scale2 = sm_scale * kLog2e;
  const __half* sk = staging_k + ((long long)b * hkv + g) * kT * kD;
  const __half* sv = staging_v + ((long long)b * hkv + g) * kT * kD;
  {
    const uint32_t w = reinterpret_cast<const uint32_t*>(q + ((long long)b * hq + h) * kD)[lane];
    sm.q[2 * lane] = fp16_bits_to_float(w & 0xFFFFu);
    sm.q[2 * lane + 1] = fp16_bits_to_float(w >> 16);
  }
  __syncthreads();
  // staging scores of tokens lane and lane + 64, split maxima and sums of lane's split
  float s0 = -INFINITY, s1 = -INFINITY;
  if (lane < n_stage) s0 = staging_dot(sk + lane * kD, sm.q) * scale2;
  if (lane + 64 < n_stage) s1 = staging_dot(sk + (lane + 64) * kD, sm.q) * scale2;
  const float* pp = partials + ((long long)b * hq + h) * nsplit * kPartialFloats;
  const float msp = lane < nsplit ? pp[lane * kPartialFloats] : -INFINITY;
  const float lsp = lane < nsplit ? pp[lane * kPartialFloats + 1] : 0.0f;
  const bool invalid = bad || __any(msp != msp);
  const float mm = wave_max(fmaxf(msp, fmaxf(s0, s1)));
  float ls = 0.0f, wsp = 0.0f, p0 = 0.0f, p1 = 0.0f;
  if (mm != -INFINITY) {
    wsp = lane < nsplit ? exp2f(msp - mm) : 0.0f;
    p0 = exp2f(s0 - mm);
    p1 = exp2f(s1 - mm);
    ls = fmaf(wsp, lsp, p0 + p1);
  }
  ls = wave_sum(ls);
  sm.w[lane] = wsp;
  sm.p[lane] = p0;
  sm.p[lane + 64] = p1;
  __syncthreads();
  // merged rotated output o~ of channels 2 lane, 2 lane + 1
  float o0 = 0.0f, o1 = 0.0f;
  if (mm != -INFINITY && !invalid) {
    const float* col = pp + 2 + 2 * lane;
#pragma unroll 4
    for (int sp = 0; sp < nsplit; ++sp) {
      const float2 v = *reinterpret_cast<const float2*>(col + sp * kPartialFloats);
      const float w = sm.w[sp];
      o0 = fmaf(w, v.x, o0);
      o1 = fmaf(w, v.y, o1);
    }
  }
  {
    const float a = o0 + o1, c = o0 - o1;
    o0 = a;
    o1 = c;
  }
  o0 = fwht_lane_stage<1>(o0, lane);   o1 = fwht_lane_stage<1>(o1, lane);
  o0 = fwht_lane_stage<2>(o0, lane);   o1 = fwht_lane_stage<2>(o1, lane);
  o0 = fwht_lane_stage<4>(o0, lane);   o1 = fwht_lane_stage<4>(o1, lane);
  o0 = fwht_lane_stage<8>(o0, lane);   o1 = fwht_lane_stage<8>(o1, lane);
  o0 = fwht_lane_stage<16>(o0, lane);  o1 = fwht_lane_stage<16>(o1, lane);
  o0 = fwht_lane_stage<32>(o0, lane);  o1 = fwht_lane_stage<32>(o1, lane);
  // raw staging output
  float r0 = 0.0f, r1 = 0.0f;
  const uint32_t* vcol = reinterpret_cast<const uint32_t*>(sv) + lane;
  for (int t = 0; t < n_stage; ++t) {
    const uint32_t w = vcol[t * (kD / 2)];
    const float pt = sm.p[t];
    r0 = fmaf(pt, fp16_bits_to_float(w & 0xFFFFu), r0);
    r1 = fmaf(pt, fp16_bits_to_float(w >> 16), r1);
  }
  float2 res = make_float2(0.0f, 0.0f);
  if (invalid) {
    res = make_float2(NAN, NAN);
  } else if (ls > 0.0f) {
    res.x = fmaf(o0, 0.08838834764831845f, r0) / ls;
    res.y = fmaf(o1, 0.08838834764831845f, r1) / ls;
  }
  reinterpret_cast<float2*>(out + ((long long)b * hq + h) * kD)[lane] = res;
}

}  // namespace

int decode_splits(int batch, int hkv, int max_blocks) {
  const long long pairs = (long long)batch * hkv;
  // about 512 workgroups (2048 waves: one round at 2 waves per SIMD on 256 CUs)
  long long s = (512 + pairs - 1) / (pairs > 0 ? pairs : 1);
  const long long per_wave = (max_blocks + kWaves - 1) / kWaves;   // >= one tile per wave
  if (s > per_wave) s = per_wave;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_decode(const __half* q, int hq, int hkv, const uint8_t* pool,
                         long long num_blocks, const int32_t* block_table, int max_blocks,
                         const int32_t* seq_lens, const __half* staging_k,
                         const __half* staging_v, float sm_scale, float* out, float* partials,
                         int splits, int batch, hipStream_t stream) {
  const int ngroups = (hq / hkv + kHeadGroup - 1) / kHeadGroup;
  hipLaunchKernelGGL(decode_tiles_kernel, dim3(splits, hkv * ngroups, batch), dim3(kTThreads),
                     0, stream, q, hq, hkv, pool, num_blocks, block_table, max_blocks, seq_lens,
                     sm_scale, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel, dim3(hq, batch), dim3(kMThreads), 0, stream, q, hq,
                     hkv, max_blocks, seq_lens, staging_k, staging_v, sm_scale, partials, splits,
                     out);
  return hipGetLastError();
}

}  // namespace kvarn
