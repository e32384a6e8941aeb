// KVarN paged decode attention over packed K4/V2 tiles (read path) for gfx950.
//
// [GR] "The four-stage pipeline" (groundy.com, "Huawei's KVarN puts KV-cache quantization
// inside vLLM's backend"), stage 4: scales are applied when a tile is read for attention.
// Nothing is dequantised to memory. Because the rotation H of stage 1 is orthonormal and
// symmetric, q . k = (qH) . (kH); so per tile, with q_rot = qH:
//   q~_j   = q_rot_j * c-hat^K_j                        (per-channel key scale into the query)
//   s_t    = sm * (s-hat^K_t * <q~, codeK_t> + z-hat^K_t * sum_j q~_j)
//                                                       (per-token key scale into the score)
//   acc_j  = sum_t (p_t s-hat^V_t) codeV_tj,  beta = sum_t p_t z-hat^V_t
//   o~_j  += c-hat^V_j * (acc_j + beta)                 (value scales into the probabilities
//                                                        and the per-tile partial output)
// with an online (running max / running sum) softmax across tiles, and the raw fp16 staging
// tokens attended with the unrotated query into a second, unrotated accumulator sharing the
// same max and sum. Each sequence's tiles are split over several workgroups (flash-decoding
// style); a merge kernel combines the splits by log-sum-exp, rotates the packed-tile part of
// the output back (o~ H) and normalises.
//
// This version computes the dot products on the vector ALUs in fp32: one workgroup of 256
// threads per (split, KV head, sequence) walks its tiles one by one; scores use thread
// (token, channel half), the value products thread (channel, head parity).

#include "kvarn_device.hpp"
#include "kvarn_kernels.hpp"

namespace kvarn {

namespace {

constexpr int kDThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

struct DecSmem {
  float qrot[kMaxGroup][kD];
  float qraw[kMaxGroup][kD];
  float qt[kMaxGroup][kD];
  float sc[kMaxGroup][kT];
  uint8_t cv[kT][kD];
  float asum[kMaxGroup];
  float m[kMaxGroup], l[kMaxGroup], alpha[kMaxGroup], beta[kMaxGroup];
  float kc[kD], ks[kT], kz[kT], vc[kD], vs[kT], vz[kT];
};

// Online-softmax update of heads handled by this wave; sc holds log2-domain scores for the
// first n tokens. Replaces sc[g][t] by p_t * (vs ? vs[t] : 1) and records alpha, beta.
__device__ __forceinline__ void softmax_update(DecSmem& sm, int group, int n, bool packed) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int g = wave; g < group; g += kDThreads / 64) {
    const float s0 = lane < n ? sm.sc[g][lane] : -INFINITY;
    const float s1 = lane + 64 < n ? sm.sc[g][lane + 64] : -INFINITY;
    const float mt = wave_max(fmaxf(s0, s1));
    const float mold = sm.m[g];
    const float mnew = fmaxf(mold, mt);
    const float alpha = (mold == -INFINITY) ? 0.0f : exp2f(mold - mnew);
    const float p0 = lane < n ? exp2f(s0 - mnew) : 0.0f;
    const float p1 = lane + 64 < n ? exp2f(s1 - mnew) : 0.0f;
    const float lsum = wave_sum(p0 + p1);
    float beta = 0.0f;
    if (packed) {
      beta = wave_sum(p0 * sm.vz[lane] + p1 * sm.vz[lane + 64]);
      sm.sc[g][lane] = p0 * sm.vs[lane];
      sm.sc[g][lane + 64] = p1 * sm.vs[lane + 64];
    } else {
      sm.sc[g][lane] = p0;
      sm.sc[g][lane + 64] = p1;
    }
    if (lane == 0) {
      sm.m[g] = mnew;
      sm.l[g] = alpha * sm.l[g] + lsum;
      sm.alpha[g] = alpha;
      sm.beta[g] = beta;
    }
  }
}

__global__ void __launch_bounds__(kDThreads)
decode_kernel(const __half* __restrict__ q, int hq, int hkv, const uint8_t* __restrict__ pool,
              long long num_blocks, const int32_t* __restrict__ block_table, int max_blocks,
              const int32_t* __restrict__ seq_lens, const __half* __restrict__ staging_k,
              const __half* __restrict__ staging_v, float sm_scale,
              float* __restrict__ partials) {
  __shared__ DecSmem sm;
  const int split = blockIdx.x, nsplit = gridDim.x;
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int group = hq / hkv;
  const int len = seq_lens[b];
  bool bad = len < 0 || (len >> 7) > max_blocks;
  const int n_full = bad ? 0 : (len >> 7);
  const int n_stage = bad ? 0 : (len & (kT - 1));
  const int chunk = (n_full + nsplit - 1) / nsplit;
  const int i0 = min(split * chunk, n_full), i1 = min(i0 + chunk, n_full);
  const bool do_stage = (split == nsplit - 1) && n_stage > 0;
  const float scale2 = sm_scale * kLog2e;

  // queries: raw and rotated (128-point FWHT in LDS, scaled by 2^-3.5)
  for (int idx = tid; idx < group * kD; idx += kDThreads) {
    const int gg = idx >> 7, j = idx & (kD - 1);
    const float v = __half2float(q[((long long)b * hq + g * group + gg) * kD + j]);
    sm.qraw[gg][j] = v;
    sm.qrot[gg][j] = v;
  }
  if (tid < group) {
    sm.m[tid] = -INFINITY;
    sm.l[tid] = 0.0f;
  }
  __syncthreads();
  for (int h = 1; h < kD; h <<= 1) {
    for (int p = tid; p < group * (kD / 2); p += kDThreads) {
      const int gg = p / (kD / 2), pi = p % (kD / 2);
      const int i = (pi / h) * 2 * h + (pi % h);
      const float a = sm.qrot[gg][i], c = sm.qrot[gg][i + h];
      sm.qrot[gg][i] = a + c;
      sm.qrot[gg][i + h] = a - c;
    }
    __syncthreads();
  }
  for (int idx = tid; idx < group * kD; idx += kDThreads)
    sm.qrot[idx >> 7][idx & (kD - 1)] *= 0.08838834764831845f;

  const int t = tid >> 1, hf = tid & 1;        // score mapping
  const int jj = tid & (kD - 1), gh = tid >> 7;  // value mapping: heads gh, gh + 2, ...
  float orot[kMaxGroup / 2], oraw[kMaxGroup / 2];
#pragma unroll
  for (int k = 0; k < kMaxGroup / 2; ++k) orot[k] = oraw[k] = 0.0f;

  for (int i = i0; i < i1; ++i) {
    const long long blk = block_table[(long long)b * max_blocks + i];
    if (blk < 0 || blk >= num_blocks) {
      bad = true;
      break;
    }
    const uint8_t* rec = pool + (blk * hkv + g) * (long long)kTileBytes;
    __syncthreads();   // previous tile fully consumed (also orders the query setup)
    if (tid < kD) {
      sm.kc[tid] = e4m3_to_float(rec[kKMetaOff + kCRel + tid]);
      sm.ks[tid] = e4m3_to_float(rec[kKMetaOff + kSRel + tid]);
      sm.kz[tid] = fp16_bits_to_float(reinterpret_cast<const uint16_t*>(rec + kKMetaOff + kZRel)[tid]);
      sm.vc[tid] = e4m3_to_float(rec[kVMetaOff + kCRel + tid]);
      sm.vs[tid] = e4m3_to_float(rec[kVMetaOff + kSRel + tid]);
      sm.vz[tid] = fp16_bits_to_float(reinterpret_cast<const uint16_t*>(rec + kVMetaOff + kZRel)[tid]);
    }
    {
      const uint4 w4 = reinterpret_cast<const uint4*>(rec + kVCodesOff)[tid];
      const uint32_t wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int w = 4 * tid + e;
        const int kb = w >> 8, ln = (w >> 2) & 63, d = w & 3;
        const int s = ln >> 4, n = ln & 15;
        const int tb = 32 * kb + 16 * (d >> 1) + 4 * s + ((d & 1) << 1);
#pragma unroll
        for (int odd = 0; odd < 2; ++odd)
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
            sm.cv[tb + odd][16 * nb + n] = (wv[e] >> (2 * nb + 16 * odd)) & 3u;
      }
    }
    __syncthreads();
    for (int idx = tid; idx < group * kD; idx += kDThreads)
      sm.qt[idx >> 7][idx & (kD - 1)] = sm.qrot[idx >> 7][idx & (kD - 1)] * sm.kc[idx & (kD - 1)];
    __syncthreads();
    {
      const int lane = tid & 63, wave = tid >> 6;
      for (int gg = wave; gg < group; gg += 4) {
        const float a = wave_sum(sm.qt[gg][lane] + sm.qt[gg][lane + 64]);
        if (lane == 0) sm.asum[gg] = a;
      }
    }
    // key codes of token t, channels 64 hf .. 64 hf + 63
    float kcode[64];
    {
      const uint4* kp = reinterpret_cast<const uint4*>(rec + kKCodesOff + t * 64 + hf * 32);
      const uint4 a = kp[0], c = kp[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int qn = 0; qn < 8; ++qn) kcode[8 * k + qn] = (float)((w[k] >> (4 * qn)) & 15u);
    }
    __syncthreads();
    for (int gg = 0; gg < group; ++gg) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < 64; ++e) dot = fmaf(sm.qt[gg][hf * 64 + e], kcode[e], dot);
      dot += __shfl_xor(dot, 1);
      if (hf == 0) sm.sc[gg][t] = (sm.ks[t] * dot + sm.kz[t] * sm.asum[gg]) * scale2;
    }
    __syncthreads();
    softmax_update(sm, group, kT, true);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxGroup / 2; ++k) {
      const int gg = gh + 2 * k;
      if (gg < group) {
        float acc = 0.0f;
        for (int tt = 0; tt < kT; ++tt) acc = fmaf(sm.sc[gg][tt], (float)sm.cv[tt][jj], acc);
        orot[k] = sm.alpha[gg] * orot[k] + sm.vc[jj] * (acc + sm.beta[gg]);
        oraw[k] *= sm.alpha[gg];
      }
    }
  }

  if (do_stage && !bad) {
    __syncthreads();
    const __half* sk = staging_k + ((long long)b * hkv + g) * kT * kD;
    const __half* sv = staging_v + ((long long)b * hkv + g) * kT * kD;
    float kr[64];
    if (t < n_stage) {
      const uint4* kp = reinterpret_cast<const uint4*>(sk + t * kD + hf * 64);
#pragma unroll
      for (int k = 0; k < 8; ++k) unpack_h8(kp[k], kr + 8 * k);
    } else {
#pragma unroll
      for (int e = 0; e < 64; ++e) kr[e] = 0.0f;
    }
    for (int gg = 0; gg < group; ++gg) {
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < 64; ++e) dot = fmaf(sm.qraw[gg][hf * 64 + e], kr[e], dot);
      dot += __shfl_xor(dot, 1);
      if (hf == 0) sm.sc[gg][t] = dot * scale2;
    }
    __syncthreads();
    softmax_update(sm, group, n_stage, false);
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kMaxGroup / 2; ++k) {
      const int gg = gh + 2 * k;
      if (gg < group) {
        float acc = 0.0f;
        for (int tt = 0; tt < n_stage; ++tt)
          acc = fmaf(sm.sc[gg][tt], __half2float(sv[tt * kD + jj]), acc);
        oraw[k] = sm.alpha[gg] * oraw[k] + acc;
        orot[k] *= sm.alpha[gg];
      }
    }
  }

  __syncthreads();
  // partial of (b, head, split): m, l, o~[128], o_raw[128]
  for (int gg = tid; gg < group; gg += kDThreads) {
    float* p = partials + (((long long)b * hq + g * group + gg) * nsplit + split) * kPartialFloats;
    p[0] = bad ? NAN : sm.m[gg];
    p[1] = bad ? NAN : sm.l[gg];
  }
#pragma unroll
  for (int k = 0; k < kMaxGroup / 2; ++k) {
    const int gg = gh + 2 * k;
    if (gg < group) {
      float* p = partials + (((long long)b * hq + g * group + gg) * nsplit + split) * kPartialFloats;
      p[2 + jj] = orot[k];
      p[2 + kD + jj] = oraw[k];
    }
  }
}

// grid (hq, batch), 128 threads: log-sum-exp merge of the splits, o~ H + o_raw, / l.
__global__ void __launch_bounds__(kD)
merge_kernel(const float* __restrict__ partials, int hq, int nsplit, float* __restrict__ out) {
  __shared__ float buf[kD];
  const int h = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
  const float* base = partials + ((long long)b * hq + h) * nsplit * kPartialFloats;
  float mmax = -INFINITY;
  bool nan = false;
  for (int s = 0; s < nsplit; ++s) {
    const float m = base[s * kPartialFloats];
    nan |= (m != m);
    mmax = fmaxf(mmax, m);
  }
  float lsum = 0.0f, orot = 0.0f, oraw = 0.0f;
  if (mmax != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float* p = base + s * kPartialFloats;
      const float w = exp2f(p[0] - mmax);
      lsum = fmaf(w, p[1], lsum);
      orot = fmaf(w, p[2 + j], orot);
      oraw = fmaf(w, p[2 + kD + j], oraw);
    }
  }
  buf[j] = orot;
  __syncthreads();
  for (int hh = 1; hh < kD; hh <<= 1) {
    float v = 0.0f;
    const float mine = buf[j], other = buf[j ^ hh];
    v = (j & hh) ? (other - mine) : (mine + other);
    __syncthreads();
    buf[j] = v;
    __syncthreads();
  }
  float o = 0.0f;
  if (nan) {
    o = NAN;
  } else if (lsum > 0.0f) {
    o = (buf[j] * 0.08838834764831845f + oraw) / lsum;
  }
  out[((long long)b * hq + h) * kD + j] = o;
}

}  // namespace

int decode_splits(int batch, int hkv, int max_blocks) {
  const long long pairs = (long long)batch * hkv;
  long long s = (1024 + pairs - 1) / (pairs > 0 ? pairs : 1);
  if (s > max_blocks) s = max_blocks;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_decode(const __half* q, int hq, int hkv, const uint8_t* pool,
                         long long num_blocks, const int32_t* block_table, int max_blocks,
                         const int32_t* seq_lens, const __half* staging_k,
                         const __half* staging_v, float sm_scale, float* out, float* partials,
                         int splits, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(decode_kernel, dim3(splits, hkv, batch), dim3(kDThreads), 0, stream, q, hq,
                     hkv, pool, num_blocks, block_table, max_blocks, seq_lens, staging_k,
                     staging_v, sm_scale, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_kernel, dim3(hq, batch), dim3(kD), 0, stream, partials, hq, splits,
                     out);
  return hipGetLastError();
}

}  // namespace kvarn
