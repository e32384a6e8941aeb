// Read-only HBM probes for gfx950: the achievable read bandwidth, streaming and in whole tile
// records at random places, beside which the decode kernel's fraction of the 8 TB/s peak can
// be judged. Not part of the codec: they are built into their own library
// (libkvarn_probe.so), which only the benchmark loads.
//
// Every lane streams 16-byte loads through a grid-stride loop with kInFlight loads issued
// before any is consumed, folds them into an XOR, and writes only if the XOR equals a value
// the caller says it will not (so the loads stay live and nothing else is written).

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(kThreads)
read_probe_kernel(const u32x4* __restrict__ buf, unsigned long long n16, uint32_t never,
                  uint32_t* __restrict__ out) {
  const unsigned long long stride = (unsigned long long)gridDim.x * kThreads;
  unsigned long long i = (unsigned long long)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 w[kInFlight];
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) w[k] = __builtin_nontemporal_load(buf + i + k * stride);
#pragma unroll
    for (int k = 0; k < kInFlight; ++k) acc ^= w[k].x ^ w[k].y ^ w[k].z ^ w[k].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 w = buf[i];
    acc ^= w.x ^ w.y ^ w.z ^ w.w;
  }
  if (acc == never) out[0] = acc;
}

// One wave per workgroup reads `per_wave` whole records of kLoads KiB (record index list
// idx[wave * per_wave ...], each clamped below nrec so every access stays in the buffer),
// 16 bytes per lane per load: 1 KiB per wave instruction, all of a record's loads issued before
// any is consumed. The access pattern of the decode's tile loads.
template <int kLoads>
__global__ void __launch_bounds__(64)
record_probe_kernel(const uint8_t* __restrict__ buf, const int32_t* __restrict__ idx,
                    int per_wave, long long nrec, uint32_t never, uint32_t* __restrict__ out) {
  const int lane = threadIdx.x;
  const int32_t* my = idx + (long long)blockIdx.x * per_wave;
  uint32_t acc = 0;
  for (int t = 0; t < per_wave; ++t) {
    long long r = my[t];
    if (r < 0 || r >= nrec) r = 0;
    const u32x4* rec = reinterpret_cast<const u32x4*>(buf + r * (kLoads * 1024LL)) + lane;
    u32x4 w[kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) w[k] = rec[64 * k];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) acc ^= w[k].x ^ w[k].y ^ w[k].z ^ w[k].w;
  }
  if (acc == never) out[0] = acc;
}

}  // namespace

// Whole-record reads: `waves` one-wave workgroups, each reading per_wave records of rec_bytes
// (13,312 or 65,536 — the packed and fp16 tile records) whose indices idx[0 .. waves *
// per_wave) lists (device memory); buf holds buf_bytes (16-byte aligned).
extern "C" __attribute__((visibility("default")))
int kvarn_probe_records(const void* buf, unsigned long long buf_bytes, int rec_bytes,
                        const int32_t* idx, int waves, int per_wave, uint32_t never, void* out,
                        void* stream) {
  if (buf == nullptr || idx == nullptr || out == nullptr || waves < 1 || per_wave < 1 ||
      (reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || buf_bytes < (unsigned long long)rec_bytes)
    return 2;
  const long long nrec = (long long)(buf_bytes / (unsigned long long)rec_bytes);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  uint32_t* o = static_cast<uint32_t*>(out);
  if (rec_bytes == 13 * 1024)
    hipLaunchKernelGGL(record_probe_kernel<13>, dim3((unsigned)waves), dim3(64), 0, s, b, idx,
                       per_wave, nrec, never, o);
  else if (rec_bytes == 64 * 1024)
    hipLaunchKernelGGL(record_probe_kernel<64>, dim3((unsigned)waves), dim3(64), 0, s, b, idx,
                       per_wave, nrec, never, o);
  else
    return 2;
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" __attribute__((visibility("default")))
int kvarn_probe_read(const void* buf, unsigned long long bytes, int workgroups, uint32_t never,
                     void* out, void* stream) {
  if (buf == nullptr || out == nullptr || workgroups < 1 || (bytes & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return 2;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                     bytes / 16, never, static_cast<uint32_t*>(out));
  return hipGetLastError() == hipSuccess ? 0 : 5;
}
