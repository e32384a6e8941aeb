// Read-only HBM streaming probe for gfx950: the achievable read bandwidth beside which the
// decode kernel's fraction of the 8 TB/s peak can be judged. Not part of the codec: it is
// built into its own library (libkvarn_probe.so), which only the benchmark loads.
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

}  // namespace

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
