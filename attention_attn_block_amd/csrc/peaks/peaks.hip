// Measured peaks of one gfx950 GPU, the denominators next to the published
// ones in the benchmark's roofline: a loop of bf16 matrix-core products with
// no memory traffic, and a streaming 16-byte copy.  Not part of the attention
// library (built into libdit_peaks.so); the benchmark times each launch with
// HIP events.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;  // 8 waves, two per SIMD, as the attention kernel
constexpr int kChains = 4;     // independent accumulators per wave
constexpr int kRounds = 4;     // rounds over the chains per loop iteration

// Each wave issues iters x kRounds rounds of kChains independent 32x32x16
// bf16 products (32768 flops each) from registers, then every lane stores one
// float so the products stay live.  sink holds gridDim.x * kThreads floats.
__global__ __launch_bounds__(kThreads, 2) void mfma_loop(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1.0f / (1 + ((lane + i) & 7)));
    b[i] = (__bf16)(0.5f / (1 + ((lane * 3 + i) & 7)));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < kRounds; ++r)
#pragma unroll
      for (int c = 0; c < kChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// dst[i] = src[i] for n 16-byte units: workgroup b copies units
// [b * 256 * U, (b + 1) * 256 * U), lane t the units t, t + 256, ..., all U
// non-temporal loads issued before the stores.
constexpr int kCopyThreads = 256;
template <int U>
__global__ __launch_bounds__(kCopyThreads) void copy16(const u32x4* __restrict__ src,
                                                      u32x4* __restrict__ dst, long long n) {
  const long long base = (long long)blockIdx.x * kCopyThreads * U + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const long long i = base + (long long)k * kCopyThreads;
    if (i < n) v[k] = __builtin_nontemporal_load(src + i);
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const long long i = base + (long long)k * kCopyThreads;
    if (i < n) __builtin_nontemporal_store(v[k], dst + i);
  }
}

}  // namespace

extern "C" {

// Flops of one dit_peak_mfma_bf16 launch: workgroups x 8 waves x iters x
// 4 rounds x 4 chains x 32768.
double dit_peak_mfma_flops(int workgroups, int iters) {
  return (double)workgroups * (kThreads / 64) * iters * kRounds * kChains * 32768.0;
}

// The matrix-core loop on `workgroups` workgroups; sink: workgroups * 512
// floats of device memory.  Returns a hipError_t value (0 on success).
int dit_peak_mfma_bf16(int workgroups, int iters, float* sink, hipStream_t stream) {
  if (workgroups <= 0 || iters <= 0 || !sink) return (int)hipErrorInvalidValue;
  mfma_loop<<<dim3((unsigned)workgroups), kThreads, 0, stream>>>(iters, sink);
  return (int)hipGetLastError();
}

// Copy `bytes` (a positive multiple of 16; both pointers 16-byte aligned)
// with `unroll` (1, 2 or 4) units per lane.
int dit_peak_copy(const void* src, void* dst, long long bytes, int unroll, hipStream_t stream) {
  if (!src || !dst || bytes <= 0 || (bytes & 15) || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15))
    return (int)hipErrorInvalidValue;
  if (unroll != 1 && unroll != 2 && unroll != 4) return (int)hipErrorInvalidValue;
  const long long n = bytes / 16;
  const long long per = (long long)kCopyThreads * unroll;
  const long long blocks = (n + per - 1) / per;
  if (blocks > 0x7fffffffLL) return (int)hipErrorInvalidValue;
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  const dim3 grid((unsigned)blocks);
  if (unroll == 1) copy16<1><<<grid, kCopyThreads, 0, stream>>>(s, d, n);
  else if (unroll == 2) copy16<2><<<grid, kCopyThreads, 0, stream>>>(s, d, n);
  else copy16<4><<<grid, kCopyThreads, 0, stream>>>(s, d, n);
  return (int)hipGetLastError();
}

}  // extern "C"
