// Memory-bound steps of the hot path: the log-sum-exp merge of two partial
// attention results, the PipeFusion patch splice, and the classifier-free
// guidance combine.  All three stream HBM with 16-byte (dwordx4) accesses,
// one contiguous 16-byte group per lane, so every wave-wide load or store
// covers whole contiguous cache lines.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "launch.h"

namespace dit {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// Log-sum-exp merge, in place into a ("SwiftFusion: Scalable Sequence
// Parallelism for Distributed Inference of Diffusion Transformers on GPUs",
// sections 1-2: each KV block that arrives is folded into the device's
// running result).
//
// Each row is handled by `lpr` consecutive lanes of one wave (16 bytes per
// lane), `rpw` rows per wave.  Keeping a row inside one wave makes the
// in-place update of LSE_a safe: every lane of the row reads LSE_a before the
// row's first lane writes it, in program order within the wave.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(void* Oa_,
                                                            float* La,
                                                            const void* Ob_,
                                                            const float* Lb, long long rows,
                                                            int d, int lpr, int rpw) {
  constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte group
  const int lane = threadIdx.x & 63;
  const long long wave = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int rg = lane / lpr;
  const int ch = lane - rg * lpr;
  if (rg >= rpw) return;
  const long long row = wave * rpw + rg;
  if (row >= rows) return;

  const float la = La[row];
  const float lb = Lb[row];
  const size_t off = (size_t)row * d + (size_t)ch * E;

  float a[E], b[E];
  if constexpr (BF16) {
    const bf16x8 va = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(Oa_) + off);
    const bf16x8 vb = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(Ob_) + off);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      a[i] = (float)va[i];
      b[i] = (float)vb[i];
    }
  } else {
    const f32x4 va = *reinterpret_cast<const f32x4*>(static_cast<const float*>(Oa_) + off);
    const f32x4 vb = *reinterpret_cast<const f32x4*>(static_cast<const float*>(Ob_) + off);
#pragma unroll
    for (int i = 0; i < E; ++i) {
      a[i] = va[i];
      b[i] = vb[i];
    }
  }

  float l_new, r[E];
  if (lb == -INFINITY) {        // empty b: a is already the result ...
    if (la != -INFINITY) return;
    l_new = -INFINITY;          // ... unless both are empty: O = 0
#pragma unroll
    for (int i = 0; i < E; ++i) r[i] = 0.f;
  } else if (la == -INFINITY) { // empty a: take b
    l_new = lb;
#pragma unroll
    for (int i = 0; i < E; ++i) r[i] = b[i];
  } else {
    const float m = fmaxf(la, lb);
    const float wa = expf(la - m);
    const float wb = expf(lb - m);
    const float sum = wa + wb;
    const float inv = 1.f / sum;
#pragma unroll
    for (int i = 0; i < E; ++i) r[i] = fmaf(wa, a[i], wb * b[i]) * inv;
    l_new = m + logf(sum);
  }

  if constexpr (BF16) {
    bf16x8 vr;
#pragma unroll
    for (int i = 0; i < E; ++i) vr[i] = (__bf16)r[i];
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(Oa_) + off) = vr;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(Oa_) + off) = f32x4{r[0], r[1], r[2], r[3]};
  }
  if (ch == 0) La[row] = l_new;
}

// ---------------------------------------------------------------------------
// PipeFusion splice (xDiT abstract): the fresh K and V of this device's patch
// overwrite their rows of the persistent KV buffer.  blockIdx.z picks K or V,
// blockIdx.y the (batch, head) segment.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void splice2_kernel(const u32x4* __restrict__ src0,
                                                          u32x4* __restrict__ dst0,
                                                          const u32x4* __restrict__ src1,
                                                          u32x4* __restrict__ dst1,
                                                          long long seg_units,
                                                          long long dst_seg_stride,
                                                          long long dst_offset) {
  const u32x4* src = blockIdx.z ? src1 : src0;
  u32x4* dst = blockIdx.z ? dst1 : dst0;
  const long long seg = blockIdx.y;
  const u32x4* s = src + seg * seg_units;
  u32x4* t = dst + seg * dst_seg_stride + dst_offset;
  const long long stride = (long long)gridDim.x * kThreads;
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < seg_units; i += stride)
    t[i] = s[i];
}

// ---------------------------------------------------------------------------
// Classifier-free guidance ("Accelerating Diffusion via Hybrid Data-Pipeline
// Parallelism Based on Conditional Guidance Scheduling", Technische
// Zusammenfassung, 2.A): out = u + s (c - u), evaluated as s c + (1 - s) u
// with one fused multiply-add so that s = 1 returns c and s = 0 returns u
// exactly in fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void cfg_kernel(const float* u,
                                                      const float* c, float* out,
                                                      long long n, float s) {
  const long long n4 = n >> 2;
  const long long stride = (long long)gridDim.x * kThreads;
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  const f32x4* u4 = reinterpret_cast<const f32x4*>(u);
  const f32x4* c4 = reinterpret_cast<const f32x4*>(c);
  f32x4* o4 = reinterpret_cast<f32x4*>(out);
  const float t = 1.f - s;
  for (long long i = gid; i < n4; i += stride) {
    const f32x4 a = u4[i], b = c4[i];
    o4[i] = f32x4{fmaf(s, b[0], t * a[0]), fmaf(s, b[1], t * a[1]), fmaf(s, b[2], t * a[2]),
                  fmaf(s, b[3], t * a[3])};
  }
  const long long tail = n - (n4 << 2);
  if (gid < tail) {
    const long long i = (n4 << 2) + gid;
    out[i] = fmaf(s, c[i], t * u[i]);
  }
}

}  // namespace

hipError_t launch_lse_merge(void* Oa, float* La, const void* Ob, const float* Lb,
                            long long rows, int d, bool bf16, hipStream_t stream) {
  const int E = bf16 ? 8 : 4;
  int lpr = d / E;                       // lanes per row; d is a multiple of 8
  int rpw = 64 / lpr;                    // whole rows per wave
  if (lpr > 64) return hipErrorInvalidValue;
  const long long waves = (rows + rpw - 1) / rpw;
  const long long blocks = (waves + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (bf16)
    lse_merge_kernel<true><<<dim3((unsigned)blocks), kThreads, 0, stream>>>(Oa, La, Ob, Lb, rows, d, lpr, rpw);
  else
    lse_merge_kernel<false><<<dim3((unsigned)blocks), kThreads, 0, stream>>>(Oa, La, Ob, Lb, rows, d, lpr, rpw);
  return hipGetLastError();
}

hipError_t launch_splice2(const void* src0, void* dst0, const void* src1, void* dst1, int nseg,
                          long long seg_units, long long dst_seg_stride, long long dst_offset,
                          hipStream_t stream) {
  long long bx = (seg_units + kThreads * 4 - 1) / (kThreads * 4);  // ~4 groups per lane
  if (bx < 1) bx = 1;
  if (bx > 65535) bx = 65535;
  if (nseg > 65535) return hipErrorInvalidValue;
  splice2_kernel<<<dim3((unsigned)bx, (unsigned)nseg, 2), kThreads, 0, stream>>>(
      static_cast<const u32x4*>(src0), static_cast<u32x4*>(dst0), static_cast<const u32x4*>(src1),
      static_cast<u32x4*>(dst1), seg_units, dst_seg_stride, dst_offset);
  return hipGetLastError();
}

hipError_t launch_cfg(const float* u, const float* c, float* out, long long n, float s,
                      hipStream_t stream) {
  const long long n4 = n >> 2;
  long long blocks = (n4 + kThreads * 4 - 1) / (kThreads * 4);
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  cfg_kernel<<<dim3((unsigned)blocks), kThreads, 0, stream>>>(u, c, out, n, s);
  return hipGetLastError();
}

}  // namespace dit
