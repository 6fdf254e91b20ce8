// Memory-bound steps of the hot path: the log-sum-exp merge of two partial
// attention results, the PipeFusion patch splice, and the classifier-free
// guidance combine.  All three stream HBM with 16-byte (dwordx4) accesses,
// one contiguous 16-byte group per lane, so every wave-wide load or store
// covers whole contiguous cache lines.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "launch.h"

namespace dit {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Log-sum-exp merge, in place into a ("SwiftFusion: Scalable Sequence
// Parallelism for Distributed Inference of Diffusion Transformers on GPUs",
// sections 1-2: each KV block that arrives is folded into the device's
// running result).
//
// Each row is handled by `lpr` consecutive lanes of one wave (16 bytes per
// lane), `rpw` rows per wave pass; a wave makes U passes over consecutive
// row groups and issues all of its loads before any arithmetic, so every lane
// keeps 2 U 16-byte loads in flight.  Keeping a row inside one wave makes the
// in-place update of LSE_a safe: every lane of the row reads LSE_a before the
// row's first lane writes it, in program order within the wave.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ T ld(const T* p, bool nt) {
  return nt ? __builtin_nontemporal_load(p) : *p;
}
template <typename T>
__device__ __forceinline__ void st(T* p, T v, bool nt) {
  if (nt) __builtin_nontemporal_store(v, p); else *p = v;
}

template <bool BF16, int U, bool NT>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(void* Oa_, float* La, const void* Ob_,
                                                            const float* Lb, long long rows,
                                                            int d, int lpr, int rpw) {
  constexpr int E = BF16 ? 8 : 4;  // elements per 16-byte group
  typedef typename std::conditional<BF16, bf16x8, f32x4>::type vec;
  typedef typename std::conditional<BF16, __bf16, float>::type elt;
  const int lane = threadIdx.x & 63;
  const long long wave = (long long)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int rg = lane / lpr;
  const int ch = lane - rg * lpr;
  if (rg >= rpw) return;
  elt* Oa = static_cast<elt*>(Oa_);
  const elt* Ob = static_cast<const elt*>(Ob_);

  float la[U], lb[U];
  vec va[U], vb[U];
  size_t off[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const long long row = (wave * U + u) * rpw + rg;
    ok[u] = row < rows;
    off[u] = (size_t)row * d + (size_t)ch * E;
    if (ok[u]) {
      la[u] = La[row];
      lb[u] = Lb[row];
      va[u] = ld(reinterpret_cast<const vec*>(Oa + off[u]), NT);
      vb[u] = ld(reinterpret_cast<const vec*>(Ob + off[u]), NT);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (!ok[u]) continue;
    const long long row = (wave * U + u) * rpw + rg;
    float l_new, r[E];
    if (lb[u] == -INFINITY) {        // empty b: a is already the result ...
      if (la[u] != -INFINITY) continue;
      l_new = -INFINITY;             // ... unless both are empty: O = 0
#pragma unroll
      for (int i = 0; i < E; ++i) r[i] = 0.f;
    } else if (la[u] == -INFINITY) { // empty a: take b
      l_new = lb[u];
#pragma unroll
      for (int i = 0; i < E; ++i) r[i] = (float)vb[u][i];
    } else {
      // Hardware exp2 / log2 / reciprocal (about 1 ulp each): every lane of
      // the row evaluates them, so their cost matters for a streaming kernel.
      const float m = fmaxf(la[u], lb[u]);
      const float wa = __builtin_amdgcn_exp2f((la[u] - m) * kLog2e);
      const float wb = __builtin_amdgcn_exp2f((lb[u] - m) * kLog2e);
      const float sum = wa + wb;
      const float inv = __builtin_amdgcn_rcpf(sum);
#pragma unroll
      for (int i = 0; i < E; ++i) r[i] = fmaf(wa, (float)va[u][i], wb * (float)vb[u][i]) * inv;
      l_new = fmaf(__builtin_amdgcn_logf(sum), kLn2, m);
    }
    vec vr;
#pragma unroll
    for (int i = 0; i < E; ++i) vr[i] = (elt)r[i];
    st(reinterpret_cast<vec*>(Oa + off[u]), vr, NT);
    if (ch == 0) La[row] = l_new;
  }
}

// ---------------------------------------------------------------------------
// PipeFusion splice (xDiT abstract): the fresh K and V of this device's patch
// overwrite their rows of the persistent KV buffer.  The patch is one run of
// rows per (batch, head), or several evenly spaced runs (a band of spatial
// rows across every frame of a video); each (batch, head, run) is a segment.
// blockIdx.z picks K or V; blockIdx.y strides over the segments.
// ---------------------------------------------------------------------------
template <int U>
__global__ __launch_bounds__(kThreads) void splice2_kernel(const u32x4* __restrict__ src0,
                                                          u32x4* __restrict__ dst0,
                                                          const u32x4* __restrict__ src1,
                                                          u32x4* __restrict__ dst1,
                                                          long long nseg, int n_runs,
                                                          long long run_units,
                                                          long long dst_bh_stride,
                                                          long long dst_run_stride,
                                                          long long dst_offset) {
  const u32x4* src = blockIdx.z ? src1 : src0;
  u32x4* dst = blockIdx.z ? dst1 : dst0;
  for (long long seg = blockIdx.y; seg < nseg; seg += gridDim.y) {
    const long long bh = seg / n_runs;
    const long long r = seg - bh * n_runs;
    const u32x4* s = src + seg * run_units;
    u32x4* t = dst + bh * dst_bh_stride + r * dst_run_stride + dst_offset;
    // Each pass moves U groups per lane, all loads issued before the stores
    // (plain accesses: the fresh patch is usually cache-resident).
    const long long pass = (long long)gridDim.x * kThreads * U;
    for (long long b0 = (long long)blockIdx.x * kThreads * U + threadIdx.x; b0 < run_units;
         b0 += pass) {
      u32x4 v[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const long long i = b0 + (long long)k * kThreads;
        if (i < run_units) v[k] = s[i];
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const long long i = b0 + (long long)k * kThreads;
        if (i < run_units) t[i] = v[k];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Classifier-free guidance ("Accelerating Diffusion via Hybrid Data-Pipeline
// Parallelism Based on Conditional Guidance Scheduling", Technische
// Zusammenfassung, 2.A): out = u + s (c - u), evaluated as s c + (1 - s) u
// with one fused multiply-add so that s = 1 returns c and s = 0 returns u
// exactly in fp32.
// ---------------------------------------------------------------------------
template <int U, bool NT>
__global__ __launch_bounds__(kThreads) void cfg_kernel(const float* u, const float* c, float* out,
                                                      long long n, float s) {
  // Block b covers float4 groups [b * kThreads * U, (b + 1) * kThreads * U);
  // lane t takes groups t, t + kThreads, ... so each load instruction is a
  // contiguous 4 KiB per workgroup.  All loads are issued before the stores.
  const long long n4 = n >> 2;
  const long long base = (long long)blockIdx.x * kThreads * U + threadIdx.x;
  const f32x4* u4 = reinterpret_cast<const f32x4*>(u);
  const f32x4* c4 = reinterpret_cast<const f32x4*>(c);
  f32x4* o4 = reinterpret_cast<f32x4*>(out);
  const float t = 1.f - s;
  f32x4 a[U], b[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const long long i = base + (long long)k * kThreads;
    if (i < n4) {
      a[k] = ld(u4 + i, NT);
      b[k] = ld(c4 + i, NT);
    }
  }
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const long long i = base + (long long)k * kThreads;
    if (i < n4)
      st(o4 + i, f32x4{fmaf(s, b[k][0], t * a[k][0]), fmaf(s, b[k][1], t * a[k][1]),
                       fmaf(s, b[k][2], t * a[k][2]), fmaf(s, b[k][3], t * a[k][3])}, NT);
  }
  const long long tail = n - (n4 << 2);
  if (blockIdx.x == 0 && threadIdx.x < tail) {
    const long long i = (n4 << 2) + threadIdx.x;
    out[i] = fmaf(s, c[i], t * u[i]);
  }
}

// ---------------------------------------------------------------------------
// CFG combine fused with the discrepancy signal Hybridiff switches its
// parallel phases on ("Accelerating Diffusion via Hybrid Data-Pipeline
// Parallelism Based on Conditional Guidance Scheduling", Technische
// Zusammenfassung, 2.B).  The page names a relative MAE between the
// conditional and unconditional noise without a formula; the reading used is
// sum|c - u| / sum|u| over the whole tensor.  Each workgroup reduces its
// float4 groups (wave shuffles, then LDS across the 4 waves) to two partial
// sums; a one-workgroup second pass adds the partials in index order, so the
// result is deterministic.
// ---------------------------------------------------------------------------
constexpr int kRelmaeGroupsPerBlock = kThreads * 4;  // float4 groups per workgroup

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__global__ __launch_bounds__(kThreads) void cfg_relmae_kernel(const float* u, const float* c,
                                                             float* out, long long n, float s,
                                                             float* work) {
  __shared__ float red[2][kThreads / 64];
  const long long n4 = n >> 2;
  const f32x4* u4 = reinterpret_cast<const f32x4*>(u);
  const f32x4* c4 = reinterpret_cast<const f32x4*>(c);
  f32x4* o4 = reinterpret_cast<f32x4*>(out);
  const float t = 1.f - s;
  float num = 0.f, den = 0.f;
  const long long base = (long long)blockIdx.x * kRelmaeGroupsPerBlock + threadIdx.x;
  // All of the lane's loads first: `out` may be `u` or `c` itself, and the
  // compiler cannot move a load above an earlier store that might alias it,
  // so a load-compute-store loop would make one HBM round trip per group.
  // Aliasing is only ever exact (same index), so each group's store still
  // follows its own loads.
  constexpr int kG = kRelmaeGroupsPerBlock / kThreads;
  f32x4 a[kG], b[kG];
#pragma unroll
  for (int k = 0; k < kG; ++k) {
    const long long i = base + (long long)k * kThreads;
    if (i < n4) {
      a[k] = __builtin_nontemporal_load(u4 + i);
      b[k] = __builtin_nontemporal_load(c4 + i);
    }
  }
#pragma unroll
  for (int k = 0; k < kG; ++k) {
    const long long i = base + (long long)k * kThreads;
    if (i < n4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        num += fabsf(b[k][e] - a[k][e]);
        den += fabsf(a[k][e]);
      }
      __builtin_nontemporal_store(f32x4{fmaf(s, b[k][0], t * a[k][0]), fmaf(s, b[k][1], t * a[k][1]),
                                        fmaf(s, b[k][2], t * a[k][2]), fmaf(s, b[k][3], t * a[k][3])},
                                  o4 + i);
    }
  }
  if (blockIdx.x == 0 && threadIdx.x < n - (n4 << 2)) {  // scalar tail
    const long long i = (n4 << 2) + threadIdx.x;
    num += fabsf(c[i] - u[i]);
    den += fabsf(u[i]);
    out[i] = fmaf(s, c[i], t * u[i]);
  }
  num = wave_sum(num);
  den = wave_sum(den);
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = num;
    red[1][threadIdx.x >> 6] = den;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      a += red[0][w];
      b += red[1][w];
    }
    work[2 * blockIdx.x] = a;
    work[2 * blockIdx.x + 1] = b;
  }
}

constexpr int kFinishThreads = 1024;  // one workgroup: as many loads in flight as it can hold

__global__ __launch_bounds__(kFinishThreads) void relmae_finish_kernel(const float* work, int nblk,
                                                                      float* relmae) {
  __shared__ double red[2][kFinishThreads / 64];
  double num = 0.0, den = 0.0;
  // Lane t adds entries t, t + kFinishThreads, ... in that order;
  // eight (num, den) pairs are loaded before they are added, and entries past
  // the end add +0, so the order (and the result) is fixed.
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2* w2 = reinterpret_cast<const f32x2*>(work);
  constexpr int kU = 8;
  for (int i0 = threadIdx.x; i0 < nblk; i0 += kFinishThreads * kU) {
    f32x2 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u * kFinishThreads;
      v[u] = i < nblk ? w2[i] : f32x2{0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      num += v[u][0];
      den += v[u][1];
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    num += __shfl_xor(num, o, 64);
    den += __shfl_xor(den, o, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    red[0][threadIdx.x >> 6] = num;
    red[1][threadIdx.x >> 6] = den;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0, b = 0.0;
    for (int w = 0; w < kFinishThreads / 64; ++w) {
      a += red[0][w];
      b += red[1][w];
    }
    // 0/0 (identical all-zero paths) reads as no discrepancy.
    *relmae = (a == 0.0) ? 0.f : (float)(a / b);
  }
}

}  // namespace

// Measured on MI355X (cold HBM, 600+ MB working sets): one row group / one
// float4 group per lane with non-temporal loads and stores streams best
// (merge 5.4 TB/s, CFG 6.4 TB/s); deeper unrolling and cached accesses were
// slower.  The splice moves two 16-byte groups per lane per pass with both
// loads issued first (77% of HBM peak; one group per pass reached 66%).
constexpr int kMergeUnroll = 1;
constexpr bool kMergeNT = true;
constexpr int kCfgUnroll = 1;
constexpr bool kCfgNT = true;
constexpr int kSpliceUnroll = 2;

hipError_t launch_lse_merge(void* Oa, float* La, const void* Ob, const float* Lb,
                            long long rows, int d, bool bf16, hipStream_t stream) {
  const int E = bf16 ? 8 : 4;
  const int lpr = d / E;                 // lanes per row; d is a multiple of 8
  if (lpr > 64) return hipErrorInvalidValue;
  const int rpw = 64 / lpr;              // whole rows per wave pass
  const long long waves = (rows + (long long)rpw * kMergeUnroll - 1) / ((long long)rpw * kMergeUnroll);
  const long long blocks = (waves + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (bf16)
    lse_merge_kernel<true, kMergeUnroll, kMergeNT><<<dim3((unsigned)blocks), kThreads, 0, stream>>>(
        Oa, La, Ob, Lb, rows, d, lpr, rpw);
  else
    lse_merge_kernel<false, kMergeUnroll, kMergeNT><<<dim3((unsigned)blocks), kThreads, 0, stream>>>(
        Oa, La, Ob, Lb, rows, d, lpr, rpw);
  return hipGetLastError();
}

hipError_t launch_splice2(const void* src0, void* dst0, const void* src1, void* dst1,
                          long long n_bh, int n_runs, long long run_units,
                          long long dst_bh_stride, long long dst_run_stride,
                          long long dst_offset, hipStream_t stream) {
  if (n_bh <= 0 || n_runs <= 0 || run_units <= 0) return hipErrorInvalidValue;
  const long long nseg = n_bh * n_runs;
  long long bx = (run_units + kThreads * kSpliceUnroll - 1) / (kThreads * kSpliceUnroll);
  if (bx > 65535) bx = 65535;
  // Segments past the y range of the grid are taken by the kernel's stride loop.
  const long long by = nseg < 65535 ? nseg : 65535;
  splice2_kernel<kSpliceUnroll><<<dim3((unsigned)bx, (unsigned)by, 2), kThreads, 0, stream>>>(
      static_cast<const u32x4*>(src0), static_cast<u32x4*>(dst0), static_cast<const u32x4*>(src1),
      static_cast<u32x4*>(dst1), nseg, n_runs, run_units, dst_bh_stride, dst_run_stride,
      dst_offset);
  return hipGetLastError();
}

hipError_t launch_cfg(const float* u, const float* c, float* out, long long n, float s,
                      hipStream_t stream) {
  const long long n4 = n >> 2;
  long long blocks = (n4 + (long long)kThreads * kCfgUnroll - 1) / ((long long)kThreads * kCfgUnroll);
  if (blocks < 1) blocks = 1;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  cfg_kernel<kCfgUnroll, kCfgNT><<<dim3((unsigned)blocks), kThreads, 0, stream>>>(u, c, out, n, s);
  return hipGetLastError();
}

}  // namespace dit

namespace dit {

long long cfg_relmae_work_floats(long long n) {
  const long long n4 = n >> 2;
  long long blocks = (n4 + kRelmaeGroupsPerBlock - 1) / kRelmaeGroupsPerBlock;
  if (blocks < 1) blocks = 1;
  return 2 * blocks;
}

hipError_t launch_cfg_relmae(const float* u, const float* c, float* out, long long n, float s,
                             float* work, float* relmae, hipStream_t stream) {
  const long long blocks = cfg_relmae_work_floats(n) / 2;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  cfg_relmae_kernel<<<dim3((unsigned)blocks), kThreads, 0, stream>>>(u, c, out, n, s, work);
  relmae_finish_kernel<<<dim3(1), kFinishThreads, 0, stream>>>(work, (int)blocks, relmae);
  return hipGetLastError();
}

}  // namespace dit

// ---------------------------------------------------------------------------
// cfg_combine_relmae without a caller workspace: the per-workgroup partial
// sums go to a fixed device array of this library instead.  Every GPU the
// library runs on holds its own copy of the array (loaded with the code
// object, kept until the process ends).  Host code must not pass the array's
// name to a kernel -- on the host it is only a stand-in -- so the device
// address is looked up once per device with hipGetSymbolAddress (that device
// current) and cached; kernels receive that address.  Calls that overlap on
// one GPU share the array and race.  Nothing in it needs to start at zero:
// the first pass writes every entry the second pass reads.
// ---------------------------------------------------------------------------
static __device__ __align__(256) float scratch[dit::kRelmaeStaticFloats];

namespace dit {
namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's `scratch`, or null on failure.
float* scratch_on(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || !addr) return nullptr;
  p = static_cast<float*>(addr);
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}
}  // namespace

hipError_t launch_cfg_relmae_static(const float* u, const float* c, float* out, long long n,
                                    float s, float* relmae, hipStream_t stream) {
  if (cfg_relmae_work_floats(n) > kRelmaeStaticFloats) return hipErrorInvalidValue;
  int dev = 0;
  if (stream) {
    hipDevice_t sd;
    const hipError_t e = hipStreamGetDevice(stream, &sd);
    if (e != hipSuccess) return e;
    dev = sd;
  } else {
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
  }
  float* work = scratch_on(dev);
  if (!work) return hipErrorInvalidSymbol;
  return launch_cfg_relmae(u, c, out, n, s, work, relmae, stream);
}

}  // namespace dit
