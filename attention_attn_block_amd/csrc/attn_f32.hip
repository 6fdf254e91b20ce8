// Block attention over float32 Q/K/V with float32 output.
//
// Same definition as the bfloat16 path (softmax(Q K^T * scale) V and the
// natural log-sum-exp per query row), computed on the vector ALU in plain
// fp32 so that no product is rounded below fp32.  This path serves fp32
// callers and small shapes; it is not the throughput path.
//
// One wave per workgroup, one query row per lane.  K/V tiles of 32 keys are
// staged in LDS by the whole wave and read back as broadcasts (all lanes read
// the same key), so there are no bank conflicts.  Online softmax in the log2
// domain, as in the matrix-core kernel.

#include <hip/hip_runtime.h>

#include "launch.h"

namespace dit {
namespace {

constexpr int kRows = 64;  // query rows per workgroup (one wave)
constexpr int kTile = 32;  // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D, bool MERGE>
__global__ __launch_bounds__(kRows) void attn_fwd_f32_kernel(const float* __restrict__ Q,
                                                             const float* __restrict__ K,
                                                             const float* __restrict__ V,
                                                             float* __restrict__ O,
                                                             float* __restrict__ LSE, int Nq,
                                                             int Nkv, int n_qtiles, float c2) {
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  const int bh = blockIdx.x / n_qtiles;
  const int qt = blockIdx.x - bh * n_qtiles;
  const int tid = threadIdx.x;
  const int row = qt * kRows + tid;
  const int rl = row < Nq ? row : Nq - 1;
  const float* Kh = K + (size_t)bh * Nkv * D;
  const float* Vh = V + (size_t)bh * Nkv * D;

  float q[D], o[D];
#pragma unroll
  for (int t = 0; t < D; ++t) {
    q[t] = Q[((size_t)bh * Nq + rl) * D + t];
    o[t] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;

  for (int kv0 = 0; kv0 < Nkv; kv0 += kTile) {
    __syncthreads();
    for (int i = tid; i < kTile * D; i += kRows) {
      const int key = i / D, t = i - key * D;
      int r = kv0 + key;
      r = r < Nkv ? r : Nkv - 1;
      ks[key][t] = Kh[(size_t)r * D + t];
      vs[key][t] = Vh[(size_t)r * D + t];
    }
    __syncthreads();
    const int nk = Nkv - kv0 < kTile ? Nkv - kv0 : kTile;

    float s[kTile];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int t = 0; t < D; ++t) dot = fmaf(q[t], ks[j][t], dot);
      s[j] = j < nk ? dot * c2 : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < D; ++t) o[t] *= alpha;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const float p = __builtin_amdgcn_exp2f(s[j] - m_new);
      l_run += p;
#pragma unroll
      for (int t = 0; t < D; ++t) o[t] = fmaf(p, vs[j][t], o[t]);
    }
    m_run = m_new;
  }

  if (row < Nq) {
    // MERGE folds this block's partial into the running (O, LSE) of the row
    // (log-sum-exp identity; LSE = -inf there marks an empty accumulator).
    const size_t lrow = (size_t)bh * Nq + row;
    const float lse_b = m_run + __builtin_amdgcn_logf(l_run);  // log2 units
    float wb = 1.f / l_run, wa = 0.f, lse_new = lse_b;
    bool has_a = false;
    if constexpr (MERGE) {
      const float la = LSE[lrow] * kLog2e;
      has_a = la != -INFINITY;
      if (has_a) {
        const float m = fmaxf(la, lse_b);
        const float ea = __builtin_amdgcn_exp2f(la - m), eb = __builtin_amdgcn_exp2f(lse_b - m);
        wa = ea / (ea + eb);
        wb = eb / (ea + eb) / l_run;
        lse_new = m + __builtin_amdgcn_logf(ea + eb);
      }
    }
#pragma unroll
    for (int t = 0; t < D; ++t) {
      float* p = O + lrow * D + t;
      float v = o[t] * wb;
      if (MERGE && has_a) v = fmaf(wa, *p, v);
      *p = v;
    }
    LSE[lrow] = lse_new * kLn2;
  }
}

template <int D>
hipError_t launch_d(const float* Q, const float* K, const float* V, float* O, float* LSE, int BH,
                    int Nq, int Nkv, float scale, bool merge, hipStream_t stream) {
  const int n_qtiles = (Nq + kRows - 1) / kRows;
  const dim3 grid((unsigned)(n_qtiles * BH));
  if (merge)
    attn_fwd_f32_kernel<D, true><<<grid, kRows, 0, stream>>>(Q, K, V, O, LSE, Nq, Nkv, n_qtiles, scale * kLog2e);
  else
    attn_fwd_f32_kernel<D, false><<<grid, kRows, 0, stream>>>(Q, K, V, O, LSE, Nq, Nkv, n_qtiles, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                           int BH, int Nq, int Nkv, int d, float scale, bool merge,
                           hipStream_t stream) {
  switch (d) {
#define DIT_CASE(DD) \
  case DD:           \
    return launch_d<DD>(Q, K, V, O, LSE, BH, Nq, Nkv, scale, merge, stream);
    DIT_CASE(8) DIT_CASE(16) DIT_CASE(24) DIT_CASE(32) DIT_CASE(40) DIT_CASE(48) DIT_CASE(56)
    DIT_CASE(64) DIT_CASE(72) DIT_CASE(80) DIT_CASE(88) DIT_CASE(96) DIT_CASE(104) DIT_CASE(112)
    DIT_CASE(120) DIT_CASE(128)
#undef DIT_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace dit
