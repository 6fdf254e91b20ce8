// Block attention over bfloat16 Q/K/V on gfx950 matrix cores.
//
// Computes O = softmax(Q K^T * scale) V and LSE = ln sum exp(scale Q K^T) for
// one query block against one KV block -- the unit of work a sequence-
// parallel DiT device repeats per KV block ("SwiftFusion: Scalable Sequence
// Parallelism for Distributed Inference of Diffusion Transformers on GPUs",
// sections 1-2; "xDiT: an Inference Engine for Diffusion Transformers (DiTs)
// with Massive Parallelism", abstract).  The key loop is the usual one-pass
// online softmax: a running row maximum and normaliser, with the output
// rescaled whenever the maximum grows, so each KV tile is read once.
//
// Work decomposition (CDNA4, wave64):
//  * A workgroup owns 128 query rows of one (batch, head); each of its four
//    waves owns 32 rows for the whole key loop.
//  * Both contractions run on v_mfma_f32_32x32x16_bf16 in the transposed
//    form S^T = K Q^T and O^T = V^T P^T.  In the 32x32 accumulator layout a
//    lane then holds 16 values of ONE query row (column = lane % 32), so the
//    softmax row max / row sum are in-register reductions plus a single
//    exchange with lane ^ 32, and P never leaves registers: the S^T
//    accumulator registers are exactly the B operand of the PV product once
//    the keys inside each 16-key chunk are visited in the order the
//    accumulator holds them.
//  * K tiles live in LDS row-major (padded rows, conflict-free 16-byte reads
//    of the A operand).  V tiles are written to LDS transposed (d-major) with
//    the same in-chunk key order as P, so the A operand of the PV product is
//    again one 16-byte read per lane.
//  * KV tiles of 64 keys are double-buffered in LDS: the next tile's global
//    loads are issued before the current tile's matrix work and written to the
//    other buffer after it, with one barrier per tile.
//  * Workgroup ids are remapped so that all query tiles of a head run on the
//    same XCD (ids are dealt round-robin over the 8 XCDs), sharing that XCD's
//    L2 for the head's K/V stream.
// Scores are kept in the log2 domain (scale * log2 e folded into one FMA) and
// exponentiated with v_exp_f32; the LSE is converted back to natural log.
// P is rounded to bfloat16 (RNE, v_cvt_pk_bf16_f32) for the PV product; the
// normaliser is summed from the fp32 values.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace dit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;   // 4 waves
constexpr int kBr = 128;        // query rows per workgroup
constexpr int kBc = 64;         // keys per KV tile
constexpr int kVs = kBc + 8;    // transposed-V LDS row stride (elements)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Geo {
  static constexpr int kChunks = (D + 15) / 16;     // 16-wide slices of the QK^T contraction
  static constexpr bool kHalfTail = (D % 16) == 8;  // last slice has 8 real columns
  static constexpr int kDTiles = (D + 31) / 32;     // 32-row tiles of O^T
  static constexpr int kOct = D / 8;                // 16-byte groups per row in memory
  static constexpr int kKs = kChunks * 16 + 8;      // K LDS row stride (elements)
  static constexpr int kKElems = kBc * kKs;
  static constexpr int kVElems = kDTiles * 32 * kVs;
  static constexpr int kKItems = kBc * kOct;        // 16-byte K groups per tile
  static constexpr int kKLoads = (kKItems + kThreads - 1) / kThreads;
  static constexpr int kVItems = (kBc / 4) * kOct;  // (key quad, 16-byte group) items per V tile
  static constexpr int kVLoads = (kVItems + kThreads - 1) / kThreads;
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Value held by lane ^ 32.  v_permlane32_swap(x, x) leaves lanes 0-31 with
// (x[l], x[l+32]) and lanes 32-63 with (x[l-32], x[l]); callers combine the
// pair symmetrically, so own and partner value need not be told apart.
struct Pair {
  float a, b;
};
__device__ __forceinline__ Pair swap32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float max_with_partner32(float x) {
  const Pair p = swap32(x);
  return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float sum_with_partner32(float x) {
  const Pair p = swap32(x);
  return p.a + p.b;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Position of key k (0..63 within a tile) in the transposed-V row.  Inside
// each 16-key chunk the accumulator of S^T gives lanes 0-31 keys
// {0-3, 8-11} and lanes 32-63 keys {4-7, 12-15}; the B operand of the PV
// product takes 8 consecutive slots per half-wave, so key quads 1 and 2 of
// every chunk swap places.
__device__ __forceinline__ int vt_quad_pos(int kq) {
  const int c = kq >> 2, q = kq & 3;
  return 16 * c + 4 * (((q & 1) << 1) | (q >> 1));
}

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    void* __restrict__ Out, float* __restrict__ LSE, int Nq, int Nkv, int n_qtiles, float c2) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][G::kKElems];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][G::kVElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // XCD-aware remap: workgroup ids are dealt round-robin over the 8 XCDs, so
  // give each XCD a contiguous range of (head, query tile) work items.
  const int nblk = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + slot;
  const int bh = logical / n_qtiles;
  const int qt = logical - bh * n_qtiles;

  const __bf16* Qh = Q + (size_t)bh * Nq * D;
  const __bf16* Kh = K + (size_t)bh * Nkv * D;
  const __bf16* Vh = V + (size_t)bh * Nkv * D;

  const int my_q = qt * kBr + wave * 32 + l32;
  const int q_ld = my_q < Nq ? my_q : Nq - 1;

  // Q^T as the B operand: lane holds Q[my_q][16c + 8hi .. +7].
  bf16x8 qf[G::kChunks];
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) {
    if (G::kHalfTail && c == G::kChunks - 1 && hi) {
      qf[c] = bf16x8{};
    } else {
      qf[c] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)q_ld * D + 16 * c + 8 * hi);
    }
  }

  u32x4 kreg[G::kKLoads];
  u32x4 vreg[G::kVLoads][4];

  auto load_tile = [&](int kv0) {
#pragma unroll
    for (int j = 0; j < G::kKLoads; ++j) {
      const int i = tid + kThreads * j;
      if (i < G::kKItems) {
        const int key = i / G::kOct, oc = i - key * G::kOct;
        int row = kv0 + key;
        row = row < Nkv ? row : Nkv - 1;
        kreg[j] = *reinterpret_cast<const u32x4*>(Kh + (size_t)row * D + 8 * oc);
      }
    }
#pragma unroll
    for (int j = 0; j < G::kVLoads; ++j) {
      const int i = tid + kThreads * j;
      if (i < G::kVItems) {
        const int kq = i / G::kOct, oc = i - kq * G::kOct;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int row = kv0 + 4 * kq + r;
          row = row < Nkv ? row : Nkv - 1;
          vreg[j][r] = *reinterpret_cast<const u32x4*>(Vh + (size_t)row * D + 8 * oc);
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < G::kKLoads; ++j) {
      const int i = tid + kThreads * j;
      if (i < G::kKItems) {
        const int key = i / G::kOct, oc = i - key * G::kOct;
        *reinterpret_cast<u32x4*>(&k_lds[buf][key * G::kKs + 8 * oc]) = kreg[j];
      }
    }
#pragma unroll
    for (int j = 0; j < G::kVLoads; ++j) {
      const int i = tid + kThreads * j;
      if (i < G::kVItems) {
        const int kq = i / G::kOct, oc = i - kq * G::kOct;
        const int pos = vt_quad_pos(kq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          u32x2 pk;
          if ((e & 1) == 0) {
            pk.x = (vreg[j][0][w] & 0xffffu) | (vreg[j][1][w] << 16);
            pk.y = (vreg[j][2][w] & 0xffffu) | (vreg[j][3][w] << 16);
          } else {
            pk.x = (vreg[j][0][w] >> 16) | (vreg[j][1][w] & 0xffff0000u);
            pk.y = (vreg[j][2][w] >> 16) | (vreg[j][3][w] & 0xffff0000u);
          }
          *reinterpret_cast<u32x2*>(&v_lds[buf][(8 * oc + e) * kVs + pos]) = pk;
        }
      }
    }
  };

  f32x16 acc[G::kDTiles];
#pragma unroll
  for (int t = 0; t < G::kDTiles; ++t) acc[t] = f32x16{};
  float m_run = -INFINITY;  // running row max, log2 units
  float l_run = 0.f;        // this lane's share of the running normaliser

  const int n_tiles = (Nkv + kBc - 1) / kBc;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int kv0 = t * kBc;
    if (t + 1 < n_tiles) load_tile(kv0 + kBc);

    // S^T = K Q^T for 64 keys (two 32-key accumulators).
    f32x16 s[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      s[kt] = f32x16{};
#pragma unroll
      for (int c = 0; c < G::kChunks; ++c) {
        bf16x8 a;
        if (G::kHalfTail && c == G::kChunks - 1 && hi) {
          a = bf16x8{};
        } else {
          a = *reinterpret_cast<const bf16x8*>(&k_lds[buf][(kt * 32 + l32) * G::kKs + 16 * c + 8 * hi]);
        }
        s[kt] = mfma32(a, qf[c], s[kt]);
      }
    }

    // Keys past the end of the block (last tile only) get zero weight.
    if (kv0 + kBc > Nkv) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key >= Nkv) s[kt][r] = -INFINITY;
        }
    }

    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = max_with_partner32(mx);
    const float m_new = fmaxf(m_run, mx * c2);
    const float alpha = fast_exp2(m_run - m_new);
    const float neg_m = -m_new;

    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(s[kt][r], c2, neg_m));
        s[kt][r] = p;
        psum += p;
      }
    l_run = fmaf(l_run, alpha, psum);
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;

    // O^T += V^T P^T, 16 keys per product.
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      bf16x8 pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = (__bf16)s[ch >> 1][8 * (ch & 1) + j];
#pragma unroll
      for (int dt = 0; dt < G::kDTiles; ++dt) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&v_lds[buf][(dt * 32 + l32) * kVs + 16 * ch + 8 * hi]);
        acc[dt] = mfma32(a, pb, acc[dt]);
      }
    }

    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = sum_with_partner32(l_run);
  if (my_q < Nq) {
    const float inv = 1.f / l_tot;
    const size_t orow = ((size_t)bh * Nq + my_q) * D;
#pragma unroll
    for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + 8 * g + 4 * hi;
        if (d0 < D) {
          const float o0 = acc[dt][4 * g + 0] * inv, o1 = acc[dt][4 * g + 1] * inv;
          const float o2 = acc[dt][4 * g + 2] * inv, o3 = acc[dt][4 * g + 3] * inv;
          if constexpr (OUT_F32) {
            *reinterpret_cast<f32x4*>(static_cast<float*>(Out) + orow + d0) = f32x4{o0, o1, o2, o3};
          } else {
            bf16x4 v = {(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3};
            *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(Out) + orow + d0) = v;
          }
        }
      }
    if (hi == 0) LSE[(size_t)bh * Nq + my_q] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D>
hipError_t launch_d(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH,
                    int Nq, int Nkv, float scale, bool out_f32, hipStream_t stream) {
  const int n_qtiles = (Nq + kBr - 1) / kBr;
  const dim3 grid((unsigned)(n_qtiles * BH));
  const float c2 = scale * kLog2e;
  const __bf16* q = static_cast<const __bf16*>(Q);
  const __bf16* k = static_cast<const __bf16*>(K);
  const __bf16* v = static_cast<const __bf16*>(V);
  if (out_f32) {
    attn_fwd_bf16_kernel<D, true><<<grid, kThreads, 0, stream>>>(q, k, v, O, LSE, Nq, Nkv, n_qtiles, c2);
  } else {
    attn_fwd_bf16_kernel<D, false><<<grid, kThreads, 0, stream>>>(q, k, v, O, LSE, Nq, Nkv, n_qtiles, c2);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int BH, int Nq, int Nkv, int d, float scale, bool out_f32,
                            hipStream_t stream) {
  switch (d) {
#define DIT_CASE(DD) \
  case DD:           \
    return launch_d<DD>(Q, K, V, O, LSE, BH, Nq, Nkv, scale, out_f32, stream);
    DIT_CASE(8) DIT_CASE(16) DIT_CASE(24) DIT_CASE(32) DIT_CASE(40) DIT_CASE(48) DIT_CASE(56)
    DIT_CASE(64) DIT_CASE(72) DIT_CASE(80) DIT_CASE(88) DIT_CASE(96) DIT_CASE(104) DIT_CASE(112)
    DIT_CASE(120) DIT_CASE(128)
#undef DIT_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace dit
