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
// P is rounded to bfloat16 (RNE, v_cvt_pk_bf16_f32) for the PV product and
// the normaliser sums those same bf16 weights (v_dot2_f32_bf16 against ones),
// so the output is an exactly normalised combination of the values.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

namespace dit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;   // 4 waves
constexpr int kBr = 128;        // query rows per workgroup
constexpr int kBc = 64;         // keys per KV tile
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
  static constexpr int kKItems = kBc * kOct;        // 16-byte K (or V) groups per tile
  static constexpr int kKLoads = (kKItems + kThreads - 1) / kThreads;
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

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i names a row of 4 consecutive bf16; lane i then receives element
// (i % 4) of the rows named by lanes 4k + i/4, k = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const __bf16* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

// Row stride (elements) of the row-major V tile in LDS.  A row must hold the
// 32 * kDTiles columns the transposing reads touch; the stride is chosen
// congruent to 64 or 192 bytes modulo 256 so that the four 64-byte row pieces
// one half-wave reads fall in distinct banks.
constexpr int v_stride(int dtiles) { return dtiles == 1 ? 32 : dtiles <= 3 ? 96 : 160; }

// Rescale threshold (log2 units): the running maximum used for the
// exponentials is only moved when a row's score maximum exceeds it by more
// than this, so most tiles skip rescaling the output accumulator.  Weights
// stay below 2^8 and the result is unchanged in exact arithmetic.
constexpr float kTau = 8.f;

template <int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    void* __restrict__ Out, float* __restrict__ LSE, int Nq, int Nkv, int n_qtiles, float c2) {
  using G = Geo<D>;
  constexpr int kVsr = v_stride(G::kDTiles);
  __shared__ __attribute__((aligned(16))) __bf16 k_lds[2][G::kKElems];
  __shared__ __attribute__((aligned(16))) __bf16 v_lds[2][kBc * kVsr];

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

  // K and V tiles are staged through registers: 16-byte groups, row-major.
  // Lane-constant parts of the global and LDS addresses are computed once.
  constexpr bool kFullLoads = (G::kKItems % kThreads) == 0;
  u32x4 kreg[G::kKLoads];
  u32x4 vreg[G::kKLoads];
  int g_off[G::kKLoads];     // element offset of this lane's group inside a tile
  int g_key[G::kKLoads];     // key of that group inside the tile
  int ks_off[G::kKLoads];    // LDS element offsets (K, V)
  int vs_off[G::kKLoads];
#pragma unroll
  for (int j = 0; j < G::kKLoads; ++j) {
    const int i = tid + kThreads * j;
    const int key = i / G::kOct, oc = i - key * G::kOct;
    g_key[j] = key;
    g_off[j] = key * D + 8 * oc;
    ks_off[j] = key * G::kKs + 8 * oc;
    vs_off[j] = key * kVsr + 8 * oc;
  }
  auto active = [&](int j) { return kFullLoads || tid + kThreads * j < G::kKItems; };

  auto load_tile = [&](int kv0) {
    const __bf16* kt = Kh + (size_t)kv0 * D;
    const __bf16* vt = Vh + (size_t)kv0 * D;
    if (kv0 + kBc <= Nkv) {
#pragma unroll
      for (int j = 0; j < G::kKLoads; ++j)
        if (active(j)) {
          kreg[j] = *reinterpret_cast<const u32x4*>(kt + g_off[j]);
          vreg[j] = *reinterpret_cast<const u32x4*>(vt + g_off[j]);
        }
    } else {  // ragged last tile: clamp rows to the block (their weights are zeroed)
#pragma unroll
      for (int j = 0; j < G::kKLoads; ++j)
        if (active(j)) {
          const int over = kv0 + g_key[j] - (Nkv - 1);
          const int back = over > 0 ? over * D : 0;
          kreg[j] = *reinterpret_cast<const u32x4*>(kt + g_off[j] - back);
          vreg[j] = *reinterpret_cast<const u32x4*>(vt + g_off[j] - back);
        }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < G::kKLoads; ++j)
      if (active(j)) {
        *reinterpret_cast<u32x4*>(&k_lds[buf][ks_off[j]]) = kreg[j];
        *reinterpret_cast<u32x4*>(&v_lds[buf][vs_off[j]]) = vreg[j];
      }
  };

  // Per-lane part of the transposing V reads (see lds_read_tr16): lane group
  // g = lane / 16 reads keys 4 (g / 2) + (lane % 16) / 4 of each 8-key half
  // chunk, columns 16 (g % 2) + 4 (lane % 4) of each 32-column d tile.
  const int vg = lane >> 4, vi = lane & 15;
  const int v_lane_off = (4 * (vg >> 1) + (vi >> 2)) * kVsr + 16 * (vg & 1) + 4 * (vi & 3);

  f32x16 acc[G::kDTiles];
#pragma unroll
  for (int t = 0; t < G::kDTiles; ++t) acc[t] = f32x16{};
  float m_ref = 0.f;   // reference row max for the exponentials, log2 units
  float l_run = 0.f;   // this lane's share of the running normaliser (bf16 weights)

  const int n_tiles = (Nkv + kBc - 1) / kBc;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};

  // One 64-key tile.  FIRST: the reference max is set from this tile's
  // maximum.  Later tiles form t = s * c2 - m_ref first (an FMA per score,
  // needed for the exponent anyway), take the row max of t, and only move the
  // reference when some row's max exceeds it by kTau.
  auto tile_step = [&](auto buf_c, auto first_c, int t, bool has_next) {
    constexpr int buf = decltype(buf_c)::value;
    constexpr bool first = decltype(first_c)::value;
    const int kv0 = t * kBc;
    if (has_next) load_tile(kv0 + kBc);

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

    if constexpr (first) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] *= c2;
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
      m_ref = max_with_partner32(mx);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] -= m_ref;
    } else {
      const float neg_m = -m_ref;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = fmaf(s[kt][r], c2, neg_m);
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
      mx = max_with_partner32(mx);
      const bool grow = mx > kTau;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float delta = grow ? mx : 0.f;
        const float alpha = fast_exp2(-delta);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
        m_ref += delta;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kt][r] -= delta;
      }
    }

    // O^T += V^T P^T, 16 keys per product.  Slot j of half-wave h holds key
    // 8 (j / 4) + 4 h + j % 4 of the chunk on both operands.  The normaliser
    // sums the same bf16 weights the product uses.
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      bf16x8 pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = (__bf16)fast_exp2(s[ch >> 1][8 * (ch & 1) + j]);
      ls0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0], pb[1]}, ones, ls0, false);
      ls1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[2], pb[3]}, ones, ls1, false);
      ls0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[4], pb[5]}, ones, ls0, false);
      ls1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[6], pb[7]}, ones, ls1, false);
#pragma unroll
      for (int dt = 0; dt < G::kDTiles; ++dt) {
        const __bf16* vp = &v_lds[buf][v_lane_off + 16 * ch * kVsr + 32 * dt];
        const bf16x4 lo = lds_read_tr16(vp);
        const bf16x4 up = lds_read_tr16(vp + 8 * kVsr);
        const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
        acc[dt] = mfma32(a, pb, acc[dt]);
      }
    }
    l_run += ls0 + ls1;

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using First = std::true_type;
  using Later = std::false_type;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  tile_step(I0{}, First{}, 0, n_tiles > 1);
  int t = 1;
  for (; t + 2 <= n_tiles; t += 2) {
    tile_step(I1{}, Later{}, t, true);
    tile_step(I0{}, Later{}, t + 1, t + 2 < n_tiles);
  }
  if (t < n_tiles) tile_step(I1{}, Later{}, t, false);

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
    if (hi == 0) LSE[(size_t)bh * Nq + my_q] = (m_ref + fast_log2(l_tot)) * kLn2;
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
