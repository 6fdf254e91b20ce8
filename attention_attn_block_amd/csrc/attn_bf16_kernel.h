// Block attention over bfloat16 Q/K/V on gfx950 matrix cores (kernel template;
// instantiated per head dim in attn_bf16_d*.hip, dispatched in attn_bf16.hip).
//
// Computes O = softmax(Q K^T * scale) V and LSE = ln sum exp(scale Q K^T) for
// one query block against one KV block -- the unit of work a sequence-
// parallel DiT device repeats per KV block ("SwiftFusion: Scalable Sequence
// Parallelism for Distributed Inference of Diffusion Transformers on GPUs",
// sections 1-2; "xDiT: an Inference Engine for Diffusion Transformers (DiTs)
// with Massive Parallelism", abstract).  The key loop is a one-pass online
// softmax: a reference row maximum and a running normaliser, with the output
// rescaled only when a row's scores outgrow the reference by a fixed margin
// (lazy rescaling, see kTau), so each KV tile is read once.
//
// Work decomposition (CDNA4, wave64):
//  * A workgroup owns 256 query rows of one (batch, head); each of its eight
//    waves owns 32 rows for the whole key loop.  Waves w and w + 4 share a
//    SIMD (two waves per SIMD, one workgroup per CU).
//  * Both contractions run on v_mfma_f32_32x32x16_bf16 in the transposed
//    form S^T = K Q^T and O^T = V^T P^T.  In the 32x32 accumulator layout a
//    lane then holds 16 values of ONE query row (column = lane % 32), shared
//    with lane ^ 32 only: the row max (taken at the first tile and on a
//    rescale) and each lane's share of the row sum are in-register
//    reductions, combined with lane ^ 32 by one exchange, and the two
//    shares of the sum are added once, in the epilogue.  P never leaves
//    registers: the S^T
//    accumulator registers are exactly the B operand of the PV product once
//    the keys inside each 16-key chunk are visited in the order the
//    accumulator holds them.
//  * K and V tiles of 64 keys move from HBM straight into LDS with
//    buffer_load_dwordx4 ... lds (no staging registers), double-buffered, in
//    16-byte units swizzled so that both LDS read patterns are bank-conflict
//    free.  V stays row-major; the PV operand is read with the transposing
//    ds_read_b64_tr_b16.
//  * Ping-pong: each wave alternates a matrix phase (tile t+1's scores and
//    tile t's PV product, K one tile ahead of V) with a vector phase (tile
//    t+1's weights), and the two waves of a SIMD run these phases half a tile
//    apart, separated by workgroup barriers, so one wave's softmax runs while
//    the other keeps the matrix core busy.  Each wave group issues tile
//    loads in its vector phase (K by one group, V by the other).  Inside the
//    matrix phase the LDS
//    operand reads run several products ahead of their use (kKDepth,
//    kVDepth).
//  * Workgroup ids are remapped so that all query tiles of a head run on the
//    same XCD (ids are dealt round-robin over the 8 XCDs), sharing that XCD's
//    L2 for the head's K/V stream.
//  * Plain launch: one workgroup per query tile.  Split launch (SPLIT): a
//    fixed grid shares the (query tile, key tile) units evenly, so a query
//    tile's key range may be cut into pieces on different workgroups whose
//    partials are combined through a caller workspace (see the kernel's
//    SPLIT notes).  Each workgroup loops over its pieces with the same
//    pipeline.
// Scores are kept in the log2 domain (scale * log2 e folded into one FMA) and
// exponentiated with v_exp_f32; the LSE is converted back to natural log.
// P is rounded to bfloat16 (RNE, v_cvt_pk_bf16_f32) for the PV product.  The
// normaliser is the fp32 sum of the fp32 weights before that rounding, added
// with ordinary v_add_f32: on gfx950 the dot instructions (v_dot2_f32_bf16)
// issue to the matrix pipe, so a wave waiting on one stalls its whole vector
// phase behind the other wave's MFMAs.  When d is not a multiple of 32 the
// fast path instead takes the normaliser from padding rows of the PV product
// (the sum of the bf16 weights; see kOnesRow).

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "launch.h"

namespace dit {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 512;   // 8 waves: two per SIMD, ping-pong
constexpr int kDmaThreads = 256;  // each tile is loaded by one group of 4 waves
constexpr int kBc = 64;         // keys per KV tile (a multiple of 32)
constexpr int kMaxPieces = kAttnMaxPieces;  // SPLIT: workgroups per query tile, at most
constexpr int kKT = kBc / 32;   // 32-key score accumulators per tile
constexpr int kCH = kBc / 16;   // 16-key chunks of the PV product per tile
constexpr int kWavesPerSimd = 2;  // with one query group per wave
constexpr int kGroups = 1;        // query groups of 32 rows per wave
// Software prefetch: K-operand LDS reads issued this many score products
// ahead of their use, V-operand reads this many PV products ahead.
constexpr int kKDepth = 4;
constexpr int kVDepth = 2;
// Word 3 of a raw (stride 0) buffer resource on gfx9-family GPUs: 32-bit
// data format; out-of-range reads return zero.
constexpr int kBufferFlags = 0x00020000;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int D>
struct Geo {
  static constexpr int kChunks = (D + 15) / 16;     // 16-wide slices of the QK^T contraction
  static constexpr bool kHalfTail = (D % 16) == 8;  // last slice has 8 real columns
  static constexpr int kDTiles = (D + 31) / 32;     // 32-row tiles of O^T
  static constexpr int kOct = D / 8;                // 16-byte groups per row in memory
  static constexpr int kKItems = kBc * kOct;        // 16-byte K (or V) groups per tile
  static constexpr int kKLoads = (kKItems + kDmaThreads - 1) / kDmaThreads;
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

// 16-byte-unit swizzles of the LDS tiles (row = key inside the tile; stored
// column = global column ^ swz).  Only for power-of-two units per row; other
// head dims keep plain row-major order.
//  swz_k: the K operand read has 16 consecutive lanes on 16 consecutive rows
//         at one column -> spread them over 16 distinct unit slots.
//  swz_v: a transposing read has 4 consecutive rows x 4 consecutive units per
//         half-wave -> give each of the 4 rows its own 4-unit slot group.
template <int kOct>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (kOct == 16) return row & 15;
  else if constexpr (kOct == 8) return (row >> 1) & 7;
  else if constexpr (kOct == 4) return (row >> 2) & 3;
  else if constexpr (kOct == 2) return (row >> 3) & 1;
  else return 0;
}
template <int kOct>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (kOct == 16) return 4 * (row & 3);
  else if constexpr (kOct == 8) return 4 * ((row >> 1) & 1);
  else return 0;
}

// d = 72: a row is 9 units (36 of the 64 four-byte LDS banks), which no XOR
// swizzle permutes.  A transposing V read pass covers 4 rows x 4 units, so
// the V tile places the units of row r at the slots given by a table indexed
// by r mod 4 (found by exhaustive search) that sends each pass to 16 distinct
// 4-bank groups.  v9_slot(r, u) is the slot of unit u, v9_unit its inverse
// (4-bit entries; unit 8 is the last).
__device__ __forceinline__ int v9_slot(int r, int u) {
  const unsigned long long t = r == 0 ? 0x387654210ull : r == 1 ? 0x876543210ull
                             : r == 2 ? 0x87216543ull : 0x576108432ull;
  return (int)((t >> (4 * u)) & 15);
}
__device__ __forceinline__ int v9_unit(int r, int s) {
  const unsigned long long t = r == 0 ? 0x765438210ull : r == 1 ? 0x876543210ull
                             : r == 2 ? 0x763210548ull : 0x376821054ull;
  return (int)((t >> (4 * s)) & 15);
}

// Lazy rescaling.  The reference max m_ref used for the exponentials is not
// tracked per tile.  A lane's 32 weights of a tile are accepted while their
// sum (needed for the normaliser anyway) is at most kLaneSumLimit, which
// bounds every weight by 2^14 -- harmless in bf16 and in the fp32
// accumulators.  A larger sum (or inf) sends the wave down the rare path: the
// rows whose maximum exceeds the reference by more than kTau (log2 units) move
// the reference to that maximum and rescale what they accumulated.  The
// result is unchanged in exact arithmetic.
constexpr float kTau = 8.f;
constexpr float kLaneSumLimit = 16.f * kKT * 512.f;

// Max over this lane's kKT x 16 scores of a tile.
__device__ __forceinline__ float row_max(const f32x16* s) {
  float mx = s[0][0];
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
  return mx;
}

// NG = query groups of 32 rows per wave.  NG = 2 lets every K and V operand
// read from LDS feed twice the matrix work, but needs one wave per SIMD and
// about 500 registers.  Built with hand-placed registers (O and Q in AGPRs,
// the softmax interleaved with the wave's own PV products) it gave the same
// bits and ran 20% slower: one wave does not hide its vector work behind its
// own MFMAs, two waves in ping-pong hide about half of it.  kGroups is 1, and
// the ping-pong schedule assumes one group.
//
// SPLIT: the grid is a fixed number of workgroups that share the
// (query tile, key tile) work evenly, so a query tile's key range may be cut
// between up to kMaxPieces workgroups (the launcher checks).  Each piece ends
// with its own partial (O, LSE); the partials of a tile are combined with the
// log-sum-exp identity by whichever piece arrives last, through the caller's
// workspace.
//
// MULTI: the keys are the concatenation of n_blocks KV blocks of Nkv keys each,
// held in separate buffers (blk): one launch for a whole ring step whose
// blocks are resident.  Key tile t of the concatenation is local tile
// t % tpb of block t / tpb (tpb = key tiles per block); the quotient is a
// scalar multiply-high by div_magic = ceil(2^32 / tpb) (tpb >= 2), exact for
// the sizes the launcher admits.  Without MULTI, K and V are one block.
template <int D, int NG, bool OUT_F32, bool MERGE, bool SPLIT, bool MULTI>
__global__ __launch_bounds__(kThreads, NG == 1 ? kWavesPerSimd : 1) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    void* __restrict__ Out, float* __restrict__ LSE, int Nq, int Nkv, int n_qtiles, float c2,
    int n_items, char* __restrict__ ws, KVBlocks blk, int n_blocks, unsigned div_magic) {
  using G = Geo<D>;
  constexpr int kRowsWG = (kThreads / 64) * 32 * NG;  // query rows per workgroup
  // K and V tiles: kBc rows of kOct 16-byte units each, unit-swizzled (see
  // swz_k / swz_v), plus slack for the transposing reads of the last rows.
  constexpr int kTileUnits = kBc * G::kOct;
  constexpr int kBufUnits = kTileUnits + 16;
  // Ones row.  When d is not a multiple of 32 the PV product computes
  // padding rows of O^T (d pads to 32 kDTiles); the transposing V reads of
  // those rows are pointed at a region of bf16 ones, so each padding row of
  // O^T accumulates the row sum of the weights: the normaliser comes out of
  // the matrix cores, and the fast vector phase needs no sums (see w_phase).
  // The region lies past the four tile buffers and is sized so that the
  // address of every padding read -- a fixed offset of two buffers plus
  // kOnesSkew units from either V buffer, plus the chunk and half-chunk
  // offsets -- lands in it.  The skew moves the padding reads to other banks
  // than the real V reads of the same pass (none conflict at d = 72).
  constexpr bool kOnesRow = (D % 32) != 0;
  // fp32 output at d = 128 (a ring step's block partials) leaves through LDS
  // in whole lines; see the epilogue.
  constexpr bool kStagedOut = OUT_F32 && !MERGE && !SPLIT && D == 128 && NG == 1;
  // bf16 output at d = 72 likewise, through a linear copy of the wave's rows.
  constexpr bool kStagedBf16 = !OUT_F32 && !MERGE && !SPLIT && D == 72 && NG == 1;
  constexpr int kOnesSkew = 8;
  constexpr int kOnesUnits = kOnesRow ? kBufUnits + kOnesSkew + 56 * G::kOct + 1 : 0;
  __shared__ u32x4 lds_all[4 * kBufUnits + kOnesUnits];
  u32x4 (*const k_lds)[kBufUnits] = reinterpret_cast<u32x4 (*)[kBufUnits]>(lds_all);
  u32x4 (*const v_lds)[kBufUnits] = k_lds + 2;
  __shared__ unsigned s_arrive;  // SPLIT: counter value seen by this workgroup

  // All kernel arguments in one scalar-load round trip: without this the
  // key loop's entry test splits them into three dependent ones (about
  // 0.3 us per call).
  asm volatile("" ::"s"(Q), "s"(K), "s"(V), "s"(Out), "s"(LSE), "s"(Nq), "s"(Nkv), "s"(gridDim.x));
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
  const int tpb = (Nkv + kBc - 1) / kBc;               // key tiles of one block
  const int n_all = MULTI ? n_blocks * tpb : tpb;      // key tiles of the whole key range

  // Work units are (query tile, key tile) pairs in query-tile-major order;
  // this workgroup owns units [u, u_end).  Unsplit: exactly one query tile.
  long long u, u_end;
  if constexpr (SPLIT) {
    const long long total = (long long)n_items * n_all;
    u = total * logical / nblk;
    u_end = total * (logical + 1) / nblk;
  } else {
    u = (long long)logical * n_all;
    u_end = u + n_all;
  }
  // Tile staging: global -> LDS directly (buffer_load_dwordx4 ... lds, no
  // registers), by the four waves of one group (w = wave mod 4).  Wave w's
  // j-th load writes LDS units 64 (4j + w) .. +63, lane i the unit
  // 64 (4j + w) + i; the unit stored there is row p / kOct, stored column
  // p % kOct, which holds global column (p % kOct) ^ swz(row).
  const int wv = __builtin_amdgcn_readfirstlane(wave & 3);
  const int dtid = tid & (kDmaThreads - 1);
  // Byte offsets of this lane's unit inside a full K / V tile (fixed for the
  // whole key loop).
  unsigned koff[G::kKLoads], voff[G::kKLoads];
#pragma unroll
  for (int j = 0; j < G::kKLoads; ++j) {
    const int pu = dtid + kDmaThreads * j;
    const int row = pu / G::kOct, col = pu - row * G::kOct;
    koff[j] = (unsigned)(row * D + 8 * (col ^ swz_k<G::kOct>(row))) * 2u;
    const int vcol = G::kOct == 9 ? v9_unit(row & 3, col) : (col ^ swz_v<G::kOct>(row));
    voff[j] = (unsigned)(row * D + 8 * vcol) * 2u;
  }
  // One tile, as buffer loads against a resource that covers exactly the
  // tile's rows inside the block: in the ragged last tile the rows past the
  // block fall outside the resource, are not read, and land in LDS as zeros
  // (their keys are masked).
  auto dma_tile = [&](auto is_v, const __bf16* base, u32x4* lds, int kv0) {
    constexpr bool kV = decltype(is_v)::value;
    // The tile base is one scalar address; the halves come back from
    // readfirstlane as int and are widened as unsigned.  The wave index is
    // re-read here so the LDS destinations are recomputed per tile instead of
    // held in registers.
    const uint64_t tba = reinterpret_cast<uint64_t>(base + (size_t)kv0 * D);
    const void* tb = reinterpret_cast<const void*>(
        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(tba >> 32)) << 32) |
        (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)tba));
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(tb), (short)0, (Nkv - kv0 < kBc ? Nkv - kv0 : kBc) * D * 2, kBufferFlags);
    int wvl = wv;
    asm volatile("" : "+s"(wvl));
#pragma unroll
    for (int j = 0; j < G::kKLoads; ++j) {
      const int first_unit = 64 * ((kDmaThreads / 64) * j + wvl);
      // Wave-uniform skip of loads past the tile; when the tile is not a
      // whole number of 64-unit wave loads, the lanes past its end must not
      // load.
      const bool lane_in = (kTileUnits % 64 == 0) || dtid + kDmaThreads * j < kTileUnits;
      if (kTileUnits % kDmaThreads == 0 || (first_unit < kTileUnits && lane_in)) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)(lds + first_unit), 16,
            (int)(kV ? voff[j] : koff[j]), 0, 0, 0);
      }
    }
  };
  using IsK = std::integral_constant<bool, false>;
  using IsV = std::integral_constant<bool, true>;
  // All of this wave's tile loads have landed in LDS (before a barrier).
  auto dma_wait = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // K operand addresses: row kt*32 + l32, global column 2c + hi.
  const int sk = swz_k<G::kOct>(l32);
  int k_unit[G::kChunks];
#pragma unroll
  for (int c = 0; c < G::kChunks; ++c) k_unit[c] = l32 * G::kOct + (((2 * c + hi) ^ sk) % G::kOct);

  if constexpr (kOnesRow) {
    // Written once; no tile load ever touches this region.  The first piece's
    // prologue barrier orders these stores before any read.
    const u32x4 one4 = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    for (int i = tid; i < kOnesUnits; i += kThreads) lds_all[4 * kBufUnits + i] = one4;
  }

  while (u < u_end) {
    // One piece: key tiles [t_beg, t_end) of query tile `item`.
    // The piece's indices are the same in every lane; the compiler computes
    // the 64-bit division in vector registers, so they are made scalar here
    // once (everything derived from them then stays in scalar registers).
    const int item = __builtin_amdgcn_readfirstlane((int)(u / n_all));
    const int t_beg = __builtin_amdgcn_readfirstlane((int)(u - (long long)item * n_all));
    const int t_end = __builtin_amdgcn_readfirstlane(
        (int)(u_end - u < (long long)(n_all - t_beg) ? t_beg + (u_end - u) : n_all));
    u += t_end - t_beg;
    const int bh = item / n_qtiles;
    const int qt = item - bh * n_qtiles;
    const int kvb = t_beg * kBc;  // first key of the piece

    const __bf16* Qh = Q + (size_t)bh * Nq * D;
    const __bf16* Kh = K + (size_t)bh * Nkv * D;
    const __bf16* Vh = V + (size_t)bh * Nkv * D;
    // Source of key tile t of the piece: the (batch, head) slice of its block
    // and the tile's first key inside that block.
    // (The tile index is wave-uniform; readfirstlane keeps the block lookup
    // and the tile's buffer resource in scalar registers.)
    auto tile_block = [&](int t) -> int {
      if constexpr (MULTI) {
        const unsigned ta = (unsigned)__builtin_amdgcn_readfirstlane(t_beg + t);
        return tpb == 1 ? (int)ta : (int)__umulhi(ta, div_magic);
      } else {
        return 0;
      }
    };
    auto tile_kv0 = [&](int t) -> int {
      if constexpr (MULTI)
        return (__builtin_amdgcn_readfirstlane(t_beg + t) - tile_block(t) * tpb) * kBc;
      else return kvb + t * kBc;
    };
    auto tile_k = [&](int t) -> const __bf16* {
      if constexpr (MULTI) return static_cast<const __bf16*>(blk.k[tile_block(t)]) + (size_t)bh * Nkv * D;
      else return Kh;
    };
    auto tile_v = [&](int t) -> const __bf16* {
      if constexpr (MULTI) return static_cast<const __bf16*>(blk.v[tile_block(t)]) + (size_t)bh * Nkv * D;
      else return Vh;
    };

    // Query rows of this lane, one per group; Q^T as the B operand: lane holds
    // Q[row][16c + 8hi .. +7].
    int my_q[NG];
    bf16x8 qf[NG][G::kChunks];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      my_q[g] = qt * kRowsWG + (wave * NG + g) * 32 + l32;
      const int q_ld = my_q[g] < Nq ? my_q[g] : Nq - 1;
#pragma unroll
      for (int c = 0; c < G::kChunks; ++c) {
        if (G::kHalfTail && c == G::kChunks - 1 && hi) {
          qf[g][c] = bf16x8{};
        } else {
          qf[g][c] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)q_ld * D + 16 * c + 8 * hi);
        }
      }
    }

    // S^T = K Q^T for the kBc keys of the K tile in LDS buffer `buf`; each K
    // operand read feeds the products of all NG query groups.
    auto qk = [&](int buf, f32x16 (*s)[kKT]) {
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int g = 0; g < NG; ++g) s[g][kt] = f32x16{};
#pragma unroll
      for (int c = 0; c < G::kChunks; ++c) {
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
          // In a half-filled last chunk the upper half-wave's K operand holds
          // another unit of the same row (finite data): its Q operand is zero.
          const bf16x8 a = __builtin_bit_cast(bf16x8, k_lds[buf][kt * 32 * G::kOct + k_unit[c]]);
#pragma unroll
          for (int g = 0; g < NG; ++g) s[g][kt] = mfma32(a, qf[g][c], s[g][kt]);
        }
      }
    };
    // Keys past the end of the block (last tile only) get zero weight.
    auto mask_tail = [&](f32x16 (*s)[kKT], int kv0) {
      if (kv0 + kBc > Nkv) {
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kv0 + kt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (key >= Nkv) s[g][kt][r] = -INFINITY;
            }
      }
    };

    // Transposing V reads (see lds_read_tr16): in lane group q = lane / 16,
    // lane i names row 4 (q / 2) + i / 4 of each 8-key half chunk and columns
    // 16 (q % 2) + 4 (i % 4) .. +3 of each 32-column d tile.  The row's swizzle
    // depends on i / 4 only, so each d tile gets one lane-constant offset.
    const int vq = lane >> 4, vi = lane & 15;
    const int v_row = 4 * (vq >> 1) + (vi >> 2);
    const int sv = swz_v<G::kOct>(v_row);
    int v_off[G::kDTiles];  // bf16 element offsets inside a V buffer
#pragma unroll
    for (int dt = 0; dt < G::kDTiles; ++dt) {
      const int unit = 4 * dt + 2 * (vq & 1) + ((vi & 3) >> 1);
      if (kOnesRow && unit >= G::kOct) {
        // A padding row of O^T: read the ones region (two buffers and
        // kOnesSkew units past this V buffer, whichever it is; see kOnesUnits).
        v_off[dt] = (2 * kBufUnits + kOnesSkew) * 8 + 4 * (vi & 1);
        continue;
      }
      const int slot = G::kOct == 9 ? v9_slot(v_row & 3, unit) : (unit ^ sv);
      v_off[dt] = (v_row * G::kOct + slot) * 8 + 4 * (vi & 1);
    }

    f32x16 acc[NG][G::kDTiles];
    float l_run[NG];   // this lane's share of each row's normaliser (exact path)
    float l_ch[NG][4];  // the same on the fast path, as four running chains of adds
    float m_ref[NG];   // reference row max for the exponentials, log2 units
    float l_fin[NG];   // each row's normaliser at the end of the key loop
    const int n_tiles = t_end - t_beg;  // key tiles of this piece
    // Accumulator element of a lane that holds a padding row of O^T (row
    // 32 (kDTiles - 1) + 8 (e / 4) + 4 hi + e % 4 >= d for both half-waves).
    constexpr int kOnesElt = 4 * ((D - 32 * (G::kDTiles - 1)) / 8);

    // Ping-pong schedule.  Waves w and w + 4 share a SIMD.  Group A (waves 0-3)
    // and group B (waves 4-7) run the same per-wave pipeline one slot apart, so
    // while one wave of a SIMD is in its matrix phase the other is in its vector
    // phase.  Per tile t a wave runs
    //   M(t):   S(t+1) = K(t+1) Q^T and O^T += V(t)^T P(t)^T  (matrix cores, LDS)
    //   W(t+1): exponent form, weights P(t+1), normaliser, rare rescale  (VALU)
    // Group A runs M(k) in slot 2k and W(k+1) in slot 2k+1; group B runs M(k) in
    // slot 2k+1 and W(k+1) in slot 2k+2.  Every slot ends with a barrier that
    // every wave executes (the slot count is the same for the whole workgroup).
    // K(t) and V(t) live in LDS buffer t % 2.  Each group issues tile loads
    // in its own vector phase: group B starts K(k+2) in slot 2k, group A
    // starts V(k+1) in slot 2k+1, each into the buffer whose last readers ran
    // in slot 2k-1.  Slot 2k+1 ends by waiting for both (the barrier of slot
    // 2k does not wait).
    const int grp = wave >> 2;
    f32x16 s_nxt[NG][kKT];
    bf16x8 pb[NG][kCH];

    // W(t): scores of tile t (raw, in s_nxt) -> weights pb, normaliser share.
    // The normaliser adds the fp32 weights before their rounding to bf16, in
    // plain adds (no dot instructions: those wait for the matrix pipe).
    // kSafe = false, the fast path: nothing bounds the weights per tile (a
    // non-finite normaliser after the key loop sends the piece to the exact
    // path); with the ones row the normaliser comes out of the PV product
    // and the phase computes the weights alone.  kFirst: tile 0, which sets
    // the reference max.
    auto w_phase = [&](auto safe_c, auto first_c, int t) __attribute__((always_inline)) {
      constexpr bool kSafe = decltype(safe_c)::value;
      constexpr bool kFirst = decltype(first_c)::value;
      mask_tail(s_nxt, tile_kv0(t));
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if constexpr (kFirst) {  // reference max from tile 0
          l_run[g] = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) l_ch[g][c] = 0.f;
          m_ref[g] = max_with_partner32(row_max(s_nxt[g])) * c2;
        }
        const float neg_m = -m_ref[g];
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) s_nxt[g][kt][r] = fmaf(s_nxt[g][kt][r], c2, neg_m);
      }
      if constexpr (!kSafe) {
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int ch = 0; ch < kCH; ++ch)
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
              const float e0 = fast_exp2(s_nxt[g][ch >> 1][8 * (ch & 1) + j]);
              const float e1 = fast_exp2(s_nxt[g][ch >> 1][8 * (ch & 1) + j + 1]);
              pb[g][ch][j] = (__bf16)e0;
              pb[g][ch][j + 1] = (__bf16)e1;
              // Four chains that run on across tiles (no per-tile total).
              if constexpr (!kOnesRow) l_ch[g][j >> 1] += e0 + e1;
            }
        return;
      }
      float ls[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        // This lane's share of the tile's normaliser also bounds every weight
        // the lane holds.  Four independent chains.
        float lc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ch = 0; ch < kCH; ++ch)
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const float e0 = fast_exp2(s_nxt[g][ch >> 1][8 * (ch & 1) + j]);
            const float e1 = fast_exp2(s_nxt[g][ch >> 1][8 * (ch & 1) + j + 1]);
            pb[g][ch][j] = (__bf16)e0;
            pb[g][ch][j + 1] = (__bf16)e1;
            lc[j >> 1] += e0 + e1;
          }
        ls[g] = (lc[0] + lc[1]) + (lc[2] + lc[3]);
      }
      // Rare: a lane's share of a row's sum exceeds the limit (so some weight
      // there exceeds 2^9), i.e. the row's scores grew well past its reference
      // max.  Rows whose tile max exceeds the reference by more than kTau move
      // the reference to it, rescale what they accumulated and recompute this
      // tile's weights.
      bool any_big = false;
#pragma unroll
      for (int g = 0; g < NG; ++g) any_big |= !(ls[g] <= kLaneSumLimit);
      if (kSafe && __builtin_amdgcn_ballot_w64(any_big)) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const float mx = max_with_partner32(row_max(s_nxt[g]));
          const bool grow = mx > kTau;
          const float delta = grow ? mx : 0.f;
          const float alpha = fast_exp2(-delta);
          l_run[g] *= alpha;
#pragma unroll
          for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[g][dt][r] *= alpha;
          m_ref[g] += delta;
          // Recompute the tile's weights against the moved reference (a row
          // that did not grow has delta = 0 and gets the same weights back).
          float lc0 = 0.f, lc1 = 0.f;
#pragma unroll
          for (int ch = 0; ch < kCH; ++ch)
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
              const float e0 = fast_exp2(s_nxt[g][ch >> 1][8 * (ch & 1) + j] - delta);
              const float e1 = fast_exp2(s_nxt[g][ch >> 1][8 * (ch & 1) + j + 1] - delta);
              pb[g][ch][j] = (__bf16)e0;
              pb[g][ch][j + 1] = (__bf16)e1;
              if (j & 2) lc1 += e0 + e1; else lc0 += e0 + e1;
            }
          ls[g] = lc0 + lc1;
        }
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) l_run[g] += ls[g];
    };

    // M(t) with K(t+1) in buffer kb and V(t) in buffer vb (compile-time).
    auto m_phase = [&](auto kb_c, auto vb_c, int t) __attribute__((always_inline)) {
      constexpr int kb = decltype(kb_c)::value, vbi = decltype(vb_c)::value;
      __builtin_amdgcn_s_setprio(1);
      if (t + 1 < n_tiles) {
        // S^T = K Q^T for tile t + 1; K-operand reads kKD products ahead, the
        // two 32-key accumulators alternate.
        constexpr int kQK = kKT * G::kChunks;
        constexpr int kKD = kKDepth;
        bf16x8 kr[kQK];
        auto kread = [&](int i) -> bf16x8 {
          const int c = i / kKT, kt = i % kKT;
          return __builtin_bit_cast(bf16x8, k_lds[kb][kt * 32 * G::kOct + k_unit[c]]);
        };
#pragma unroll
        for (int i = 0; i < kKD && i < kQK; ++i) kr[i] = kread(i);
        __builtin_amdgcn_sched_group_barrier(0x100, kKD, 0);
#pragma unroll
        for (int i = 0; i < kQK; ++i) {
          if (i + kKD < kQK) kr[i + kKD] = kread(i + kKD);
          const int c = i / kKT, kt = i % kKT;
#pragma unroll
          for (int g = 0; g < NG; ++g)
            s_nxt[g][kt] = mfma32(kr[i], qf[g][c], c == 0 ? f32x16{} : s_nxt[g][kt]);
          if (i + kKD < kQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, NG, 0);                    // MFMA
        }
      }
      // O^T += V^T P^T for tile t (16 keys per product).  Slot j of half-wave h
      // holds key 8 (j / 4) + 4 h + j % 4 of the chunk on both operands; the
      // two transposing reads of a product are issued kVD products ahead.
      const __bf16* vbase = reinterpret_cast<const __bf16*>(v_lds[vbi]);
      constexpr int kPV = kCH * G::kDTiles;
      constexpr int kVD = kVDepth;
      bf16x8 vr[kPV];
      auto vread = [&](int j) -> bf16x8 {
        const int ch = j / G::kDTiles, dt = j % G::kDTiles;
        const __bf16* vp = vbase + v_off[dt] + 16 * ch * G::kOct * 8;
        const bf16x4 lo = lds_read_tr16(vp);
        const bf16x4 up = lds_read_tr16(vp + 8 * G::kOct * 8);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
      };
#pragma unroll
      for (int j = 0; j < kVD && j < kPV; ++j) vr[j] = vread(j);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kVD, 1);
#pragma unroll
      for (int j = 0; j < kPV; ++j) {
        if (j + kVD < kPV) vr[j + kVD] = vread(j + kVD);
        const int ch = j / G::kDTiles, dt = j % G::kDTiles;
#pragma unroll
        for (int g = 0; g < NG; ++g) acc[g][dt] = mfma32(vr[j], pb[g][ch], acc[g][dt]);
        if (j + kVD < kPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, NG, 1);                    // MFMA
      }
      __builtin_amdgcn_s_setprio(0);
    };

    // The whole key loop of the piece: prologue, then the slots.  Leaves the
    // piece's (acc, m_ref, l_fin).
    auto pipeline = [&](auto safe_c) __attribute__((always_inline)) {
    constexpr bool kSafe = decltype(safe_c)::value;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int t = 0; t < G::kDTiles; ++t) acc[g][t] = f32x16{};
    if (grp == 1) {
      dma_tile(IsK{}, tile_k(0), k_lds[0], tile_kv0(0));
      dma_tile(IsV{}, tile_v(0), v_lds[0], tile_kv0(0));
      if (n_tiles > 1) dma_tile(IsK{}, tile_k(1), k_lds[1], tile_kv0(1));
    }
    dma_wait();
    __syncthreads();
    qk(0, s_nxt);
    // Slot 0 loads K tile 2 into the buffer tile 0 was just read from: every
    // wave must have finished those reads first.
    __syncthreads();

    w_phase(safe_c, std::true_type{}, 0);

    // One slot; p = slot index mod 4 (compile-time), so the buffer of every
    // tile a slot touches is known: in slots 4j + {0, 1} tile k is even, in
    // slots 4j + {2, 3} odd (k = slot / 2 rounded down).
    auto run_slot = [&](auto p_c, int s) __attribute__((always_inline)) {
      constexpr int p = decltype(p_c)::value;
      constexpr int kpar = p >> 1;  // parity of k
      using KP = std::integral_constant<int, kpar>;
      using KQ = std::integral_constant<int, kpar ^ 1>;
      const int k = s >> 1;
      if constexpr ((p & 1) == 0) {
        if (grp == 1) {  // group B is in its vector phase in even slots
          if (k + 2 < n_tiles) dma_tile(IsK{}, tile_k(k + 2), k_lds[kpar], tile_kv0(k + 2));
        }
        if (grp == 0) {
          if (k < n_tiles) m_phase(KQ{}, KP{}, k);
        } else {
          if (k >= 1 && k < n_tiles) w_phase(safe_c, std::false_type{}, k);
        }
      } else {
        if (grp == 0) {  // group A is in its vector phase in odd slots
          if (k + 1 < n_tiles) dma_tile(IsV{}, tile_v(k + 1), v_lds[kpar ^ 1], tile_kv0(k + 1));
          if (k + 1 < n_tiles) w_phase(safe_c, std::false_type{}, k + 1);
        } else {
          if (k < n_tiles) m_phase(KQ{}, KP{}, k);
        }
        dma_wait();
      }
      if constexpr ((p & 1) == 0) {
        // Even slot: its tile loads are read two slots later, after the odd
        // slot's wait, so they may stay in flight across this barrier.  A
        // workgroup release fence (__syncthreads) would wait for them here;
        // only this wave's LDS reads have to be complete.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      } else {
        __syncthreads();
      }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    for (int s = 0; s < 2 * n_tiles; s += 4) {
      run_slot(P0{}, s);
      run_slot(P1{}, s + 1);
      run_slot(P2{}, s + 2);
      run_slot(P3{}, s + 3);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g)
      l_fin[g] = kSafe      ? sum_with_partner32(l_run[g])
                 : kOnesRow ? acc[g][G::kDTiles - 1][kOnesElt]
                            : sum_with_partner32((l_ch[g][0] + l_ch[g][1]) + (l_ch[g][2] + l_ch[g][3]));
    };  // pipeline

    // Fast path first.  Its weights are exp2 of (score - reference max of the
    // first tile) with no per-tile bound: a row whose scores later outgrow
    // that reference by 128 (log2 units) or more overflows, which shows as a
    // non-finite normaliser.  Then the whole workgroup runs the piece again
    // with the per-tile bound and lazy rescale (the loop has drained: its
    // last slot waited for every tile load and ended with a barrier).
    pipeline(std::false_type{});
    bool bad = false;
#pragma unroll
    for (int g = 0; g < NG; ++g) bad |= !(l_fin[g] < INFINITY);
    if (__syncthreads_or(bad)) pipeline(std::true_type{});

    if (!SPLIT || (t_beg == 0 && t_end == n_all)) {
      float st_wb = 0.f;  // the staged bf16 epilogue's row weight (NG = 1)
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float l_tot = l_fin[g];
        if (my_q[g] < Nq) {
          // This block's partial: O_b = acc / l_tot, LSE_b = m_ref + log2 l_tot
          // (log2 units).  MERGE folds it into the running (Out, LSE) of the row
          // with the log-sum-exp identity; LSE = -inf there marks an empty
          // accumulator whose O is not read.
          const size_t lrow = (size_t)bh * Nq + my_q[g];
          const float lse_b = m_ref[g] + fast_log2(l_tot);
          float wb = 1.f / l_tot, wa = 0.f, lse_new = lse_b;
          bool has_a = false;
          if constexpr (MERGE) {
            const float la = LSE[lrow] * kLog2e;
            has_a = la != -INFINITY;
            if (has_a) {
              const float m = fmaxf(la, lse_b);
              const float ea = fast_exp2(la - m), eb = fast_exp2(lse_b - m);
              const float inv = 1.f / (ea + eb);
              wa = ea * inv;
              wb = eb * inv / l_tot;
              lse_new = m + fast_log2(ea + eb);
            }
          }
          const size_t orow = lrow * D;
          st_wb = wb;
#pragma unroll
          for (int dt = 0; dt < (kStagedOut || kStagedBf16 ? 0 : G::kDTiles); ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int d0 = dt * 32 + 8 * q4 + 4 * hi;
              if (d0 < D) {
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = acc[g][dt][4 * q4 + e] * wb;
                if constexpr (OUT_F32) {
                  f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(Out) + orow + d0);
                  if (MERGE && has_a) {
                    const f32x4 a = *p;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = fmaf(wa, a[e], o[e]);
                  }
                  *p = f32x4{o[0], o[1], o[2], o[3]};
                } else {
                  bf16x4* p = reinterpret_cast<bf16x4*>(static_cast<__bf16*>(Out) + orow + d0);
                  if (MERGE && has_a) {
                    const bf16x4 a = *p;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = fmaf(wa, (float)a[e], o[e]);
                  }
                  *p = bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
                }
              }
            }
          if (hi == 0) LSE[lrow] = lse_new * kLn2;
        }
      }
      if constexpr (kStagedOut) {
        // Written straight from the accumulators, each store would cover 32-byte
        // pieces of 32 rows (two lanes per row), 32 cache-line requests per
        // instruction.  Instead each wave passes its rows through its own 8 KB
        // slice of the tile buffers (idle since the key loop's last barrier),
        // two 32-column tiles at a time, and every store then writes whole
        // 128-byte lines of 4 rows.  Unit u (16 bytes) of slice row r sits at
        // u ^ (r % 16): each 16-lane pass of the writes and of the reads meets
        // 16 different units.
        static_assert(kThreads / 64 * 512 <= 4 * kBufUnits, "staging slices fit the tile buffers");
        u32x4* slice = lds_all + wave * 512;
        const float wb0 = 1.f / l_fin[0];
        const int q_base = qt * kRowsWG + wave * 32;
        float* out_rows = static_cast<float*>(Out) + ((size_t)bh * Nq + q_base) * D;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int dd = 0; dd < 2; ++dd)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int u = dd * 8 + 2 * q4 + hi;
              const f32x16& a = acc[0][2 * h + dd];
              slice[l32 * 16 + (u ^ (l32 & 15))] = __builtin_bit_cast(
                  u32x4, f32x4{a[4 * q4] * wb0, a[4 * q4 + 1] * wb0, a[4 * q4 + 2] * wb0,
                               a[4 * q4 + 3] * wb0});
            }
          // The reads take other lanes' writes: wave-ordered LDS, made visible
          // to the compiler by the clobber.
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
          for (int it = 0; it < 8; ++it) {
            const int r = it * 4 + (lane >> 4), c = lane & 15;
            const u32x4 v4 = slice[r * 16 + (c ^ (r & 15))];
            if (q_base + r < Nq)
              *reinterpret_cast<u32x4*>(out_rows + (size_t)r * D + h * 64 + c * 4) = v4;
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // before the slice is rewritten
        }
      }
      if constexpr (kStagedBf16) {
        // The wave's 32 rows are one contiguous range of Out (32 * D bf16).
        // Stored from the accumulators, each store would cover 16-byte pieces
        // of 32 rows.  Instead the lanes' 8-byte pieces go to a linear copy of
        // that range in the wave's own part of the (idle) tile buffers, and
        // the wave then copies it out in consecutive 16-byte units, whole
        // lines per store.  A row's 144 bytes are 9 whole units.
        static_assert((kThreads / 64) * 32 * D * 2 <= 4 * kBufUnits * 16, "copies fit the tile buffers");
        static_assert((D * 2) % 16 == 0, "a unit never straddles two rows");
        char* slice = reinterpret_cast<char*>(lds_all) + wave * (32 * D * 2);
#pragma unroll
        for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = dt * 32 + 8 * q4 + 4 * hi;
            if (d0 < D) {
              const f32x16& a = acc[0][dt];
              *reinterpret_cast<bf16x4*>(slice + (l32 * D + d0) * 2) =
                  bf16x4{(__bf16)(a[4 * q4] * st_wb), (__bf16)(a[4 * q4 + 1] * st_wb),
                         (__bf16)(a[4 * q4 + 2] * st_wb), (__bf16)(a[4 * q4 + 3] * st_wb)};
            }
          }
        // The reads take other lanes' writes: wave-ordered LDS, made visible
        // to the compiler by the clobber.
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        constexpr int kUnits = 32 * D * 2 / 16;
        const int q_base = qt * kRowsWG + wave * 32;
        __bf16* out_base = static_cast<__bf16*>(Out) + ((size_t)bh * Nq + q_base) * D;
#pragma unroll
        for (int k = 0; k < (kUnits + 63) / 64; ++k) {
          const int unit = k * 64 + lane;
          if (unit < kUnits && q_base + unit / (D / 8) < Nq)
            *reinterpret_cast<u32x4*>(out_base + unit * 8) =
                *reinterpret_cast<const u32x4*>(slice + unit * 16);
        }
      }
    } else {
      // One of the k (2..kMaxPieces) pieces of a query tile whose key range
      // is cut between workgroups; piece j holds the j-th key range.  All
      // partials take one representation -- O normalised, in fp32, and LSE in
      // log2 units -- and are combined in key order, so the result is the same
      // bits whichever piece combines.
      // A partial is stored in the accumulators' own lane order, so that every
      // store and load of the exchange moves 1 KB of contiguous memory: O in
      // 1 KB units ((wave * NG + g) * kDTiles + dt) * 4 + q4, lane l at byte
      // 16 l of its unit, holding row (wave * NG + g) * 32 + l % 32 and
      // columns dt * 32 + 8 q4 + 4 (l / 32) .. +3 (units past d are never
      // written or read); then the LSE of row r at byte kOBytes + 4 r.
      constexpr int kOBytes = (kThreads / 64) * NG * G::kDTiles * 4 * 1024;
      constexpr int kSlotBytes = kOBytes + kRowsWG * 4;
      static_assert(kSlotBytes <= kAttnSplitSlotBytes, "a partial must fit its workspace slot");
      constexpr long long kSlotStride = kAttnSplitSlotBytes / 4;  // floats between slots
      auto o_off = [&](int g, int dt, int q4) {
        return ((((wave * NG + g) * G::kDTiles + dt) * 4 + q4) * 64 + lane) * 16;
      };
      const long long total = (long long)n_items * n_all;
      // Workgroup whose range holds unit x (ranges start at total * w / nblk).
      auto owner = [&](long long x) { return ((x + 1) * nblk + total - 1) / total - 1; };
      const long long w_first = owner((long long)item * n_all);
      const int n_pieces = (int)(owner((long long)item * n_all + n_all - 1) - w_first + 1);
      const int j_piece = (int)(logical - w_first);
      // This tile's workspace record: arrival counter, then the partial slots.
      char* rec = ws + (size_t)item * kAttnSplitItemBytes;
      float* slots = reinterpret_cast<float*>(rec + 256);
      float lse_own[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const float l_tot = l_fin[g];
        lse_own[g] = m_ref[g] + fast_log2(l_tot);
        const float inv = 1.f / l_tot;
#pragma unroll
        for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[g][dt][r] *= inv;
      }
      // Partials are written and read with device-coherent buffer accesses
      // (sc1, the encoding of device-scope atomic loads and stores: coherent
      // across the per-XCD L2s), so the exchange needs no L2 write-back or
      // invalidate -- those would also drop the K/V tiles other workgroups are
      // reusing from L2.
      auto slot_rsrc = [&](int j) {
        return __builtin_amdgcn_make_buffer_rsrc(slots + (size_t)j * kSlotStride, (short)0,
                                                 kSlotBytes, kBufferFlags);
      };
      constexpr int kCoherent = 16;  // sc1
      auto publish = [&]() {
        const __amdgpu_buffer_rsrc_t own = slot_rsrc(j_piece);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (my_q[g] >= Nq) continue;
          const int row = (wave * NG + g) * 32 + l32;
#pragma unroll
          for (int dt = 0; dt < G::kDTiles; ++dt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int d0 = dt * 32 + 8 * q4 + 4 * hi;
              if (d0 < D)
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, f32x4{acc[g][dt][4 * q4], acc[g][dt][4 * q4 + 1],
                                                    acc[g][dt][4 * q4 + 2], acc[g][dt][4 * q4 + 3]}),
                    own, o_off(g, dt, q4), 0, kCoherent);
            }
          if (hi == 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(lse_own[g]), own,
                                                  kOBytes + row * 4, 0, kCoherent);
        }
      };
      // Arrival on the tile's counter (0 before the first piece arrives; the
      // combining piece sets it back to 0).  The low 16 bits count arrivals,
      // bit 16 says piece 0 has published.
      //   piece j > 0: publish, add 1; combine iff the counter was
      //                2^16 + (k - 1) (piece 0 published, every other piece in).
      //   piece 0:     add 1; combine iff it was k - 1 (every other piece has
      //                published).  Otherwise publish, add 2^16, and combine iff
      //                the arrivals then numbered k.
      // Piece 0 ends its workgroup's range and usually arrives last, so it
      // usually combines without publishing.  Exactly one piece combines, only
      // after every other partial is published, and no workgroup ever waits
      // for another.  The counter is a relaxed device-scope atomic; each
      // arrival first waits until this workgroup's coherent stores are
      // acknowledged.
      unsigned* cnt = reinterpret_cast<unsigned*>(rec);
      auto arrive = [&](unsigned add) -> unsigned {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // own published stores acknowledged
        __syncthreads();
        if (tid == 0)
          s_arrive = __hip_atomic_fetch_add(cnt, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        return s_arrive;
      };
      constexpr unsigned kPublished0 = 1u << 16;
      const unsigned others = (unsigned)n_pieces - 1u;
      bool combine;
      if (j_piece > 0) {
        publish();
        combine = arrive(1u) == kPublished0 + others;
      } else {
        const unsigned first = arrive(1u);
        if (first == others) {
          combine = true;
        } else {
          publish();
          combine = (arrive(kPublished0) & 0xffffu) == others + 1u;
        }
      }
      if (combine) {
        if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (my_q[g] >= Nq) continue;
          const int row = (wave * NG + g) * 32 + l32;
          const size_t lrow = (size_t)bh * Nq + my_q[g];
          // Weights of the pieces: e_j = 2^(L_j - m), normalised by their sum.
          // Every slot of the tile is read (all are inside the workspace) and
          // the ones that are not another piece's published partial are
          // replaced by selects, so the loads issue back to back without
          // branches between them.
          float lp[kMaxPieces], wp[kMaxPieces];
#pragma unroll
          for (int j = 0; j < kMaxPieces; ++j)
            lp[j] = j < n_pieces ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                       slot_rsrc(j), kOBytes + row * 4, 0, kCoherent))
                                 : 0.f;
          float m = -INFINITY;
#pragma unroll
          for (int j = 0; j < kMaxPieces; ++j) {
            lp[j] = j == j_piece ? lse_own[g] : (j < n_pieces ? lp[j] : -INFINITY);
            m = fmaxf(m, lp[j]);
          }
          float esum = 0.f;
#pragma unroll
          for (int j = 0; j < kMaxPieces; ++j) {
            wp[j] = j < n_pieces ? fast_exp2(lp[j] - m) : 0.f;
            esum += wp[j];
          }
          const float einv = 1.f / esum;
#pragma unroll
          for (int j = 0; j < kMaxPieces; ++j) wp[j] *= einv;
          const float lse_b = m + fast_log2(esum);
          // Fold into the running (Out, LSE) as in the unsplit epilogue.
          float wa = 0.f, wb = 1.f, lse_new = lse_b;
          bool has_a = false;
          if constexpr (MERGE) {
            const float la = LSE[lrow] * kLog2e;
            has_a = la != -INFINITY;
            if (has_a) {
              const float m2 = fmaxf(la, lse_b);
              const float ea = fast_exp2(la - m2), eb = fast_exp2(lse_b - m2);
              const float inv2 = 1.f / (ea + eb);
              wa = ea * inv2;
              wb = eb * inv2;
              lse_new = m2 + fast_log2(ea + eb);
            }
          }
          const size_t orow = lrow * D;
#pragma unroll
          for (int dt = 0; dt < G::kDTiles; ++dt) {
            // One 32-column tile of each other slot (slot i, or i + 1 from this
            // piece's own on), loaded back to back.
            f32x4 pv[kMaxPieces - 1][4];
#pragma unroll
            for (int i = 0; i < kMaxPieces - 1; ++i) {
              if (i < n_pieces - 1) {  // workgroup-uniform
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                  const int d0 = dt * 32 + 8 * q4 + 4 * hi;
                  pv[i][q4] = d0 < D
                                  ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                        slot_rsrc(i + (i >= j_piece)), o_off(g, dt, q4), 0, kCoherent))
                                  : f32x4{};
                }
              } else {
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) pv[i][q4] = f32x4{};
              }
            }
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              const int d0 = dt * 32 + 8 * q4 + 4 * hi;
              if (d0 < D) {
                float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < kMaxPieces; ++j) {
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    // piece j: own below, else slot j (j < own) or loaded entry j - 1
                    const float lo = j < kMaxPieces - 1 ? pv[j < kMaxPieces - 1 ? j : 0][q4][e] : 0.f;
                    const float up = j > 0 ? pv[j > 0 ? j - 1 : 0][q4][e] : 0.f;
                    const float pj = j == j_piece ? acc[g][dt][4 * q4 + e]
                                                  : (j >= n_pieces ? 0.f : (j < j_piece ? lo : up));
                    o[e] = fmaf(wp[j], pj, o[e]);
                  }
                }
                if constexpr (OUT_F32) {
                  f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(Out) + orow + d0);
                  if (MERGE && has_a) {
                    const f32x4 a = *p;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = fmaf(wa, a[e], wb * o[e]);
                  }
                  *p = f32x4{o[0], o[1], o[2], o[3]};
                } else {
                  bf16x4* p = reinterpret_cast<bf16x4*>(static_cast<__bf16*>(Out) + orow + d0);
                  if (MERGE && has_a) {
                    const bf16x4 a = *p;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = fmaf(wa, (float)a[e], wb * o[e]);
                  }
                  *p = bf16x4{(__bf16)o[0], (__bf16)o[1], (__bf16)o[2], (__bf16)o[3]};
                }
              }
            }
          }
          if (hi == 0) LSE[lrow] = lse_new * kLn2;
        }
      }
    }
    if constexpr (SPLIT) __syncthreads();  // LDS is reused by the next piece
  }  // piece loop
}

}  // namespace

// Launch for one head dim (explicitly instantiated in the attn_bf16_d*.hip
// files so the instantiations compile in parallel).  split_grid > 0 selects
// the SPLIT kernel on that many workgroups, with `ws` laid out as
// attn_split_workspace_bytes describes (one record per query tile).  A
// non-null `blocks` selects the MULTI kernel over blocks->n blocks of Nkv
// keys (K and V unused); merge is then not supported.
template <int D>
hipError_t launch_bf16_d(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH,
                         int Nq, int Nkv, float scale, bool out_f32, bool merge, int split_grid,
                         void* ws, const KVBlocks* blocks, hipStream_t stream) {
  constexpr int NG = kGroups;
  constexpr int kRowsWG = (kThreads / 64) * 32 * NG;
  static_assert(kRowsWG == kAttnRowsPerTile && kBc == kAttnKeysPerTile,
                "the split planner's tile sizes must match the kernel's");
  const int n_qtiles = (Nq + kRowsWG - 1) / kRowsWG;
  const int n_items = n_qtiles * BH;
  const float c2 = scale * kLog2e;
  const __bf16* q = static_cast<const __bf16*>(Q);
  const __bf16* k = static_cast<const __bf16*>(K);
  const __bf16* v = static_cast<const __bf16*>(V);
  using Kern = void (*)(const __bf16*, const __bf16*, const __bf16*, void*, float*, int, int, int,
                        float, int, char*, KVBlocks, int, unsigned);
  const bool split = split_grid > 0;
  const bool multi = blocks != nullptr;
  if (multi && merge) return hipErrorInvalidValue;
  // [out_f32][merge][split], then [out_f32][split] for the block sets
  static constexpr Kern kKernels[2][2][2] = {
      {{attn_fwd_bf16_kernel<D, NG, false, false, false, false>, attn_fwd_bf16_kernel<D, NG, false, false, true, false>},
       {attn_fwd_bf16_kernel<D, NG, false, true, false, false>, attn_fwd_bf16_kernel<D, NG, false, true, true, false>}},
      {{attn_fwd_bf16_kernel<D, NG, true, false, false, false>, attn_fwd_bf16_kernel<D, NG, true, false, true, false>},
       {attn_fwd_bf16_kernel<D, NG, true, true, false, false>, attn_fwd_bf16_kernel<D, NG, true, true, true, false>}}};
  static constexpr Kern kMulti[2][2] = {
      {attn_fwd_bf16_kernel<D, NG, false, false, false, true>, attn_fwd_bf16_kernel<D, NG, false, false, true, true>},
      {attn_fwd_bf16_kernel<D, NG, true, false, false, true>, attn_fwd_bf16_kernel<D, NG, true, false, true, true>}};
  const Kern kern = multi ? kMulti[out_f32][split] : kKernels[out_f32][merge][split];
  KVBlocks blk{};
  int n_blocks = 1;
  unsigned magic = 0;
  if (multi) {
    blk = *blocks;
    n_blocks = blocks->n;
    const unsigned tpb = (unsigned)((Nkv + kBc - 1) / kBc);
    magic = tpb > 1 ? (unsigned)(((1ull << 32) + tpb - 1) / tpb) : 0u;  // ceil(2^32 / tpb)
  }
  const dim3 grid((unsigned)(split ? split_grid : n_items));
  kern<<<grid, kThreads, 0, stream>>>(q, k, v, O, LSE, Nq, Nkv, n_qtiles, c2, n_items,
                                      split ? static_cast<char*>(ws) : nullptr, blk, n_blocks, magic);
  return hipGetLastError();
}

}  // namespace dit
