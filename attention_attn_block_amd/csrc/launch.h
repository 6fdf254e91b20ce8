// Internal launchers shared by the C-ABI layer (abi.hip) and the kernel
// files.  Callers have validated every argument; these only pick a kernel
// instantiation, size the grid and enqueue on `stream`.
#pragma once

#include <hip/hip_runtime.h>

namespace dit {

// Query rows per workgroup and keys per K/V tile of the bf16 attention kernel,
// and the most workgroups a split launch may share one query tile between.
constexpr int kAttnRowsPerTile = 256;
constexpr int kAttnKeysPerTile = 64;
constexpr int kAttnMaxPieces = 4;

// Workspace of the split launch: one record of kAttnSplitItemBytes per query
// tile, the same size and layout for every shape and head dim, so that a
// workspace made for one call serves any later call with no more query tiles
// (at any head dim) without a counter ever landing on another call's
// partials.  Record i, at byte i * kAttnSplitItemBytes:
//   [0, 4)                          arrival counter (uint32, zero between calls)
//   [256 + j * kAttnSplitSlotBytes)  partial j < kAttnMaxPieces of the tile:
//                                    fp32 O rows [256][d], then LSE [256]
constexpr long long kAttnSplitSlotBytes = (long long)kAttnRowsPerTile * (128 + 1) * 4;
constexpr long long kAttnSplitItemBytes = 256 + kAttnMaxPieces * kAttnSplitSlotBytes;
inline long long attn_split_workspace_bytes(long long n_items) {
  return n_items * kAttnSplitItemBytes;
}

// Workgroup count for the split launch on a device with n_cu compute units,
// or 0 when the plain one-tile-per-workgroup grid should be used: it already
// fills at least 95% of its waves of workgroups, the block has fewer than
// min_key_tiles key tiles, or an even share would cut some query tile into
// more than kAttnMaxPieces pieces.
int attn_split_grid(long long n_items, int Nkv, int n_cu, int min_key_tiles);

// Key tiles below which a split costs more than it gains (measured on MI355X:
// the exchange of partials adds round trips to every workgroup's path that a
// 2048-key block cannot hide; from 6144 keys the split is 9-22% faster).
constexpr int kAttnSplitMinKeyTiles = 96;

// The KV blocks of one ring step, resident on the device: block i's K and V
// are [B, H, Nkv, d] buffers of their own.  Passed to the kernel by value.
constexpr int kAttnMaxBlocks = 16;
struct KVBlocks {
  const void* k[kAttnMaxBlocks];
  const void* v[kAttnMaxBlocks];
  int n;
};
// Keys per block of a block set, at most: keeps the kernel's scalar division
// of a key-tile index by the tiles per block exact (tile index x tiles per
// block < 2^32).
constexpr int kAttnMaxBlockKeys = 1 << 20;

// Attention with bfloat16 Q/K/V (matrix cores), fp32 or bf16 output.  With
// `merge`, (O, LSE) hold a running partial that the block's result is folded
// into (LSE = -inf: empty) instead of being overwritten.  A non-null `ws`
// (attn_split_workspace_bytes, counters zero) allows the split launch for
// blocks of at least kAttnSplitMinKeyTiles key tiles, or of any length with
// force_split.
hipError_t launch_attn_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int BH, int Nq, int Nkv, int d, float scale, bool out_f32, bool merge,
                            void* ws, bool force_split, hipStream_t stream);

// The same over the concatenation of a block set (blocks->n blocks of Nkv
// keys each, at most kAttnMaxBlockKeys), in one launch; no merge.
hipError_t launch_attn_bf16_blocks(const void* Q, const KVBlocks* blocks, void* O, float* LSE,
                                   int BH, int Nq, int Nkv, int d, float scale, bool out_f32,
                                   void* ws, bool force_split, hipStream_t stream);

// Attention with float32 Q/K/V/O (vector ALU, no reduced-precision products);
// `merge` as for launch_attn_bf16.
hipError_t launch_attn_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                           int BH, int Nq, int Nkv, int d, float scale, bool merge,
                           hipStream_t stream);

// In-place log-sum-exp merge a <- a (+) b over `rows` rows of width d.
hipError_t launch_lse_merge(void* Oa, float* La, const void* Ob, const float* Lb,
                            long long rows, int d, bool bf16, hipStream_t stream);

// Copy n_bh * n_runs segments of `run_units` 16-byte units from src (packed,
// segment s at unit s * run_units) into dst, where segment s = bh * n_runs + r
// starts at unit bh * dst_bh_stride + r * dst_run_stride + dst_offset.  Two
// independent copies (K and V) run in one launch.  Any segment count.
hipError_t launch_splice2(const void* src0, void* dst0, const void* src1, void* dst1,
                          long long n_bh, int n_runs, long long run_units,
                          long long dst_bh_stride, long long dst_run_stride,
                          long long dst_offset, hipStream_t stream);

// out = u + s * (c - u) over n floats.
hipError_t launch_cfg(const float* u, const float* c, float* out, long long n, float s,
                      hipStream_t stream);

// CFG combine plus rel-MAE = sum|c - u| / sum|u|: per-block partial sums go to
// `work` (cfg_relmae_work_floats(n) floats), a second launch reduces them in
// a fixed order and writes the ratio to *relmae.
long long cfg_relmae_work_floats(long long n);
hipError_t launch_cfg_relmae(const float* u, const float* c, float* out, long long n, float s,
                             float* work, float* relmae, hipStream_t stream);

// The same with the partial sums in the library's own device array of
// kRelmaeStaticFloats floats (one per GPU) instead of a caller workspace:
// n up to kRelmaeStaticMaxN.  Allocates nothing.
constexpr long long kRelmaeStaticFloats = 1LL << 16;            // 256 KiB
constexpr long long kRelmaeStaticMaxN = kRelmaeStaticFloats / 2 * 4096;  // 2^27
hipError_t launch_cfg_relmae_static(const float* u, const float* c, float* out, long long n,
                                    float s, float* relmae, hipStream_t stream);

}  // namespace dit
