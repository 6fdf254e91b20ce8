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

// Workspace of the split launch for `n_items` query tiles of head dim d: one
// arrival counter per tile (uint32, zero between calls), then kAttnMaxPieces
// fp32 partials per tile (O rows, then LSE).
struct AttnSplitLayout {
  long long part_offset;  // bytes; the counters occupy [0, part_offset)
  long long bytes;        // total
};
inline AttnSplitLayout attn_split_layout(long long n_items, int d) {
  const long long counters = (n_items * 4 + 255) / 256 * 256;
  const long long part = (long long)kAttnRowsPerTile * (d + 1) * 4;
  return {counters, counters + n_items * kAttnMaxPieces * part};
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

// Attention with bfloat16 Q/K/V (matrix cores), fp32 or bf16 output.  With
// `merge`, (O, LSE) hold a running partial that the block's result is folded
// into (LSE = -inf: empty) instead of being overwritten.  A non-null `ws`
// (attn_split_layout bytes, counters zero) allows the split launch for blocks
// of at least kAttnSplitMinKeyTiles key tiles, or of any length with
// force_split.
hipError_t launch_attn_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int BH, int Nq, int Nkv, int d, float scale, bool out_f32, bool merge,
                            void* ws, bool force_split, hipStream_t stream);

// Attention with float32 Q/K/V/O (vector ALU, no reduced-precision products);
// `merge` as for launch_attn_bf16.
hipError_t launch_attn_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                           int BH, int Nq, int Nkv, int d, float scale, bool merge,
                           hipStream_t stream);

// In-place log-sum-exp merge a <- a (+) b over `rows` rows of width d.
hipError_t launch_lse_merge(void* Oa, float* La, const void* Ob, const float* Lb,
                            long long rows, int d, bool bf16, hipStream_t stream);

// Copy `nseg` segments of `seg_units` 16-byte units from src (packed) into
// dst, where segment i starts at unit i * dst_seg_stride + dst_offset.
// Two independent copies (K and V) run in one launch.
hipError_t launch_splice2(const void* src0, void* dst0, const void* src1, void* dst1,
                          int nseg, long long seg_units, long long dst_seg_stride,
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

}  // namespace dit
