// Internal launchers shared by the C-ABI layer (abi.hip) and the kernel
// files.  Callers have validated every argument; these only pick a kernel
// instantiation, size the grid and enqueue on `stream`.
#pragma once

#include <hip/hip_runtime.h>

namespace dit {

// Attention with bfloat16 Q/K/V (matrix cores), fp32 or bf16 output.  With
// `merge`, (O, LSE) hold a running partial that the block's result is folded
// into (LSE = -inf: empty) instead of being overwritten.
hipError_t launch_attn_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int BH, int Nq, int Nkv, int d, float scale, bool out_f32, bool merge,
                            hipStream_t stream);

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
