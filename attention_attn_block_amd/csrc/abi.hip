// C ABI of libdit_attn: argument validation and dispatch.
//
// Every check runs before any HIP runtime call, so a rejected call touches
// neither the device nor the stream (and the checks can be exercised on a
// machine without a GPU).  Accepted calls enqueue their kernels on the
// caller's stream and return without synchronising.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/dit_attn.h"
#include "launch.h"

static_assert(DIT_RELMAE_NOALLOC_MAX_N == dit::kRelmaeStaticMaxN,
              "the header's limit must match the library's scratch array");
static_assert(DIT_MAX_KV_BLOCKS == dit::kAttnMaxBlocks && DIT_MAX_BLOCK_KEYS == dit::kAttnMaxBlockKeys,
              "the header's block-set limits must match the kernel's");

namespace {

constexpr long long kMaxI32 = 0x7fffffffLL;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na && nb && x < y + nb && y < x + na;
}

bool dtype_ok(int t) { return t == DIT_F32 || t == DIT_BF16; }
size_t elt_size(dit_dtype_t t) { return t == DIT_BF16 ? 2 : 4; }
bool head_dim_ok(int d) { return d >= 8 && d <= 128 && d % 8 == 0; }

dit_status_t from_hip(hipError_t e) { return e == hipSuccess ? DIT_OK : DIT_ERR_HIP; }

// Shared checks of the attention calls; fills the byte sizes of each tensor.
dit_status_t check_attn(const void* Q, const void* K, const void* V, const void* O,
                        const float* LSE, int B, int H, int Nq, int Nkv, int d, float scale,
                        int in_dtype, int out_dtype, size_t* q_bytes, size_t* kv_bytes,
                        size_t* o_bytes, size_t* l_bytes) {
  if (!Q || !K || !V || !O || !LSE) return DIT_ERR_INVALID_ARG;
  if (B <= 0 || H <= 0 || Nq <= 0 || Nkv <= 0 || d <= 0) return DIT_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return DIT_ERR_INVALID_ARG;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return DIT_ERR_INVALID_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return DIT_ERR_INVALID_ARG;
  if (!head_dim_ok(d)) return DIT_ERR_UNSUPPORTED;
  if (in_dtype == DIT_F32 && out_dtype != DIT_F32) return DIT_ERR_UNSUPPORTED;
  const long long bh = (long long)B * H;
  // Work items (query tiles of 64 rows at the finest) must fit a 1-D grid.
  if (bh > kMaxI32 || bh * ((Nq + 63) / 64) > kMaxI32) return DIT_ERR_UNSUPPORTED;
  const size_t ie = elt_size((dit_dtype_t)in_dtype), oe = elt_size((dit_dtype_t)out_dtype);
  *q_bytes = (size_t)bh * Nq * d * ie;
  *kv_bytes = (size_t)bh * Nkv * d * ie;
  *o_bytes = (size_t)bh * Nq * d * oe;
  *l_bytes = (size_t)bh * Nq * sizeof(float);
  return DIT_OK;
}

bool outputs_clash(const void* O, size_t ob, const float* L, size_t lb, const void* const* ins,
                   const size_t* in_bytes, int n_in) {
  if (overlaps(O, ob, L, lb)) return true;
  for (int i = 0; i < n_in; ++i)
    if (overlaps(O, ob, ins[i], in_bytes[i]) || overlaps(L, lb, ins[i], in_bytes[i])) return true;
  return false;
}

dit_status_t run_attn(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH,
                      int Nq, int Nkv, int d, float scale, int in_dtype, int out_dtype, bool merge,
                      void* ws, bool force_split, hipStream_t stream) {
  if (in_dtype == DIT_BF16)
    return from_hip(dit::launch_attn_bf16(Q, K, V, O, LSE, BH, Nq, Nkv, d, scale,
                                          out_dtype == DIT_F32, merge, ws, force_split, stream));
  return from_hip(dit::launch_attn_f32(static_cast<const float*>(Q), static_cast<const float*>(K),
                                       static_cast<const float*>(V), static_cast<float*>(O), LSE,
                                       BH, Nq, Nkv, d, scale, merge, stream));
}

// The patch step for a patch of n_runs runs of run_len buffer rows, run r at
// rows [p0 + r * run_stride, +run_len) (one run: a contiguous patch), with an
// optional split workspace (null: plain launch).
dit_status_t patch_fwd(const void* Q_p, const void* K_p, const void* V_p, void* K_buf, void* V_buf,
                       void* O, float* LSE, int B, int H, int run_len, int n_runs, int run_stride,
                       int N, int p0, int d, float scale, dit_dtype_t in_dtype,
                       dit_dtype_t out_dtype, void* ws, long long ws_bytes, hipStream_t stream);

}  // namespace

extern "C" {

dit_status_t attn_block_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int B, int H, int Nq, int Nkv, int d, float scale,
                            dit_dtype_t in_dtype, dit_dtype_t out_dtype, hipStream_t stream) {
  size_t qb, kvb, ob, lb;
  const dit_status_t st = check_attn(Q, K, V, O, LSE, B, H, Nq, Nkv, d, scale, (int)in_dtype,
                                     (int)out_dtype, &qb, &kvb, &ob, &lb);
  if (st != DIT_OK) return st;
  const void* ins[3] = {Q, K, V};
  const size_t inb[3] = {qb, kvb, kvb};
  if (outputs_clash(O, ob, LSE, lb, ins, inb, 3)) return DIT_ERR_INVALID_ARG;
  return run_attn(Q, K, V, O, LSE, B * H, Nq, Nkv, d, scale, in_dtype, out_dtype, false, nullptr,
                  false, stream);
}

dit_status_t attn_block_fwd_merge(const void* Q, const void* K, const void* V, void* O_acc,
                                  float* LSE_acc, int B, int H, int Nq, int Nkv, int d,
                                  float scale, dit_dtype_t in_dtype, dit_dtype_t acc_dtype,
                                  hipStream_t stream) {
  size_t qb, kvb, ob, lb;
  const dit_status_t st = check_attn(Q, K, V, O_acc, LSE_acc, B, H, Nq, Nkv, d, scale,
                                     (int)in_dtype, (int)acc_dtype, &qb, &kvb, &ob, &lb);
  if (st != DIT_OK) return st;
  const void* ins[3] = {Q, K, V};
  const size_t inb[3] = {qb, kvb, kvb};
  if (outputs_clash(O_acc, ob, LSE_acc, lb, ins, inb, 3)) return DIT_ERR_INVALID_ARG;
  return run_attn(Q, K, V, O_acc, LSE_acc, B * H, Nq, Nkv, d, scale, in_dtype, acc_dtype, true,
                  nullptr, false, stream);
}

long long attn_block_workspace_bytes(int B, int H, int Nq, int Nkv, int d) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nkv <= 0 || !head_dim_ok(d)) return 0;
  const long long items = (long long)B * H * ((Nq + dit::kAttnRowsPerTile - 1) / dit::kAttnRowsPerTile);
  return dit::attn_split_workspace_bytes(items);
}

dit_status_t attn_block_fwd_ws(const void* Q, const void* K, const void* V, void* O_acc,
                               float* LSE_acc, int B, int H, int Nq, int Nkv, int d, float scale,
                               dit_dtype_t in_dtype, dit_dtype_t out_dtype, int flags,
                               void* workspace, long long workspace_bytes, hipStream_t stream) {
  size_t qb, kvb, ob, lb;
  const dit_status_t st = check_attn(Q, K, V, O_acc, LSE_acc, B, H, Nq, Nkv, d, scale,
                                     (int)in_dtype, (int)out_dtype, &qb, &kvb, &ob, &lb);
  if (st != DIT_OK) return st;
  if (flags & ~(DIT_WS_MERGE | DIT_WS_FORCE_SPLIT)) return DIT_ERR_INVALID_ARG;
  const long long need = attn_block_workspace_bytes(B, H, Nq, Nkv, d);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return DIT_ERR_INVALID_ARG;
  const void* ins[3] = {Q, K, V};
  const size_t inb[3] = {qb, kvb, kvb};
  if (outputs_clash(O_acc, ob, LSE_acc, lb, ins, inb, 3)) return DIT_ERR_INVALID_ARG;
  const void* all[5] = {Q, K, V, O_acc, LSE_acc};
  const size_t allb[5] = {qb, kvb, kvb, ob, lb};
  for (int i = 0; i < 5; ++i)
    if (overlaps(workspace, (size_t)need, all[i], allb[i])) return DIT_ERR_INVALID_ARG;
  return run_attn(Q, K, V, O_acc, LSE_acc, B * H, Nq, Nkv, d, scale, in_dtype, out_dtype,
                  (flags & DIT_WS_MERGE) != 0, workspace, (flags & DIT_WS_FORCE_SPLIT) != 0, stream);
}

dit_status_t attn_ring_fwd(const void* Q, const void* const* K_blocks,
                          const void* const* V_blocks, int n_blocks, void* O, float* LSE, int B,
                          int H, int Nq, int Nkv_block, int d, float scale, dit_dtype_t in_dtype,
                          dit_dtype_t out_dtype, int flags, void* workspace,
                          long long workspace_bytes, hipStream_t stream) {
  if (!K_blocks || !V_blocks) return DIT_ERR_INVALID_ARG;
  if (n_blocks < 1 || n_blocks > DIT_MAX_KV_BLOCKS) return DIT_ERR_INVALID_ARG;
  for (int i = 0; i < n_blocks; ++i)
    if (!K_blocks[i] || !V_blocks[i]) return DIT_ERR_INVALID_ARG;
  size_t qb, kvb, ob, lb;
  dit_status_t st = check_attn(Q, K_blocks[0], V_blocks[0], O, LSE, B, H, Nq, Nkv_block, d, scale,
                               (int)in_dtype, (int)out_dtype, &qb, &kvb, &ob, &lb);
  if (st != DIT_OK) return st;
  for (int i = 1; i < n_blocks; ++i)
    if (!aligned16(K_blocks[i]) || !aligned16(V_blocks[i])) return DIT_ERR_INVALID_ARG;
  if (flags & ~DIT_WS_FORCE_SPLIT) return DIT_ERR_INVALID_ARG;
  if (in_dtype != DIT_BF16) return DIT_ERR_UNSUPPORTED;
  if (Nkv_block > dit::kAttnMaxBlockKeys) return DIT_ERR_UNSUPPORTED;
  const long long keys = (long long)n_blocks * ((Nkv_block + dit::kAttnKeysPerTile - 1) /
                                                dit::kAttnKeysPerTile) * dit::kAttnKeysPerTile;
  if (keys > kMaxI32) return DIT_ERR_UNSUPPORTED;
  // Outputs overlap nothing that is read: Q and every block.
  if (overlaps(O, ob, LSE, lb) || overlaps(O, ob, Q, qb) || overlaps(LSE, lb, Q, qb))
    return DIT_ERR_INVALID_ARG;
  for (int i = 0; i < n_blocks; ++i) {
    const void* kv[2] = {K_blocks[i], V_blocks[i]};
    for (int j = 0; j < 2; ++j)
      if (overlaps(O, ob, kv[j], kvb) || overlaps(LSE, lb, kv[j], kvb)) return DIT_ERR_INVALID_ARG;
  }
  if (workspace) {
    const long long need = attn_block_workspace_bytes(B, H, Nq, Nkv_block, d);
    if (workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
      return DIT_ERR_INVALID_ARG;
    if (overlaps(workspace, (size_t)need, Q, qb) || overlaps(workspace, (size_t)need, O, ob) ||
        overlaps(workspace, (size_t)need, LSE, lb))
      return DIT_ERR_INVALID_ARG;
    for (int i = 0; i < n_blocks; ++i)
      if (overlaps(workspace, (size_t)need, K_blocks[i], kvb) ||
          overlaps(workspace, (size_t)need, V_blocks[i], kvb))
        return DIT_ERR_INVALID_ARG;
  }
  dit::KVBlocks blocks{};
  blocks.n = n_blocks;
  for (int i = 0; i < n_blocks; ++i) {
    blocks.k[i] = K_blocks[i];
    blocks.v[i] = V_blocks[i];
  }
  return from_hip(dit::launch_attn_bf16_blocks(Q, &blocks, O, LSE, B * H, Nq, Nkv_block, d, scale,
                                               out_dtype == DIT_F32, workspace,
                                               (flags & DIT_WS_FORCE_SPLIT) != 0, stream));
}

dit_status_t attn_lse_merge(void* O_a, float* LSE_a, const void* O_b, const float* LSE_b,
                            long long rows, int d, dit_dtype_t o_dtype, hipStream_t stream) {
  if (!O_a || !LSE_a || !O_b || !LSE_b) return DIT_ERR_INVALID_ARG;
  if (rows <= 0 || d <= 0) return DIT_ERR_INVALID_ARG;
  if (!dtype_ok((int)o_dtype)) return DIT_ERR_INVALID_ARG;
  if (!aligned16(O_a) || !aligned16(LSE_a) || !aligned16(O_b) || !aligned16(LSE_b))
    return DIT_ERR_INVALID_ARG;
  if (!head_dim_ok(d)) return DIT_ERR_UNSUPPORTED;
  if (rows > (kMaxI32 * 4LL)) return DIT_ERR_UNSUPPORTED;
  const size_t ob = (size_t)rows * d * elt_size(o_dtype), lb = (size_t)rows * sizeof(float);
  const bool same_o = O_a == O_b, same_l = LSE_a == LSE_b;
  if (same_o != same_l) return DIT_ERR_INVALID_ARG;          // half-aliased pair
  if (!same_o && (overlaps(O_a, ob, O_b, ob) || overlaps(LSE_a, lb, LSE_b, lb)))
    return DIT_ERR_INVALID_ARG;
  if (overlaps(O_a, ob, LSE_a, lb) || overlaps(O_a, ob, LSE_b, lb) || overlaps(O_b, ob, LSE_a, lb))
    return DIT_ERR_INVALID_ARG;
  return from_hip(dit::launch_lse_merge(O_a, LSE_a, O_b, LSE_b, rows, d, o_dtype == DIT_BF16, stream));
}

dit_status_t attn_patch_fwd(const void* Q_p, const void* K_p, const void* V_p, void* K_buf,
                            void* V_buf, void* O, float* LSE, int B, int H, int Np, int N, int p0,
                            int d, float scale, dit_dtype_t in_dtype, dit_dtype_t out_dtype,
                            hipStream_t stream) {
  return patch_fwd(Q_p, K_p, V_p, K_buf, V_buf, O, LSE, B, H, Np, 1, Np, N, p0, d, scale,
                   in_dtype, out_dtype, nullptr, 0, stream);
}

dit_status_t attn_patch_fwd_ws(const void* Q_p, const void* K_p, const void* V_p, void* K_buf,
                               void* V_buf, void* O, float* LSE, int B, int H, int Np, int N,
                               int p0, int d, float scale, dit_dtype_t in_dtype,
                               dit_dtype_t out_dtype, void* workspace, long long workspace_bytes,
                               hipStream_t stream) {
  if (!workspace) return DIT_ERR_INVALID_ARG;
  return patch_fwd(Q_p, K_p, V_p, K_buf, V_buf, O, LSE, B, H, Np, 1, Np, N, p0, d, scale,
                   in_dtype, out_dtype, workspace, workspace_bytes, stream);
}

dit_status_t attn_patch_fwd_strided(const void* Q_p, const void* K_p, const void* V_p,
                                    void* K_buf, void* V_buf, void* O, float* LSE, int B, int H,
                                    int run_len, int n_runs, int run_stride, int N, int p0, int d,
                                    float scale, dit_dtype_t in_dtype, dit_dtype_t out_dtype,
                                    void* workspace, long long workspace_bytes,
                                    hipStream_t stream) {
  return patch_fwd(Q_p, K_p, V_p, K_buf, V_buf, O, LSE, B, H, run_len, n_runs, run_stride, N, p0,
                   d, scale, in_dtype, out_dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {
dit_status_t patch_fwd(const void* Q_p, const void* K_p, const void* V_p, void* K_buf, void* V_buf,
                       void* O, float* LSE, int B, int H, int run_len, int n_runs, int run_stride,
                       int N, int p0, int d, float scale, dit_dtype_t in_dtype,
                       dit_dtype_t out_dtype, void* ws, long long ws_bytes, hipStream_t stream) {
  if (!K_p || !V_p || !K_buf || !V_buf) return DIT_ERR_INVALID_ARG;
  if (N <= 0 || run_len <= 0 || n_runs <= 0 || p0 < 0) return DIT_ERR_INVALID_ARG;
  // Runs must not overlap (and go forward); the last must end inside the buffer.
  if (n_runs > 1 && run_stride < run_len) return DIT_ERR_INVALID_ARG;
  const long long last_end = (long long)p0 + (long long)(n_runs - 1) * (n_runs > 1 ? run_stride : 0) +
                             run_len;
  if (last_end > N) return DIT_ERR_INVALID_ARG;
  // The runs are disjoint rows of [0, N), so Np <= N fits an int.
  const int Np = (int)((long long)run_len * n_runs);
  size_t qb, kvb, ob, lb;
  const dit_status_t st = check_attn(Q_p, K_buf, V_buf, O, LSE, B, H, Np, N, d, scale,
                                     (int)in_dtype, (int)out_dtype, &qb, &kvb, &ob, &lb);
  if (st != DIT_OK) return st;
  if (!aligned16(K_p) || !aligned16(V_p)) return DIT_ERR_INVALID_ARG;
  const size_t pb = qb;  // fresh K/V patches have the query patch's shape
  if (overlaps(K_buf, kvb, V_buf, kvb)) return DIT_ERR_INVALID_ARG;
  const void* bufs[2] = {K_buf, V_buf};
  const void* fresh[3] = {Q_p, K_p, V_p};
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 3; ++j)
      if (overlaps(bufs[i], kvb, fresh[j], pb)) return DIT_ERR_INVALID_ARG;
  const void* ins[5] = {Q_p, K_p, V_p, K_buf, V_buf};
  const size_t inb[5] = {pb, pb, pb, kvb, kvb};
  if (outputs_clash(O, ob, LSE, lb, ins, inb, 5)) return DIT_ERR_INVALID_ARG;
  if (ws) {
    const long long need = attn_block_workspace_bytes(B, H, Np, N, d);
    if (ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 255u)) return DIT_ERR_INVALID_ARG;
    const void* all[7] = {Q_p, K_p, V_p, K_buf, V_buf, O, LSE};
    const size_t allb[7] = {pb, pb, pb, kvb, kvb, ob, lb};
    for (int i = 0; i < 7; ++i)
      if (overlaps(ws, (size_t)need, all[i], allb[i])) return DIT_ERR_INVALID_ARG;
  }

  const long long row_units = (long long)d * (long long)elt_size(in_dtype) / 16;
  hipError_t e = dit::launch_splice2(K_p, K_buf, V_p, V_buf, (long long)B * H, n_runs,
                                     (long long)run_len * row_units, (long long)N * row_units,
                                     (long long)(n_runs > 1 ? run_stride : 0) * row_units,
                                     (long long)p0 * row_units, stream);
  if (e != hipSuccess) return DIT_ERR_HIP;
  return run_attn(Q_p, K_buf, V_buf, O, LSE, B * H, Np, N, d, scale, in_dtype, out_dtype, false,
                  ws, false, stream);
}
}  // namespace

extern "C" {

dit_status_t cfg_combine(const float* eps_u, const float* eps_c, float* out, long long n, float s,
                         hipStream_t stream) {
  if (!eps_u || !eps_c || !out) return DIT_ERR_INVALID_ARG;
  if (n <= 0 || !isfinite(s)) return DIT_ERR_INVALID_ARG;
  if (!aligned16(eps_u) || !aligned16(eps_c) || !aligned16(out)) return DIT_ERR_INVALID_ARG;
  const size_t nb = (size_t)n * sizeof(float);
  if (out != eps_u && overlaps(out, nb, eps_u, nb)) return DIT_ERR_INVALID_ARG;
  if (out != eps_c && overlaps(out, nb, eps_c, nb)) return DIT_ERR_INVALID_ARG;
  return from_hip(dit::launch_cfg(eps_u, eps_c, out, n, s, stream));
}

long long cfg_combine_relmae_workspace(long long n) {
  return n > 0 ? dit::cfg_relmae_work_floats(n) : 0;
}

dit_status_t cfg_combine_relmae(const float* eps_u, const float* eps_c, float* out, long long n,
                                float s, float* workspace, float* relmae, hipStream_t stream) {
  if (!eps_u || !eps_c || !out || !workspace || !relmae) return DIT_ERR_INVALID_ARG;
  if (n <= 0 || !isfinite(s)) return DIT_ERR_INVALID_ARG;
  if (!aligned16(eps_u) || !aligned16(eps_c) || !aligned16(out) || !aligned16(workspace) ||
      !aligned16(relmae))
    return DIT_ERR_INVALID_ARG;
  const size_t nb = (size_t)n * sizeof(float);
  const size_t wb = (size_t)dit::cfg_relmae_work_floats(n) * sizeof(float);
  if (out != eps_u && overlaps(out, nb, eps_u, nb)) return DIT_ERR_INVALID_ARG;
  if (out != eps_c && overlaps(out, nb, eps_c, nb)) return DIT_ERR_INVALID_ARG;
  const void* all[3] = {eps_u, eps_c, out};
  for (int i = 0; i < 3; ++i)
    if (overlaps(workspace, wb, all[i], nb) || overlaps(relmae, 4, all[i], nb))
      return DIT_ERR_INVALID_ARG;
  if (overlaps(workspace, wb, relmae, 4)) return DIT_ERR_INVALID_ARG;
  return from_hip(dit::launch_cfg_relmae(eps_u, eps_c, out, n, s, workspace, relmae, stream));
}

dit_status_t cfg_combine_relmae_noalloc(const float* eps_u, const float* eps_c, float* out,
                                        long long n, float s, float* relmae, hipStream_t stream) {
  if (!eps_u || !eps_c || !out || !relmae) return DIT_ERR_INVALID_ARG;
  if (n <= 0 || !isfinite(s)) return DIT_ERR_INVALID_ARG;
  if (!aligned16(eps_u) || !aligned16(eps_c) || !aligned16(out) || !aligned16(relmae))
    return DIT_ERR_INVALID_ARG;
  if (n > DIT_RELMAE_NOALLOC_MAX_N) return DIT_ERR_UNSUPPORTED;
  const size_t nb = (size_t)n * sizeof(float);
  if (out != eps_u && overlaps(out, nb, eps_u, nb)) return DIT_ERR_INVALID_ARG;
  if (out != eps_c && overlaps(out, nb, eps_c, nb)) return DIT_ERR_INVALID_ARG;
  const void* all[3] = {eps_u, eps_c, out};
  for (int i = 0; i < 3; ++i)
    if (overlaps(relmae, 4, all[i], nb)) return DIT_ERR_INVALID_ARG;
  return from_hip(dit::launch_cfg_relmae_static(eps_u, eps_c, out, n, s, relmae, stream));
}

const char* dit_status_string(dit_status_t status) {
  switch (status) {
    case DIT_OK:
      return "DIT_OK: success";
    case DIT_ERR_INVALID_ARG:
      return "DIT_ERR_INVALID_ARG: invalid argument (null, non-positive size, misaligned or "
             "overlapping buffer, bad scale, patch out of range or unknown dtype)";
    case DIT_ERR_UNSUPPORTED:
      return "DIT_ERR_UNSUPPORTED: valid but unsupported (head dim, dtype pairing or size)";
    case DIT_ERR_HIP:
      return "DIT_ERR_HIP: the HIP kernel launch failed";
  }
  return "unknown dit_status_t value";
}

}  // extern "C"
