/*
 * dit_attn -- the per-device attention step of parallel DiT inference on one
 * AMD Instinct MI355X (gfx950), as a C ABI.
 *
 * The calls follow the problem as the pages state it:
 *  - attention over image-patch tokens is where DiT inference spends its time
 *    ("xDiT: an Inference Engine for Diffusion Transformers (DiTs) with
 *    Massive Parallelism", abstract);
 *  - sequence parallelism hands each device its queries plus a series of KV
 *    blocks whose partial results must be combined -- Ring attention passes
 *    the blocks between neighbours and Torus attention starts on each chunk as
 *    it arrives ("SwiftFusion: Scalable Sequence Parallelism for Distributed
 *    Inference of Diffusion Transformers on GPUs", sections 1 and 2);
 *  - PipeFusion, the patch-level pipeline, has a device attend its patch's
 *    queries to the whole image's KV (xDiT abstract), and Orchestra gives
 *    devices patches of unequal size ("Spatio-Temporal Parallelism for
 *    Diffusion Model Inference on Heterogeneous Multi-GPU Systems", abstract);
 *  - CFG parallelism runs the conditional and unconditional paths apart and
 *    only their noise predictions meet ("Accelerating Diffusion via Hybrid
 *    Data-Pipeline Parallelism Based on Conditional Guidance Scheduling",
 *    Technische Zusammenfassung, 2.A).
 * No page writes a formula; each call below states the textbook definition it
 * computes.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer is a device pointer owned by the caller and must be 16-byte
 *    aligned.  The library allocates no memory and keeps no per-call state;
 *    the calls that need scratch (cfg_combine_relmae, attn_block_fwd_ws,
 *    attn_patch_fwd_ws, attn_patch_fwd_strided with a workspace) take it
 *    from the caller, except
 *    cfg_combine_relmae_noalloc, which uses a fixed array of the library.
 *  - Work is enqueued on `stream` (0 = the null stream) and returns without
 *    synchronising.  Calls on different streams may run concurrently.
 *  - Tensors are row-major and contiguous: [B, H, N, d] with d innermost;
 *    log-sum-exp arrays are [B, H, N] float32.
 *  - Supported head dims: d a multiple of 8 with 8 <= d <= 128.
 *  - Element types: DIT_BF16 (bfloat16) or DIT_F32 (float32).  bfloat16
 *    inputs may produce bfloat16 or float32 outputs; float32 inputs produce
 *    float32 outputs.  Arithmetic is float32 throughout (bfloat16 matrix-core
 *    products accumulate in float32).
 *  - All argument checks run before any HIP call; a rejected call touches
 *    neither the device nor the stream.  Return codes:
 *      DIT_OK               enqueued;
 *      DIT_ERR_INVALID_ARG  null pointer, non-positive size, misaligned or
 *                           overlapping buffers, bad scale, patch out of range,
 *                           unknown dtype value;
 *      DIT_ERR_UNSUPPORTED  valid but not implemented (d, dtype pairing, sizes
 *                           beyond 32-bit indexing);
 *      DIT_ERR_HIP          the kernel launch failed.
 *    Faults inside a kernel surface at the caller's next synchronisation.
 *  - Log-sum-exp values are natural logarithms.  LSE = -inf marks an empty
 *    partial result in attn_lse_merge.
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DIT_OK = 0,
  DIT_ERR_INVALID_ARG = 1,
  DIT_ERR_UNSUPPORTED = 2,
  DIT_ERR_HIP = 3
} dit_status_t;

typedef enum { DIT_F32 = 0, DIT_BF16 = 1 } dit_dtype_t;

/*
 * Block attention: one query block against one KV block.
 *
 *   O[b,h,i,:] = sum_j softmax_j(scale * <Q[b,h,i,:], K[b,h,j,:]>) V[b,h,j,:]
 *   LSE[b,h,i] = ln sum_j exp(scale * <Q[b,h,i,:], K[b,h,j,:]>)
 *
 * This is the unit of work a sequence-parallel device repeats for every KV
 * block it receives (SwiftFusion, sections 1-2; xDiT abstract).  No mask or
 * bias: DiT self-attention over patches is bidirectional.
 *   Q: [B,H,Nq,d] in_dtype;  K, V: [B,H,Nkv,d] in_dtype      (read only)
 *   O: [B,H,Nq,d] out_dtype; LSE: [B,H,Nq] float32          (written)
 *   B, H, Nq, Nkv >= 1;  scale > 0 and finite (usually 1/sqrt(d)).
 * O and LSE must not overlap Q, K, V or each other.
 */
dit_status_t attn_block_fwd(const void* Q, const void* K, const void* V,
                            void* O, float* LSE,
                            int B, int H, int Nq, int Nkv, int d, float scale,
                            dit_dtype_t in_dtype, dit_dtype_t out_dtype,
                            hipStream_t stream);

/*
 * Fused ring step: block attention of Q against this KV block, folded into a
 * running partial (O_acc, LSE_acc) in the kernel epilogue.  The result equals
 * attn_block_fwd into temporaries followed by attn_lse_merge(O_acc, LSE_acc,
 * O_tmp, LSE_tmp), without writing or re-reading the block partial.  This is
 * the per-device step of Ring and Torus attention, which fold each KV block
 * (or chunk) as it arrives (SwiftFusion, sections 1-2).
 *   Q: [B,H,Nq,d], K, V: [B,H,Nkv,d] in_dtype              (read only)
 *   O_acc: [B,H,Nq,d] acc_dtype, LSE_acc: [B,H,Nq] float32  (read and written)
 * A row with LSE_acc = -inf is empty: its O_acc is not read and the block's
 * result is stored (so the first block needs no separate call: fill LSE_acc
 * with -inf).  Same argument rules and return codes as attn_block_fwd.
 */
dit_status_t attn_block_fwd_merge(const void* Q, const void* K, const void* V,
                                  void* O_acc, float* LSE_acc,
                                  int B, int H, int Nq, int Nkv, int d, float scale,
                                  dit_dtype_t in_dtype, dit_dtype_t acc_dtype,
                                  hipStream_t stream);

/* Flags of attn_block_fwd_ws. */
enum {
  DIT_WS_MERGE = 1,       /* fold into (O_acc, LSE_acc) as attn_block_fwd_merge */
  DIT_WS_FORCE_SPLIT = 2  /* split whenever the grid allows, whatever the block length */
};

/*
 * attn_block_fwd (flags without DIT_WS_MERGE) or attn_block_fwd_merge (with
 * it) with a workspace that lets the library share one query tile's keys
 * between up to four workgroups.  A block with few query tiles of 256 rows
 * (for example 24 heads x 2048 queries: 192 tiles on 256 compute units)
 * leaves part of the GPU idle when each tile is one workgroup; the workspace
 * call instead gives every compute unit an equal share of (query tile,
 * 64-key tile) work, and the partials of a cut tile are combined with the
 * log-sum-exp identity of attn_lse_merge (SwiftFusion, sections 1-2: blocks
 * over disjoint keys combine in any grouping).  Which piece combines depends
 * on timing, but the combination takes a fixed order, so repeated calls give
 * identical bits.  Results agree with the plain calls to within rounding
 * (not bit for bit).  The split is taken for blocks of at least 6144 keys
 * (shorter blocks gain less from the fuller grid than the exchange of
 * partials costs) unless DIT_WS_FORCE_SPLIT is set; shapes the plain grid
 * already fills, and fp32 inputs, always run the plain path.
 *   Q, K, V, O_acc, LSE_acc, dtypes: as attn_block_fwd / attn_block_fwd_merge
 *   workspace: device memory of at least attn_block_workspace_bytes(...)
 *              bytes, 256-byte aligned, owned by the caller, overlapping no
 *              tensor.  It must be zero-filled before its first use; every
 *              call leaves its arrival counters at zero again, so a workspace
 *              made for one shape serves any later call with no more query
 *              tiles, at any head dim.  One workspace serves one call at a
 *              time (calls that share a workspace on different streams race).
 * Returns DIT_ERR_INVALID_ARG for a null, short, misaligned or overlapping
 * workspace or unknown flags, otherwise as attn_block_fwd.
 * attn_block_workspace_bytes returns the workspace size for a shape, or 0 for
 * a non-positive size or an unsupported d: one record of 528640 bytes per
 * 256-row query tile (B * H * ceil(Nq / 256) records), whatever the head dim
 * -- an arrival counter in the record's first 256 bytes, then four float32
 * partials of 256 x (128 + 1).  A counter therefore sits at the same place
 * for every shape and never under another call's partials.
 */
long long attn_block_workspace_bytes(int B, int H, int Nq, int Nkv, int d);
dit_status_t attn_block_fwd_ws(const void* Q, const void* K, const void* V,
                               void* O_acc, float* LSE_acc,
                               int B, int H, int Nq, int Nkv, int d, float scale,
                               dit_dtype_t in_dtype, dit_dtype_t out_dtype, int flags,
                               void* workspace, long long workspace_bytes,
                               hipStream_t stream);

/*
 * One device's share of a Ring or Torus attention step in one launch: the
 * queries against the concatenation of every KV block of the step, with the
 * blocks resident on the device in buffers of their own (SwiftFusion,
 * sections 1-2: the device folds every block's partial into its output;
 * blocks over disjoint keys combine in any grouping).  The result is
 * attention over all n_blocks * Nkv_block keys, the same as attn_block_fwd
 * per block folded with attn_lse_merge, up to rounding, without writing or
 * re-reading any block partial and with one launch's fixed cost instead of
 * n_blocks.  A query tile's key range runs across the blocks in order; with
 * a workspace the range may be shared between workgroups as for
 * attn_block_fwd_ws.
 *   Q: [B,H,Nq,d] bfloat16 (read only)
 *   K_blocks, V_blocks: HOST arrays of n_blocks device pointers, each a
 *     [B,H,Nkv_block,d] bfloat16 buffer (read only; blocks may repeat)
 *   O: [B,H,Nq,d] out_dtype; LSE: [B,H,Nq] float32 (written)
 *   1 <= n_blocks <= DIT_MAX_KV_BLOCKS; 1 <= Nkv_block <= DIT_MAX_BLOCK_KEYS;
 *   flags: 0 or DIT_WS_FORCE_SPLIT; workspace: NULL (one workgroup per query
 *   tile) or as for attn_block_fwd_ws.
 * Returns DIT_ERR_UNSUPPORTED for float32 inputs (use attn_block_fwd_merge per
 * block) and for Nkv_block above the limit; otherwise as attn_block_fwd_ws.
 * O and LSE must not overlap Q, any block or the workspace.
 */
#define DIT_MAX_KV_BLOCKS 16
#define DIT_MAX_BLOCK_KEYS (1 << 20)
dit_status_t attn_ring_fwd(const void* Q, const void* const* K_blocks,
                           const void* const* V_blocks, int n_blocks,
                           void* O, float* LSE,
                           int B, int H, int Nq, int Nkv_block, int d, float scale,
                           dit_dtype_t in_dtype, dit_dtype_t out_dtype, int flags,
                           void* workspace, long long workspace_bytes,
                           hipStream_t stream);

/*
 * Log-sum-exp merge of two partials over disjoint key sets, in place into a.
 *
 * Per row r (rows = B*H*Nq):
 *   LSE_b = -inf           : a unchanged (an empty partial is the identity),
 *                            except that two empty partials give O_a <- 0
 *   LSE_a = -inf           : a <- b
 *   otherwise m = max(LSE_a, LSE_b), w_a = e^(LSE_a-m), w_b = e^(LSE_b-m),
 *             O_a <- (w_a O_a + w_b O_b) / (w_a + w_b),
 *             LSE_a <- m + ln(w_a + w_b).
 * This folds the result of each arriving KV block into a device's running
 * output (SwiftFusion, sections 1-2).
 *   O_a: [rows, d] o_dtype, LSE_a: [rows] float32     (read and written)
 *   O_b: [rows, d] o_dtype, LSE_b: [rows] float32     (read only)
 *   rows >= 1.  b may equal a exactly (O_b == O_a and LSE_b == LSE_a);
 *   any other overlap between a and b is rejected.
 */
dit_status_t attn_lse_merge(void* O_a, float* LSE_a,
                            const void* O_b, const float* LSE_b,
                            long long rows, int d, dit_dtype_t o_dtype,
                            hipStream_t stream);

/*
 * PipeFusion patch step: splice the fresh patch into the device's KV buffer,
 * then attend the patch queries to the whole buffer.
 *
 *   K_buf[b,h,p0+i,:] <- K_p[b,h,i,:],  V_buf[b,h,p0+i,:] <- V_p[b,h,i,:]
 *                                                  for 0 <= i < Np (bit copy)
 *   (O, LSE) <- attn_block_fwd(Q_p, K_buf, V_buf) over all N buffer rows.
 * Rows of the buffer outside [p0, p0+Np) keep whatever the caller left there
 * (stale KV from the previous denoising step) (xDiT abstract).  Any Np >= 1
 * at any offset is accepted, so devices may hold patches of unequal size
 * (Orchestra, abstract).
 *   Q_p, K_p, V_p: [B,H,Np,d] in_dtype       (read only)
 *   K_buf, V_buf:  [B,H,N,d] in_dtype        (rows [p0,p0+Np) overwritten)
 *   O: [B,H,Np,d] out_dtype; LSE: [B,H,Np] float32   (written)
 *   1 <= Np, 0 <= p0, p0 + Np <= N;  scale > 0 and finite.
 * The fresh patch must not overlap the buffers; O and LSE must overlap
 * nothing else.
 */
dit_status_t attn_patch_fwd(const void* Q_p, const void* K_p, const void* V_p,
                            void* K_buf, void* V_buf,
                            void* O, float* LSE,
                            int B, int H, int Np, int N, int p0, int d, float scale,
                            dit_dtype_t in_dtype, dit_dtype_t out_dtype,
                            hipStream_t stream);

/*
 * attn_patch_fwd with a split workspace (as attn_block_fwd_ws without flags):
 * the attention over the buffer may share its query tiles' keys between
 * workgroups.  A patch whose query tiles fill part of a wave of workgroups
 * gains from it (for example 24 heads x 4096 patch queries, PipeFusion on 8
 * devices over 32768 tokens: 384 tiles of 256 rows, 1.5 waves on 256
 * compute units).  Patches of unequal size (Orchestra, abstract) make such
 * fractions common.
 *   workspace: at least attn_block_workspace_bytes(B, H, Np, N, d) bytes,
 *              256-byte aligned, zero-filled before its first use, owned by
 *              the caller, overlapping no tensor; one call at a time.
 * Otherwise as attn_patch_fwd.
 */
dit_status_t attn_patch_fwd_ws(const void* Q_p, const void* K_p, const void* V_p,
                               void* K_buf, void* V_buf,
                               void* O, float* LSE,
                               int B, int H, int Np, int N, int p0, int d, float scale,
                               dit_dtype_t in_dtype, dit_dtype_t out_dtype,
                               void* workspace, long long workspace_bytes,
                               hipStream_t stream);

/*
 * PipeFusion patch step for a patch made of several evenly spaced runs of
 * buffer rows.  The pages split the image into patches (xDiT abstract) of
 * possibly unequal size (Orchestra, abstract) without fixing their shape; a
 * band of spatial rows across every frame of a video is, in frame-major
 * token order, one run of rows per frame:
 *   run r (0 <= r < n_runs) covers buffer rows
 *       [p0 + r * run_stride, p0 + r * run_stride + run_len),
 *   and the patch tensors hold the runs back to back (Np = n_runs * run_len
 *   rows; patch row r * run_len + i is buffer row p0 + r * run_stride + i).
 *   K_buf/V_buf: every run's rows <- the run's rows of K_p/V_p (bit copy);
 *   then (O, LSE) <- attn_block_fwd(Q_p, K_buf, V_buf) over all N rows.
 *   Q_p, K_p, V_p: [B,H,Np,d] in_dtype                 (read only)
 *   K_buf, V_buf:  [B,H,N,d] in_dtype                  (the runs' rows overwritten)
 *   O: [B,H,Np,d] out_dtype; LSE: [B,H,Np] float32     (written)
 *   run_len >= 1, n_runs >= 1, p0 >= 0; with n_runs > 1, run_stride >=
 *   run_len (runs in order, never overlapping; run_stride is not used when
 *   n_runs == 1); p0 + (n_runs - 1) * run_stride + run_len <= N; otherwise
 *   DIT_ERR_INVALID_ARG.
 *   workspace: NULL for the plain launch, or as for attn_patch_fwd_ws (at
 *   least attn_block_workspace_bytes(B, H, Np, N, d) bytes, zero-filled
 *   before its first use).
 * With n_runs == 1 this is attn_patch_fwd (workspace NULL) or
 * attn_patch_fwd_ws with Np = run_len.  Buffers and overlap rules as
 * attn_patch_fwd.
 */
dit_status_t attn_patch_fwd_strided(const void* Q_p, const void* K_p, const void* V_p,
                                    void* K_buf, void* V_buf,
                                    void* O, float* LSE,
                                    int B, int H, int run_len, int n_runs, int run_stride,
                                    int N, int p0, int d, float scale,
                                    dit_dtype_t in_dtype, dit_dtype_t out_dtype,
                                    void* workspace, long long workspace_bytes,
                                    hipStream_t stream);

/*
 * Classifier-free guidance combine of the unconditional and conditional
 * noise predictions (Hybridiff, Technische Zusammenfassung, 2.A):
 *   out[i] = eps_u[i] + s * (eps_c[i] - eps_u[i]),
 * evaluated in fp32 as fma(s, eps_c[i], (1 - s) * eps_u[i]) so that s = 1
 * returns eps_c and s = 0 returns eps_u bit for bit (finite inputs).
 *   eps_u, eps_c, out: [n] float32, n >= 1, s finite.
 *   out may be exactly eps_u or exactly eps_c; no other overlap.
 */
dit_status_t cfg_combine(const float* eps_u, const float* eps_c, float* out,
                         long long n, float s, hipStream_t stream);

/*
 * CFG combine fused with the cond/uncond discrepancy signal.  Hybridiff
 * switches between its sequential and parallel phases on a relative mean
 * absolute error between the conditional and unconditional noise
 * ("Accelerating Diffusion via Hybrid Data-Pipeline Parallelism ...",
 * Technische Zusammenfassung, 2.B); the page gives no formula, and the
 * reading used here is
 *   relmae = sum_i |eps_c[i] - eps_u[i]| / sum_i |eps_u[i]|   (0 if both are 0)
 * out is computed exactly as cfg_combine computes it.  The sums are reduced
 * per workgroup into `workspace`, then in a fixed order (deterministic).
 *   eps_u, eps_c, out: [n] float32 (out may be exactly eps_u or eps_c)
 *   workspace: device float32 array of cfg_combine_relmae_workspace(n) entries,
 *              owned by the caller, scratch (contents on return unspecified)
 *   relmae: device pointer to one float32, written
 * workspace and relmae must not overlap the tensors or each other.
 */
long long cfg_combine_relmae_workspace(long long n);
dit_status_t cfg_combine_relmae(const float* eps_u, const float* eps_c, float* out,
                                long long n, float s, float* workspace, float* relmae,
                                hipStream_t stream);

/*
 * cfg_combine_relmae for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same result, bit for bit, with the per-workgroup partial
 * sums kept in a fixed 256 KiB device array inside the library instead of a
 * caller workspace.  Each GPU the library runs on holds its own copy of that
 * array until the process ends; the call itself allocates nothing.  Calls
 * that overlap on one GPU (other streams, other threads) share the array and
 * race: the caller must order them.
 *   eps_u, eps_c, out, relmae: as cfg_combine_relmae;
 *   1 <= n <= DIT_RELMAE_NOALLOC_MAX_N (2^27); larger n returns
 *   DIT_ERR_UNSUPPORTED.
 * Returns DIT_ERR_HIP if the array's device address cannot be obtained on the
 * stream's device or the launch fails.
 */
#define DIT_RELMAE_NOALLOC_MAX_N (1LL << 27)
dit_status_t cfg_combine_relmae_noalloc(const float* eps_u, const float* eps_c, float* out,
                                        long long n, float s, float* relmae,
                                        hipStream_t stream);

/* Static English text for a status code (never NULL). */
const char* dit_status_string(dit_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */
