/*
 * A plain C caller of libdit_attn (no Python, no torch): device memory from
 * hipMalloc, calls through include/dit_attn.h only.  Used by the GPU tests to
 * check the ABI from a native client against the fp64 oracle.
 *
 *   abi_client <in.bin> <out.bin>
 *
 * in.bin  : int32 B, H, Nq, Nkv, d, nblocks; float32 scale;
 *           Q [B,H,Nq,d], K, V [B,H,Nkv,d] as bfloat16 bit patterns (uint16).
 * out.bin : for each of (full attention, unfused block fold, fused block fold,
 *           full attention through attn_block_fwd_ws with a forced split):
 *           O [B,H,Nq,d] float32 then LSE [B,H,Nq] float32.
 * The KV rows are cut into `nblocks` consecutive blocks of near-equal length.
 * Exit status 0 on success; any failing call prints its status text.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../include/dit_attn.h"

#define HIP_OK(x)                                                         \
  do {                                                                    \
    hipError_t e_ = (x);                                                  \
    if (e_ != hipSuccess) {                                               \
      fprintf(stderr, "%s:%d HIP error %s\n", __FILE__, __LINE__,         \
              hipGetErrorString(e_));                                     \
      return 1;                                                           \
    }                                                                     \
  } while (0)
#define DIT_OK_OR_FAIL(x)                                                 \
  do {                                                                    \
    dit_status_t s_ = (x);                                                \
    if (s_ != DIT_OK) {                                                   \
      fprintf(stderr, "%s:%d %s\n", __FILE__, __LINE__,                   \
              dit_status_string(s_));                                     \
      return 1;                                                           \
    }                                                                     \
  } while (0)

static int read_all(FILE* f, void* p, size_t n) { return fread(p, 1, n, f) == n ? 0 : 1; }

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s in.bin out.bin\n", argv[0]);
    return 2;
  }
  FILE* fi = fopen(argv[1], "rb");
  if (!fi) return 2;
  int32_t hdr[6];
  float scale;
  if (read_all(fi, hdr, sizeof hdr) || read_all(fi, &scale, sizeof scale)) return 2;
  const int B = hdr[0], H = hdr[1], Nq = hdr[2], Nkv = hdr[3], d = hdr[4], nb = hdr[5];
  if (B < 1 || H < 1 || Nq < 1 || Nkv < 1 || nb < 1 || nb > Nkv) return 2;
  const size_t BH = (size_t)B * H;
  const size_t nq = BH * Nq * d, nkv = BH * Nkv * d;
  uint16_t* hq = (uint16_t*)malloc(nq * 2);
  uint16_t* hk = (uint16_t*)malloc(nkv * 2);
  uint16_t* hv = (uint16_t*)malloc(nkv * 2);
  if (!hq || !hk || !hv) return 2;
  if (read_all(fi, hq, nq * 2) || read_all(fi, hk, nkv * 2) || read_all(fi, hv, nkv * 2)) return 2;
  fclose(fi);

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  void *dq, *dk, *dv, *dkb, *dvb;
  float *o_full, *l_full, *o_acc, *l_acc, *o_tmp, *l_tmp, *o_fus, *l_fus, *o_ws, *l_ws;
  void* ws;
  HIP_OK(hipMalloc(&dq, nq * 2));
  HIP_OK(hipMalloc(&dk, nkv * 2));
  HIP_OK(hipMalloc(&dv, nkv * 2));
  HIP_OK(hipMalloc(&dkb, nkv * 2));
  HIP_OK(hipMalloc(&dvb, nkv * 2));
  HIP_OK(hipMalloc((void**)&o_full, nq * 4));
  HIP_OK(hipMalloc((void**)&o_acc, nq * 4));
  HIP_OK(hipMalloc((void**)&o_tmp, nq * 4));
  HIP_OK(hipMalloc((void**)&o_fus, nq * 4));
  HIP_OK(hipMalloc((void**)&l_full, BH * Nq * 4));
  HIP_OK(hipMalloc((void**)&l_acc, BH * Nq * 4));
  HIP_OK(hipMalloc((void**)&l_tmp, BH * Nq * 4));
  HIP_OK(hipMalloc((void**)&l_fus, BH * Nq * 4));
  HIP_OK(hipMalloc((void**)&o_ws, nq * 4));
  HIP_OK(hipMalloc((void**)&l_ws, BH * Nq * 4));
  const long long ws_bytes = attn_block_workspace_bytes(B, H, Nq, Nkv, d);
  if (ws_bytes <= 0) return 2;
  HIP_OK(hipMalloc(&ws, (size_t)ws_bytes));
  HIP_OK(hipMemset(ws, 0, (size_t)ws_bytes)); /* counters start at zero */
  HIP_OK(hipMemcpy(dq, hq, nq * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, hk, nkv * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, hv, nkv * 2, hipMemcpyHostToDevice));

  /* 1. full attention */
  DIT_OK_OR_FAIL(attn_block_fwd(dq, dk, dv, o_full, l_full, B, H, Nq, Nkv, d, scale, DIT_BF16,
                                DIT_F32, st));

  /* 4. the same through the workspace call (split where the grid allows) */
  DIT_OK_OR_FAIL(attn_block_fwd_ws(dq, dk, dv, o_ws, l_ws, B, H, Nq, Nkv, d, scale, DIT_BF16,
                                   DIT_F32, DIT_WS_FORCE_SPLIT, ws, ws_bytes, st));

  /* 2./3. block folds: copy each block into contiguous [B,H,n,d] buffers */
  float* ninf = (float*)malloc(BH * Nq * 4);
  for (size_t i = 0; i < BH * Nq; ++i) ninf[i] = -INFINITY;
  HIP_OK(hipMemcpyAsync(l_fus, ninf, BH * Nq * 4, hipMemcpyHostToDevice, st));
  int start = 0;
  for (int j = 0; j < nb; ++j) {
    const int stop = (int)(((long long)Nkv * (j + 1)) / nb);
    const int n = stop - start;
    const size_t row_bytes = (size_t)d * 2;
    HIP_OK(hipMemcpy2DAsync(dkb, (size_t)n * row_bytes, (char*)dk + (size_t)start * row_bytes,
                            (size_t)Nkv * row_bytes, (size_t)n * row_bytes, BH,
                            hipMemcpyDeviceToDevice, st));
    HIP_OK(hipMemcpy2DAsync(dvb, (size_t)n * row_bytes, (char*)dv + (size_t)start * row_bytes,
                            (size_t)Nkv * row_bytes, (size_t)n * row_bytes, BH,
                            hipMemcpyDeviceToDevice, st));
    if (j == 0) {
      DIT_OK_OR_FAIL(attn_block_fwd(dq, dkb, dvb, o_acc, l_acc, B, H, Nq, n, d, scale, DIT_BF16,
                                    DIT_F32, st));
    } else {
      DIT_OK_OR_FAIL(attn_block_fwd(dq, dkb, dvb, o_tmp, l_tmp, B, H, Nq, n, d, scale, DIT_BF16,
                                    DIT_F32, st));
      DIT_OK_OR_FAIL(attn_lse_merge(o_acc, l_acc, o_tmp, l_tmp, (long long)BH * Nq, d, DIT_F32, st));
    }
    DIT_OK_OR_FAIL(attn_block_fwd_merge(dq, dkb, dvb, o_fus, l_fus, B, H, Nq, n, d, scale,
                                        DIT_BF16, DIT_F32, st));
    HIP_OK(hipStreamSynchronize(st)); /* block buffers are reused */
    start = stop;
  }

  /* a rejected call must not disturb the stream or the results */
  if (attn_block_fwd(NULL, dk, dv, o_full, l_full, B, H, Nq, Nkv, d, scale, DIT_BF16, DIT_F32,
                     st) != DIT_ERR_INVALID_ARG)
    return 3;
  HIP_OK(hipStreamSynchronize(st));

  FILE* fo = fopen(argv[2], "wb");
  if (!fo) return 2;
  float* ho = (float*)malloc(nq * 4);
  float* hl = (float*)malloc(BH * Nq * 4);
  float* outs[4][2] = {{o_full, l_full}, {o_acc, l_acc}, {o_fus, l_fus}, {o_ws, l_ws}};
  for (int r = 0; r < 4; ++r) {
    HIP_OK(hipMemcpy(ho, outs[r][0], nq * 4, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(hl, outs[r][1], BH * Nq * 4, hipMemcpyDeviceToHost));
    if (fwrite(ho, 4, nq, fo) != nq || fwrite(hl, 4, BH * Nq, fo) != BH * Nq) return 2;
  }
  fclose(fo);
  printf("abi_client ok\n");
  return 0;
}
