// Head-dim dispatch of the bf16 attention launches (kernel in
// attn_bf16_kernel.h; instantiations in attn_bf16_d*.hip) and the planner of
// the split launch.
#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.h"

namespace dit {

template <int D>
hipError_t launch_bf16_d(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH,
                         int Nq, int Nkv, float scale, bool out_f32, bool merge, int split_grid,
                         void* ws, const KVBlocks* blocks, hipStream_t stream);

int attn_split_grid(long long n_items, int Nkv, int n_cu, int min_key_tiles) {
  const int n_all = (Nkv + kAttnKeysPerTile - 1) / kAttnKeysPerTile;
  if (n_cu <= 0 || n_items <= 0 || n_all < 4 || n_all < min_key_tiles) return 0;
  // One workgroup per CU at a time (the kernel's registers allow no more).
  const long long waves = (n_items + n_cu - 1) / n_cu;
  const long long grid = waves * n_cu;
  if (n_items * 100 >= grid * 95 || grid > (1LL << 24)) return 0;
  // Workgroup w owns units [total * w / grid, total * (w + 1) / grid); every
  // range must be non-empty and every query tile within kAttnMaxPieces ranges.
  const long long total = n_items * n_all;
  if (total < grid) return 0;
  auto owner = [&](long long x) { return ((x + 1) * grid + total - 1) / total - 1; };
  for (long long i = 0; i < n_items; ++i)
    if (owner(i * n_all + n_all - 1) - owner(i * n_all) + 1 > kAttnMaxPieces) return 0;
  return (int)grid;
}

namespace {
// Compute units of the device a stream runs on, queried once per device.
int device_cus(hipStream_t stream) {
  static std::atomic<int> cache[64];
  // The device the work runs on is the stream's, which need not be the
  // current one; the null stream runs on the current device.
  int dev = 0;
  if (stream) {
    hipDevice_t sd;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return 0;
    dev = sd;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return 0;
  }
  if (dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace

namespace {
hipError_t dispatch(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH, int Nq,
                    int Nkv, int d, float scale, bool out_f32, bool merge, int split_grid, void* ws,
                    const KVBlocks* blocks, hipStream_t stream) {
  switch (d) {
#define DIT_CASE(DD) \
  case DD:           \
    return launch_bf16_d<DD>(Q, K, V, O, LSE, BH, Nq, Nkv, scale, out_f32, merge, split_grid, ws, blocks, stream);
    DIT_CASE(8) DIT_CASE(16) DIT_CASE(24) DIT_CASE(32) DIT_CASE(40) DIT_CASE(48) DIT_CASE(56)
    DIT_CASE(64) DIT_CASE(72) DIT_CASE(80) DIT_CASE(88) DIT_CASE(96) DIT_CASE(104) DIT_CASE(112)
    DIT_CASE(120) DIT_CASE(128)
#undef DIT_CASE
    default:
      return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_attn_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int BH, int Nq, int Nkv, int d, float scale, bool out_f32, bool merge,
                            void* ws, bool force_split, hipStream_t stream) {
  const long long n_items = (long long)BH * ((Nq + kAttnRowsPerTile - 1) / kAttnRowsPerTile);
  const int split_grid =
      ws ? attn_split_grid(n_items, Nkv, device_cus(stream), force_split ? 0 : kAttnSplitMinKeyTiles) : 0;
  return dispatch(Q, K, V, O, LSE, BH, Nq, Nkv, d, scale, out_f32, merge, split_grid, ws, nullptr,
                  stream);
}

hipError_t launch_attn_bf16_blocks(const void* Q, const KVBlocks* blocks, void* O, float* LSE,
                                   int BH, int Nq, int Nkv, int d, float scale, bool out_f32,
                                   void* ws, bool force_split, hipStream_t stream) {
  if (!blocks || blocks->n < 1 || blocks->n > kAttnMaxBlocks || Nkv > kAttnMaxBlockKeys)
    return hipErrorInvalidValue;
  const long long n_items = (long long)BH * ((Nq + kAttnRowsPerTile - 1) / kAttnRowsPerTile);
  // The planner sees the concatenation: n blocks of whole key tiles each.
  const long long tpb = (Nkv + kAttnKeysPerTile - 1) / kAttnKeysPerTile;
  const long long keys = (long long)blocks->n * tpb * kAttnKeysPerTile;
  if (keys > 0x7fffffffLL) return hipErrorInvalidValue;
  const int split_grid = ws ? attn_split_grid(n_items, (int)keys, device_cus(stream),
                                              force_split ? 0 : kAttnSplitMinKeyTiles)
                            : 0;
  return dispatch(Q, nullptr, nullptr, O, LSE, BH, Nq, Nkv, d, scale, out_f32, false, split_grid,
                  ws, blocks, stream);
}

}  // namespace dit
