// Explicit instantiations of the bf16 attention launch for head dims 8, 16, 24, 32, 40, 48.
#include "attn_bf16_kernel.h"

namespace dit {
template hipError_t launch_bf16_d<8>(const void*, const void*, const void*, void*, float*, int, int, int, float, bool, bool, int, void*, const KVBlocks*, hipStream_t);
template hipError_t launch_bf16_d<16>(const void*, const void*, const void*, void*, float*, int, int, int, float, bool, bool, int, void*, const KVBlocks*, hipStream_t);
template hipError_t launch_bf16_d<24>(const void*, const void*, const void*, void*, float*, int, int, int, float, bool, bool, int, void*, const KVBlocks*, hipStream_t);
template hipError_t launch_bf16_d<32>(const void*, const void*, const void*, void*, float*, int, int, int, float, bool, bool, int, void*, const KVBlocks*, hipStream_t);
template hipError_t launch_bf16_d<40>(const void*, const void*, const void*, void*, float*, int, int, int, float, bool, bool, int, void*, const KVBlocks*, hipStream_t);
template hipError_t launch_bf16_d<48>(const void*, const void*, const void*, void*, float*, int, int, int, float, bool, bool, int, void*, const KVBlocks*, hipStream_t);
}  // namespace dit
