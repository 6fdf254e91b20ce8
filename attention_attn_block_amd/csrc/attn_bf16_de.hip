// Explicit instantiations of the bf16 attention launch for head dims 120, 128.
#include "attn_bf16_kernel.h"

namespace dit {
template hipError_t launch_bf16_d<120>(const void*, const void*, const void*, void*, float*, int, int, int, float, bool, bool, int, void*, const KVBlocks*, hipStream_t);
template hipError_t launch_bf16_d<128>(const void*, const void*, const void*, void*, float*, int, int, int, float, bool, bool, int, void*, const KVBlocks*, hipStream_t);
}  // namespace dit
