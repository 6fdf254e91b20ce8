// Head-dim dispatch of the bf16 attention launches (kernel in
// attn_bf16_kernel.h; instantiations in attn_bf16_d*.hip).
#include <hip/hip_runtime.h>

#include "launch.h"

namespace dit {

template <int D>
hipError_t launch_bf16_d(const void* Q, const void* K, const void* V, void* O, float* LSE, int BH,
                         int Nq, int Nkv, float scale, bool out_f32, bool merge,
                         hipStream_t stream);

hipError_t launch_attn_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int BH, int Nq, int Nkv, int d, float scale, bool out_f32, bool merge,
                            hipStream_t stream) {
  switch (d) {
#define DIT_CASE(DD) \
  case DD:           \
    return launch_bf16_d<DD>(Q, K, V, O, LSE, BH, Nq, Nkv, scale, out_f32, merge, stream);
    DIT_CASE(8) DIT_CASE(16) DIT_CASE(24) DIT_CASE(32) DIT_CASE(40) DIT_CASE(48) DIT_CASE(56)
    DIT_CASE(64) DIT_CASE(72) DIT_CASE(80) DIT_CASE(88) DIT_CASE(96) DIT_CASE(104) DIT_CASE(112)
    DIT_CASE(120) DIT_CASE(128)
#undef DIT_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace dit
