// bf16 grouped GEMMs: the 256-row tiles (each wave a 128 x 128 accumulator
// block in AGPRs).  The kernel is in gemm_bf16_kernel.h; this unit uses the
// default (AGPR-form) MFMA code generation.
#include "gemm_bf16_kernel.h"

namespace moe {

hipError_t launch_gemm_bf16_tall(int mode, const GemmArgs& a, int T, hipStream_t s, const int32_t* tiles_all) {
  switch (mode) {
    case MODE_GATEUP: return launch_v2<MODE_GATEUP, 256, 2, 2>(a, T, s, tiles_all);
    case MODE_DOWN_SHARED: return launch_v2<MODE_DOWN_SHARED, 256, 2, 2>(a, T, s, tiles_all);
    case MODE_DOWN_ROUTED: return launch_v2<MODE_DOWN_ROUTED, 256, 2, 2>(a, T, s, tiles_all);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
