// bf16 grouped GEMMs for prefill-sized token counts: the 64- and 128-row
// tiles, and the entry point that picks a tile height (the 256-row tiles live
// in gemm_bf16_tall.hip).  The kernel is in gemm_bf16_kernel.h.
//
// This unit is compiled with VGPR-form MFMAs (-amdgpu-mfma-vgpr-form=1): the
// accumulators of these tiles (64 / 128 registers) fit in VGPRs, and with the
// AGPR form the register allocator copied them between registers on every
// iteration of the main loop.
#include "gemm_bf16_kernel.h"

namespace moe {

bool bf16_v2_supported(int K, int N, int N_shared) {
  return K % (2 * BK) == 0 && N % 64 == 0 && N_shared % 64 == 0;
}

hipError_t launch_gemm_bf16_v2(int mode, int bm, const GemmArgs& a, int T, hipStream_t s,
                               const int32_t* tiles_all) {
  if (bm == 256) return launch_gemm_bf16_tall(mode, a, T, s, tiles_all);
  const bool b128 = bm == 128;
  switch (mode) {
    case MODE_GATEUP:
      return b128 ? launch_v2<MODE_GATEUP, 128, 2, 2>(a, T, s, tiles_all)
                  : launch_v2<MODE_GATEUP, 64, 1, 4>(a, T, s, tiles_all);
    case MODE_DOWN_SHARED:
      return b128 ? launch_v2<MODE_DOWN_SHARED, 128, 2, 2>(a, T, s, tiles_all)
                  : launch_v2<MODE_DOWN_SHARED, 64, 1, 4>(a, T, s, tiles_all);
    case MODE_DOWN_ROUTED:
      return b128 ? launch_v2<MODE_DOWN_ROUTED, 128, 2, 2>(a, T, s, tiles_all)
                  : launch_v2<MODE_DOWN_ROUTED, 64, 1, 4>(a, T, s, tiles_all);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
