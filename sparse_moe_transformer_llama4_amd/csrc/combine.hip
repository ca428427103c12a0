// Combine of the routed and the shared expert outputs when the two down GEMMs
// run unordered (on two streams): out[t][c] = r[t][c] + y[t][c] in fp32,
// rounded to bf16 for bf16 outputs; y may hold several K-split partials of
// the shared output, added in order (a dense layer has no r) (superteams.ai "Llama 4", routing sketch:
// the layer returns the shared expert's output plus the routed one).  r is the
// routed expert's output in token order (each row written once by the routed
// down GEMM), y the shared expert's.  It is the same fp32 addition, operand
// order included, that the routed down epilogue performs when it adds y
// itself, so both schedules give identical results.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void combine_kernel(const f32x4* r, const f32x4* y, int parts, void* out,
                                                      int64_t n4, int out_bf16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4; i += stride) {
    f32x4 v = r ? r[i] + y[i] : y[i];
    for (int q = 1; q < parts; ++q) v += y[q * n4 + i];
    if (out_bf16) {
      const uint32_t lo = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
      const uint32_t hi = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
      reinterpret_cast<uint2*>(out)[i] = make_uint2(lo, hi);
    } else {
      reinterpret_cast<f32x4*>(out)[i] = v;
    }
  }
}

}  // namespace

hipError_t launch_combine(const float* r, const float* y, int parts, void* out, int64_t n, int out_bf16,
                          hipStream_t s) {
  if (n % 4 != 0 || parts < 1) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(combine_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     reinterpret_cast<const f32x4*>(r), reinterpret_cast<const f32x4*>(y), parts, out, n4, out_bf16);
  return hipGetLastError();
}

}  // namespace moe
