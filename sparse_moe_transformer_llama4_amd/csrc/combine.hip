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

// The same with k routed picks per token (slot rows t*k + j of r, written
// once each by the routed down GEMM): out[t] = y[t] (its partials in order)
// + r[t*k] + r[t*k + 1] + ... + r[t*k + k - 1], in fp32, in this order.
__global__ __launch_bounds__(256) void combine_topk_kernel(const f32x4* r, int k, const f32x4* y, int parts,
                                                           void* out, int64_t n4, int d4, int out_bf16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n4; i += stride) {
    const int64_t t = i / d4;
    const int64_t c = i - t * d4;
    f32x4 v = y[i];
    for (int q = 1; q < parts; ++q) v += y[q * n4 + i];
    for (int j = 0; j < k; ++j) v += r[(t * k + j) * d4 + c];
    if (out_bf16) {
      const uint32_t lo = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
      const uint32_t hi = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
      reinterpret_cast<uint2*>(out)[i] = make_uint2(lo, hi);
    } else {
      reinterpret_cast<f32x4*>(out)[i] = v;
    }
  }
}

// SwiGLU over summed K-split partials of the gate/up GEMM (the same SiLU and
// products as the gate/up epilogue): thread -> 4 consecutive columns.
__global__ __launch_bounds__(256) void swiglu_parts_kernel(const float* gu, int parts, int T, int N, uint16_t* h) {
  const int n4 = N / 4;
  const int64_t total = static_cast<int64_t>(T) * n4;
  const int64_t pstride = static_cast<int64_t>(T) * 2 * N;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t t = i / n4;
    const int c = static_cast<int>(i - t * n4) * 4;
    const float* g0 = gu + t * 2 * N + c;
    f32x4 g = *reinterpret_cast<const f32x4*>(g0);
    f32x4 u = *reinterpret_cast<const f32x4*>(g0 + N);
    for (int q = 1; q < parts; ++q) {
      g += *reinterpret_cast<const f32x4*>(g0 + q * pstride);
      u += *reinterpret_cast<const f32x4*>(g0 + q * pstride + N);
    }
    uint16_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = f32_to_bf16(silu_f(g[j]) * u[j]);
    *reinterpret_cast<uint2*>(h + t * N + c) =
        make_uint2(v[0] | (static_cast<uint32_t>(v[1]) << 16), v[2] | (static_cast<uint32_t>(v[3]) << 16));
  }
}

}  // namespace

hipError_t launch_swiglu_parts(const float* gu, int parts, int T, int N, uint16_t* h, hipStream_t s) {
  if (N % 4 != 0 || parts < 1) return hipErrorInvalidValue;
  const int64_t total = static_cast<int64_t>(T) * (N / 4);
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(swiglu_parts_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, gu, parts, T, N, h);
  return hipGetLastError();
}

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

hipError_t launch_combine_topk(const float* r, int k, const float* y, int parts, void* out, int T, int d,
                               int out_bf16, hipStream_t s) {
  if (d % 4 != 0 || parts < 1 || k < 1) return hipErrorInvalidValue;
  const int64_t n4 = static_cast<int64_t>(T) * (d / 4);
  if (n4 == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(combine_topk_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     reinterpret_cast<const f32x4*>(r), k, reinterpret_cast<const f32x4*>(y), parts, out, n4, d / 4,
                     out_bf16);
  return hipGetLastError();
}

}  // namespace moe
