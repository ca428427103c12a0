// Routing stage of the Llama 4 MoE block on gfx950:
//   router GEMM (fp32 logits) -> top-1 (lowest index among maxima) ->
//   sigmoid gate -> per-workgroup expert histogram -> column scan to expert
//   offsets + per-group tile tables -> stable permutation (tokens grouped by
//   expert, ascending token index inside a group).
//
// The router is one logit per expert and the choice is the argmax
// (superteams.ai "Llama 4", section "Mixture of Experts: Why Total and
// Active Parameters Diverge"); the gate is the sigmoid of the chosen logit,
// applied to the routed expert's input (KerasFormers "Llama 4", section
// "What is unusual about the block").
#include "common.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------- e4m3

// float -> OCP e4m3fn code, round to nearest even, saturating at +-448.
// Written from the format definition (4 significant bits, exponent bias 7,
// subnormal quantum 2^-9, largest finite 448 = code 0x7E).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(v);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0.015625f) {                     // below 2^-6: subnormal grid of 2^-9
    const float q = rintf(a * 512.0f);     // exact scaling, RNE; q in [0, 8]
    return sign | static_cast<uint32_t>(q);
  }
  const uint32_t ua = __float_as_uint(a);
  int e = static_cast<int>(ua >> 23) - 127;
  const uint32_t m = ua & 0x7FFFFFu;
  const uint32_t r = m + 0x7FFFFu + ((m >> 20) & 1u);  // drop 20 mantissa bits, ties to even
  e += static_cast<int>(r >> 23);
  const uint32_t mant = (r >> 20) & 7u;
  if (e > 8 || (e == 8 && mant == 7u)) return sign | 0x7Eu;
  return sign | (static_cast<uint32_t>(e + 7) << 3) | mant;
}

// ---------------------------------------------------------------- router

template <int DT> struct RouterT;
template <> struct RouterT<DT_BF16> {
  static constexpr int KC = 64;     // K elements staged per chunk
  static constexpr int KSTEP = 32;  // K of one MFMA
};
template <> struct RouterT<DT_F32> {
  static constexpr int KC = 32;
  static constexpr int KSTEP = 4;
};

// One workgroup = 4 waves = 64 tokens; each wave computes a 16 x Ep logit
// tile with 16x16 MFMAs (Ep = E rounded up to 16).  The router weight chunk
// [KC x E] is staged in LDS transposed to [E][KC] so that every lane reads
// its K-contiguous MFMA operand with one LDS access.
template <int DT>
__global__ __launch_bounds__(256) void router_kernel(RouterArgs a) {
  using R = RouterT<DT>;
  constexpr int KC = R::KC;
  constexpr int PITCH = KC + 8;  // elements per LDS row (padding breaks bank aliasing)
  using Elem = typename std::conditional<DT == DT_BF16, uint16_t, float>::type;
  __shared__ Elem wt[256 * PITCH];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, d = a.d, T = a.T;
  const int Ep = (E + 15) & ~15;
  const int nf = Ep >> 4;
  const int t0 = blockIdx.x * kRouteTokens + wave * 16;
  const int trow = min(t0 + (lane & 15), T - 1);
  const Elem* xrow = reinterpret_cast<const Elem*>(a.x) + static_cast<int64_t>(trow) * d;
  const Elem* wr = reinterpret_cast<const Elem*>(a.wr);

  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // zero the padding rows E..Ep-1 once
  for (int i = tid; i < (Ep - E) * PITCH; i += 256) wt[E * PITCH + i] = Elem(0);

  for (int k0 = 0; k0 < d; k0 += KC) {
    __syncthreads();
    for (int i = tid; i < KC * E; i += 256) {
      const int k = i / E, e = i - k * E;
      wt[e * PITCH + k] = wr[static_cast<int64_t>(k0 + k) * E + e];
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KC; ks += R::KSTEP) {
      if constexpr (DT == DT_BF16) {
        const int kk = ks + (lane >> 4) * 8;
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(xrow + k0 + kk);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j < nf) {
            const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&wt[(j * 16 + (lane & 15)) * PITCH + kk]);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[j], 0, 0, 0);
          }
        }
      } else {
        const int kk = ks + (lane >> 4);
        const float av = xrow[k0 + kk];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j < nf) {
            const float bv = wt[(j * 16 + (lane & 15)) * PITCH + kk];
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[j], 0, 0, 0);
          }
        }
      }
    }
  }

  // Lane holds logits of rows 4*(lane/16)+q, column j*16 + lane%16.
  // Per row: best (value, index) over this lane's columns (ascending), then
  // across the 16 lanes of the row group; ties go to the lower index.
  const int col0 = lane & 15;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float best = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (j < nf) {
        const int e = j * 16 + col0;
        if (e < E) {
          float v = acc[j][q];
          if (a.bias) v += a.bias[e];
          if (v > best) { best = v; bi = e; }
        }
      }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      const float ov = __shfl_xor(best, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
    }
    bi = min(bi, E - 1);  // only reachable with non-finite logits (outside the contract)
    const int t = t0 + 4 * (lane >> 4) + q;
    if (col0 == 0 && t < T) {
      a.idx[t] = bi;
      a.gate[t] = 1.0f / (1.0f + expf(-best));
    }
  }

  // per-workgroup histogram
  __shared__ int hist[256];
  for (int e = tid; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  if (tid < kRouteTokens) {
    const int t = blockIdx.x * kRouteTokens + tid;
    if (t < T) atomicAdd(&hist[a.idx[t]], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) a.hist[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
}

// Per-token e4m3 quantisation of x (bf16): s = fp32(max|x_t|) / 448 (1 for
// a zero row), code = e4m3(x / s).  One wave per token row.
__global__ __launch_bounds__(256) void quant_x_kernel(const uint16_t* x, int T, int d, uint8_t* xq,
                                                      float* sx) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint16_t* row = x + static_cast<int64_t>(t) * d;
  float amax = 0.f;
  for (int k = lane * 8; k < d; k += 64 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      amax = fmaxf(amax, fabsf(__uint_as_float(w[i] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
  const float s = amax > 0.f ? amax / 448.0f : 1.0f;
  if (lane == 0) sx[t] = s;
  uint8_t* qrow = xq + static_cast<int64_t>(t) * d;
  for (int k = lane * 8; k < d; k += 64 * 8) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      lo |= f32_to_e4m3(__uint_as_float(w[i] << 16) / s) << (16 * i);
      lo |= f32_to_e4m3(__uint_as_float(w[i] & 0xFFFF0000u) / s) << (16 * i + 8);
      hi |= f32_to_e4m3(__uint_as_float(w[i + 2] << 16) / s) << (16 * i);
      hi |= f32_to_e4m3(__uint_as_float(w[i + 2] & 0xFFFF0000u) / s) << (16 * i + 8);
    }
    *reinterpret_cast<uint2*>(qrow + k) = make_uint2(lo, hi);
  }
}

// Per-row e4m3 quantisation of fp32 h rows with a precomputed row max:
// s = max|h| / 448 (1 for a zero row), code = e4m3(h / s).
__global__ __launch_bounds__(256) void quant_h_kernel(const float* h, const uint32_t* amax, int rows,
                                                      int n, uint8_t* hq, float* sh) {
  const int r = blockIdx.x;
  if (r >= rows) return;
  const float am = __uint_as_float(amax[r]);
  const float s = am > 0.f ? am / 448.0f : 1.0f;
  if (blockIdx.y == 0 && threadIdx.x == 0) sh[r] = s;
  const int k = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (k >= n) return;
  const float* src = h + static_cast<int64_t>(r) * n + k;
  const float4 v0 = *reinterpret_cast<const float4*>(src);
  const float4 v1 = *reinterpret_cast<const float4*>(src + 4);
  const uint32_t lo = f32_to_e4m3(v0.x / s) | (f32_to_e4m3(v0.y / s) << 8) | (f32_to_e4m3(v0.z / s) << 16) |
                      (f32_to_e4m3(v0.w / s) << 24);
  const uint32_t hi = f32_to_e4m3(v1.x / s) | (f32_to_e4m3(v1.y / s) << 8) | (f32_to_e4m3(v1.z / s) << 16) |
                      (f32_to_e4m3(v1.w / s) << 24);
  *reinterpret_cast<uint2*>(hq + static_cast<int64_t>(r) * n + k) = make_uint2(lo, hi);
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------- scan

// Block-wide exclusive scan of one int per thread (256 threads).
__device__ int block_exclusive_scan(int v, int* sm, int* total) {
  const int tid = threadIdx.x;
  sm[tid] = v;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int o = tid >= off ? sm[tid - off] : 0;
    __syncthreads();
    sm[tid] += o;
    __syncthreads();
  }
  const int incl = sm[tid];
  if (total) *total = sm[255];
  __syncthreads();
  return incl - v;
}

// One workgroup: column scan of the per-workgroup histograms.
//   hist[b][e] <- offsets[e] + sum_{b' < b} hist[b'][e]   (base of block b in group e)
//   counts[e], offsets[e]
//   tiles[i][g] = sum_{g' < g} ceil(n_g' / BM_i) for g = 0..E+1, where group E
//   is the shared expert (n_E = T) and entry E+1 is the total.
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  __shared__ int sm[256];
  const int e = threadIdx.x;
  const int E = a.E;
  int running = 0;
  if (e < E) {
    for (int b = 0; b < a.nblocks; ++b) {
      int* p = a.hist + static_cast<int64_t>(b) * E + e;
      const int c = *p;
      *p = running;
      running += c;
    }
  }
  const int cnt = e < E ? running : 0;
  int total = 0;
  const int off = block_exclusive_scan(cnt, sm, &total);
  if (e < E) {
    a.counts[e] = cnt;
    a.offsets[e] = off;
    for (int b = 0; b < a.nblocks; ++b) a.hist[static_cast<int64_t>(b) * E + e] += off;
  }
  if (e == 0) a.offsets[E] = total;
  for (int i = 0; i < kNumBM; ++i) {
    const int bm = bm_of(i);
    const int mt = (cnt + bm - 1) / bm;
    int tot = 0;
    const int start = block_exclusive_scan(mt, sm, &tot);
    int* tt = a.tiles + i * (E + 2);
    if (e < E) tt[e] = start;
    if (e == 0) {
      tt[E] = tot;                            // the shared group follows the routed ones
      tt[E + 1] = tot + (a.T + bm - 1) / bm;
    }
  }
}

// Stable position of every token: perm[base[b][e] + rank] = t, where rank
// counts earlier tokens of the same workgroup routed to the same expert.
__global__ __launch_bounds__(64) void perm_kernel(const int32_t* idx, const int32_t* base, int T, int E,
                                                  int32_t* perm) {
  __shared__ int ids[kRouteTokens];
  const int t = blockIdx.x * kRouteTokens + threadIdx.x;
  ids[threadIdx.x] = t < T ? idx[t] : -1;
  __syncthreads();
  if (t >= T) return;
  const int e = ids[threadIdx.x];
  int rank = 0;
  for (int j = 0; j < static_cast<int>(threadIdx.x); ++j) rank += ids[j] == e;
  perm[base[static_cast<int64_t>(blockIdx.x) * E + e] + rank] = t;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_router(const RouterArgs& a, int x_dtype, hipStream_t s) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  if (x_dtype == DT_BF16)
    hipLaunchKernelGGL(router_kernel<DT_BF16>, dim3(nb), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(router_kernel<DT_F32>, dim3(nb), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_perm(const int32_t* idx, const int32_t* base, int T, int E, int32_t* perm,
                       hipStream_t s) {
  const int nb = (T + kRouteTokens - 1) / kRouteTokens;
  hipLaunchKernelGGL(perm_kernel, dim3(nb), dim3(kRouteTokens), 0, s, idx, base, T, E, perm);
  return hipGetLastError();
}

hipError_t launch_quant_x(const uint16_t* x, int T, int d, uint8_t* xq, float* sx, hipStream_t s) {
  hipLaunchKernelGGL(quant_x_kernel, dim3((T + 3) / 4), dim3(256), 0, s, x, T, d, xq, sx);
  return hipGetLastError();
}

hipError_t launch_quant_h(const float* h, const uint32_t* amax, int rows, int n, uint8_t* hq,
                          float* sh, hipStream_t s) {
  hipLaunchKernelGGL(quant_h_kernel, dim3(rows, (n + 2047) / 2048), dim3(256), 0, s, h, amax, rows, n,
                     hq, sh);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, p, n,
                     v);
  return hipGetLastError();
}

}  // namespace moe
