// The RMSNorm in front of the block fused with the router GEMM (gfx950).
//
// The norm (llm-architectures-explained "Llama 4 Maverick", table "Every
// architecture field": RMSNorm before the MLP; KerasFormers "Llama 4",
// Llama4Model arguments: norm_eps) and the router (superteams.ai "Llama 4",
// routing sketch: one logit per expert) both read every row of x once; here
// one pass does both:
//   xn[t, j]   = x[t, j] * r_t * w[j],  r_t = 1 / sqrt(mean_j x[t, j]^2 + eps),
//                rounded once (RNE) to bf16 (fp64 sum of squares, r_t and
//                product, rounded to odd in fp32 before the bf16 rounding:
//                the correctly rounded value to ties closer than 2^-52);
//   logit[t,e] = sum_j xn[t, j] * W_router[j, e]  (fp32; the bias and the
//                top-k are left to the routing finish kernels);
// and, for e4m3 weights, xn's per-token e4m3 codes and scales
// (s = fp32 max|xn_t| / 448, code = e4m3(xn / s)).  Without the norm
// (NORM = false: a block with e4m3 weights and no RMSNorm in front) the same
// kernel quantises x itself and computes its logits, so x is read once for
// the router and the codes.
//
// Layout: a workgroup of 4 waves takes 16 rows; wave q holds columns
// [q d/4, (q+1) d/4) of those rows in registers, already in the operand
// layout of v_mfma_f32_16x16x32_bf16 (lane l: row l % 16, 8 consecutive
// columns 8 (l / 16) + 32 s for K step s).  So each element of x is loaded
// once, the row sums are reduced across the lanes and waves, the rows are
// normalised and stored in place, and the same registers feed the MFMA.  The
// router weight is read as B fragments from a copy packed per call
// (wr_pack_kernel: fragment (K step, 16 experts) = 64 lanes x 16 bytes,
// contiguous): every 16 rows read all of it from L2 (1.3 MB at d = 5120,
// E = 128), so the fragments stream through a per-wave LDS ring of 16 slots
// filled by direct-to-LDS loads (no VGPRs), 16 KB in flight per wave.  The
// four waves' partial logits (one K quarter each) are added in a fixed order
// through LDS.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kNRRows = 16;   // rows per workgroup
constexpr int kRing = 16;     // router weight fragments in flight per wave

typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8_t;

template <int N>
__device__ __forceinline__ void nr_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Direct-to-LDS 16-byte load of lane l's bytes [16 l, 16 l + 16) of a 1 KB
// fragment at `sbase` (wave-uniform) into LDS m0 + 16 l; it writes no VGPR.
__device__ __forceinline__ void nr_dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// Wr [d][E] bf16 -> pk[(ks * e16 + nf) * 64 + l] = the 8 values
// Wr[32 ks + 8 (l / 16) + i][16 nf + l % 16], i = 0..7 (0 past column E).
__global__ __launch_bounds__(64) void wr_pack_kernel(const uint16_t* wr, int d, int E, int e16, uint4* pk) {
  const int ks = blockIdx.x, nf = blockIdx.y, l = threadIdx.x;
  const int col = 16 * nf + (l & 15);
  const int k0 = 32 * ks + 8 * (l >> 4);
  uint32_t v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = col < E ? wr[static_cast<int64_t>(k0 + 2 * i) * E + col] : 0u;
    const uint32_t hi = col < E ? wr[static_cast<int64_t>(k0 + 2 * i + 1) * E + col] : 0u;
    v[i] = lo | (hi << 16);
  }
  pk[(static_cast<int64_t>(ks) * e16 + nf) * 64 + l] = make_uint4(v[0], v[1], v[2], v[3]);
}

struct NormRouteArgs {
  const uint16_t* x;   // [T][d] bf16
  const uint16_t* w;   // [d] bf16 gain
  int T, d, E, e16;
  float eps;
  const uint4* wr_pack;
  uint16_t* xn;        // [T][d]
  uint8_t* xq;         // [T][d] e4m3 codes (QUANT)
  float* sx;           // [T] (QUANT)
  float* logits;       // [T][E] fp32
};

// MAXS: K steps of 32 per wave the registers hold (d / 128 <= MAXS);
// NF: 16-expert fragments the accumulators hold (E <= 16 NF).
// Two workgroups per CU, except the norm at d > 2048: its row registers and
// fp64 temporaries need more than 256 VGPRs, so one workgroup per CU, whose
// waves then also have the 256 AGPRs (used by the allocator instead of
// scratch memory).
template <bool NORM, bool QUANT, int MAXS, int NF>
__global__ __launch_bounds__(256, (NORM && MAXS > 16) ? 1 : 2) void norm_route_kernel(NormRouteArgs a) {
  static_assert(NORM || QUANT, "without the norm the kernel is the router + x quantisation");
  static_assert(4 * kNRRows * NF * 16 * 4 <= 4 * kRing * 1024, "partial logits fit the ring");
  __shared__ uint4 gain[MAXS * 16];                       // d / 8 chunks of 8 values
  __shared__ double red_ss[4][kNRRows];
  __shared__ float red_am[4][kNRRows];
  // each wave's ring of kRing router weight fragments (1 KB each); after the
  // MFMAs it holds the partial logits [4 waves][16 rows][NF * 16]
  __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * kRing * 1024];
  const int tid = threadIdx.x, lane = tid & 63, q = tid >> 6;
  const int row = lane & 15, g = lane >> 4;
  const int T = a.T, d = a.d, nks = d >> 7;
  const int t0 = blockIdx.x * kNRRows;
  const int t = t0 + row;
  const bool live = t < T;
  const int kq = q * (d >> 2) + 8 * g;                    // this lane's first column
  const uint16_t* xrow = a.x + static_cast<int64_t>(min(t, T - 1)) * d + kq;

  uint4 xr[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s)
    if (s < nks) xr[s] = *reinterpret_cast<const uint4*>(xrow + 32 * s);
  if constexpr (NORM)
    for (int i = tid; i < (d >> 3); i += 256) gain[i] = reinterpret_cast<const uint4*>(a.w)[i];

  auto unpack = [](const uint4& u4, float (&v)[8]) {
    const uint32_t u[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  };

  float amax = 0.f;
  if constexpr (NORM) {
  // sum of squares (fp64: squares of bf16 values are exact), over the lane,
  // its row's four lane groups, then the four waves in order
  double ssp[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s < nks) {
      float v[8];
      unpack(xr[s], v);
#pragma unroll
      for (int i = 0; i < 8; ++i) ssp[i & 3] = fma(static_cast<double>(v[i]), static_cast<double>(v[i]), ssp[i & 3]);
    }
  }
  double ss = (ssp[0] + ssp[1]) + (ssp[2] + ssp[3]);
  ss += __shfl_xor(ss, 16, 64);
  ss += __shfl_xor(ss, 32, 64);
  if (g == 0) red_ss[q][row] = ss;
  __syncthreads();   // also publishes the gain
  const double tot = ((red_ss[0][row] + red_ss[1][row]) + red_ss[2][row]) + red_ss[3][row];
  const double r = 1.0 / sqrt(tot / static_cast<double>(d) + static_cast<double>(a.eps));

  // normalise in place, store the rows
  uint16_t* xnrow = a.xn + static_cast<int64_t>(t) * d + kq;
  const int gq = (q * (d >> 2)) >> 3;                     // this wave's first gain chunk
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    if (s < nks) {
      float v[8], wv[8], yf[8];
      unpack(xr[s], v);
      unpack(gain[gq + 4 * s + g], wv);
      // x r w in fp64 (within 2^-52 of the exact value), rounded to odd in
      // fp32: the bf16 rounding below is then the correct rounding of the
      // fp64 value.  Branch-free, so the row loop unrolls with the row in
      // registers (~6 us of VALU work on the largest shape)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        yf[i] = f64_to_f32_odd(static_cast<double>(v[i]) * r * static_cast<double>(wv[i]));
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] = static_cast<uint32_t>(f32_to_bf16(yf[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(yf[2 * i + 1])) << 16);
        if constexpr (QUANT)
          amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(o[i] << 16)), fabsf(__uint_as_float(o[i] & 0xFFFF0000u))));
      }
      xr[s] = make_uint4(o[0], o[1], o[2], o[3]);
      if (live) *reinterpret_cast<uint4*>(xnrow + 32 * s) = xr[s];
    }
    // one chunk at a time: interleaving chunks would hold their fp64
    // temporaries beside the row and spill it
    __builtin_amdgcn_sched_barrier(0);
  }
  } else {
    // no norm: the codes are those of x itself
#pragma unroll
    for (int s = 0; s < MAXS; ++s)
      if (s < nks) {
        float v[8];
        unpack(xr[s], v);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
      }
  }

  if constexpr (QUANT) {
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    if (g == 0) red_am[q][row] = amax;
    __syncthreads();
    const float am = fmaxf(fmaxf(red_am[0][row], red_am[1][row]), fmaxf(red_am[2][row], red_am[3][row]));
    const float sc = am > 0.f ? am / 448.0f : 1.0f;
    if (live && q == 0 && g == 0) a.sx[t] = sc;
    uint8_t* qrow = a.xq + static_cast<int64_t>(t) * d + kq;
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      if (s < nks) {
        float y[8];
        unpack(xr[s], y);
        if (live)
          *reinterpret_cast<uint2*>(qrow + 32 * s) =
              make_uint2(e4m3x4(y[0] / sc, y[1] / sc, y[2] / sc, y[3] / sc),
                         e4m3x4(y[4] / sc, y[5] / sc, y[6] / sc, y[7] / sc));
      }
    }
  }

  // router: this wave's K quarter against each 16-expert fragment in turn.
  // The weight fragments (in order nf-major: f = nf * nks + s) stream through
  // the wave's LDS ring: loads complete in order, so once only kRing - 1 are
  // outstanding fragment f has landed; its slot is refilled with fragment
  // f + kRing as soon as it is in registers.  Two accumulators over
  // alternate K steps keep the MFMA chain short.
  const int e16 = a.e16;
  const int qu = __builtin_amdgcn_readfirstlane(q);   // the wave index, as the scalar it is
  // fragment (nf, s) of this wave: K step q nks + s, experts 16 nf..
  const uint8_t* wq = reinterpret_cast<const uint8_t*>(a.wr_pack) + static_cast<int64_t>(qu) * nks * e16 * 1024;
  const int64_t sstep = static_cast<int64_t>(e16) * 1024;
  const uint32_t ring_w = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring)) + qu * (kRing * 1024);
  const uint32_t voff = static_cast<uint32_t>(lane) * 16;
  // the next fragment to fetch, as (pnf, ps), advanced one step per fetch
  // (past the last fragment the last one is fetched again, unused)
  int pnf = 0, ps = 0;
  auto fetch = [&](uint32_t slot) {
    const bool past = pnf >= e16;
    nr_dma16(wq + (past ? (nks - 1) * sstep + (e16 - 1) * 1024 : ps * sstep + pnf * 1024), voff, slot);
    if (++ps == nks) {
      ps = 0;
      ++pnf;
    }
  };
  nr_wait_vmcnt<0>();   // the row stores have drained: vmcnt now counts the ring alone
#pragma unroll
  for (int f = 0; f < kRing; ++f) fetch(ring_w + f * 1024);
  f32x4 acc[NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    acc[nf] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (nf < e16) {
      f32x4 acc1 = acc[nf];
#pragma unroll
      for (int s = 0; s < MAXS; ++s) {
        if (s < nks) {
          const int f = nf * nks + s;
          const uint32_t slot = ring_w + static_cast<uint32_t>(f & (kRing - 1)) * 1024;
          nr_wait_vmcnt<kRing - 1>();
          __builtin_amdgcn_sched_barrier(0);
          const bf16x8 bf = *(const lds_bf16x8_t*)(uintptr_t)(slot + voff);
          __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the fragment is in registers
          __builtin_amdgcn_sched_barrier(0);
          fetch(slot);   // fragment f + kRing
          const bf16x8 af = __builtin_bit_cast(bf16x8, xr[s]);
          if (s & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc1, 0, 0, 0);
          else acc[nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[nf], 0, 0, 0);
        }
      }
      acc[nf] = acc[nf] + acc1;
    }
  }
  nr_wait_vmcnt<0>();
  __syncthreads();   // every wave is done with its ring: it now holds the partial logits
  // partial sums (lane l holds rows 4 (l / 16) + i of column l % 16), then
  // the four K quarters added in order
  typedef float PartRow[kNRRows][NF * 16];
  PartRow* part = reinterpret_cast<PartRow*>(ring);
#pragma unroll
  for (int nf = 0; nf < NF; ++nf)
    if (nf < e16)
#pragma unroll
      for (int i = 0; i < 4; ++i) part[q][4 * g + i][16 * nf + row] = acc[nf][i];
  __syncthreads();
  const int E = a.E;
  for (int i = tid; i < kNRRows * E; i += 256) {
    const int rr = i / E, e = i - rr * E;
    if (t0 + rr < T)
      a.logits[static_cast<int64_t>(t0 + rr) * E + e] = ((part[0][rr][e] + part[1][rr][e]) + part[2][rr][e]) + part[3][rr][e];
  }
}

template <int MAXS, int NF>
hipError_t launch_nr(const NormRouteArgs& a, hipStream_t s) {
  const unsigned nb = static_cast<unsigned>((a.T + kNRRows - 1) / kNRRows);
  if (!a.w) hipLaunchKernelGGL((norm_route_kernel<false, true, MAXS, NF>), dim3(nb), dim3(256), 0, s, a);
  else if (a.xq) hipLaunchKernelGGL((norm_route_kernel<true, true, MAXS, NF>), dim3(nb), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((norm_route_kernel<true, false, MAXS, NF>), dim3(nb), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int MAXS>
hipError_t launch_nr_e(const NormRouteArgs& a, hipStream_t s) {
  if (a.e16 <= 1) return launch_nr<MAXS, 1>(a, s);
  if (a.e16 <= 2) return launch_nr<MAXS, 2>(a, s);
  if (a.e16 <= 4) return launch_nr<MAXS, 4>(a, s);
  return launch_nr<MAXS, 8>(a, s);
}

}  // namespace

bool norm_route_supported(int x_dtype, int d, int E) {
  return x_dtype == DT_BF16 && d > 0 && d % 128 == 0 && d <= 128 * 40 && E >= 1 && E <= 128;
}

size_t norm_route_pack_bytes(int d, int E) {
  return static_cast<size_t>(d / 32) * ((E + 15) / 16) * 64 * 16;
}

hipError_t launch_norm_route(const void* x, const void* w, int T, int d, int E, float eps, const void* wr,
                             void* wr_pack, void* xn, uint8_t* xq, float* sx, float* logits, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int e16 = (E + 15) / 16;
  hipLaunchKernelGGL(wr_pack_kernel, dim3(d / 32, e16), dim3(64), 0, s, static_cast<const uint16_t*>(wr), d, E, e16,
                     static_cast<uint4*>(wr_pack));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  NormRouteArgs a{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), T, d, E, e16, eps,
                  static_cast<const uint4*>(wr_pack), static_cast<uint16_t*>(xn), xq, sx, logits};
  if (!w && (!xq || !sx)) return hipErrorInvalidValue;   // no norm: the x quantisation with the router
  const int nks = d / 128;
  if (nks <= 8) return launch_nr_e<8>(a, s);
  if (nks <= 16) return launch_nr_e<16>(a, s);
  return launch_nr_e<40>(a, s);
}

}  // namespace moe
