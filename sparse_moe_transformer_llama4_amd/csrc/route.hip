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
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------- e4m3

// ---------------------------------------------------------------- router

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short r_s16x4;
typedef __attribute__((address_space(3))) r_s16x4 r_lds_s16x4;

// Partial logits of 64 tokens x all experts over one K slice of d.
// Workgroup = 4 waves x 16 tokens; grid = (token blocks, K slices).  The
// router weight rows of each 64-deep K chunk are staged in LDS as they sit in
// memory ([K][E], expert-contiguous, rows padded by 32 bytes); bf16 operands
// are read back with the LDS transpose read (one expert column's 4 K values
// per lane), fp32 ones with plain 4-byte reads (one K value per lane).
// Tokens come straight from global memory into the MFMA registers.
template <int DT>
__global__ __launch_bounds__(256) void router_partial_kernel(RouterArgs a, int kslice, float* part) {
  using Elem = typename std::conditional<DT == DT_BF16, uint16_t, float>::type;
  constexpr int ES = sizeof(Elem);
  constexpr int KC = DT == DT_BF16 ? 64 : 32;          // K rows per staged chunk
  constexpr int KSTEP = DT == DT_BF16 ? 32 : 4;        // K per MFMA
  __shared__ __attribute__((aligned(16))) uint8_t wt[KC * (256 * 4 + 32)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = a.E, d = a.d, T = a.T;
  const int Ep = (E + 15) & ~15;
  const int nf = Ep >> 4;
  const int pitch = Ep * ES + 32;                       // bytes per staged row
  const int t0 = blockIdx.x * kRouteTokens + wave * 16;
  const int trow = min(t0 + (lane & 15), T - 1);
  const int ks0 = blockIdx.y * kslice;
  const int ks1 = min(d, ks0 + kslice);
  const Elem* xrow = reinterpret_cast<const Elem*>(a.x) + static_cast<int64_t>(trow) * d;
  const Elem* wr = reinterpret_cast<const Elem*>(a.wr);

  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int chunk_elems = KC * E;                       // contiguous in [d][E]
  const bool vec_ok = (E * ES) % 16 == 0;
  for (int k0 = ks0; k0 < ks1; k0 += KC) {
    __syncthreads();
    const Elem* src = wr + static_cast<int64_t>(k0) * E;
    if (vec_ok) {
      const int rowv = E * ES / 16;                     // 16-byte pieces per row
      for (int i = tid; i < KC * rowv; i += 256) {
        const int r = i / rowv, c = i - r * rowv;
        *reinterpret_cast<i32x4*>(&wt[r * pitch + c * 16]) =
            *reinterpret_cast<const i32x4*>(reinterpret_cast<const uint8_t*>(src) + (static_cast<int64_t>(r) * E * ES + c * 16));
      }
    } else {
      for (int i = tid; i < chunk_elems; i += 256) {
        const int r = i / E, c = i - r * E;
        *reinterpret_cast<Elem*>(&wt[r * pitch + c * ES]) = src[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KC; ks += KSTEP) {
      if constexpr (DT == DT_BF16) {
        const int kk = ks + (lane >> 4) * 8;
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(xrow + k0 + kk);
        const int s = lane & 15;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j < nf) {
            const uint8_t* p0 = &wt[(kk + (s >> 2)) * pitch + (j * 16 + 4 * (s & 3)) * 2];
            const r_s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((r_lds_s16x4*)(p0));
            const r_s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((r_lds_s16x4*)(p0 + 4 * pitch));
            typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
            const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, v), acc[j], 0, 0, 0);
          }
        }
      } else {
        const int kk = ks + (lane >> 4);
        const float av = xrow[k0 + kk];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j < nf) {
            const float bv = *reinterpret_cast<const float*>(&wt[kk * pitch + (j * 16 + (lane & 15)) * 4]);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[j], 0, 0, 0);
          }
        }
      }
    }
  }
  // partial logits: lane holds rows 4*(lane/16)+q of column j*16 + lane%16
  float* out = part + static_cast<int64_t>(blockIdx.y) * T * E;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < nf) {
      const int e = j * 16 + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + 4 * (lane >> 4) + q;
        if (e < E && t < T) out[static_cast<int64_t>(t) * E + e] = acc[j][q];
      }
    }
  }
}

// The k largest logits of a token, best first; among equal logits the lower
// expert index ranks first (experts arrive in ascending order: a new logit
// must exceed a kept one to pass it, a displaced one moves down one rank).
// k = 1 is the argmax with ties to the lowest index.
struct TopK {
  float v[kMaxTopK];
  int i[kMaxTopK];
};
__device__ __forceinline__ void topk_init(TopK& b) {
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    b.v[j] = -INFINITY;
    b.i[j] = 0x7fffffff;
  }
}
__device__ __forceinline__ void topk_push(TopK& b, float x, int e, int k) {
  float cv = x;
  int ci = e;
  bool moving = false;   // cv is a displaced entry (ranked ahead of the rest)
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    if (j < k && (moving || cv > b.v[j])) {
      const float tv = b.v[j];
      const int ti = b.i[j];
      b.v[j] = cv;
      b.i[j] = ci;
      cv = tv;
      ci = ti;
      moving = true;
    }
  }
}

// Sum of the K-slice partials in slice order (deterministic), bias, top-k
// (lowest index among equal logits), sigmoid gate of each pick, and the
// per-workgroup histogram of picks (64 tokens per workgroup, the blocking
// the permutation uses).  Token t's j-th pick is slot t * k + j.
// The workgroup's 64 x E logits are first staged in LDS by coalesced loads,
// several in flight per thread (one thread walking its token's row with
// dependent global loads took ~60 us per workgroup at E = 128).  Wave q then
// ranks quarter q of every token's experts, and wave 0 pushes the other
// quarters' rankings, best first and in quarter order, into its own: every
// entry of a later quarter has a higher index than those of the earlier
// ones, so among equal logits the lower index stays ahead, and the result is
// the ranking of the whole row.
constexpr int kFinishPitch = 257;   // floats per staged row: the 64 lanes of a wave read distinct banks
__global__ __launch_bounds__(256) void router_finish_kernel(RouterArgs a, int nsplit, const float* part) {
  __shared__ float lg[kRouteTokens * kFinishPitch];
  __shared__ float qv[3][kRouteTokens][kMaxTopK];
  __shared__ int qi[3][kRouteTokens][kMaxTopK];
  __shared__ int hist[256];
  const int tid = threadIdx.x;
  const int E = a.E, T = a.T, k = a.k;
  const int t0 = blockIdx.x * kRouteTokens;
  const int nt = min(kRouteTokens, T - t0);
  const int n = nt * E;   // this block's logits: part[s][t0 * E + i], i < n
  hist[tid] = 0;
  for (int i0 = tid; i0 < n; i0 += 4 * 256) {
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nsplit; ++s) {
      const float* ps = part + (static_cast<int64_t>(s) * T + t0) * E;
      float x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = i0 + 256 * u < n ? ps[i0 + 256 * u] : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] += x[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + 256 * u;
      if (i < n) {
        const int r = i / E, e = i - r * E;
        float y = v[u];
        if (a.bias) y += a.bias[e];
        lg[r * kFinishPitch + e] = y;
      }
    }
  }
  __syncthreads();
  const int q = tid >> 6, r = tid & 63;
  const int seg = (E + 3) >> 2;
  const int e0 = min(E, q * seg), e1 = min(E, e0 + seg);
  TopK b;
  topk_init(b);
  if (r < nt)
    for (int e = e0; e < e1; ++e) topk_push(b, lg[r * kFinishPitch + e], e, k);
  if (q > 0) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      qv[q - 1][r][j] = b.v[j];
      qi[q - 1][r][j] = b.i[j];
    }
  }
  __syncthreads();
  if (q == 0 && r < nt) {
    for (int qq = 0; qq < 3; ++qq)
      for (int j = 0; j < k; ++j) topk_push(b, qv[qq][r][j], qi[qq][r][j], k);
    const int t = t0 + r;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k) break;
      const int bi = min(b.i[j], E - 1);   // only reachable with non-finite logits (outside the contract)
      a.idx[static_cast<int64_t>(t) * k + j] = bi;
      a.gate[static_cast<int64_t>(t) * k + j] = 1.0f / (1.0f + expf(-b.v[j]));
      atomicAdd(&hist[bi], 1);
    }
  }
  __syncthreads();
  if (tid < E) a.hist[static_cast<int64_t>(blockIdx.x) * E + tid] = hist[tid];
}

// Per-token e4m3 quantisation of x (bf16): s = fp32(max|x_t|) / 448 (1 for
// a zero row), code = e4m3(x / s).  One wave per token row, the row held in
// registers between the max and the quantisation when d <= 64 * 8 * NC
// (NC > 0), else read twice (NC = 0).  With
// zero_a / zero_b non-null it also clears the row's entries of the two max
// |h| arrays the gate/up epilogues accumulate into: zero_a[t] and
// zero_b[t * kb + j], j < kb.
template <int NC>
__global__ __launch_bounds__(256) void quant_x_kernel(const uint16_t* x, int T, int d, uint8_t* xq, float* sx,
                                                      uint32_t* zero_a, uint32_t* zero_b, int kb) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (zero_a && lane == 0) zero_a[t] = 0u;
  if (zero_b && lane < kb) zero_b[static_cast<int64_t>(t) * kb + lane] = 0u;
  const uint16_t* row = x + static_cast<int64_t>(t) * d;
  uint8_t* qrow = xq + static_cast<int64_t>(t) * d;
  if constexpr (NC == 0) {
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
    for (int k = lane * 8; k < d; k += 64 * 8) {
      const uint4 v = *reinterpret_cast<const uint4*>(row + k);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      float q[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q[2 * i] = __uint_as_float(w[i] << 16) / s;
        q[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u) / s;
      }
      *reinterpret_cast<uint2*>(qrow + k) = make_uint2(e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7]));
    }
    return;
  }
  constexpr int NR = NC > 0 ? NC : 1;
  uint4 v[NR];
#pragma unroll
  for (int c = 0; c < NR; ++c) {
    const int k = (lane + 64 * c) * 8;
    v[c] = k < d ? *reinterpret_cast<const uint4*>(row + k) : make_uint4(0u, 0u, 0u, 0u);
  }
  float amax = 0.f;
#pragma unroll
  for (int c = 0; c < NR; ++c) {
    const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
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
#pragma unroll
  for (int c = 0; c < NR; ++c) {
    const int k = (lane + 64 * c) * 8;
    if (k >= d) continue;
    const uint32_t w[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
    float q[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = __uint_as_float(w[i] << 16) / s;
      q[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u) / s;
    }
    *reinterpret_cast<uint2*>(qrow + k) = make_uint2(e4m3x4(q[0], q[1], q[2], q[3]), e4m3x4(q[4], q[5], q[6], q[7]));
  }
}

// RMSNorm of the block's input rows, the normalisation that precedes the
// feed-forward block (llm-architectures-explained "Llama 4 Maverick", table
// "Every architecture field": RMSNorm, placed before the MLP; KerasFormers
// "Llama 4", Llama4Model arguments: norm_eps = 1e-5):
//   xn[t, j] = x[t, j] * r_t * w[j],  r_t = 1 / sqrt(mean_j x[t, j]^2 + eps),
// rounded once (RNE) to x's dtype; the block then reads xn in place of x.
// The rounded rows are those of the exact value (to ties closer than ~1e-15
// relative), so the router's argmax and the e4m3 codes downstream are
// decided on the same rows as an exact computation would give:
//   - the sum of squares and r_t are fp64 (squares of bf16 / fp32 values
//     are exact in fp64);
//   - bf16 rows: y = (x * fp32(r_t)) * w in fp32 is within 2 fp32 ulps of
//     the exact value, which settles the bf16 rounding unless y's low 16
//     bits lie within 4 of the halfway pattern 0x8000; those elements (about
//     1 in 8000) are recomputed in fp64 and rounded to odd in fp32 before
//     the bf16 rounding (no double-rounding error);
//   - fp32 rows: fp64 throughout, one rounding to fp32.
// With QUANT (bf16 rows feeding e4m3 weights) the same pass also writes xn's
// per-token e4m3 codes and scales (s = fp32 max|xn_t| / 448, code =
// e4m3(xn / s) with an IEEE fp32 division), so the normalised rows are not
// read back for the quantisation.  One wave per row.

template <int XDT, bool QUANT, int NCH>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* x, const void* w, int T, int d, float eps,
                                                      void* xn, uint8_t* xq, float* sx) {
  static_assert(XDT == DT_BF16 || !QUANT, "e4m3 codes come from bf16 rows");
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  constexpr int V = XDT == DT_BF16 ? 8 : 4;   // elements per 16-byte chunk
  constexpr int ES = XDT == DT_BF16 ? 2 : 4;  // bytes per element
  // NCH chunks per lane are held in registers (the launcher picks the
  // smallest instance that holds the row, 16 at most: fewer registers, more
  // rows in flight): a row of up to 64 * V * NCH elements is loaded once,
  // all its loads in flight together.  Longer rows are walked in groups of
  // NCH chunks per lane: the sum of squares reads them once, the output
  // pass again (from L2); with QUANT the output pass of a long row also
  // recomputes its values after the max pass.
  const int step = 64 * V;
  const int nch = (d + step - 1) / step;
  const bool resident = nch <= NCH;
  const uint8_t* xrow = static_cast<const uint8_t*>(x) + static_cast<int64_t>(t) * d * ES;
  const uint8_t* wrow = static_cast<const uint8_t*>(w);
  // the gain, the same for every row: staged in LDS once per workgroup for
  // a resident row (chunk c of lane l at c * 64 + l), so the registers hold
  // x alone and more rows are in flight
  __shared__ uint4 wl[NCH * 64];
  if (resident)
    for (int i = threadIdx.x; i < nch * 64; i += 256)
      if (i * V < d) wl[i] = *reinterpret_cast<const uint4*>(wrow + static_cast<int64_t>(i) * V * ES);
  __syncthreads();
  if (t >= T) return;
  uint4 xr[NCH];
  auto valid = [&](int g0, int c) { return g0 + c < nch && (g0 + c) * step + lane * V < d; };
  auto load_group = [&](int g0) {
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (valid(g0, c)) xr[c] = *reinterpret_cast<const uint4*>(xrow + static_cast<int64_t>((g0 + c) * step + lane * V) * ES);
  };
  auto wchunk = [&](int g0, int c) -> uint4 {
    if (resident) return wl[c * 64 + lane];
    return *reinterpret_cast<const uint4*>(wrow + static_cast<int64_t>((g0 + c) * step + lane * V) * ES);
  };
  auto unpack = [](const uint4& q, float (&v)[V]) {
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
    if constexpr (XDT == DT_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(u[i] << 16);
        v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(u[i]);
    }
  };

  // pass 1: sum of squares (fp64; four independent partial sums per lane
  // keep the dependent FMA chains short)
  double ssp[4] = {0.0, 0.0, 0.0, 0.0};
  for (int g0 = 0; g0 < nch; g0 += NCH) {
    load_group(g0);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      if (valid(g0, c)) {
        float v[V];
        unpack(xr[c], v);
#pragma unroll
        for (int i = 0; i < V; ++i)
          ssp[i & 3] = fma(static_cast<double>(v[i]), static_cast<double>(v[i]), ssp[i & 3]);
      }
  }
  double ss = (ssp[0] + ssp[1]) + (ssp[2] + ssp[3]);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m, 64);
  const double r = 1.0 / sqrt(ss / static_cast<double>(d) + static_cast<double>(eps));
  const float r32 = static_cast<float>(r);

  // the normalised values of chunk c, as stored (rounded once to the row dtype)
  auto normed = [&](int g0, int c, float (&y)[V]) {
    float v[V], wv[V];
    unpack(xr[c], v);
    unpack(wchunk(g0, c), wv);
    if constexpr (XDT == DT_BF16) {
      float yf[V];
      bool near = false;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        yf[i] = (v[i] * r32) * wv[i];
        near |= ((__float_as_uint(yf[i]) & 0xFFFFu) - 0x7FFCu) <= 8u;
      }
      if (near) {   // some value within 4 of the bf16 halfway pattern: decide those in fp64
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (((__float_as_uint(yf[i]) & 0xFFFFu) - 0x7FFCu) <= 8u)
            yf[i] = f64_to_f32_odd(static_cast<double>(v[i]) * r * static_cast<double>(wv[i]));
      }
#pragma unroll
      for (int i = 0; i < V; ++i) y[i] = __uint_as_float(static_cast<uint32_t>(f32_to_bf16(yf[i])) << 16);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i)
        y[i] = static_cast<float>(static_cast<double>(v[i]) * r * static_cast<double>(wv[i]));
    }
  };
  auto pack_bf16 = [](const float (&y)[V]) -> uint4 {
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (__float_as_uint(y[2 * i]) >> 16) | (__float_as_uint(y[2 * i + 1]) & 0xFFFF0000u);
    return make_uint4(o[0], o[1], o[2], o[3]);
  };
  auto out_index = [&](int g0, int c) { return static_cast<int64_t>(t) * d + (g0 + c) * step + lane * V; };

  if constexpr (!QUANT) {
    // pass 2: the normalised rows
    for (int g0 = 0; g0 < nch; g0 += NCH) {
      if (!resident) load_group(g0);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (!valid(g0, c)) continue;
        float y[V];
        normed(g0, c, y);
        if constexpr (XDT == DT_BF16)
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(xn) + out_index(g0, c)) = pack_bf16(y);
        else
          *reinterpret_cast<float4*>(static_cast<float*>(xn) + out_index(g0, c)) = make_float4(y[0], y[1], y[2], y[3]);
      }
    }
  } else {
    // pass 2: the normalised rows and their largest magnitude; a resident
    // row keeps its bf16 values in place of x for the codes
    float amax = 0.f;
    for (int g0 = 0; g0 < nch; g0 += NCH) {
      if (!resident) load_group(g0);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (!valid(g0, c)) continue;
        float y[V];
        normed(g0, c, y);
#pragma unroll
        for (int i = 0; i < V; ++i) amax = fmaxf(amax, fabsf(y[i]));
        const uint4 yb = pack_bf16(y);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(xn) + out_index(g0, c)) = yb;
        if (resident) xr[c] = yb;
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    if (lane == 0) sx[t] = s;
    // pass 3: e4m3 codes of the normalised rows
    for (int g0 = 0; g0 < nch; g0 += NCH) {
      if (!resident) load_group(g0);
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        if (!valid(g0, c)) continue;
        float y[V];
        if (resident) unpack(xr[c], y);
        else normed(g0, c, y);
#pragma unroll
        for (int i = 0; i < V; ++i) y[i] = y[i] / s;
        *reinterpret_cast<uint2*>(xq + out_index(g0, c)) =
            make_uint2(e4m3x4(y[0], y[1], y[2], y[3]), e4m3x4(y[4], y[5], y[6], y[7]));
      }
    }
  }
}

// Per-row e4m3 quantisation of h with the row max the gate/up epilogues
// gathered from its fp32 values: s = max|h| / 448 (1 for a zero row), code =
// e4m3(h / s).  h arrives in 24 bits (each fp32 pattern rounded at bit 8:
// bits 31..16 in `h`, bits 15..8 in `h_lo`), a relative change of at most
// 2^-16, below the fp8 MFMA's own accumulation error.
__global__ __launch_bounds__(256) void quant_h_kernel(const uint16_t* h, const uint8_t* h_lo, const uint32_t* amax,
                                                      int rows, int n, uint8_t* hq, float* sh) {
  const int r = blockIdx.x;
  if (r >= rows) return;
  const float am = __uint_as_float(amax[r]);
  const float s = am > 0.f ? am / 448.0f : 1.0f;
  if (blockIdx.y == 0 && threadIdx.x == 0) sh[r] = s;
  const int k = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (k >= n) return;
  const int64_t o = static_cast<int64_t>(r) * n + k;
  const uint4 v = *reinterpret_cast<const uint4*>(h + o);
  const uint2 b = *reinterpret_cast<const uint2*>(h_lo + o);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  const uint32_t lb[2] = {b.x, b.y};
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t hi = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    const uint32_t lo = (lb[i >> 2] >> (8 * (i & 3))) & 0xFFu;
    y[i] = __uint_as_float((hi << 16) | (lo << 8)) / s;
  }
  *reinterpret_cast<uint2*>(hq + o) = make_uint2(e4m3x4(y[0], y[1], y[2], y[3]), e4m3x4(y[4], y[5], y[6], y[7]));
}

__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// ---------------------------------------------------------------- scan

// Exclusive scans over a 256-thread workgroup of NV values per thread at
// once (wave shuffles, one barrier): v[i] -> exclusive prefix, tot[i] -> total.
template <int NV>
__device__ void block_exclusive_scan(int (&v)[NV], int (&tot)[NV], int* sm /* [NV][4] */) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) x[i] = v[i];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int n = __shfl_up(x[i], o, 64);
      if (lane >= o) x[i] += n;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < NV; ++i) sm[i * 4 + w] = x[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    int off = 0, t = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sj = sm[i * 4 + j];
      off += j < w ? sj : 0;
      t += sj;
    }
    tot[i] = t;
    v[i] = x[i] - v[i] + off;
  }
}

// Writes counts, offsets[E + 1] and the tile tables (see table_all /
// table_main / table_tail) from per-expert counts held one per thread
// (thread e < E); group E of the all / main tables is the shared expert
// (T rows) and entry E + 1 the total.
__device__ void offsets_and_tiles(int cnt, int E, int T, int32_t* counts, int32_t* offsets, int32_t* tiles,
                                  int* sm) {
  const int e = threadIdx.x;
  int v[1 + kNumTables], tot[1 + kNumTables];
  v[0] = cnt;
#pragma unroll
  for (int i = 0; i < kNumBM; ++i) {
    const int bm = bm_of(i);
    const int r = cnt % bm;
    const bool tail = r > 0 && r <= kTailRows;
    v[1 + i] = (cnt + bm - 1) / bm;
    v[1 + kNumBM + i] = tail ? cnt / bm : (cnt + bm - 1) / bm;
    v[1 + 2 * kNumBM + i] = tail ? 1 : 0;
    v[1 + 3 * kNumBM + i] = class_tiles(cnt, bm);
  }
  block_exclusive_scan<1 + kNumTables>(v, tot, sm);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = v[0];
#pragma unroll
    for (int i = 0; i < kNumTables; ++i) tiles[i * (E + 2) + e] = v[1 + i];
  }
  if (e == 0) {
    offsets[E] = tot[0];
#pragma unroll
    for (int i = 0; i < kNumTables; ++i) {
      const int shared = i >= 2 * kNumBM ? 0 : (T + bm_of(i % kNumBM) - 1) / bm_of(i % kNumBM);   // tail, class: none
      tiles[i * (E + 2) + E] = tot[1 + i];   // the shared group follows the routed ones
      tiles[i * (E + 2) + E + 1] = tot[1 + i] + shared;
    }
  }
}

// One workgroup: column scan of the per-workgroup histograms.
//   hist[b][e] <- sum_{b' < b} hist[b'][e]   (rank base of block b inside group e;
//                                          the permutation adds offsets[e])
//   counts[e], offsets[e], and the tile tables tiles[i][g] = sum_{g' < g}
//   ceil(n_g' / BM_i) for g = 0..E+1 (group E = the shared expert, n_E = T).
// Each thread owns one expert's column and walks it in chunks whose loads
// are all issued before the chunk's stores (a load after a store to the same
// array would wait a full round trip).
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a) {
  __shared__ int sm[(1 + kNumTables) * 4];
  const int e = threadIdx.x;
  const int E = a.E;
  int running = 0;
  if (e < E) {
    constexpr int CH = 32;
    for (int b0 = 0; b0 < a.nblocks; b0 += CH) {
      int c[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u)
        c[u] = b0 + u < a.nblocks ? a.hist[static_cast<int64_t>(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        if (b0 + u < a.nblocks) {
          a.hist[static_cast<int64_t>(b0 + u) * E + e] = running;
          running += c[u];
        }
      }
    }
  }
  offsets_and_tiles(e < E ? running : 0, E, a.T, a.counts, a.offsets, a.tiles, sm);
}

// Routing of at most 64 tokens in one workgroup: sum of the K-slice partial
// logits, bias, top-1 (lowest index), gate, counts, offsets, tile tables and
// the stable permutation, without a histogram pass.
__global__ __launch_bounds__(256) void route_small_kernel(RouterArgs a, int nsplit, const float* part,
                                                          int32_t* counts, int32_t* offsets, int32_t* tiles,
                                                          int32_t* perm) {
  __shared__ int cnt_s[256];
  __shared__ int ids[kRouteTokens * kMaxTopK];
  __shared__ int sm[(1 + kNumTables) * 4];
  __shared__ float lg[kRouteTokens * 256];
  const int tid = threadIdx.x, E = a.E, T = a.T, k = a.k;
  cnt_s[tid] = 0;
  // logits of every (token, expert) pair, the K-slice partials summed in
  // slice order; the loads of a pair are issued together (a dependent chain
  // of global loads per token took tens of microseconds)
  for (int i = tid; i < T * E; i += 256) {
    const int t = i / E, e = i - t * E;
    float v = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 16) {
      float pv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        pv[u] = s0 + u < nsplit ? part[(static_cast<int64_t>(s0 + u) * T + t) * E + e] : 0.f;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (s0 + u < nsplit) v += pv[u];
    }
    if (a.bias) v += a.bias[e];
    lg[i] = v;
  }
  __syncthreads();
  if (tid < T) {
    TopK b;
    topk_init(b);
    for (int e = 0; e < E; ++e) topk_push(b, lg[tid * E + e], e, k);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j >= k) break;
      const int bi = min(b.i[j], E - 1);   // only reachable with non-finite logits (outside the contract)
      a.idx[tid * k + j] = bi;
      a.gate[tid * k + j] = 1.0f / (1.0f + expf(-b.v[j]));
      ids[tid * k + j] = bi;
      atomicAdd(&cnt_s[bi], 1);
    }
  }
  __syncthreads();
  offsets_and_tiles(tid < E ? cnt_s[tid] : 0, E, T, counts, offsets, tiles, sm);
  __shared__ int off_s[256];
  __syncthreads();
  if (tid < E) off_s[tid] = offsets[tid];
  __syncthreads();
  // stable position of every slot (slots in ascending order within a group)
  for (int sl = tid; sl < T * k; sl += 256) {
    const int e = ids[sl];
    int rank = 0;
    for (int j = 0; j < sl; ++j) rank += ids[j] == e;
    perm[off_s[e] + rank] = sl;
  }
}

// Stable position of every slot: perm[offsets[e] + base[b][e] + rank] = slot,
// where rank counts earlier slots of the same workgroup (64 tokens, their
// k picks each) routed to the same expert.
__global__ __launch_bounds__(64) void perm_kernel(const int32_t* idx, const int32_t* base,
                                                  const int32_t* offsets, int T, int E, int k, int32_t* perm) {
  __shared__ int ids[kRouteTokens * kMaxTopK];
  const int t = blockIdx.x * kRouteTokens + threadIdx.x;
  for (int j = 0; j < k; ++j)
    ids[threadIdx.x * k + j] = t < T ? idx[static_cast<int64_t>(t) * k + j] : -1;
  __syncthreads();
  if (t >= T) return;
  for (int j = 0; j < k; ++j) {
    const int ls = threadIdx.x * k + j;
    const int e = ids[ls];
    int rank = 0;
    for (int l = 0; l < ls; ++l) rank += ids[l] == e;
    perm[offsets[e] + base[static_cast<int64_t>(blockIdx.x) * E + e] + rank] = t * k + j;
  }
}

#ifdef MOE_DEBUG
// Debug builds: the routing invariants the grouped GEMMs rely on, one thread
// per routed slot position i (plus the offsets and tile tables in block 0):
//   * idx[i] in [0, E);
//   * offsets[0] = 0, offsets[e + 1] - offsets[e] = counts[e] >= 0,
//     offsets[E] = S;
//   * perm[i] in [0, S), the slot of an expert-g pick for every position i of
//     group g, and slots increasing inside a group (the stable order; with the
//     two conditions before, perm is then a permutation of the S slots);
//   * every tile table starts at 0 and does not decrease.
// Positions are placed in groups by a search over offsets clamped to [0, E),
// so broken offsets cannot send a read out of bounds.
__global__ __launch_bounds__(256) void validate_routing_kernel(const int32_t* idx, const int32_t* counts,
                                                               const int32_t* offsets, const int32_t* perm,
                                                               const int32_t* tiles, int S, int E,
                                                               uint32_t* flags) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < S) {
    const int e = idx[i];
    MOE_DCHECK(flags, e >= 0 && e < E, kDbgIdx);
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (offsets[mid] <= i) lo = mid; else hi = mid - 1;
    }
    const int sl = perm[i];
    if (MOE_DCHECK(flags, sl >= 0 && sl < S, kDbgPerm)) {
      MOE_DCHECK(flags, idx[sl] == lo, kDbgPerm);
      if (i + 1 < S && i + 1 < offsets[lo + 1]) MOE_DCHECK(flags, perm[i + 1] > sl, kDbgPerm);
    }
  }
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < E; e += 256)
      MOE_DCHECK(flags, counts[e] >= 0 && offsets[e + 1] - offsets[e] == counts[e], kDbgOffsets);
    if (threadIdx.x == 0) MOE_DCHECK(flags, offsets[0] == 0 && offsets[E] == S, kDbgOffsets);
    for (int j = threadIdx.x; j < kNumTables * (E + 1); j += 256) {
      const int t = j / (E + 1), g = j - t * (E + 1);
      MOE_DCHECK(flags, tiles[t * (E + 2) + g + 1] >= tiles[t * (E + 2) + g], kDbgTiles);
    }
    for (int t = threadIdx.x; t < kNumTables; t += 256) MOE_DCHECK(flags, tiles[t * (E + 2)] == 0, kDbgTiles);
  }
}

// After the validation (same stream): with any flag set, every tile table
// becomes all zeros, so the grouped GEMMs find no tiles.
__global__ __launch_bounds__(256) void neutralize_tables_kernel(int32_t* tiles, int n, const uint32_t* flags) {
  if (*flags == 0u) return;
  for (int j = threadIdx.x; j < n; j += 256) tiles[j] = 0;
}

__global__ void debug_break_perm_kernel(int32_t* perm, int S) {
  if (threadIdx.x == 0 && S > 1) perm[0] = perm[S - 1];
}
#endif  // MOE_DEBUG

// ---------------------------------------------------------------- launchers

// (release builds: no-ops)
hipError_t launch_validate_routing(const int32_t* idx, const int32_t* counts, const int32_t* offsets,
                                   const int32_t* perm, int32_t* tiles, int S, int E, uint32_t* flags,
                                   hipStream_t s) {
#ifndef MOE_DEBUG
  return hipSuccess;
#else
  if (S <= 0 || E <= 0) return hipSuccess;
  hipLaunchKernelGGL(validate_routing_kernel, dim3((S + 255) / 256), dim3(256), 0, s, idx, counts, offsets, perm,
                     tiles, S, E, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(neutralize_tables_kernel, dim3(1), dim3(256), 0, s, tiles, kNumTables * (E + 2),
                     static_cast<const uint32_t*>(flags));
  return hipGetLastError();
#endif
}

hipError_t launch_debug_break_perm(int32_t* perm, int S, hipStream_t s) {
#ifndef MOE_DEBUG
  return hipSuccess;
#else
  hipLaunchKernelGGL(debug_break_perm_kernel, dim3(1), dim3(64), 0, s, perm, S);
  return hipGetLastError();
#endif
}

int router_splits(int T, int d, int x_dtype) {
  const int kc = x_dtype == DT_BF16 ? 64 : 32;
  const int nb = (T + kRouteTokens - 1) / kRouteTokens;
  int ns = 1;
  while (nb * ns < 256 && (d / kc) % (ns * 2) == 0 && d / (ns * 2) >= 2 * kc) ns *= 2;
  return ns;
}

static hipError_t launch_partials(const RouterArgs& a, int x_dtype, float* part, int ns, hipStream_t s) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  const int kslice = a.d / ns;
  if (x_dtype == DT_BF16)
    hipLaunchKernelGGL(router_partial_kernel<DT_BF16>, dim3(nb, ns), dim3(256), 0, s, a, kslice, part);
  else
    hipLaunchKernelGGL(router_partial_kernel<DT_F32>, dim3(nb, ns), dim3(256), 0, s, a, kslice, part);
  return hipGetLastError();
}

hipError_t launch_router_finish(const RouterArgs& a, int nsplit, const float* part, hipStream_t s) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  hipLaunchKernelGGL(router_finish_kernel, dim3(nb), dim3(256), 0, s, a, nsplit, part);
  return hipGetLastError();
}

hipError_t launch_router(const RouterArgs& a, int x_dtype, float* part, hipStream_t s) {
  const int nb = (a.T + kRouteTokens - 1) / kRouteTokens;
  const int ns = router_splits(a.T, a.d, x_dtype);
  hipError_t e = launch_partials(a, x_dtype, part, ns, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(router_finish_kernel, dim3(nb), dim3(256), 0, s, a, ns, part);
  return hipGetLastError();
}

hipError_t launch_route_small(const RouterArgs& a, int x_dtype, float* part, int32_t* counts, int32_t* offsets,
                              int32_t* tiles, int32_t* perm, hipStream_t s) {
  const int ns = router_splits(a.T, a.d, x_dtype);
  hipError_t e = launch_partials(a, x_dtype, part, ns, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(256), 0, s, a, ns, part, counts, offsets, tiles, perm);
  return hipGetLastError();
}

hipError_t launch_route_small_finish(const RouterArgs& a, const float* logits, int32_t* counts, int32_t* offsets,
                                     int32_t* tiles, int32_t* perm, hipStream_t s) {
  hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(256), 0, s, a, 1, logits, counts, offsets, tiles, perm);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_perm(const int32_t* idx, const int32_t* base, const int32_t* offsets, int T, int E, int k,
                       int32_t* perm, hipStream_t s) {
  if (k < 1 || k > kMaxTopK) return hipErrorInvalidValue;
  hipLaunchKernelGGL(perm_kernel, dim3((T + kRouteTokens - 1) / kRouteTokens), dim3(kRouteTokens), 0, s, idx, base,
                     offsets, T, E, k, perm);
  return hipGetLastError();
}

hipError_t launch_quant_x(const uint16_t* x, int T, int d, uint8_t* xq, float* sx, hipStream_t s, uint32_t* zero_a,
                          uint32_t* zero_b, int kb) {
  if (kb < 0 || kb > 64) return hipErrorInvalidValue;
  const dim3 g((T + 3) / 4);
  if (d <= 64 * 8 * 4)
    hipLaunchKernelGGL(quant_x_kernel<4>, g, dim3(256), 0, s, x, T, d, xq, sx, zero_a, zero_b, kb);
  else if (d <= 64 * 8 * 10)
    hipLaunchKernelGGL(quant_x_kernel<10>, g, dim3(256), 0, s, x, T, d, xq, sx, zero_a, zero_b, kb);
  else if (d <= 64 * 8 * 16)
    hipLaunchKernelGGL(quant_x_kernel<16>, g, dim3(256), 0, s, x, T, d, xq, sx, zero_a, zero_b, kb);
  else
    hipLaunchKernelGGL(quant_x_kernel<0>, g, dim3(256), 0, s, x, T, d, xq, sx, zero_a, zero_b, kb);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(int x_dtype, const void* x, const void* w, int T, int d, float eps, void* xn,
                          uint8_t* xq, float* sx, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (d % (x_dtype == DT_BF16 ? 8 : 4) != 0) return hipErrorInvalidValue;
  if (x_dtype != DT_BF16 && (x_dtype != DT_F32 || xq)) return hipErrorInvalidValue;
  const dim3 grid((T + 3) / 4);
  const int nch = (d + 64 * (x_dtype == DT_BF16 ? 8 : 4) - 1) / (64 * (x_dtype == DT_BF16 ? 8 : 4));
  auto go = [&](auto nch_c) {
    constexpr int N = decltype(nch_c)::value;
    if (x_dtype == DT_BF16 && xq)
      hipLaunchKernelGGL((rmsnorm_kernel<DT_BF16, true, N>), grid, dim3(256), 0, s, x, w, T, d, eps, xn, xq, sx);
    else if (x_dtype == DT_BF16)
      hipLaunchKernelGGL((rmsnorm_kernel<DT_BF16, false, N>), grid, dim3(256), 0, s, x, w, T, d, eps, xn, xq, sx);
    else
      hipLaunchKernelGGL((rmsnorm_kernel<DT_F32, false, N>), grid, dim3(256), 0, s, x, w, T, d, eps, xn, xq, sx);
  };
  if (nch <= 2) go(std::integral_constant<int, 2>{});
  else if (nch <= 4) go(std::integral_constant<int, 4>{});
  else if (nch <= 8) go(std::integral_constant<int, 8>{});
  else if (nch <= 10) go(std::integral_constant<int, 10>{});   // 5120-wide bf16 rows
  else go(std::integral_constant<int, 16>{});
  return hipGetLastError();
}

hipError_t launch_quant_h(const uint16_t* h, const uint8_t* h_lo, const uint32_t* amax, int rows, int n,
                          uint8_t* hq, float* sh, hipStream_t s) {
  hipLaunchKernelGGL(quant_h_kernel, dim3(rows, (n + 2047) / 2048), dim3(256), 0, s, h, h_lo, amax, rows, n,
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
