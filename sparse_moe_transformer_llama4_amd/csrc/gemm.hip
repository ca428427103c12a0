// Grouped GEMMs of the Llama 4 MoE block on gfx950 MFMA.
//
// Experts are gated MLPs: h = SiLU(u Wg) * (u Wu), y = h Wd, with a shared
// expert of the same form added to the routed one (llm-architectures-
// explained "Llama 4 Maverick", table "Every architecture field";
// superteams.ai "Llama 4", routing sketch: shared_expert(x) + routed output).
// The routed expert's input is the token scaled by the sigmoid gate
// (KerasFormers "Llama 4", "What is unusual about the block"); because the
// first layer is linear the gate is applied to the fp32 accumulator rows.
//
// One kernel template serves three launches:
//   MODE_GATEUP       groups 0..E-1: rows of x gathered through perm
//                     (expert-contiguous order), group E: the shared expert
//                     on all T rows.  A tile pairs BN/2 gate columns with
//                     the matching BN/2 up columns so the epilogue can form
//                     SiLU(g*acc_gate) * (g*acc_up) in registers.
//   MODE_DOWN_SHARED  y_s = h_s Ws_d in fp32.
//   MODE_DOWN_ROUTED  out[perm[r]] = h_r[r] W_d[e] + y_s[perm[r]]: every
//                     output row has exactly one writer (top-1), no atomics.
//
// Tiles: BM x BN per workgroup of 4 waves (WM x WN), K staged 128 bytes at
// a time through double-buffered LDS.  A rows are K-contiguous in memory;
// weights are [K][N] (N-contiguous), so the weight tile is transposed while
// it is written to LDS, and every lane then reads its K-contiguous MFMA
// operand with one LDS access.  Groups and M tiles come from a device-side
// tile table (prefix of ceil(rows / BM) per group), so the grid never
// depends on host-visible counts; surplus workgroups exit.
#include "common.h"
#include "launch.h"

namespace moe {

template <int DT> struct Elem;
template <> struct Elem<DT_BF16> {
  static constexpr int kSize = 2;
  static constexpr int kStep = 32;   // K per MFMA (v_mfma_f32_16x16x32_bf16)
  static constexpr int kLaneK = 8;   // K elements per lane per MFMA
};
template <> struct Elem<DT_F32> {
  static constexpr int kSize = 4;
  static constexpr int kStep = 4;    // v_mfma_f32_16x16x4_f32
  static constexpr int kLaneK = 1;
};
template <> struct Elem<DT_E4M3> {
  static constexpr int kSize = 1;
  static constexpr int kStep = 128;  // v_mfma_scale_f32_16x16x128_f8f6f4 (unit scales)
  static constexpr int kLaneK = 32;
};

constexpr int kKBytes = 128;            // K bytes per stage
constexpr int kPitch = kKBytes + 16;    // LDS row pitch in bytes

template <int DT>
__device__ __forceinline__ f32x4 mfma_step(const uint8_t* ap, const uint8_t* bp, f32x4 acc) {
  if constexpr (DT == DT_BF16) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(ap);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(bp);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  } else if constexpr (DT == DT_F32) {
    const float a = *reinterpret_cast<const float*>(ap);
    const float b = *reinterpret_cast<const float*>(bp);
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
  } else {
    const i32x8 a = *reinterpret_cast<const i32x8*>(ap);
    const i32x8 b = *reinterpret_cast<const i32x8*>(bp);
    // format 0 = fp8 e4m3 for both operands; E8M0 scale 127 = 1.0
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
  }
}

template <int DT, int MODE, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs p) {
  using EL = Elem<DT>;
  constexpr int ES = EL::kSize;
  constexpr int BK = kKBytes / ES;          // K elements per stage
  constexpr int VEC = 16 / ES;              // elements per 16-byte global load
  constexpr int FM = BM / WM / 16;          // 16-row fragments per wave
  constexpr int FN = BN / WN / 16;          // 16-col fragments per wave
  constexpr int A_CHUNKS = BM * kKBytes / 16 / 256;
  constexpr int B_CHUNKS = BN * kKBytes / 16 / 256;
  constexpr int B_ROW_CHUNKS = BN * ES / 16;  // 16-byte chunks per K row of the tile
  constexpr bool GATEUP = MODE == MODE_GATEUP;
  constexpr int BNH = GATEUP ? BN / 2 : BN;   // output columns per tile
  static_assert(WM * WN == 4, "4 waves");
  static_assert(!GATEUP || FN % 2 == 0, "gate/up fragment pairs");
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small");

  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * kPitch];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * kPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int E = p.E, T = p.T, K = p.K;

  // ---- tile lookup
  int g, m0, rows;
  if constexpr (MODE == MODE_DOWN_SHARED) {
    g = 0;
    m0 = blockIdx.x * BM;
    rows = T;
    if (m0 >= T) return;
  } else {
    const int mt = blockIdx.x + p.tiles[p.group_lo];
    if (mt >= p.tiles[p.group_hi]) return;
    int lo = p.group_lo, hi = p.group_hi - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.tiles[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    g = lo;
    m0 = (mt - p.tiles[g]) * BM;
    rows = (g == E) ? T : p.offsets[g + 1] - p.offsets[g];
  }
  const bool shared = (MODE == MODE_DOWN_SHARED) || (GATEUP && g == E);
  const int NH = (GATEUP && shared) ? p.N_shared : p.N;   // output width of this group
  const int n0 = blockIdx.y * BNH;
  if (n0 >= NH) return;
  if (!shared && !MOE_DCHECK_TILE(p, g, m0, rows)) return;   // debug builds: the tile is in its group
  const int row_base = shared ? 0 : p.offsets[g];          // first row of the group (permuted order)
  const int ldb = GATEUP ? 2 * NH : NH;                     // weight row length (elements)

  // ---- per-thread global source pointers
  const uint8_t* a_src[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int c = tid + i * 256;
    const int r = min(m0 + (c >> 3), rows - 1);   // clamp the ragged tail to a valid row
    int64_t arow;
    const uint8_t* base;
    if constexpr (GATEUP) {
      arow = shared ? r : slot_token(p.perm[row_base + r], p.top_k);
      base = reinterpret_cast<const uint8_t*>(shared ? p.A_shared : p.A);
    } else if constexpr (MODE == MODE_DOWN_SHARED) {
      arow = r;
      base = reinterpret_cast<const uint8_t*>(p.A_shared);
    } else {
      arow = row_base + r;
      base = reinterpret_cast<const uint8_t*>(p.A);
    }
    a_src[i] = base + arow * static_cast<int64_t>(K) * ES + (c & 7) * 16;
  }
  const uint8_t* bbase = reinterpret_cast<const uint8_t*>(shared ? p.B_shared : p.B) +
                         (shared ? 0 : static_cast<int64_t>(g) * K * ldb * ES);
  const uint8_t* b_src[B_CHUNKS];
  int b_k[B_CHUNKS], b_col[B_CHUNKS];
  bool b_ok[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    const int c = tid + i * 256;
    const int k = c / B_ROW_CHUNKS;
    const int lc = (c % B_ROW_CHUNKS) * VEC;  // local column in the tile
    int gc;                                     // global column in the weight row
    if constexpr (GATEUP) gc = lc < BNH ? n0 + lc : NH + n0 + (lc - BNH);
    else gc = n0 + lc;
    b_ok[i] = GATEUP ? true : (n0 + lc < NH);
    b_k[i] = k;
    b_col[i] = lc;
    b_src[i] = bbase + (static_cast<int64_t>(k) * ldb + (b_ok[i] ? gc : 0)) * ES;
  }

  i32x4 ra[A_CHUNKS], rb[B_CHUNKS];   // native vectors stay in VGPRs
  auto load_tiles = [&](int kt) {
    const int64_t koff = static_cast<int64_t>(kt) * kKBytes;
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) ra[i] = *reinterpret_cast<const i32x4*>(a_src[i] + koff);
    const int64_t kboff = static_cast<int64_t>(kt) * BK * ldb * ES;
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i)
      rb[i] = b_ok[i] ? *reinterpret_cast<const i32x4*>(b_src[i] + kboff) : i32x4{0, 0, 0, 0};
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int c = tid + i * 256;
      *reinterpret_cast<i32x4*>(&As[buf][(c >> 3) * kPitch + (c & 7) * 16]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
      const uint32_t w[4] = {static_cast<uint32_t>(rb[i][0]), static_cast<uint32_t>(rb[i][1]),
                             static_cast<uint32_t>(rb[i][2]), static_cast<uint32_t>(rb[i][3])};
      uint8_t* dst = &Bs[buf][b_col[i] * kPitch + b_k[i] * ES];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        if constexpr (ES == 2) {
          *reinterpret_cast<uint16_t*>(dst + j * kPitch) = static_cast<uint16_t>(w[j >> 1] >> (16 * (j & 1)));
        } else if constexpr (ES == 4) {
          *reinterpret_cast<uint32_t*>(dst + j * kPitch) = w[j];
        } else {
          dst[j * kPitch] = static_cast<uint8_t>(w[j >> 2] >> (8 * (j & 3)));
        }
      }
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // LDS column (row of Bs) of this wave's fragment j
  auto frag_col = [&](int j) -> int {
    if constexpr (GATEUP) {
      constexpr int HF = FN / 2;
      const int jj = j % HF;
      return (j < HF ? 0 : BNH) + wn * (BNH / WN) + jj * 16;
    } else {
      return wn * (BN / WN) + j * 16;
    }
  };

  const int nk = K / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  const int lrow = lane & 15;
  const int lk = (lane >> 4) * EL::kLaneK * ES;   // byte offset of this lane's K slice
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kKBytes; ks += EL::kStep * ES) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint8_t* ap = &As[cur][(wm * (BM / WM) + i * 16 + lrow) * kPitch + ks + lk];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const uint8_t* bp = &Bs[cur][(frag_col(j) + lrow) * kPitch + ks + lk];
          acc[i][j] = mfma_step<DT>(ap, bp, acc[i][j]);
        }
      }
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  16x16 accumulator layout: lane holds rows 4*(lane/16)+q
  // of column lane%16.
  const int lcol = lane & 15;
  const int rq = 4 * (lane >> 4);
  if constexpr (GATEUP) {
    constexpr int HF = FN / 2;
    const float* sB = shared ? p.sB_shared : (p.sB ? p.sB + static_cast<int64_t>(g) * 2 * NH : nullptr);
    uint32_t* amax = shared ? p.amax_shared : p.amax;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = m0 + wm * (BM / WM) + i * 16 + rq + q;
        const bool valid = r < rows;
        const int orow = row_base + min(r, rows - 1);        // output row (permuted order for routed)
        const int slot = shared ? min(r, rows - 1) : p.perm[orow];
        const int tok = shared ? slot : slot_token(slot, p.top_k);
        float scale = shared ? 1.0f : p.gate[slot];
        if constexpr (DT == DT_E4M3) scale *= (shared ? p.sA_shared : p.sA)[tok];
        float rmax = 0.f;
#pragma unroll
        for (int j = 0; j < HF; ++j) {
          const int col = n0 + wn * (BNH / WN) + j * 16 + lcol;
          float gv = acc[i][j][q] * scale;
          float uv = acc[i][j + HF][q] * scale;
          if constexpr (DT == DT_E4M3) {
            gv *= sB[col];
            uv *= sB[NH + col];
          }
          const float h = silu_f(gv) * uv;
          if (valid) {
            void* C = shared ? p.C_shared : p.C;
            const int64_t o = static_cast<int64_t>(orow) * NH + col;
            if constexpr (DT == DT_BF16) {
              reinterpret_cast<uint16_t*>(C)[o] = f32_to_bf16(h);
            } else if constexpr (DT == DT_F32) {
              reinterpret_cast<float*>(C)[o] = h;
            } else {
              // 24-bit h (the fp32 pattern rounded at bit 8: bits 31..16,
              // then 15..8); e4m3 rows are quantised afterwards from these
              // values, with the scale from the max of the fp32 values
              const uint32_t hb = __float_as_uint(h) + 0x80u;
              reinterpret_cast<uint16_t*>(C)[o] = static_cast<uint16_t>(hb >> 16);
              (shared ? p.C_shared_lo : p.C_lo)[o] = static_cast<uint8_t>(hb >> 8);
              rmax = fmaxf(rmax, fabsf(h));
            }
          }
        }
        if constexpr (DT == DT_E4M3) {
#pragma unroll
          for (int m = 1; m < 16; m <<= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, m, 64));
          if (valid && lcol == 0) atomicMax(&amax[orow], __float_as_uint(rmax));
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = m0 + wm * (BM / WM) + i * 16 + rq + q;
        if (r >= rows) continue;
        const int arow = row_base + r;   // row of A (h) = permuted row for routed
        const int orow = (MODE == MODE_DOWN_ROUTED) ? p.perm[arow] : r;
        float rs = 1.0f;
        if constexpr (DT == DT_E4M3) rs = (MODE == MODE_DOWN_ROUTED ? p.sA : p.sA_shared)[arow];
        const float* sB = nullptr;
        if constexpr (DT == DT_E4M3)
          sB = (MODE == MODE_DOWN_ROUTED) ? p.sB + static_cast<int64_t>(g) * NH : p.sB_shared;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * (BN / WN) + j * 16 + lcol;
          if (col >= NH) continue;
          float v = acc[i][j][q];
          if constexpr (DT == DT_E4M3) v *= rs * sB[col];
          const int64_t o = static_cast<int64_t>(orow) * NH + col;
          if constexpr (MODE == MODE_DOWN_SHARED) {
            reinterpret_cast<float*>(p.C_shared)[o] = v;
          } else {
            if (p.Y) v += p.Y[o];
            if (p.out_bf16) reinterpret_cast<uint16_t*>(p.C)[o] = f32_to_bf16(v);
            else reinterpret_cast<float*>(p.C)[o] = v;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- launcher

template <int DT, int MODE, int BM, int BN, int WM, int WN>
static hipError_t launch_one(const GemmArgs& a0, int grid_m_tokens, hipStream_t s, const int32_t* tiles_all) {
  GemmArgs a = a0;
  a.tiles = tiles_all + bm_index(BM) * (a.E + 2);
  int gm, nmax;
  constexpr int BNH = MODE == MODE_GATEUP ? BN / 2 : BN;
  const bool has_routed = a.group_lo < a.E;
  const bool has_shared = a.group_hi > a.E;
  const int mt_tok = (grid_m_tokens + BM - 1) / BM;
  if constexpr (MODE == MODE_DOWN_SHARED) {
    gm = mt_tok;
    nmax = a.N;
  } else {
    // sum over routed groups of ceil(n_g / BM) <= ceil(T k / BM) + E (T k routed rows); the shared
    // group adds ceil(T / BM)
    const int mt_r = (grid_m_tokens * (a.top_k > 1 ? a.top_k : 1) + BM - 1) / BM;
    gm = (has_routed ? mt_r + a.E : 0) + (has_shared ? mt_tok : 0);
    nmax = a.N;
    if (MODE == MODE_GATEUP) nmax = max(has_routed ? a.N : 0, has_shared ? a.N_shared : 0);
  }
  const int gn = (nmax + BNH - 1) / BNH;
  if (gm <= 0 || gn <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<DT, MODE, BM, BN, WM, WN>), dim3(gm, gn), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_dt(int mode, const GemmArgs& a, int grid_m_tokens, hipStream_t s, const int32_t* tiles) {
  switch (mode) {
    case MODE_GATEUP: return launch_one<DT, MODE_GATEUP, 128, 128, 2, 2>(a, grid_m_tokens, s, tiles);
    case MODE_DOWN_SHARED: return launch_one<DT, MODE_DOWN_SHARED, 128, 128, 2, 2>(a, grid_m_tokens, s, tiles);
    case MODE_DOWN_ROUTED: return launch_one<DT, MODE_DOWN_ROUTED, 128, 128, 2, 2>(a, grid_m_tokens, s, tiles);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm(int mode, int w_dtype, const GemmArgs& a, int grid_m_tokens, hipStream_t s,
                       const int32_t* tiles_all) {
  switch (w_dtype) {
    case DT_BF16: return launch_dt<DT_BF16>(mode, a, grid_m_tokens, s, tiles_all);
    case DT_F32: return launch_dt<DT_F32>(mode, a, grid_m_tokens, s, tiles_all);
    case DT_E4M3: return launch_dt<DT_E4M3>(mode, a, grid_m_tokens, s, tiles_all);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
