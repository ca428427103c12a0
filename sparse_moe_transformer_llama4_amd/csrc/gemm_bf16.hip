// bf16 grouped GEMMs for prefill-sized token counts (gfx950).
//
// Same three launches and epilogues as gemm.hip (gate/up with the SwiGLU
// epilogue over routed groups plus the shared expert; shared down; routed
// down with un-permute + combine), with a tiling sized for CDNA4:
//   * workgroup tile BM x 256 (BM = 64 / 128 / 256), K staged 64 at a time,
//     4 waves; at BM = 256 each wave owns a 128 x 128 accumulator block, so
//     LDS traffic per MFMA stays at half of what 64 x 64 blocks would need;
//   * both operands are written to LDS exactly as they sit in memory (A rows
//     K-contiguous, the weight tile N-contiguous) with 16-byte stores;
//   * the weight operand is read back with the gfx950 LDS transpose read
//     (ds_read_b64_tr_b16): each 16-lane group reads a 4 (K) x 16 (N) block
//     and every lane receives one column's 4 K values -- the MFMA operand
//     layout -- so no transpose is done in registers or with scalar stores;
//   * the weight rows are padded to 544 bytes so the four rows a 16-lane
//     group reads fall into disjoint LDS banks;
//   * double-buffered LDS: the next K stage is fetched into registers while
//     the current one feeds the MFMAs, one barrier per stage.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BN = 256;               // weight columns per tile (gate/up: 128 + 128)
constexpr int BK = 64;                // K per stage (bf16 elements)
constexpr int A_PITCH = BK * 2 + 16;  // bytes per A row in LDS
constexpr int B_PITCH = BN * 2 + 32;  // bytes per weight row in LDS

__device__ __forceinline__ bf16x8 read_b_frag(const uint8_t* bs, int kb, int col, int lane) {
  // lane s of the 16-lane group points at row kb + s/4, columns col + 4*(s%4)
  const int s = lane & 15;
  const uint8_t* p0 = bs + (kb + (s >> 2)) * B_PITCH + (col + 4 * (s & 3)) * 2;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * B_PITCH));
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int MODE, int BM, int WM, int WN>
__global__ __launch_bounds__(256, 1) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr bool GATEUP = MODE == MODE_GATEUP;
  constexpr int BNH = GATEUP ? BN / 2 : BN;
  constexpr int A_CH = BM * BK * 2 / 16 / 256;   // 16-byte chunks per thread (rows tid/8 + 32 i)
  constexpr int B_CH = BK * BN * 2 / 16 / 256;   // (K rows tid/32 + 8 i)
  static_assert(B_CH == 8, "weight chunk layout");
  static_assert(WM * WN == 4, "4 waves");
  static_assert(!GATEUP || FN % 2 == 0, "gate/up fragment pairs");

  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * A_PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BK * B_PITCH];

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
  const int NH = (GATEUP && shared) ? p.N_shared : p.N;
  const int n0 = blockIdx.y * BNH;
  if (n0 >= NH) return;
  const int row_base = shared ? 0 : p.offsets[g];
  const int ldb = GATEUP ? 2 * NH : NH;

  // ---- global sources.  A: 8 chunks of 16 bytes per row, rows (tid>>3) + 32*i
  // (gathered through perm for the routed gate/up groups), kept as 32-bit
  // element offsets.  Weights: every chunk of this thread sits in the same
  // tile column, rows (tid>>5) + 8*i, so one base address and a row stride
  // serve all of them.
  const uint16_t* abase;
  if constexpr (GATEUP) abase = reinterpret_cast<const uint16_t*>(shared ? p.A_shared : p.A);
  else if constexpr (MODE == MODE_DOWN_SHARED) abase = reinterpret_cast<const uint16_t*>(p.A_shared);
  else abase = reinterpret_cast<const uint16_t*>(p.A);
  uint32_t a_off[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int r = min(m0 + (tid >> 3) + 32 * i, rows - 1);
    int arow;
    if constexpr (GATEUP) arow = shared ? r : p.perm[row_base + r];
    else if constexpr (MODE == MODE_DOWN_SHARED) arow = r;
    else arow = row_base + r;
    a_off[i] = static_cast<uint32_t>(arow) * static_cast<uint32_t>(K) + (tid & 7) * 8;
  }
  const int lcB = (tid & 31) * 8;   // tile column of this thread's weight chunks
  int gcB;
  if constexpr (GATEUP) gcB = lcB < BNH ? n0 + lcB : NH + n0 + (lcB - BNH);
  else gcB = n0 + lcB;
  const bool b_ok = n0 + (GATEUP ? lcB % BNH : lcB) < NH;
  const uint16_t* bptr = reinterpret_cast<const uint16_t*>(shared ? p.B_shared : p.B) +
                         (shared ? 0 : static_cast<int64_t>(g) * K * ldb) +
                         static_cast<int64_t>(tid >> 5) * ldb + (b_ok ? gcB : 0);
  const int64_t b_rstride = static_cast<int64_t>(8) * ldb;     // 8 K rows between this thread's chunks
  const int64_t b_kstride = static_cast<int64_t>(BK) * ldb;    // one K stage

  i32x4 ra[A_CH], rb[B_CH];   // native vectors: kept in VGPRs (HIP's uint4 struct is not)
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  const int lrow = lane & 15;
  const int lkb = (lane >> 4) * 8;   // this lane's K offset inside a 32-wide MFMA step
  uint8_t* const a_st = &As[0][(tid >> 3) * A_PITCH + (tid & 7) * 16];
  uint8_t* const b_st = &Bs[0][(tid >> 5) * B_PITCH + (tid & 31) * 16];

#define MOE_LOAD_STAGE(kt)                                                                     \
  do {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                                           \
      ra[i] = *reinterpret_cast<const i32x4*>(abase + a_off[i] + (kt) * BK);                   \
    const uint16_t* bp_ = bptr + (kt) * b_kstride;                                             \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i)                                           \
      rb[i] = b_ok ? *reinterpret_cast<const i32x4*>(bp_ + i * b_rstride) : i32x4{0, 0, 0, 0};     \
  } while (0)
#define MOE_STORE_STAGE(buf)                                                                   \
  do {                                                                                         \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                                           \
      *reinterpret_cast<i32x4*>(a_st + (buf) * (BM * A_PITCH) + i * 32 * A_PITCH) = ra[i];     \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i)                                           \
      *reinterpret_cast<i32x4*>(b_st + (buf) * (BK * B_PITCH) + i * 8 * B_PITCH) = rb[i];      \
  } while (0)

  MOE_LOAD_STAGE(0);
  MOE_STORE_STAGE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) MOE_LOAD_STAGE(kt + 1);
    const uint8_t* as = As[cur];
    const uint8_t* bs = Bs[cur];
#pragma unroll
    for (int ks = 0; ks < BK; ks += 32) {
      bf16x8 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(as + (wm * (BM / WM) + i * 16 + lrow) * A_PITCH + (ks + lkb) * 2);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        int col;
        if constexpr (GATEUP) {
          constexpr int HF = FN / 2;
          col = (j < HF ? 0 : BNH) + wn * (BNH / WN) + (j % HF) * 16;
        } else {
          col = wn * (BN / WN) + j * 16;
        }
        bf[j] = read_b_frag(bs, ks + lkb, col, lane);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) MOE_STORE_STAGE(cur ^ 1);
    __syncthreads();
  }
#undef MOE_LOAD_STAGE
#undef MOE_STORE_STAGE

  // ---- epilogue (16x16 accumulator: lane holds rows 4*(lane/16)+q of column lane%16)
  const int lcol = lane & 15;
  const int rq = 4 * (lane >> 4);
  if constexpr (GATEUP) {
    constexpr int HF = FN / 2;
    void* C = shared ? p.C_shared : p.C;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = m0 + wm * (BM / WM) + i * 16 + rq + q;
        if (r >= rows) continue;
        const int orow = row_base + r;
        const float scale = shared ? 1.0f : p.gate[p.perm[orow]];
#pragma unroll
        for (int j = 0; j < HF; ++j) {
          const int col = n0 + wn * (BNH / WN) + j * 16 + lcol;
          if (col >= NH) continue;
          const float gv = acc[i][j][q] * scale;
          const float uv = acc[i][j + HF][q] * scale;
          reinterpret_cast<uint16_t*>(C)[static_cast<int64_t>(orow) * NH + col] = f32_to_bf16(silu_f(gv) * uv);
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
        const int arow = row_base + r;
        const int orow = (MODE == MODE_DOWN_ROUTED) ? p.perm[arow] : r;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = n0 + wn * (BN / WN) + j * 16 + lcol;
          if (col >= NH) continue;
          const int64_t o = static_cast<int64_t>(orow) * NH + col;
          const float v = acc[i][j][q];
          if constexpr (MODE == MODE_DOWN_SHARED) {
            reinterpret_cast<float*>(p.C_shared)[o] = v;
          } else {
            const float y = v + p.Y[o];
            if (p.out_bf16) reinterpret_cast<uint16_t*>(p.C)[o] = f32_to_bf16(y);
            else reinterpret_cast<float*>(p.C)[o] = y;
          }
        }
      }
    }
  }
}

template <int MODE, int BM, int WM, int WN>
hipError_t launch_v2(const GemmArgs& a0, int T, hipStream_t s, const int32_t* tiles_all) {
  GemmArgs a = a0;
  a.tiles = tiles_all + bm_index(BM) * (a.E + 2);
  constexpr int BNH = MODE == MODE_GATEUP ? BN / 2 : BN;
  int gm, nmax;
  const bool has_routed = a.group_lo < a.E;
  const bool has_shared = a.group_hi > a.E;
  if constexpr (MODE == MODE_DOWN_SHARED) {
    gm = (T + BM - 1) / BM;
    nmax = a.N;
  } else {
    // sum over routed groups of ceil(n_g / BM) <= ceil(T / BM) + E; the shared group adds ceil(T / BM)
    gm = (has_routed ? (T + BM - 1) / BM + a.E : 0) + (has_shared ? (T + BM - 1) / BM : 0);
    nmax = a.N;
    if (MODE == MODE_GATEUP) nmax = max(has_routed ? a.N : 0, has_shared ? a.N_shared : 0);
  }
  if (gm <= 0) return hipSuccess;
  const int gn = (nmax + BNH - 1) / BNH;
  hipLaunchKernelGGL((gemm_bf16_kernel<MODE, BM, WM, WN>), dim3(gm, gn), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int bm, const GemmArgs& a, int T, hipStream_t s, const int32_t* tiles) {
  switch (bm) {
    case 256: return launch_v2<MODE, 256, 2, 2>(a, T, s, tiles);
    case 128: return launch_v2<MODE, 128, 2, 2>(a, T, s, tiles);
    default: return launch_v2<MODE, 64, 1, 4>(a, T, s, tiles);
  }
}

}  // namespace

bool bf16_v2_supported(int K, int N, int N_shared) {
  return K % BK == 0 && N % 64 == 0 && N_shared % 64 == 0;
}

hipError_t launch_gemm_bf16_v2(int mode, int bm, const GemmArgs& a, int T, hipStream_t s,
                               const int32_t* tiles_all) {
  switch (mode) {
    case MODE_GATEUP: return launch_mode<MODE_GATEUP>(bm, a, T, s, tiles_all);
    case MODE_DOWN_SHARED: return launch_mode<MODE_DOWN_SHARED>(bm, a, T, s, tiles_all);
    case MODE_DOWN_ROUTED: return launch_mode<MODE_DOWN_ROUTED>(bm, a, T, s, tiles_all);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
