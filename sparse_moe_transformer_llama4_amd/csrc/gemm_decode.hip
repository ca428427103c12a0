// bf16 grouped GEMMs for decode-sized token counts (gfx950).
//
// With a few tokens per expert the block is a weight stream: every touched
// expert's W_gate_up and W_down are read once from HBM and each weight is
// used by a handful of rows.  The kernels therefore optimise bytes in
// flight, not MFMA reuse:
//   * workgroup tile = (group, 16 or 32 rows, 128 weight columns); gate/up
//     tiles pair 64 gate columns with the matching 64 up columns;
//   * wave-level split-K: each of the 4 waves streams its own quarter of K
//     through a private LDS ring (4 deep for 16-row tiles, 3 deep for 32-row
//     tiles) fed by direct-to-LDS loads (global_load_lds_dwordx4), so the
//     main loop needs no workgroup barrier -- each wave only waits for its
//     own DMA (vmcnt) -- and 80-108 KB per CU are in flight against HBM
//     latency;
//   * weight rows are 256 B in LDS; 16-byte chunk c of row r is stored at
//     c ^ (2 * (r & 3)) so the LDS transpose reads (ds_read_b64_tr_b16) of
//     four consecutive rows hit disjoint banks;
//   * the activation rows of each stage travel through the same per-wave
//     DMA ring (1-2 KB per stage), so every load in the loop is ordered by
//     the explicit waits and none by compiler-inserted ones;
//   * MFMAs only for the 16-row fragments that hold valid rows;
//   * the four K-quarter partial sums are added through LDS once at the end,
//     followed by the same epilogues as the prefill kernels (SwiGLU with the
//     gate on routed rows; fp32 shared output; un-permute + combine).
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int DBN = 128;            // weight columns per tile
constexpr int DBK = 32;             // K per stage (one MFMA step)
constexpr int ROWB = DBN * 2;       // bytes per weight row in LDS
constexpr int WSTAGE = DBK * ROWB;  // 8 KB of weights per stage
constexpr int INS = WSTAGE / 1024;  // weight DMA instructions per stage per wave (8)
constexpr int FN = DBN / 16;        // weight fragments (16 columns each)

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Direct-to-LDS 16-byte load into m0 + 16 * lane (inline asm: it writes no
// VGPR; the stage ring orders it with explicit vmcnt waits).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(g) : "memory", "m0");
}

__device__ __forceinline__ bf16x8 read_w_frag(const lds_u8* st, int kb, int col, int lane) {
  const int s = lane & 15;
  const int lbyte = (col + 4 * (s & 3)) * 2;
  const int r = kb + (s >> 2);
  const int pbyte = ((lbyte >> 4) ^ (2 * (r & 3))) * 16 + (lbyte & 15);
  const lds_u8* p0 = st + r * ROWB + pbyte;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * ROWB));
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

template <int MODE, int FMMAX>
__global__ __launch_bounds__(256, 1) void gemm_decode_kernel(GemmArgs p) {
  constexpr bool GATEUP = MODE == MODE_GATEUP;
  constexpr int BNH = GATEUP ? DBN / 2 : DBN;   // output columns per tile
  constexpr int DBM = 16 * FMMAX;               // rows per tile
  constexpr int ASTAGE = FMMAX * 1024;          // activation bytes per stage (16 rows x 64 B per KB)
  constexpr int STAGE = WSTAGE + ASTAGE;
  constexpr int DNBUF = 4;                      // per-wave ring depth (LDS: 4 x 4 x 9 KB / 4 x 4 x 10 KB)
  constexpr int LOADS = INS + FMMAX;            // DMA instructions per stage per wave
  constexpr int PART = 4 * DBM * DBN * 4;       // bytes of the final partial sums
  constexpr int RING = 4 * DNBUF * STAGE;
  constexpr int SMEM = RING > PART + 4 * DBM ? RING : PART + 4 * DBM;   // + per-row table after PART
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, T = p.T, K = p.K;

  // ---- tile lookup (DBM-row tiles)
  int g, m0, rows;
  if constexpr (MODE == MODE_DOWN_SHARED) {
    g = 0;
    m0 = blockIdx.x * DBM;
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
    m0 = (mt - p.tiles[g]) * DBM;
    rows = (g == E) ? T : p.offsets[g + 1] - p.offsets[g];
  }
  const bool shared = (MODE == MODE_DOWN_SHARED) || (GATEUP && g == E);
  const int NH = (GATEUP && shared) ? p.N_shared : p.N;
  const int n0 = blockIdx.y * BNH;
  if (n0 >= NH) return;
  const int row_base = shared ? 0 : p.offsets[g];
  const int ldb = GATEUP ? 2 * NH : NH;
  const int nvalid = min(DBM, rows - m0);
  const int fm = (nvalid + 15) >> 4;            // fragments with valid rows (uniform)

  // Per-row metadata for the epilogue (the routed gate/up's gate scale, the
  // routed down's output row), one tile row per thread, loaded now so its
  // latency hides behind the main loop.
  float row_scale = 1.0f;
  int row_out = 0;
  if (tid < DBM) {
    const int r = min(m0 + tid, rows - 1);
    if constexpr (GATEUP) {
      if (!shared) row_scale = p.gate[p.perm[row_base + r]];
    } else if constexpr (MODE == MODE_DOWN_ROUTED) {
      row_out = p.perm[row_base + r];
    }
  }

  // ---- this block's K range (split over blockIdx.z for the shared down
  // GEMM, whose single M-tile would otherwise leave most CUs idle) and this
  // wave's quarter of it
  const int nsplit = gridDim.z;
  const int kq = (K / nsplit) >> 2;             // multiple of 32
  const int k0 = static_cast<int>(blockIdx.z) * (K / nsplit) + wave * kq;
  const int ns = kq / DBK;

  // weights: DMA instruction i fills K rows 4i .. 4i+3 of the stage; lane ->
  // row 4i + lane/16, physical chunk lane%16 holds logical chunk c
  const uint16_t* wbase = reinterpret_cast<const uint16_t*>(shared ? p.B_shared : p.B) +
                          (shared ? 0 : static_cast<int64_t>(g) * K * ldb);
  int64_t w_off[INS];
#pragma unroll
  for (int i = 0; i < INS; ++i) {
    const int kr = 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ (2 * (kr & 3));
    const int lc = c * 8;
    int gc;
    if constexpr (GATEUP) gc = lc < BNH ? n0 + lc : NH + n0 + (lc - BNH);
    else gc = n0 + lc;
    const bool ok = n0 + (GATEUP ? lc % BNH : lc) < NH;
    w_off[i] = static_cast<int64_t>(k0 + kr) * ldb + (ok ? gc : 0);
  }
  const int64_t w_kstride = static_cast<int64_t>(DBK) * ldb;

  // activations: DMA instruction f fills rows 16f .. 16f+15 (64 B each) of the
  // stage's activation block; lane -> row 16f + lane/4, slot lane%4, which
  // holds logical chunk slot ^ ((row >> 1) & 3) (conflict-free fragment reads)
  const uint16_t* abase;
  if constexpr (GATEUP) abase = reinterpret_cast<const uint16_t*>(shared ? p.A_shared : p.A);
  else if constexpr (MODE == MODE_DOWN_SHARED) abase = reinterpret_cast<const uint16_t*>(p.A_shared);
  else abase = reinterpret_cast<const uint16_t*>(p.A);
  int64_t a_off[FMMAX];
#pragma unroll
  for (int f = 0; f < FMMAX; ++f) {
    const int r = min(m0 + 16 * f + (lane >> 2), rows - 1);
    int arow;
    if constexpr (GATEUP) arow = shared ? r : p.perm[row_base + r];
    else if constexpr (MODE == MODE_DOWN_SHARED) arow = r;
    else arow = row_base + r;
    a_off[f] = static_cast<int64_t>(arow) * K + k0 + (((lane & 3) ^ ((lane >> 3) & 3)) * 8);
  }

  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem)) +
                        __builtin_amdgcn_readfirstlane(wave) * (DNBUF * STAGE);
  const lds_u8* ring_p = (const lds_u8*)smem + wave * (DNBUF * STAGE);
  // this lane's A fragment slot: row lane%16 of the fragment, K chunk lane/16
  const int a_rd = WSTAGE + (lane & 15) * 64 + (((lane >> 4) ^ ((lane >> 1) & 3)) << 4);

  f32x4 acc[FMMAX][FN];
#pragma unroll
  for (int f = 0; f < FMMAX; ++f)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[f][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#define DEC_ISSUE(st)                                                                          \
  do {                                                                                         \
    const int s_ = min((st), ns - 1);                                                          \
    const uint32_t b_ = ring + static_cast<uint32_t>(((st) % DNBUF) * STAGE);                  \
    _Pragma("unroll") for (int i = 0; i < INS; ++i)                                            \
      dma16(wbase + w_off[i] + s_ * w_kstride, b_ + i * 1024);                                 \
    _Pragma("unroll") for (int f = 0; f < FMMAX; ++f)                                          \
      dma16(abase + a_off[f] + s_ * DBK, b_ + WSTAGE + f * 1024);                              \
  } while (0)
  // Stage kt: its DMA is complete once only the later stages' DMAs remain.
#define DEC_STEP(kt)                                                                           \
  do {                                                                                         \
    DEC_ISSUE((kt) + DNBUF - 1);                                                               \
    wait_vmcnt<(DNBUF - 1) * LOADS>();                                                         \
    const lds_u8* st_ = ring_p + ((kt) % DNBUF) * STAGE;                                       \
    bf16x8 wf[FN], af[FMMAX];                                                                  \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                           \
      int col_;                                                                                \
      if constexpr (GATEUP) col_ = (j < FN / 2 ? 0 : BNH) + (j % (FN / 2)) * 16;               \
      else col_ = j * 16;                                                                      \
      wf[j] = read_w_frag(st_, (lane >> 4) * 8, col_, lane);                                   \
    }                                                                                          \
    _Pragma("unroll") for (int f = 0; f < FMMAX; ++f)                                          \
      af[f] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(st_ + a_rd + f * 1024); \
    _Pragma("unroll") for (int f = 0; f < FMMAX; ++f)                                          \
      if (f < fm)                                                                              \
        _Pragma("unroll") for (int j = 0; j < FN; ++j)                                         \
          acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[f], wf[j], acc[f][j], 0, 0, 0); \
    /* this stage's slot is refilled DNBUF-1 steps later: reads must be done */                \
    __builtin_amdgcn_s_waitcnt(0xC07F);                                                        \
  } while (0)

#pragma unroll
  for (int st = 0; st < DNBUF - 1; ++st) DEC_ISSUE(st);
  for (int kt = 0; kt < ns; ++kt) DEC_STEP(kt);
  wait_vmcnt<0>();
#undef DEC_ISSUE
#undef DEC_STEP

  // ---- add the four K-quarter partial sums through LDS: wave w writes its
  // [64 x 128] fp32 partial (layout [row][col]) into smem
  __syncthreads();
  float* part = reinterpret_cast<float*>(smem);
  const int lcol = lane & 15, rq = 4 * (lane >> 4);
#pragma unroll
  for (int f = 0; f < FMMAX; ++f) {
    if (f < fm) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          part[(wave * DBM + 16 * f + rq + q) * DBN + j * 16 + lcol] = acc[f][j][q];
    }
  }
  if (tid < DBM) {
    if constexpr (GATEUP) reinterpret_cast<float*>(smem + PART)[tid] = row_scale;
    else reinterpret_cast<int*>(smem + PART)[tid] = row_out;
  }
  __syncthreads();
  auto total = [&](int r, int c) -> float {
    return part[(0 * DBM + r) * DBN + c] + part[(1 * DBM + r) * DBN + c] + part[(2 * DBM + r) * DBN + c] +
           part[(3 * DBM + r) * DBN + c];
  };

  // ---- epilogue: thread -> (row, column) pairs, columns fastest.  Fixed
  // trip count, fully unrolled, every global load ahead of the stores (the
  // compiler must assume stores through C may alias the loaded arrays, so a
  // load between stores would wait a full round trip).
  constexpr int NIT = DBM * BNH / 256;
  if constexpr (GATEUP) {
    void* C = shared ? p.C_shared : p.C;
    const float* sct = reinterpret_cast<const float*>(smem + PART);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int e = tid + 256 * it;
      const int r = e / BNH, c = e % BNH;
      const int col = n0 + c;
      if (r >= nvalid || col >= NH) continue;
      const int orow = row_base + m0 + r;
      const float gv = total(r, c) * sct[r];
      const float uv = total(r, BNH + c) * sct[r];
      reinterpret_cast<uint16_t*>(C)[static_cast<int64_t>(orow) * NH + col] = f32_to_bf16(silu_f(gv) * uv);
    }
  } else {
    const int* ot = reinterpret_cast<const int*>(smem + PART);
    float y[NIT];
    if constexpr (MODE == MODE_DOWN_ROUTED) {
      // the shared expert's output, as y_parts K-split partials summed in order
      const int nparts = p.y_parts > 1 ? p.y_parts : 1;
      const int64_t pstride = static_cast<int64_t>(T) * NH;
#pragma unroll
      for (int it = 0; it < NIT; ++it) y[it] = 0.0f;
      for (int s0 = 0; s0 < nparts; s0 += 4) {
        float yv[4][NIT];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int it = 0; it < NIT; ++it) {
            const int e = tid + 256 * it;
            const int r = e / BNH, col = n0 + e % BNH;
            yv[u][it] = (s0 + u < nparts && r < nvalid && col < NH)
                            ? p.Y[(s0 + u) * pstride + static_cast<int64_t>(ot[r]) * NH + col] : 0.0f;
          }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int it = 0; it < NIT; ++it)
            if (s0 + u < nparts) y[it] += yv[u][it];
      }
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int e = tid + 256 * it;
      const int r = e / BNH, c = e % BNH;
      const int col = n0 + c;
      if (r >= nvalid || col >= NH) continue;
      const int orow = (MODE == MODE_DOWN_ROUTED) ? ot[r] : m0 + r;
      const int64_t o = static_cast<int64_t>(orow) * NH + col;
      const float v = total(r, c);
      if constexpr (MODE == MODE_DOWN_SHARED) {
        reinterpret_cast<float*>(p.C_shared)[static_cast<int64_t>(blockIdx.z) * T * NH + o] = v;
      } else {
        const float yv = v + y[it];
        if (p.out_bf16) reinterpret_cast<uint16_t*>(p.C)[o] = f32_to_bf16(yv);
        else reinterpret_cast<float*>(p.C)[o] = yv;
      }
    }
  }
}

template <int MODE, int FMMAX>
hipError_t launch_dec(const GemmArgs& a0, int T, hipStream_t s, const int32_t* tiles_all) {
  constexpr int DBM = 16 * FMMAX;
  GemmArgs a = a0;
  a.tiles = tiles_all + bm_index(DBM) * (a.E + 2);
  constexpr int BNH = MODE == MODE_GATEUP ? DBN / 2 : DBN;
  const bool has_routed = a.group_lo < a.E;
  const bool has_shared = a.group_hi > a.E;
  const int mt_tok = (T + DBM - 1) / DBM;
  int gm, nmax = a.N;
  if constexpr (MODE == MODE_DOWN_SHARED) {
    gm = mt_tok;
  } else {
    gm = (has_routed ? mt_tok + a.E : 0) + (has_shared ? mt_tok : 0);
    if (MODE == MODE_GATEUP) nmax = max(has_routed ? a.N : 0, has_shared ? a.N_shared : 0);
  }
  if (gm <= 0) return hipSuccess;
  const int gn = (nmax + BNH - 1) / BNH;
  const int ks = (MODE == MODE_DOWN_SHARED && a.ksplit > 1) ? a.ksplit : 1;
  if (a.K % (128 * ks) != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_decode_kernel<MODE, FMMAX>), dim3(gm, gn, ks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int K) { return K % 128 == 0 && K >= 128; }

// rows32: 32-row tiles (for groups that may exceed 16 rows), else 16-row tiles.
hipError_t launch_gemm_decode(int mode, bool rows32, const GemmArgs& a, int T, hipStream_t s,
                              const int32_t* tiles_all) {
  if (rows32) {
    switch (mode) {
      case MODE_GATEUP: return launch_dec<MODE_GATEUP, 2>(a, T, s, tiles_all);
      case MODE_DOWN_SHARED: return launch_dec<MODE_DOWN_SHARED, 2>(a, T, s, tiles_all);
      case MODE_DOWN_ROUTED: return launch_dec<MODE_DOWN_ROUTED, 2>(a, T, s, tiles_all);
    }
  } else {
    switch (mode) {
      case MODE_GATEUP: return launch_dec<MODE_GATEUP, 1>(a, T, s, tiles_all);
      case MODE_DOWN_SHARED: return launch_dec<MODE_DOWN_SHARED, 1>(a, T, s, tiles_all);
      case MODE_DOWN_ROUTED: return launch_dec<MODE_DOWN_ROUTED, 1>(a, T, s, tiles_all);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
