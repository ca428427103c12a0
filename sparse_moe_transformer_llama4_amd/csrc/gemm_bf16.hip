// bf16 grouped GEMMs for prefill-sized token counts (gfx950).
//
// Same three launches and epilogues as gemm.hip (gate/up with the SwiGLU
// epilogue over routed groups plus the shared expert; shared down; routed
// down with un-permute + combine), with a tiling sized for CDNA4:
//   * workgroup tile BM x 256 (BM = 64 / 128 / 256), 4 waves; at BM = 256
//     each wave owns a 128 x 128 accumulator block (256 AGPRs), so LDS
//     traffic per MFMA is half of what 64 x 64 blocks would need;
//   * operands travel global -> LDS with the gfx950 direct-to-LDS load
//     (global_load_lds_dwordx4): no staging registers, so a 4-deep ring of
//     K = 32 stages keeps about two stages of MFMA work in front of memory
//     latency at no VGPR cost;
//   * the DMA writes 16 bytes per lane at base + 16 * lane, so the LDS layout
//     is dense; bank conflicts are avoided with XOR swizzles applied on the
//     global side (each lane fetches the chunk that belongs at its slot):
//     A rows (64 B): chunk c of row r sits at c ^ ((r >> 2) & 3);
//     weight rows (512 B): 16-byte chunk c of row r sits at c ^ (2 * (r & 3));
//   * the weight operand is read with the gfx950 LDS transpose read
//     (ds_read_b64_tr_b16): each 16-lane group reads a 4 (K) x 16 (N) block
//     and every lane receives one column's 4 K values -- the MFMA operand
//     layout -- so the N-contiguous weight tile needs no transpose anywhere;
//   * the next stage's MFMA operands are read from LDS while the current
//     stage's MFMAs run (register double buffer, loop unrolled by two), one
//     explicit vmcnt wait + s_barrier per stage, and scheduling-group hints
//     interleave the memory operations with the MFMAs.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BN = 256;   // weight columns per tile (gate/up: 128 + 128)
constexpr int BK = 32;    // K per pipeline stage (bf16) = one MFMA step
constexpr int A_ROWB = BK * 2;    // bytes per A row in LDS (dense, swizzled)
constexpr int B_ROWB = BN * 2;    // bytes per weight row in LDS (dense, swizzled)
constexpr int B_STAGE = BK * B_ROWB;

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Scheduling-group hints (masks: 0x008 MFMA, 0x020 VMEM read, 0x100 DS read):
// N groups of (one op of class M, S MFMAs).
template <int N, int M, int S>
__device__ __forceinline__ void sched_pairs() {
  if constexpr (N > 0) {
    __builtin_amdgcn_sched_group_barrier(M, 1, 0);
    if constexpr (S > 0) __builtin_amdgcn_sched_group_barrier(0x008, S, 0);
    sched_pairs<N - 1, M, S>();
  }
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt in [3:0] and
// [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15 -> no wait on those).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Direct-to-LDS 16-byte load: every lane fetches 16 bytes from `g`; they
// land at LDS byte address m0 + 16 * lane.  Written as inline asm on purpose:
// the instruction writes no VGPR, and the stage pipeline below orders it with
// explicit vmcnt waits and barriers, whereas the compiler would otherwise
// wait for every in-flight stage before each LDS transpose read.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(g) : "memory", "m0");
}

// Weight fragment of 16 columns x 8 K rows (rows kb..kb+7) for this lane:
// lane s of each 16-lane group points at row kb + s/4 (and kb + 4 + s/4),
// bytes [2*(col + 4*(s%4)), +8) of the logical row, mapped through the swizzle.
__device__ __forceinline__ bf16x8 read_b_frag(const lds_u8* bs, int kb, int col, int lane) {
  const int s = lane & 15;
  const int lbyte = (col + 4 * (s & 3)) * 2;                 // logical byte in the row
  const int r = kb + (s >> 2);                                // (r & 3) == (s >> 2) & 3
  const int pbyte = ((lbyte >> 4) ^ (2 * (r & 3))) * 16 + (lbyte & 15);
  const lds_u8* p0 = bs + r * B_ROWB + pbyte;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 4 * B_ROWB));
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
  constexpr int A_STAGE = BM * A_ROWB;
  // LDS ring depth 4 (NBUF - 2 = 2 stages in flight ahead of the MFMAs).
  // Deeper rings measured slower: at BM = 64 they cost the second resident
  // workgroup per CU (4 x 20 KB lets two share the 160 KB LDS).
  constexpr int NBUF = 4;
  constexpr int A_INS = A_STAGE / 1024 / 4;   // 1 KB DMA instructions per wave per stage (A)
  constexpr int B_INS = B_STAGE / 1024 / 4;   // (weights)
  constexpr int LOADS = A_INS + B_INS;        // VMEM instructions per wave per stage
  constexpr int JPB = FN / FM;                 // next-stage weight fragments read per A block
  static_assert(WM * WN == 4, "4 waves");
  static_assert(!GATEUP || FN % 2 == 0, "gate/up fragment pairs");
  static_assert(A_INS >= 1 && B_INS == 4, "stage layout");
  static_assert(NBUF >= 4, "pipeline depth");
  static_assert(FN % FM == 0, "weight fragments spread evenly over the A blocks");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * (A_STAGE + B_STAGE)];
  lds_u8* const As = (lds_u8*)(smem);
  lds_u8* const Bs = As + NBUF * A_STAGE;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int E = p.E, T = p.T, K = p.K;

  // ---- tile lookup with an XCD-aware order.  Workgroup ids go round-robin
  // over the 8 XCDs (each with its own L2): XCD x = id % 8 takes the N-tiles
  // [x*gn/8, (x+1)*gn/8) for every M-tile, so each weight panel is fetched by
  // one XCD, and walks them M-major so the workgroups it runs together share
  // an A panel.  Ids beyond the real tile count exit.
  const int nmt = (MODE == MODE_DOWN_SHARED) ? (T + BM - 1) / BM : p.tiles[p.group_hi] - p.tiles[p.group_lo];
  const int gn = p.n_tiles;
  const int lid = blockIdx.x;
  int mt_rel, nt;
  if (gn >= 8) {
    const int x = lid & 7, local = lid >> 3;
    const int nt_lo = (x * gn) >> 3, w = (((x + 1) * gn) >> 3) - nt_lo;
    if (local >= nmt * w) return;
    mt_rel = local / w;
    nt = nt_lo + (local - mt_rel * w);
  } else {
    if (lid >= nmt * gn) return;
    mt_rel = lid / gn;
    nt = lid - mt_rel * gn;
  }
  int g, m0, rows;
  if constexpr (MODE == MODE_DOWN_SHARED) {
    g = 0;
    m0 = mt_rel * BM;
    rows = T;
  } else {
    const int mt = mt_rel + p.tiles[p.group_lo];
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
  const int n0 = nt * BNH;
  if (n0 >= NH) return;
  const int row_base = shared ? 0 : p.offsets[g];
  const int ldb = GATEUP ? 2 * NH : NH;

  // ---- DMA sources.  A: instruction i of this wave fills tile rows
  // 16*(wave*A_INS + i) + lane/4; the lane fetches the logical chunk that the
  // swizzle places at its slot.  Rows past the group's end repeat its last
  // row (their results are never stored).
  const uint16_t* abase;
  if constexpr (GATEUP) abase = reinterpret_cast<const uint16_t*>(shared ? p.A_shared : p.A);
  else if constexpr (MODE == MODE_DOWN_SHARED) abase = reinterpret_cast<const uint16_t*>(p.A_shared);
  else abase = reinterpret_cast<const uint16_t*>(p.A);
  uint32_t a_off[A_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int tr = 16 * (wave * A_INS + i) + (lane >> 2);        // tile row
    const int c = (lane & 3) ^ ((tr >> 2) & 3);                  // logical 16-byte chunk
    const int r = min(m0 + tr, rows - 1);
    int arow;
    if constexpr (GATEUP) arow = shared ? r : p.perm[row_base + r];
    else if constexpr (MODE == MODE_DOWN_SHARED) arow = r;
    else arow = row_base + r;
    a_off[i] = static_cast<uint32_t>(arow) * static_cast<uint32_t>(K) + c * 8;
  }
  // weights: instruction i fills K rows 2*(wave*4 + i) + lane/32 of the stage;
  // the lane's slot is 16-byte chunk lane%32 of that row
  const uint16_t* bbase = reinterpret_cast<const uint16_t*>(shared ? p.B_shared : p.B) +
                          (shared ? 0 : static_cast<int64_t>(g) * K * ldb);
  int64_t b_off[B_INS];
#pragma unroll
  for (int i = 0; i < B_INS; ++i) {
    const int kr = 2 * (wave * B_INS + i) + (lane >> 5);
    const int c = (lane & 31) ^ (2 * (kr & 3));
    const int lc = c * 8;                                        // tile column
    int gc;
    if constexpr (GATEUP) gc = lc < BNH ? n0 + lc : NH + n0 + (lc - BNH);
    else gc = n0 + lc;
    const bool ok = n0 + (GATEUP ? lc % BNH : lc) < NH;
    b_off[i] = static_cast<int64_t>(kr) * ldb + (ok ? gc : 0);  // clamped columns: valid, discarded
  }
  const int64_t b_kstride = static_cast<int64_t>(BK) * ldb;
  const int nk = K / BK;   // even: K is a multiple of 64

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lrow = lane & 15;
  const int kg = lane >> 4;         // this lane's 8-wide K group inside the stage
  // A fragment i: logical row wm*(BM/WM) + 16 i + lrow, chunk kg; (row >> 2) & 3 == lrow >> 2
  const int a_rd = (wm * (BM / WM) + lrow) * A_ROWB + ((kg ^ (lrow >> 2)) << 4);

  // Operands in registers: the weight fragments of a stage (FN x 4 VGPRs) are
  // double-buffered across stages; A fragments stream one 16-row block ahead
  // (2 x 4 VGPRs), the next A block read while the current one's FN MFMAs run.
  bf16x8 fb0[FN], fb1[FN], fa[2];
  // wave-uniform LDS byte addresses of this wave's first DMA slot (A / weights)
  const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t a_lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(As)) + wave_u * (A_INS * 1024);
  const uint32_t b_lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(Bs)) + wave_u * (B_INS * 1024);

#define MOE_ISSUE(st)                                                                          \
  do {                                                                                         \
    const int s_ = min((st), nk - 1);                                                          \
    const uint32_t b_ = static_cast<uint32_t>((st) % NBUF);                                    \
    _Pragma("unroll") for (int i = 0; i < A_INS; ++i)                                          \
      dma16(abase + a_off[i] + s_ * BK, a_lds0 + b_ * A_STAGE + i * 1024);                     \
    _Pragma("unroll") for (int i = 0; i < B_INS; ++i)                                          \
      dma16(bbase + b_off[i] + s_ * b_kstride, b_lds0 + b_ * B_STAGE + i * 1024);              \
  } while (0)
#define MOE_BFRAG(FB, j, st)                                                                   \
  do {                                                                                         \
    int col_;                                                                                  \
    if constexpr (GATEUP) col_ = ((j) < FN / 2 ? 0 : BNH) + wn * (BNH / WN) + ((j) % (FN / 2)) * 16; \
    else col_ = wn * (BN / WN) + (j) * 16;                                                     \
    FB[j] = read_b_frag(Bs + ((st) % NBUF) * B_STAGE, kg * 8, col_, lane);                     \
  } while (0)
#define MOE_AFRAG(dst, i, st)                                                                  \
  dst = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(                    \
      As + ((st) % NBUF) * A_STAGE + a_rd + (i) * 16 * A_ROWB)
  // One stage: DMA of stage kt+NBUF-1; weight fragments of stage kt+1 into
  // FB2; FM blocks of FN MFMAs on stage kt (A block i+1 read during block i,
  // the last one reading block 0 of stage kt+1); then publish stage kt+2 (this
  // wave's DMA for it done, only later stages' may be in flight) with a
  // barrier that also keeps every wave's reads ahead of the next overwrite.
#define MOE_STEP(kt, FB, FB2)                                                                  \
  do {                                                                                         \
    MOE_ISSUE((kt) + NBUF - 1);                                                                \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                           \
      /* reads for the next block: A block i+1 (or block 0 of stage kt+1) and */               \
      /* JPB of stage kt+1's weight fragments; then block i's MFMAs          */               \
      if (i + 1 < FM) MOE_AFRAG(fa[(i + 1) & 1], i + 1, (kt));                                 \
      else MOE_AFRAG(fa[(i + 1) & 1], 0, (kt) + 1);                                            \
      _Pragma("unroll") for (int jj = 0; jj < JPB; ++jj) MOE_BFRAG(FB2, i * JPB + jj, (kt) + 1); \
      __builtin_amdgcn_sched_barrier(0);                                                       \
      _Pragma("unroll") for (int j = 0; j < FN; ++j)                                           \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i & 1], FB[j], acc[i][j], 0, 0, 0); \
      __builtin_amdgcn_sched_barrier(0);                                                       \
    }                                                                                          \
    wait_vmcnt<(NBUF - 3) * LOADS>();                                                          \
    __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) */                                       \
    __builtin_amdgcn_s_barrier();                                                              \
  } while (0)

  // prologue: stages 0 .. NBUF-2 in flight.  Iteration kt reads stage kt+1's
  // operands, so stages 0 and 1 must have landed (only the later stages' DMA
  // may still be in flight) before the barrier that publishes them.
#pragma unroll
  for (int st = 0; st < NBUF - 1; ++st) MOE_ISSUE(st);
  wait_vmcnt<(NBUF - 3) * LOADS>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int j = 0; j < FN; ++j) MOE_BFRAG(fb0, j, 0);
  MOE_AFRAG(fa[0], 0, 0);
  for (int kt = 0; kt < nk; kt += 2) {
    MOE_STEP(kt, fb0, fb1);
    MOE_STEP(kt + 1, fb1, fb0);
  }
  wait_vmcnt<0>();
#undef MOE_BFRAG
#undef MOE_AFRAG
#undef MOE_ISSUE
#undef MOE_STEP

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
  a.n_tiles = gn;
  // 1-D grid: enough ids for the largest per-XCD share of (M-tile bound x N-tiles)
  const int64_t nblk = gn >= 8 ? 8 * static_cast<int64_t>(gm) * ((gn + 7) / 8) : static_cast<int64_t>(gm) * gn;
  hipLaunchKernelGGL((gemm_bf16_kernel<MODE, BM, WM, WN>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, a);
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
