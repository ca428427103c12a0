// bf16 grouped GEMM kernel for prefill-sized token counts (gfx950).
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
//     A rows (64 B): chunk c of row r sits at c ^ ((r >> 1) & 3) (measured
//     conflict-free for the fragment reads; (r >> 2) & 3 halves their rate);
//     weight rows (512 B): 16-byte chunk c of row r sits at c ^ (2 * (r & 3));
//   * the weight operand is read with the gfx950 LDS transpose read
//     (ds_read_b64_tr_b16): each 16-lane group reads a 4 (K) x 16 (N) block
//     and every lane receives one column's 4 K values -- the MFMA operand
//     layout -- so the N-contiguous weight tile needs no transpose anywhere;
//   * all of the next stage's MFMA operands are read from LDS while the
//     current stage's MFMAs run (register double buffer, loop unrolled by
//     two), one explicit vmcnt wait + s_barrier per stage.
//
// Internal header: gemm_bf16_tall.hip instantiates the 256-row tiles (AGPR
// accumulators) and gemm_bf16.hip the 64- and 128-row tiles (built with
// VGPR-form MFMAs, which keeps their main loops free of accumulator copies).
#pragma once

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
// The scalar-base form is used: `sbase` is wave-uniform (SGPR pair) and each
// lane adds its own 32-bit byte offset, so advancing along K is one scalar
// add per stage and the per-lane offsets never change.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}


template <int MODE, int BM, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_bf16_kernel(GemmArgs p) {
  constexpr int FM = BM / WM / 16;
  constexpr int FN = BN / WN / 16;
  constexpr bool GATEUP = MODE == MODE_GATEUP;
  constexpr int BNH = GATEUP ? BN / 2 : BN;
  constexpr int A_STAGE = BM * A_ROWB;
  // LDS ring of NBUF stages.  A stage's slot is refilled as soon as its
  // fragments are in registers, so NBUF - 1 stages are always in flight; the
  // main loop is unrolled by the ring depth so that slot indices (and the
  // register double buffer's parity) are compile-time constants.  Fetches
  // that miss L2 take thousands of cycles under load: 128-row tiles, which
  // consume a stage every ~570 cycles, keep 5 in flight (6 x 24 KB); 256-row
  // tiles keep 4 (5 x 32 KB, the whole LDS); 64-row tiles keep 3 per
  // workgroup with two workgroups per CU (2 x 4 x 20 KB).
  constexpr int NBUF = BM == 128 ? 6 : BM == 256 ? 5 : 4;
  constexpr int NW = WM * WN;                 // waves per workgroup
  constexpr int NT = 64 * NW;                 // threads per workgroup
  constexpr int A_INS = A_STAGE / 1024 / NW;  // 1 KB DMA instructions per wave per stage (A)
  constexpr int B_INS = B_STAGE / 1024 / NW;  // (weights)
  constexpr int LOADS = A_INS + B_INS;        // VMEM instructions per wave per stage
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(!GATEUP || FN % 2 == 0, "gate/up fragment pairs");
  static_assert(A_INS >= 1 && B_INS >= 1 && A_INS * NW * 1024 == A_STAGE && B_INS * NW * 1024 == B_STAGE,
                "stage layout");

  __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * (A_STAGE + B_STAGE)];
  lds_u8* const As = (lds_u8*)(smem);
  lds_u8* const Bs = As + NBUF * A_STAGE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar registers
  const int wm = wave / WN, wn = wave % WN;
  const int E = p.E, T = p.T, K = p.K;

  // ---- tile lookup with an XCD-aware order.  Workgroup ids go round-robin
  // over the 8 XCDs (each with its own L2): XCD x = id % 8 takes the N-tiles
  // [x*gn/8, (x+1)*gn/8) for every M-tile, so each weight panel is fetched by
  // one XCD, and walks them M-major so the workgroups it runs together share
  // an A panel.  Ids beyond the real tile count exit.
  // a launch over the shared group alone addresses its tiles directly (it
  // does not read the routing tables, so it may run before routing ends)
  const bool shared_only = MODE == MODE_DOWN_SHARED || (GATEUP && p.group_lo == E);
  const int nmt = shared_only ? (T + BM - 1) / BM : p.tiles[p.group_hi] - p.tiles[p.group_lo];
  const int gn = p.n_tiles;
  const int lid = blockIdx.x;
  int mt_rel, nt;
  if (gn >= 8 && gn % 8 != 0 && gn % 4 == 0) {
    // N-tiles a multiple of 4 but not of 8 (the down GEMMs: d / 256 = 20):
    // 4 N-ranges x 2 M-halves, one rectangle per XCD, so every XCD gets the
    // same number of tiles and reads a quarter of the weight panels
    const int x = lid & 7, local = lid >> 3;
    const int w = gn >> 2, m_lo = ((x >> 2) * nmt) >> 1, m_hi = (((x >> 2) + 1) * nmt) >> 1;
    if (local >= (m_hi - m_lo) * w) return;
    mt_rel = m_lo + local / w;
    nt = (x & 3) * w + (local - (local / w) * w);
  } else if (gn >= 8) {
    const int x = lid & 7, local = lid >> 3;
    const int nt_lo = (x * gn) >> 3, w = (((x + 1) * gn) >> 3) - nt_lo;
    if (local >= nmt * w) return;
    if (w > 8 && w % 8 == 0) {
      // a wide range (d_ff = 16384: 16 N-tiles per XCD) is walked in blocks
      // of 8 N-tiles, so the workgroups running together cover ~4 M-tiles x 8
      // weight panels rather than 2 x 16 (fewer distinct panel slices per stage)
      const int blk = local / (nmt * 8), in = local - blk * (nmt * 8);
      mt_rel = in >> 3;
      nt = nt_lo + blk * 8 + (in & 7);
    } else {
      mt_rel = local / w;
      nt = nt_lo + (local - mt_rel * w);
    }
  } else {
    if (lid >= nmt * gn) return;
    mt_rel = lid / gn;
    nt = lid - mt_rel * gn;
  }
  int g, m0, rows;
  if (shared_only) {
    g = MODE == MODE_DOWN_SHARED ? 0 : E;
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
  // the shared group: its own launch (DOWN_SHARED), or group E of a gate/up
  // or routed down launch over groups .. E (the routed down then writes the
  // shared output in token order to C_shared, the routed rows to C; the
  // caller guarantees the same K, f == f_shared, for that launch)
  const bool shared = (MODE == MODE_DOWN_SHARED) || g == E;
  const int NH = (GATEUP && shared) ? p.N_shared : p.N;
  const int n0 = nt * BNH;
  if (n0 >= NH) return;
  if (!shared && !MOE_DCHECK_TILE(p, g, m0, rows)) return;   // debug builds: the tile is in its group
  const int row_base = shared ? 0 : p.offsets[g];
  const int ldb = GATEUP ? 2 * NH : NH;

  // Per-row metadata for the epilogue (the routed gate/up's gate scale, the
  // routed down's output row), one tile row per thread, loaded now so its
  // latency hides behind the main loop.
  float row_scale = 1.0f;
  int row_out = 0;
  if (tid < BM) {
    const int r = min(m0 + tid, rows - 1);
    if constexpr (GATEUP) {
      if (!shared) row_scale = p.gate[p.perm[row_base + r]];
    } else if constexpr (MODE == MODE_DOWN_ROUTED) {
      row_out = shared ? r : p.perm[row_base + r];
    }
  }

  // ---- DMA sources (byte offsets from the stage's scalar base).  A:
  // instruction i of this wave fills tile rows 16*(wave*A_INS + i) + lane/4;
  // the lane fetches the logical chunk that the swizzle places at its slot.
  // Rows past the group's end repeat its last row (their results are never
  // stored).  The caller guarantees T * K * 2 < 2^31.
  const uint8_t* a_src;
  if constexpr (GATEUP) a_src = reinterpret_cast<const uint8_t*>(shared ? p.A_shared : p.A);
  else a_src = reinterpret_cast<const uint8_t*>(shared ? p.A_shared : p.A);
  uint32_t a_voff[A_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int tr = 16 * (wave * A_INS + i) + (lane >> 2);        // tile row
    const int c = (lane & 3) ^ ((tr >> 1) & 3);                  // logical 16-byte chunk
    const int r = min(m0 + tr, rows - 1);
    int arow;
    if constexpr (GATEUP) arow = shared ? r : slot_token(p.perm[row_base + r], p.top_k);
    else if constexpr (MODE == MODE_DOWN_SHARED) arow = r;
    else arow = row_base + r;
    a_voff[i] = (static_cast<uint32_t>(arow) * static_cast<uint32_t>(K) + c * 8) * 2;
  }
  // weights: instruction i fills K rows 2*(wave*4 + i) + lane/32 of the stage;
  // the lane's slot is 16-byte chunk lane%32 of that row
  const uint8_t* b_src = reinterpret_cast<const uint8_t*>(shared ? p.B_shared : p.B) +
                         (shared ? 0 : static_cast<int64_t>(g) * K * ldb * 2);
  uint32_t b_voff[B_INS];
#pragma unroll
  for (int i = 0; i < B_INS; ++i) {
    const int kr = 2 * (wave * B_INS + i) + (lane >> 5);
    const int c = (lane & 31) ^ (2 * (kr & 3));
    const int lc = c * 8;                                        // tile column
    int gc;
    if constexpr (GATEUP) gc = lc < BNH ? n0 + lc : NH + n0 + (lc - BNH);
    else gc = n0 + lc;
    const bool ok = n0 + (GATEUP ? lc % BNH : lc) < NH;
    b_voff[i] = static_cast<uint32_t>(kr * ldb + (ok ? gc : 0)) * 2;  // clamped columns: valid, discarded
  }
  const int64_t a_kstep = static_cast<int64_t>(BK) * 2;         // bytes per stage along K
  const int64_t b_kstep = static_cast<int64_t>(BK) * ldb * 2;
  const int nk = K / BK;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- LDS read addresses: per-lane bases; slot and fragment offsets are
  // compile-time immediates of the ds_read instructions.
  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(As));
  const int lrow = lane & 15;
  const int kg = lane >> 4;         // this lane's 8-wide K group inside the stage
  // A fragment i of slot sl: row wm*(BM/WM) + 16 i + lrow, logical chunk kg at
  // a_rd + sl*A_STAGE + i*16*A_ROWB ((row >> 1) & 3 == (lrow >> 1) & 3)
  const uint32_t a_rd = ring + (wm * (BM / WM) + lrow) * A_ROWB + ((kg ^ ((lrow >> 1) & 3)) << 4);
  // weight fragment j of slot sl (16 columns x K rows 8kg..8kg+7): two
  // transpose reads at b_rd[j] + sl*B_STAGE and 4 rows further.  Lane s of
  // each 16-lane group points at row 8kg + s/4, bytes [2*(col + 4*(s%4)), +8)
  // of the logical row, mapped through the swizzle.
  // Fragments j and j + 4 are 64 (gate/up: 128) columns apart, a multiple of
  // the swizzle period, so four base registers serve all of them.
  constexpr int NBR = FN < 4 ? FN : 4;
  constexpr int B_JSTEP = GATEUP ? BNH * 2 * 4 / (FN / 2) : 64 * 2;   // bytes from fragment j to j + 4
  uint32_t b_rd[NBR];
#pragma unroll
  for (int j = 0; j < NBR; ++j) {
    int col;
    if constexpr (GATEUP) col = (j < FN / 2 ? 0 : BNH) + wn * (BNH / WN) + (j % (FN / 2)) * 16;
    else col = wn * (BN / WN) + j * 16;
    const int s4 = lane & 15;
    const int lbyte = (col + 4 * (s4 & 3)) * 2;
    const int r = kg * 8 + (s4 >> 2);                            // (r & 3) == (s4 >> 2) & 3
    const int pbyte = ((lbyte >> 4) ^ (2 * (r & 3))) * 16 + (lbyte & 15);
    b_rd[j] = ring + NBUF * A_STAGE + r * B_ROWB + pbyte;
  }
  typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
#define MOE_AREAD(FA, i, SL)                                                                   \
  FA[i] = *(const lds_bf16x8*)((const lds_u8*)(uintptr_t)a_rd + (SL) * A_STAGE + (i) * 16 * A_ROWB)
#define MOE_BREAD(FB, j, SL)                                                                   \
  do {                                                                                         \
    const lds_u8* q_ = (const lds_u8*)(uintptr_t)b_rd[(j) % NBR] + (SL) * B_STAGE + ((j) / NBR) * B_JSTEP; \
    const s16x4 lo_ = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(q_));               \
    const s16x4 hi_ = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(q_ + 4 * B_ROWB));  \
    typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8_;                  \
    const s16x8_ v_ = {lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};       \
    FB[j] = __builtin_bit_cast(bf16x8, v_);                                                    \
  } while (0)

  // wave-uniform LDS byte addresses of this wave's first DMA slot (A / weights)
  const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t a_lds0 = ring + wave_u * (A_INS * 1024);
  const uint32_t b_lds0 = ring + NBUF * A_STAGE + wave_u * (B_INS * 1024);
#define MOE_DMA_A(i, st, SL)                                                                   \
  dma16(a_src + static_cast<int64_t>(min((st), nk - 1)) * a_kstep, a_voff[i], a_lds0 + (SL) * A_STAGE + (i) * 1024)
#define MOE_DMA_B(i, st, SL)                                                                   \
  dma16(b_src + static_cast<int64_t>(min((st), nk - 1)) * b_kstep, b_voff[i], b_lds0 + (SL) * B_STAGE + (i) * 1024)

  // Operands in registers: all of a stage's fragments (FM A + FN weight
  // fragments, 4 VGPRs each) are double-buffered.
  bf16x8 fa0[FM], fa1[FM], fb0[FN], fb1[FN];
  constexpr int NMF = FM * FN;                       // MFMAs per stage
  constexpr int NOPS = FM + FN + A_INS + B_INS;      // other operations per stage

  // One stage (step kt + R, operands FA/FB in registers, its slot R % NBUF free):
  // the MFMA stream starts right after the previous barrier, and the stage's
  // other work is threaded through it in a fixed order -- first the reads of
  // stage kt+SL+1's fragments into FA2/FB2 (they must land before the stage
  // ends), then the DMA of stage kt+SL+NBUF into slot SL.  The end waits for
  // stage kt+SL+2 (this wave's part; later stages may be in flight) and for
  // the reads, and the barrier publishes that stage and frees slot SL+1.
#define MOE_STEP(R, FA, FB, FA2, FB2)                                                          \
  do {                                                                                         \
    constexpr int sl_ = (R) % NBUF, nsl_ = ((R) + 1) % NBUF;                                   \
    const int sd_ = kt + (R) + NBUF;                                                           \
    _Pragma("unroll") for (int m_ = 0; m_ < NMF; ++m_) {                                       \
      acc[m_ / FN][m_ % FN] =                                                                  \
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(FA[m_ / FN], FB[m_ % FN], acc[m_ / FN][m_ % FN], 0, 0, 0); \
      _Pragma("unroll") for (int o_ = 0; o_ < NOPS; ++o_) {                                    \
        if (o_ * NMF / NOPS == m_) {                                                           \
          if (o_ < FM) MOE_AREAD(FA2, o_, nsl_);                                               \
          else if (o_ < FM + FN) MOE_BREAD(FB2, o_ - FM, nsl_);                                \
          else if (o_ < FM + FN + A_INS) MOE_DMA_A(o_ - FM - FN, sd_, sl_);                    \
          else MOE_DMA_B(o_ - FM - FN - A_INS, sd_, sl_);                                      \
        }                                                                                      \
      }                                                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                       \
    }                                                                                          \
    wait_vmcnt<(NBUF - 2) * LOADS>();                                                          \
    __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) */                                       \
    __builtin_amdgcn_s_barrier();                                                              \
  } while (0)

  // prologue: stages 0 .. NBUF-1 in flight; stages 0 and 1 landed and
  // published; stage 0's fragments in registers and its slot released.
#pragma unroll
  for (int st = 0; st < NBUF; ++st) {
#pragma unroll
    for (int i = 0; i < A_INS; ++i) MOE_DMA_A(i, st, st);
#pragma unroll
    for (int i = 0; i < B_INS; ++i) MOE_DMA_B(i, st, st);
  }
  wait_vmcnt<(NBUF - 2) * LOADS>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < FM; ++i) MOE_AREAD(fa0, i, 0);
#pragma unroll
  for (int j = 0; j < FN; ++j) MOE_BREAD(fb0, j, 0);
  __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) */
  __builtin_amdgcn_s_barrier();
  // Unrolled by U = lcm(NBUF, 2) so that ring slots and the register
  // buffers' parity are compile-time; the tail runs the first steps of one
  // more group.
  constexpr int U = NBUF % 2 == 0 ? NBUF : 2 * NBUF;
  static_assert(U <= 10, "unrolled steps below");
#define MOE_STEPR(R)                                                                           \
  do {                                                                                         \
    if constexpr ((R) < U) {                                                                   \
      if constexpr ((R) % 2 == 0) MOE_STEP((R), fa0, fb0, fa1, fb1);                           \
      else MOE_STEP((R), fa1, fb1, fa0, fb0);                                                  \
    }                                                                                          \
  } while (0)
  int kt = 0;
  for (; kt + U <= nk; kt += U) {
    // 256-row tiles keep their accumulators in AGPRs: pinning them there at
    // each iteration keeps the register allocator from moving them between
    // AGPRs and VGPRs across iterations (hundreds of v_accvgpr copies otherwise)
    if constexpr (BM == 256) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
    }
    MOE_STEPR(0); MOE_STEPR(1); MOE_STEPR(2); MOE_STEPR(3); MOE_STEPR(4);
    MOE_STEPR(5); MOE_STEPR(6); MOE_STEPR(7); MOE_STEPR(8); MOE_STEPR(9);
  }
  const int left = nk - kt;   // 0 .. U-1
  if (left > 0) { MOE_STEPR(0);
  if (left > 1) { MOE_STEPR(1);
  if (left > 2) { MOE_STEPR(2);
  if (left > 3) { MOE_STEPR(3);
  if (left > 4) { MOE_STEPR(4);
  if (left > 5) { MOE_STEPR(5);
  if (left > 6) { MOE_STEPR(6);
  if (left > 7) { MOE_STEPR(7);
  if (left > 8) { MOE_STEPR(8); } } } } } } } } }
#undef MOE_STEPR
  wait_vmcnt<0>();
#undef MOE_AREAD
#undef MOE_BREAD
#undef MOE_DMA_A
#undef MOE_DMA_B
#undef MOE_STEP

  // ---- epilogue (16x16 accumulator: lane holds rows 4*(lane/16)+q of column
  // lane%16).  The tile goes through LDS (the ring is free once every wave's
  // DMA has landed) so that global memory sees 16-byte row chunks instead of
  // 2- or 4-byte scattered stores; the per-row metadata comes through LDS too.
  // No global load sits between two stores through C (the compiler must
  // assume they may alias, so such a load would wait a full round trip): the
  // shared expert's output is loaded for 16 chunks at a time before they are
  // stored.
  __syncthreads();
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
  typedef __attribute__((address_space(3))) float lds_f32;
  typedef __attribute__((address_space(3))) int lds_i32;
  typedef __attribute__((address_space(3))) uint16_t lds_u16;
  if (tid < BM) {
    if constexpr (GATEUP) reinterpret_cast<lds_f32*>(As)[tid] = row_scale;
    else reinterpret_cast<lds_i32*>(As)[tid] = row_out;
  }
  __syncthreads();
  lds_u8* const stage = As + 1024;        // staging area after the row table (BM * 4 <= 1 KB)
  const int lcol = lane & 15;
  const int rq = 4 * (lane >> 4);
  const int wrow = wm * (BM / WM) + rq;   // tile row of fragment 0, q = 0
  if constexpr (GATEUP && BM == 256) {
    // 256-row tiles store straight from the accumulators: the staged
    // version below upsets their register allocation (accumulator copies in
    // the main loop)
    constexpr int HF = FN / 2;
    void* C = shared ? p.C_shared : p.C;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const f32x4 sc = *(const lds_f32x4*)(As + 4 * (wrow + 16 * i));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = m0 + wrow + i * 16 + q;
        if (r >= rows) continue;
        const int orow = row_base + r;
#pragma unroll
        for (int j = 0; j < HF; ++j) {
          const int col = n0 + wn * (BNH / WN) + j * 16 + lcol;
          if (col >= NH) continue;
          const float gv = acc[i][j][q] * sc[q];
          const float uv = acc[i][j + HF][q] * sc[q];
          reinterpret_cast<uint16_t*>(C)[static_cast<int64_t>(orow) * NH + col] = f32_to_bf16(silu_f(gv) * uv);
        }
      }
    }
  } else if constexpr (GATEUP) {
    // h tile [BM][BNH] bf16, row pitch HP bytes
    constexpr int HF = FN / 2;
    constexpr int HP = BNH * 2 + 16;
    static_assert(1024 + BM * HP <= NBUF * (A_STAGE + B_STAGE), "h staging fits the ring");
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const f32x4 sc = *(const lds_f32x4*)(As + 4 * (wrow + 16 * i));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rt = wrow + i * 16 + q;
#pragma unroll
        for (int j = 0; j < HF; ++j) {
          const int ct = wn * (BNH / WN) + j * 16 + lcol;
          const float gv = acc[i][j][q] * sc[q];
          const float uv = acc[i][j + HF][q] * sc[q];
          *(lds_u16*)(stage + rt * HP + ct * 2) = f32_to_bf16(silu_f(gv) * uv);
        }
      }
    }
    __syncthreads();
    constexpr int CPR = BNH / 8;          // 16-byte chunks per row
    uint16_t* C = reinterpret_cast<uint16_t*>(shared ? p.C_shared : p.C);
    for (int k = tid; k < BM * CPR; k += NT) {
      const int r = k / CPR, cc = k - r * CPR;
      const int col = n0 + cc * 8;
      if (m0 + r < rows && col < NH)      // NH % 8 == 0: a chunk is wholly in or out
        *reinterpret_cast<i32x4*>(C + static_cast<int64_t>(row_base + m0 + r) * NH + col) =
            *(const lds_i32x4*)(stage + r * HP + cc * 16);
    }
  } else {
    // fp32 tile in passes of PR rows, [PR][BN] with row pitch FPB bytes
    constexpr int FPB = BN * 4 + 16;
    constexpr int PR = (1024 + 128 * FPB <= NBUF * (A_STAGE + B_STAGE) && BM >= 128) ? 128 : 64;
    static_assert(1024 + PR * FPB <= NBUF * (A_STAGE + B_STAGE), "fp32 staging fits the ring");
    constexpr int CPR = BN / 4;           // 16-byte chunks per row
    constexpr int NB = 16;                // chunks per thread per batch
    static_assert((PR * CPR) % (NT * NB) == 0, "whole batches per pass");
#pragma unroll
    for (int pass = 0; pass < BM / PR; ++pass) {
      if (pass > 0) __syncthreads();      // the previous pass's chunks are read
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int rt0 = wm * (BM / WM) + i * 16;          // first tile row of fragment i (uniform)
        if (rt0 / PR != pass) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rp = rt0 + rq + q - pass * PR;
#pragma unroll
          for (int j = 0; j < FN; ++j)
            *(lds_f32*)(stage + rp * FPB + (wn * (BN / WN) + j * 16 + lcol) * 4) = acc[i][j][q];
        }
      }
      __syncthreads();
      for (int k0 = tid; k0 < PR * CPR; k0 += NT * NB) {
        f32x4 y[NB];
        int orow[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int k = k0 + u * NT;
          const int r = k / CPR, cc = k - r * CPR;
          const int rt = pass * PR + r;
          if constexpr (MODE == MODE_DOWN_ROUTED) orow[u] = reinterpret_cast<const lds_i32*>(As)[rt];
          else orow[u] = m0 + rt;
          const bool ok = m0 + rt < rows && n0 + cc * 4 < NH;
          y[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (MODE == MODE_DOWN_ROUTED)
            if (ok && p.Y && !shared)
              y[u] = *reinterpret_cast<const f32x4*>(p.Y + static_cast<int64_t>(orow[u]) * NH + n0 + cc * 4);
        }
        // the batch's loads have landed before its first store: the stores
        // are conditional, and a wait the compiler placed after one of them
        // would also wait for the stores before it (one round trip each)
        wait_vmcnt<0>();
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int k = k0 + u * NT;
          const int r = k / CPR, cc = k - r * CPR;
          const int rt = pass * PR + r;
          if (m0 + rt >= rows || n0 + cc * 4 >= NH) continue;
          // routed rows without a shared output (Y null) are stored as summed
          const f32x4 acc4 = *(const lds_f32x4*)(stage + r * FPB + cc * 16);
          const f32x4 v = (MODE == MODE_DOWN_ROUTED && (!p.Y || shared)) ? acc4 : acc4 + y[u];
          const int64_t o = static_cast<int64_t>(orow[u]) * NH + n0 + cc * 4;
          if (shared) {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C_shared) + o) = v;
          } else if (p.out_bf16) {
            const uint32_t lo = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
            const uint32_t hi = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.C) + o) = make_uint2(lo, hi);
          } else {
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C) + o) = v;
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
    // sum over routed groups of ceil(n_g / BM) <= ceil(T k / BM) + E (T k routed rows); the shared
    // group adds ceil(T / BM)
    const int Tr = T * (a.top_k > 1 ? a.top_k : 1);
    gm = (has_routed ? (Tr + BM - 1) / BM + a.E : 0) + (has_shared ? (T + BM - 1) / BM : 0);
    nmax = a.N;
    if (MODE == MODE_GATEUP) nmax = max(has_routed ? a.N : 0, has_shared ? a.N_shared : 0);
  }
  if (gm <= 0) return hipSuccess;
  // a routed down launch that includes the shared group reads h_s and the
  // shared weights with the routed K: the caller passes the shared K in
  // N_shared, and it must match
  if (MODE == MODE_DOWN_ROUTED && has_shared && a.N_shared != a.K) return hipErrorInvalidValue;
  const int gn = (nmax + BNH - 1) / BNH;
  a.n_tiles = gn;
  // 1-D grid: enough ids for the largest per-XCD share of (M-tile bound x N-tiles)
  const int64_t nblk = (gn >= 8 && gn % 8 != 0 && gn % 4 == 0) ? 8 * static_cast<int64_t>((gm + 1) / 2) * (gn / 4)
                       : gn >= 8 ? 8 * static_cast<int64_t>(gm) * ((gn + 7) / 8)
                                 : static_cast<int64_t>(gm) * gn;
  hipLaunchKernelGGL((gemm_bf16_kernel<MODE, BM, WM, WN>), dim3(static_cast<unsigned>(nblk)), dim3(64 * WM * WN), 0, s,
                     a);
  return hipGetLastError();
}

}  // namespace

}  // namespace moe
