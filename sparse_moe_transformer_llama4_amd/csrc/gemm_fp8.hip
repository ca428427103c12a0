// fp8 (OCP e4m3fn) grouped GEMMs for prefill-sized token counts (gfx950).
//
// The same three launches as the bf16 kernels, on e4m3 codes with fp32
// scales: the gate/up GEMM multiplies per-token-quantised x by per-column-
// quantised W_gate_up and applies (gate x token scale x column scale) to the
// fp32 accumulator before the SwiGLU epilogue; the down GEMMs multiply the
// per-row-quantised h by per-column-quantised W_down.  MFMA:
// v_mfma_scale_f32_16x16x128_f8f6f4 (unit block scales), 32 K bytes per lane.
//   * workgroup tile 128 x 256 (gate/up: 128 gate + 128 up columns), 4 waves
//     of 64 x 128 accumulators; one pipeline stage = K 128 (one MFMA step);
//   * direct-to-LDS loads (scalar-base form) into a 3-deep ring of 48 KB
//     stages; a slot is refilled as soon as its stage's fragments are in
//     registers, so two stages are always in flight;
//   * A rows (128 B) are stored with 16-byte chunk k of row r at
//     k ^ a_swz(r & 15), a permutation found by measuring LDS read rates: the
//     fragment reads (16 rows x 16 B per 16-lane group) run at the full
//     ds_read_b128 rate, where k ^ ((r >> 1) & 7) or k ^ (r & 7) run at half;
//   * weight rows (256 B) are stored with 16-byte chunk c of row r at
//     c ^ (r & 7) ^ (8 * ((r >> 5) & 1)) (the last term keeps the two 16-lane
//     groups that one transpose read serves together, 32 rows apart, on
//     different banks; without it the reads run at 60 % of the rate) and read
//     with the gfx950 byte transpose read
//     (ds_read_b64_tr_b8): each 16-lane group reads 8 K rows x 16 columns and
//     every lane receives its column's 8 K bytes; four reads give the 32 K
//     bytes of the MFMA operand;
//   * XCD-aware tile order, one explicit vmcnt wait + s_barrier per stage,
//     and the MFMA stream with the next stage's LDS reads and the DMA
//     threaded through it, as in the bf16 kernels.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr int BN = 256, WM = 2, WN = 2;
constexpr int BK = 128;                  // K bytes per stage = one MFMA step
constexpr int NBUF = 3;
constexpr int A_ROWB = BK;               // 128 B per A row
constexpr int B_ROWB = BN;               // 256 B per weight row
constexpr int B_STAGE = BK * B_ROWB;     // 32 KB
constexpr int B_INS = B_STAGE / 1024 / 4;
constexpr int FN = BN / WN / 16;         // 8

// Chunk permutation of an A row (see the header comment): XOR of 5, 7 and 1
// selected by bits 0, 1 and 3 of the row.
__device__ __forceinline__ int a_swz(int r) {
  return ((r & 1) ? 5 : 0) ^ ((r & 2) ? 7 : 0) ^ ((r & 8) ? 1 : 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// Direct-to-LDS 16-byte load into m0 + 16 * lane (inline asm: it writes no
// VGPR; the stage ring orders it with explicit vmcnt waits and barriers).
// Scalar-base form: `sbase` is wave-uniform and each lane adds its own 32-bit
// byte offset, so advancing along K is one scalar add per stage.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// Maximum of v over the 16 lanes of its DPP row (lanes 16 r .. 16 r + 15),
// returned in every lane of the row: lane pairs, quad pairs, the two quads of
// each half, the two halves (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror; every source lane is in the row).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)));
  return v;
}


// Four fp32 h values in the 24-bit form the quantisation pass reads: each
// value's bit pattern rounded at bit 8 (half a unit added to the magnitude,
// the low 8 bits then dropped), bits 31..16 (four uint16, in order) to `hi`,
// bits 15..8 (four bytes) to `lo`.
__device__ __forceinline__ void store_h24(uint16_t* hi, uint8_t* lo, f32x4 v) {
  const uint32_t b0 = __float_as_uint(v[0]) + 0x80u, b1 = __float_as_uint(v[1]) + 0x80u,
                 b2 = __float_as_uint(v[2]) + 0x80u, b3 = __float_as_uint(v[3]) + 0x80u;
  *reinterpret_cast<uint2*>(hi) = make_uint2(__builtin_amdgcn_perm(b1, b0, 0x07060302u),
                                             __builtin_amdgcn_perm(b3, b2, 0x07060302u));
  *reinterpret_cast<uint32_t*>(lo) =
      __builtin_amdgcn_perm(__builtin_amdgcn_perm(b3, b2, 0x00000501u), __builtin_amdgcn_perm(b1, b0, 0x00000501u),
                            0x05040100u);
}

// BM = 128 or 160 rows (the 160-row gate/up tile takes a group of up to 160
// rows whole where 128-row tiles would add a second, nearly empty tile)
template <int MODE, int BM>
__global__ __launch_bounds__(256, 1) void gemm_fp8_kernel(GemmArgs p) {
  constexpr bool GATEUP = MODE == MODE_GATEUP;
  constexpr int BNH = GATEUP ? BN / 2 : BN;
  constexpr int A_STAGE = BM * A_ROWB;   // 16 / 20 KB
  constexpr int A_INS = A_STAGE / 1024 / 4;
  constexpr int LOADS = A_INS + B_INS;
  constexpr int FM = BM / WM / 16;       // 4 / 5
  static_assert((BM == 128 || BM == 160) && A_INS * 4 * 1024 == A_STAGE, "tile rows");
  static_assert(NBUF * (A_STAGE + B_STAGE) <= 160 * 1024, "ring fits the LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NBUF * (A_STAGE + B_STAGE)];
  lds_u8* const As = (lds_u8*)(smem);
  lds_u8* const Bs = As + NBUF * A_STAGE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar registers
  const int wm = wave / WN, wn = wave % WN;
  const int E = p.E, T = p.T, K = p.K;

  // ---- XCD-aware tile lookup (as in the bf16 kernels)
  const int nmt = (MODE == MODE_DOWN_SHARED) ? (T + BM - 1) / BM : p.tiles[p.group_hi] - p.tiles[p.group_lo];
  const int gn = p.n_tiles;
  const int lid = blockIdx.x;
  int mt_rel, nt;
  if (gn >= 8 && gn % 8 != 0 && gn % 4 == 0) {
    // N-tiles a multiple of 4 but not of 8 (the down GEMMs: d / 256 = 20):
    // 4 N-ranges x 2 M-halves, one rectangle per XCD (as in the bf16 kernels)
    const int x = lid & 7, local = lid >> 3;
    const int w = gn >> 2, m_lo = ((x >> 2) * nmt) >> 1, m_hi = (((x >> 2) + 1) * nmt) >> 1;
    if (local >= (m_hi - m_lo) * w) return;
    mt_rel = m_lo + local / w;
    nt = (x & 3) * w + (local - (local / w) * w);
  } else if (gn >= 8) {
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
  if (!shared && !MOE_DCHECK_TILE(p, g, m0, rows)) return;   // debug builds: the tile is in its group
  const int row_base = shared ? 0 : p.offsets[g];
  const int ldb = GATEUP ? 2 * NH : NH;   // weight row length in bytes

  // Per-row metadata for the epilogue, one tile row per thread, loaded now so
  // its latency hides behind the main loop: the row's scale (gate/up: the
  // routing gate times the token's activation scale; down: the scale of h)
  // and, for the routed down, the token the row belongs to.
  float row_scale = 1.0f;
  int row_out = 0;
  if (tid < BM) {
    const int r = min(m0 + tid, rows - 1);
    if constexpr (GATEUP) {
      const int slot = shared ? r : p.perm[row_base + r];
      row_scale = (shared ? 1.0f : p.gate[slot]) * (shared ? p.sA_shared : p.sA)[shared ? slot : slot_token(slot, p.top_k)];
    } else if constexpr (MODE == MODE_DOWN_SHARED) {
      row_scale = p.sA_shared[r];
    } else {
      row_scale = p.sA[row_base + r];
      row_out = p.perm[row_base + r];
    }
  }

  // ---- DMA sources.  A: instruction i fills tile rows 8*(wave*A_INS + i) + lane/8,
  // the lane fetching the logical chunk its slot holds under the swizzle.
  const uint8_t* a_src;
  if constexpr (GATEUP) a_src = reinterpret_cast<const uint8_t*>(shared ? p.A_shared : p.A);
  else if constexpr (MODE == MODE_DOWN_SHARED) a_src = reinterpret_cast<const uint8_t*>(p.A_shared);
  else a_src = reinterpret_cast<const uint8_t*>(p.A);
  uint32_t a_voff[A_INS];   // byte offsets (the caller guarantees T * K < 2^31)
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int tr = 8 * (wave * A_INS + i) + (lane >> 3);
    const int c = (lane & 7) ^ a_swz(tr & 15);
    const int r = min(m0 + tr, rows - 1);
    int arow;
    if constexpr (GATEUP) arow = shared ? r : slot_token(p.perm[row_base + r], p.top_k);
    else if constexpr (MODE == MODE_DOWN_SHARED) arow = r;
    else arow = row_base + r;
    a_voff[i] = static_cast<uint32_t>(arow) * static_cast<uint32_t>(K) + c * 16;
  }
  // weights: instruction i fills K rows 4*(wave*B_INS + i) + lane/16; slot = chunk lane%16
  const uint8_t* b_src = reinterpret_cast<const uint8_t*>(shared ? p.B_shared : p.B) +
                         (shared ? 0 : static_cast<int64_t>(g) * K * ldb);
  uint32_t b_voff[B_INS];
#pragma unroll
  for (int i = 0; i < B_INS; ++i) {
    const int kr = 4 * (wave * B_INS + i) + (lane >> 4);
    const int c = (lane & 15) ^ (kr & 7) ^ (((kr >> 5) & 1) << 3);
    const int lc = c * 16;
    int gc;
    if constexpr (GATEUP) gc = lc < BNH ? n0 + lc : NH + n0 + (lc - BNH);
    else gc = n0 + lc;
    const bool ok = n0 + (GATEUP ? lc % BNH : lc) < NH;
    b_voff[i] = static_cast<uint32_t>(kr * ldb + (ok ? gc : 0));   // clamped columns are never stored
  }
  const int64_t b_kstep = static_cast<int64_t>(BK) * ldb;
  const int nk = K / BK;

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- LDS read addresses: per-lane bases, slot and fragment offsets as
  // immediates.
  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(As));
  const int lrow = lane & 15, kg = lane >> 4;
  // A fragment i of slot sl: row wm*64 + 16 i + lrow, logical chunks 2 kg and
  // 2 kg + 1 (row & 15 == lrow) at a_rd0/1 + sl*A_STAGE + i*16*A_ROWB
  const uint32_t a_rd0 = ring + (wm * (BM / WM) + lrow) * A_ROWB + (((2 * kg) ^ a_swz(lrow)) << 4);
  const uint32_t a_rd1 = ring + (wm * (BM / WM) + lrow) * A_ROWB + (((2 * kg + 1) ^ a_swz(lrow)) << 4);
  // weight fragment j of slot sl (32 K bytes of one column per lane): four
  // byte-transpose reads at b_rd[j] + sl*B_STAGE + 8 q rows.  Lane s of
  // 16-lane group g points at row 32 g + s/2 (+ 8 q), 8 bytes of the 16-byte
  // chunk holding its column block; rows of one read share (row & 7) = s/2
  // and (row >> 5) & 1 = g & 1.
  uint32_t b_rd[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int col;
    if constexpr (GATEUP) col = (j < FN / 2 ? 0 : BNH) + wn * (BNH / WN) + (j % (FN / 2)) * 16;
    else col = wn * (BN / WN) + j * 16;
    const int s = lane & 15, g = lane >> 4;
    const int pchunk = (col >> 4) ^ ((s >> 1) & 7) ^ ((g & 1) << 3);
    b_rd[j] = ring + NBUF * A_STAGE + (32 * g + (s >> 1)) * B_ROWB + pchunk * 16 + 8 * (s & 1);
  }
  typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
#define F8_AREAD(FA, i, SL)                                                                    \
  do {                                                                                         \
    const i32x4 lo_ = *(const lds_i32x4*)((const lds_u8*)(uintptr_t)a_rd0 + (SL) * A_STAGE + (i) * 16 * A_ROWB); \
    const i32x4 hi_ = *(const lds_i32x4*)((const lds_u8*)(uintptr_t)a_rd1 + (SL) * A_STAGE + (i) * 16 * A_ROWB); \
    FA[i] = i32x8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};             \
  } while (0)
#define F8_BREAD(FB, j, SL)                                                                    \
  do {                                                                                         \
    const lds_u8* q_ = (const lds_u8*)(uintptr_t)b_rd[j] + (SL) * B_STAGE;                     \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                            \
      const i32x2 v_ = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(q_ + 8 * q * B_ROWB)); \
      FB[j][2 * q] = v_[0];                                                                    \
      FB[j][2 * q + 1] = v_[1];                                                                \
    }                                                                                          \
  } while (0)
  const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t a_lds0 = ring + wave_u * (A_INS * 1024);
  const uint32_t b_lds0 = ring + NBUF * A_STAGE + wave_u * (B_INS * 1024);
#define F8_DMA_A(i, st, SL)                                                                    \
  dma16(a_src + static_cast<int64_t>(min((st), nk - 1)) * BK, a_voff[i], a_lds0 + (SL) * A_STAGE + (i) * 1024)
#define F8_DMA_B(i, st, SL)                                                                    \
  dma16(b_src + static_cast<int64_t>(min((st), nk - 1)) * b_kstep, b_voff[i], b_lds0 + (SL) * B_STAGE + (i) * 1024)

  // Operands in registers: all of a stage's fragments double-buffered; the
  // 160-row tile (ASB) keeps one set of A fragments, each refilled with the
  // next stage's fragment right after its last MFMA of the stage (the
  // registers of a second set would not fit beside its 160 accumulators).
  constexpr bool ASB = BM == 160;
  i32x8 fa0[FM], fa1[FM], fb0[FN], fb1[FN];
  i32x8 (&fa_odd)[FM] = ASB ? fa0 : fa1;
  constexpr int NMF = FM * FN;
  constexpr int NOPS = (ASB ? 0 : FM) + FN + A_INS + B_INS;   // spread through the MFMA stream
  // One stage (step kt + R, slot R % NBUF free, operands FA/FB): the MFMA
  // stream starts right after the previous barrier; the reads of the next
  // stage's fragments and then the DMA of stage kt + R + NBUF into the free
  // slot are threaded through it; the end waits for stage kt + R + 2 and the
  // reads, and the barrier publishes that stage and frees the next slot.
#define F8_STEP(R, FA, FB, FA2, FB2)                                                           \
  do {                                                                                         \
    constexpr int sl_ = (R) % NBUF, nsl_ = ((R) + 1) % NBUF;                                   \
    const int sd_ = kt + (R) + NBUF;                                                           \
    _Pragma("unroll") for (int m_ = 0; m_ < NMF; ++m_) {                                       \
      acc[m_ / FN][m_ % FN] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(               \
          FA[m_ / FN], FB[m_ % FN], acc[m_ / FN][m_ % FN], 0, 0, 0, 127, 0, 127);              \
      if constexpr (ASB)                                                                       \
        if (m_ % FN == FN - 1) F8_AREAD(FA, m_ / FN, nsl_);                                    \
      _Pragma("unroll") for (int o_ = 0; o_ < NOPS; ++o_) {                                    \
        if (o_ * NMF / NOPS == m_) {                                                           \
          const int u_ = o_ + (ASB ? FM : 0);                                                  \
          if (u_ < FM) F8_AREAD(FA2, u_, nsl_);                                                \
          else if (u_ < FM + FN) F8_BREAD(FB2, u_ - FM, nsl_);                                 \
          else if (u_ < FM + FN + A_INS) F8_DMA_A(u_ - FM - FN, sd_, sl_);                     \
          else F8_DMA_B(u_ - FM - FN - A_INS, sd_, sl_);                                       \
        }                                                                                      \
      }                                                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                       \
    }                                                                                          \
    wait_vmcnt<(NBUF - 2) * LOADS>();                                                          \
    __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) */                                       \
    __builtin_amdgcn_s_barrier();                                                              \
  } while (0)

  // prologue: stages 0 .. NBUF-1 in flight; 0 and 1 landed and published;
  // stage 0's fragments in registers and its slot released
#pragma unroll
  for (int st = 0; st < NBUF; ++st) {
#pragma unroll
    for (int i = 0; i < A_INS; ++i) F8_DMA_A(i, st, st);
#pragma unroll
    for (int i = 0; i < B_INS; ++i) F8_DMA_B(i, st, st);
  }
  wait_vmcnt<(NBUF - 2) * LOADS>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < FM; ++i) F8_AREAD(fa0, i, 0);
#pragma unroll
  for (int j = 0; j < FN; ++j) F8_BREAD(fb0, j, 0);
  __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) */
  __builtin_amdgcn_s_barrier();
  // unrolled by 6 = ring depth x register parity: slots and buffers are
  // compile-time; the accumulators are pinned to AGPRs at each iteration
  // (otherwise the register allocator rotates them with v_accvgpr copies)
  static_assert(NBUF == 3, "the loop below is unrolled by 2 x the ring depth");
  int kt = 0;
  for (; kt + 6 <= nk; kt += 6) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
    F8_STEP(0, fa0, fb0, fa_odd, fb1);
    F8_STEP(1, fa_odd, fb1, fa0, fb0);
    F8_STEP(2, fa0, fb0, fa_odd, fb1);
    F8_STEP(3, fa_odd, fb1, fa0, fb0);
    F8_STEP(4, fa0, fb0, fa_odd, fb1);
    F8_STEP(5, fa_odd, fb1, fa0, fb0);
  }
  if (kt < nk) {
    F8_STEP(0, fa0, fb0, fa_odd, fb1);
    if (kt + 1 < nk) {
      F8_STEP(1, fa_odd, fb1, fa0, fb0);
      if (kt + 2 < nk) {
        F8_STEP(2, fa0, fb0, fa_odd, fb1);
        if (kt + 3 < nk) {
          F8_STEP(3, fa_odd, fb1, fa0, fb0);
          if (kt + 4 < nk) F8_STEP(4, fa0, fb0, fa_odd, fb1);
        }
      }
    }
  }
  wait_vmcnt<0>();
#undef F8_AREAD
#undef F8_BREAD
#undef F8_DMA_A
#undef F8_DMA_B
#undef F8_STEP

  // ---- epilogue (16x16 accumulator: lane holds rows 4*(lane/16)+q of column
  // lane%16).  No global load sits between two stores through C (the compiler
  // must assume they may alias, so each would wait a full round trip): the
  // column scales are loaded first and the row metadata comes through LDS
  // (the ring is free once every wave's DMA has landed).
  const int lcol = lane & 15;
  const int rq = 4 * (lane >> 4);
  const int wrow = wm * (BM / WM) + rq;   // tile row of fragment 0, q = 0
  constexpr int BNW = BNH / WN;           // output columns per wave
  float csc[FN];                          // column scales of this lane's fragments
  {
    const float* sB = GATEUP ? (shared ? p.sB_shared : p.sB + static_cast<int64_t>(g) * 2 * NH)
                             : (MODE == MODE_DOWN_ROUTED ? p.sB + static_cast<int64_t>(g) * NH : p.sB_shared);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int jj = GATEUP ? j % (FN / 2) : j;
      const int col = n0 + wn * BNW + jj * 16 + lcol;
      csc[j] = col < NH ? sB[(GATEUP && j >= FN / 2 ? NH : 0) + col] : 0.0f;
    }
  }
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
  __syncthreads();
  if (tid < BM) {
    reinterpret_cast<__attribute__((address_space(3))) float*>(As)[tid] = row_scale;
    reinterpret_cast<__attribute__((address_space(3))) int*>(As)[BM + tid] = row_out;
    reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(As)[2 * BM + tid] = 0u;
  }
  __syncthreads();
  // The tile goes through LDS (after the row tables) so that global memory
  // sees 16-byte row chunks instead of scattered 4-byte stores.
  typedef __attribute__((address_space(3))) float lds_f32;
  typedef __attribute__((address_space(3))) int lds_i32;
  constexpr int TABB = (12 * BM + 1023) / 1024 * 1024;  // three row tables, rounded to 1 KB
  lds_u8* const stage = As + TABB;
  if constexpr (GATEUP) {
    // h tile [BM][BNH] fp32 (row pitch HP bytes) and each row's max |h|: over
    // this lane's HF columns, then over the 16 lanes of the row (DPP), then
    // over the two waves of the row (LDS atomic max on the bit patterns of
    // non-negative floats); then rows to global memory in 24 bits (the max
    // is that of the fp32 values) and one atomic per row.  Columns past NH
    // hold h = 0 (zero column scales).
    constexpr int HF = FN / 2;
    constexpr int HP = BNH * 4 + 16;
    static_assert(TABB + BM * HP <= NBUF * (A_STAGE + B_STAGE), "h staging fits the ring");
    float mx[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const f32x4 sc = *(const lds_f32x4*)(As + 4 * (wrow + 16 * i));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int rt = wrow + i * 16 + q;
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < HF; ++j) {
          const float gv = acc[i][j][q] * sc[q] * csc[j];
          const float uv = acc[i][j + HF][q] * sc[q] * csc[j + HF];
          const float h = silu_f(gv) * uv;
          *(lds_f32*)(stage + rt * HP + (wn * BNW + j * 16 + lcol) * 4) = h;
          m = fmaxf(m, fabsf(h));
        }
        mx[i][q] = row16_max(m);
      }
    }
    if (lcol == 15) {
      uint32_t* const rmax = reinterpret_cast<uint32_t*>(smem) + 2 * BM;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) atomicMax(rmax + wrow + i * 16 + q, __float_as_uint(mx[i][q]));
    }
    __syncthreads();
    constexpr int CPR = BNH / 4;          // 4-column chunks per row (32)
    static_assert((BM * CPR) % 256 == 0, "whole passes");
    uint16_t* C = reinterpret_cast<uint16_t*>(shared ? p.C_shared : p.C);
    uint8_t* Clo = shared ? p.C_shared_lo : p.C_lo;
    uint32_t* amax = shared ? p.amax_shared : p.amax;
    if (tid < BM && m0 + tid < rows)
      atomicMax(&amax[row_base + m0 + tid], reinterpret_cast<const lds_u32*>(As)[2 * BM + tid]);
    // thread: chunk tid % 32 of rows tid / 32 + 8 u, NU rows read before any
    // is stored; each chunk leaves in the 24-bit form (8 + 4 bytes)
    constexpr int NPASS = BM * CPR / 256, NU = NPASS % 8 == 0 ? 8 : 5;
    static_assert(CPR == 32 && NPASS % NU == 0, "whole batches of rows");
    const int cc = tid & 31, col = n0 + cc * 4;
#pragma unroll
    for (int u0 = 0; u0 < NPASS; u0 += NU) {
      f32x4 v[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) v[u] = *(const lds_f32x4*)(stage + ((tid >> 5) + 8 * (u0 + u)) * HP + cc * 16);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int r = (tid >> 5) + 8 * (u0 + u);
        if (m0 + r < rows && col < NH) {
          const int64_t o = static_cast<int64_t>(row_base + m0 + r) * NH + col;
          store_h24(C + o, Clo + o, v[u]);
        }
      }
    }
  } else {
    // scaled fp32 tile [PR][BN] (row pitch FPB bytes) in passes of PR rows
    // (160-row tiles: two passes, one per wave row), then 16-byte chunks:
    // shared down stores them; routed down adds the shared expert's output.
    // Thread: chunk tid % 64 of pass rows tid / 64 + 4 u.  The routed down
    // loads its chunks of that output for the pass before the pass's staging
    // writes, so their latency overlaps the staging, and before the pass's
    // stores: a load issued after a store would make its wait cover the
    // store's round trip too.
    constexpr int FPB = BN * 4 + 16;
    constexpr int PR = TABB + BM * FPB <= NBUF * (A_STAGE + B_STAGE) ? BM : BM / WM;
    static_assert(TABB + PR * FPB <= NBUF * (A_STAGE + B_STAGE), "fp32 staging fits the ring");
    constexpr int CPR = BN / 4;
    constexpr int NPR = PR * CPR / 256;   // chunks per thread and pass (20 / 32)
    static_assert(CPR == 64 && (PR * CPR) % 256 == 0, "rows of 64 chunks, whole passes");
    const int cc = tid & 63, col = n0 + cc * 4;
    const lds_i32* const orows = reinterpret_cast<const lds_i32*>(As) + BM;
#pragma unroll
    for (int pass = 0; pass < BM / PR; ++pass) {
      // (unconditional loads: the rows past the group repeat its last
      // token, a column past NH reads column 0; neither is stored)
      f32x4 y[MODE == MODE_DOWN_ROUTED ? NPR : 1];
      if constexpr (MODE == MODE_DOWN_ROUTED) {
        const int ycol = col < NH ? col : 0;
#pragma unroll
        for (int u = 0; u < NPR; ++u) {
          y[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (p.Y) y[u] = *reinterpret_cast<const f32x4*>(p.Y + static_cast<int64_t>(orows[pass * PR + (tid >> 6) + 4 * u]) * NH + ycol);
        }
      }
      if (pass > 0) __syncthreads();      // the previous pass's chunks are read
      if (PR == BM || wm == pass) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const f32x4 sc = *(const lds_f32x4*)(As + 4 * (wrow + 16 * i));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int rp = wrow + i * 16 + q - pass * PR;
#pragma unroll
            for (int j = 0; j < FN; ++j)
              *(lds_f32*)(stage + rp * FPB + (wn * BNW + j * 16 + lcol) * 4) = acc[i][j][q] * sc[q] * csc[j];
          }
        }
      }
      __syncthreads();
      // every load of this pass has landed before the first store: the
      // stores are conditional, and a wait placed by the compiler after one
      // of them would also wait for the stores before it
      wait_vmcnt<0>();
      if constexpr (MODE == MODE_DOWN_ROUTED) {
        if (p.out_bf16) {
#pragma unroll
          for (int u = 0; u < NPR; ++u) {
            const int r = (tid >> 6) + 4 * u, rt = pass * PR + r;
            if (m0 + rt >= rows || col >= NH) continue;
            const f32x4 v = *(const lds_f32x4*)(stage + r * FPB + cc * 16) + y[u];
            const uint32_t lo = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
            const uint32_t hi = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.C) + static_cast<int64_t>(orows[rt]) * NH + col) =
                make_uint2(lo, hi);
          }
        } else {
#pragma unroll
          for (int u = 0; u < NPR; ++u) {
            const int r = (tid >> 6) + 4 * u, rt = pass * PR + r;
            if (m0 + rt >= rows || col >= NH) continue;
            const f32x4 v = *(const lds_f32x4*)(stage + r * FPB + cc * 16) + y[u];
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C) + static_cast<int64_t>(orows[rt]) * NH + col) = v;
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < NPR; ++u) {
          const int r = (tid >> 6) + 4 * u, rt = pass * PR + r;
          if (m0 + rt >= rows || col >= NH) continue;
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C_shared) + static_cast<int64_t>(m0 + rt) * NH + col) =
              *(const lds_f32x4*)(stage + r * FPB + cc * 16);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- 256 x 256 tiles
//
// The same three GEMMs on 256 x 256 workgroup tiles, for MFMA-bound work (the
// shared expert's gate/up and down GEMMs): each of the 4 waves owns a
// 128 x 128 accumulator block of 16 v_mfma_scale_f32_32x32x64_f8f6f4
// fragments (256 AGPRs), which reads 2/3 of the LDS bytes per FLOP that the
// 64 x 128 (or 80 x 128) blocks of the tiles above read, and half the L2
// bytes.  K = 64 bytes per stage (16 KB of A + 16 KB of weights) in a 5-deep
// ring, the whole LDS: four stages (~2 us of MFMA work) in flight, for
// operands that come from the last-level cache rather than L2.
//   * A rows (64 B): 16-byte chunk c of row r at c ^ ((r >> 1) & 3) ^
//     ((r >> 4) & 1); a lane's operand is 32 K bytes of one row (two
//     ds_read_b128).  The bf16 tiles' c ^ ((r >> 1) & 3) left a 2-way bank
//     conflict here (lanes 0-31 read 32 rows at one chunk, where the bf16
//     fragment reads 16 rows at two chunks): SQ_LDS_BANK_CONFLICT measured
//     29-31 % of the LDS-active cycles with it, 0 with the extra term;
//   * weight rows (256 B): chunk c of row r at c ^ (2 (r & 7)).  A byte
//     transpose read serves two 16-lane groups that read the same 8 K rows
//     at the adjacent column chunks 2m and 2m + 1; with this swizzle the
//     first lands on chunks {2m ^ even} and the second on {2m + 1 ^ even},
//     disjoint halves of the banks;
//   * 32 x 32 accumulator layout: lane l holds column l % 32 of rows
//     8 (i / 4) + 4 (l / 32) + i % 4, i = 0..15.
__device__ __forceinline__ int tall_a_swz(int r) { return ((r >> 1) & 3) ^ ((r >> 4) & 1); }

template <int MODE>
__global__ __launch_bounds__(256, 1) void gemm_fp8_tall_kernel(GemmArgs p) {
  typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
  constexpr int BM = 256;
  constexpr bool GATEUP = MODE == MODE_GATEUP;
  constexpr int BNH = GATEUP ? BN / 2 : BN;
  constexpr int TK = 64;                         // K bytes per stage
  constexpr int TNBUF = 5;
  constexpr int TA_ROWB = TK;
  constexpr int TA_STAGE = BM * TA_ROWB;         // 16 KB
  constexpr int TB_STAGE = TK * BN;              // 16 KB
  constexpr int TA_INS = TA_STAGE / 1024 / 4;    // 1 KB DMA instructions per wave per stage
  constexpr int TB_INS = TB_STAGE / 1024 / 4;
  constexpr int TLOADS = TA_INS + TB_INS;
  constexpr int FM = 4, FN = 4;                  // 32 x 32 fragments per wave
  static_assert(TNBUF * (TA_STAGE + TB_STAGE) <= 160 * 1024, "ring fits the LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[TNBUF * (TA_STAGE + TB_STAGE)];
  lds_u8* const As = (lds_u8*)(smem);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: scalar registers
  const int wm = wave >> 1, wn = wave & 1;
  const int E = p.E, T = p.T, K = p.K;

  // ---- XCD-aware tile lookup (as in the tiles above).  A launch of the
  // shared group alone (group_lo == E) reads no tile tables, so it can run
  // before the routing has written them.
  const bool shared_only = MODE != MODE_DOWN_SHARED && p.group_lo == E;
  const int nmt = (MODE == MODE_DOWN_SHARED || shared_only) ? (T + BM - 1) / BM
                                                            : p.tiles[p.group_hi] - p.tiles[p.group_lo];
  const int gn = p.n_tiles;
  const int lid = blockIdx.x;
  int mt_rel, nt;
  if (gn >= 8 && gn % 8 != 0 && gn % 4 == 0) {
    const int x = lid & 7, local = lid >> 3;
    const int w = gn >> 2, m_lo = ((x >> 2) * nmt) >> 1, m_hi = (((x >> 2) + 1) * nmt) >> 1;
    if (local >= (m_hi - m_lo) * w) return;
    mt_rel = m_lo + local / w;
    nt = (x & 3) * w + (local - (local / w) * w);
  } else if (gn >= 8) {
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
  } else if (shared_only) {
    g = E;
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
  if (!shared && !MOE_DCHECK_TILE(p, g, m0, rows)) return;   // debug builds: the tile is in its group
  const int row_base = shared ? 0 : p.offsets[g];
  const int ldb = GATEUP ? 2 * NH : NH;

  // per-row metadata for the epilogue, one tile row per thread
  float row_scale = 1.0f;
  int row_out = 0;
  {
    const int r = min(m0 + tid, rows - 1);
    if constexpr (GATEUP) {
      const int slot = shared ? r : p.perm[row_base + r];
      row_scale = (shared ? 1.0f : p.gate[slot]) * (shared ? p.sA_shared : p.sA)[shared ? slot : slot_token(slot, p.top_k)];
    } else if constexpr (MODE == MODE_DOWN_SHARED) {
      row_scale = p.sA_shared[r];
    } else {
      row_scale = p.sA[row_base + r];
      row_out = p.perm[row_base + r];
    }
  }

  // ---- DMA sources.  A: instruction i of wave w fills tile rows
  // 16 (w TA_INS + i) + lane / 4, the lane fetching the chunk its slot holds.
  const uint8_t* a_src;
  if constexpr (GATEUP) a_src = reinterpret_cast<const uint8_t*>(shared ? p.A_shared : p.A);
  else if constexpr (MODE == MODE_DOWN_SHARED) a_src = reinterpret_cast<const uint8_t*>(p.A_shared);
  else a_src = reinterpret_cast<const uint8_t*>(p.A);
  uint32_t a_voff[TA_INS];   // (the caller guarantees T * K < 2^31)
#pragma unroll
  for (int i = 0; i < TA_INS; ++i) {
    const int tr = 16 * (wave * TA_INS + i) + (lane >> 2);
    const int c = (lane & 3) ^ tall_a_swz(tr);
    const int r = min(m0 + tr, rows - 1);
    int arow;
    if constexpr (GATEUP) arow = shared ? r : slot_token(p.perm[row_base + r], p.top_k);
    else if constexpr (MODE == MODE_DOWN_SHARED) arow = r;
    else arow = row_base + r;
    a_voff[i] = static_cast<uint32_t>(arow) * static_cast<uint32_t>(K) + c * 16;
  }
  // weights: instruction i of wave w fills K rows 4 (w TB_INS + i) + lane / 16
  const uint8_t* b_src = reinterpret_cast<const uint8_t*>(shared ? p.B_shared : p.B) +
                         (shared ? 0 : static_cast<int64_t>(g) * K * ldb);
  uint32_t b_voff[TB_INS];
#pragma unroll
  for (int i = 0; i < TB_INS; ++i) {
    const int kr = 4 * (wave * TB_INS + i) + (lane >> 4);
    const int c = (lane & 15) ^ (2 * (kr & 7));
    const int lc = c * 16;
    int gc;
    if constexpr (GATEUP) gc = lc < BNH ? n0 + lc : NH + n0 + (lc - BNH);
    else gc = n0 + lc;
    const bool ok = n0 + (GATEUP ? lc % BNH : lc) < NH;
    b_voff[i] = static_cast<uint32_t>(kr * ldb + (ok ? gc : 0));   // clamped columns are never stored
  }
  const int64_t b_kstep = static_cast<int64_t>(TK) * ldb;
  const int nk = K / TK;

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // ---- LDS read addresses
  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(As));
  const int l32 = lane & 31, kh = lane >> 5;
  // A fragment i of slot sl: row wm 128 + 32 i + l32, logical chunks 2 kh and
  // 2 kh + 1 (the row's (r >> 1) & 3 equals (l32 >> 1) & 3)
  const int aswz = tall_a_swz(l32);   // (bits 0..4 of the row: the fragment base is a multiple of 32)
  const uint32_t a_rd0 = ring + (wm * 128 + l32) * TA_ROWB + (((2 * kh) ^ aswz) << 4);
  const uint32_t a_rd1 = ring + (wm * 128 + l32) * TA_ROWB + (((2 * kh + 1) ^ aswz) << 4);
  // weight fragment j: 32 columns; lane group gg = lane / 16 reads the 16
  // columns 16 (gg & 1) of it at K rows 32 (gg >> 1) + 8 q + s / 2, bytes
  // 8 (s & 1) of the chunk, s = lane % 16; four reads (q) give 32 K bytes
  uint32_t b_rd[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int gg = lane >> 4, s = lane & 15;
    int col;
    if constexpr (GATEUP) col = (j < FN / 2 ? 0 : BNH) + wn * (BNH / 2) + (j % (FN / 2)) * 32 + 16 * (gg & 1);
    else col = wn * (BN / 2) + j * 32 + 16 * (gg & 1);
    const int kr = 32 * (gg >> 1) + (s >> 1);
    b_rd[j] = ring + TNBUF * TA_STAGE + kr * BN + (((col >> 4) ^ (2 * (kr & 7))) << 4) + 8 * (s & 1);
  }
  typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
#define T8_AREAD(FA, i, SL)                                                                    \
  do {                                                                                         \
    const i32x4 lo_ = *(const lds_i32x4*)((const lds_u8*)(uintptr_t)a_rd0 + (SL) * TA_STAGE + (i) * 32 * TA_ROWB); \
    const i32x4 hi_ = *(const lds_i32x4*)((const lds_u8*)(uintptr_t)a_rd1 + (SL) * TA_STAGE + (i) * 32 * TA_ROWB); \
    FA[i] = i32x8{lo_[0], lo_[1], lo_[2], lo_[3], hi_[0], hi_[1], hi_[2], hi_[3]};             \
  } while (0)
#define T8_BREAD(FB, j, SL)                                                                    \
  do {                                                                                         \
    const lds_u8* q_ = (const lds_u8*)(uintptr_t)b_rd[j] + (SL) * TB_STAGE;                    \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                            \
      const i32x2 v_ = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(q_ + 8 * q * BN));  \
      FB[j][2 * q] = v_[0];                                                                    \
      FB[j][2 * q + 1] = v_[1];                                                                \
    }                                                                                          \
  } while (0)
  const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t a_lds0 = ring + wave_u * (TA_INS * 1024);
  const uint32_t b_lds0 = ring + TNBUF * TA_STAGE + wave_u * (TB_INS * 1024);
#define T8_DMA_A(i, st, SL)                                                                    \
  dma16(a_src + static_cast<int64_t>(min((st), nk - 1)) * TK, a_voff[i], a_lds0 + (SL) * TA_STAGE + (i) * 1024)
#define T8_DMA_B(i, st, SL)                                                                    \
  dma16(b_src + static_cast<int64_t>(min((st), nk - 1)) * b_kstep, b_voff[i], b_lds0 + (SL) * TB_STAGE + (i) * 1024)

  i32x8 fa0[FM], fa1[FM], fb0[FN], fb1[FN];
  constexpr int NMF = FM * FN;
  constexpr int NOPS = FM + FN + TA_INS + TB_INS;
#define T8_STEP(R, FA, FB, FA2, FB2)                                                           \
  do {                                                                                         \
    constexpr int sl_ = (R) % TNBUF, nsl_ = ((R) + 1) % TNBUF;                                 \
    const int sd_ = kt + (R) + TNBUF;                                                          \
    _Pragma("unroll") for (int m_ = 0; m_ < NMF; ++m_) {                                       \
      acc[m_ / FN][m_ % FN] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(               \
          FA[m_ / FN], FB[m_ % FN], acc[m_ / FN][m_ % FN], 0, 0, 0, 127, 0, 127);              \
      _Pragma("unroll") for (int o_ = 0; o_ < NOPS; ++o_) {                                    \
        if (o_ * NMF / NOPS == m_) {                                                           \
          if (o_ < FM) T8_AREAD(FA2, o_, nsl_);                                                \
          else if (o_ < FM + FN) T8_BREAD(FB2, o_ - FM, nsl_);                                 \
          else if (o_ < FM + FN + TA_INS) T8_DMA_A(o_ - FM - FN, sd_, sl_);                    \
          else T8_DMA_B(o_ - FM - FN - TA_INS, sd_, sl_);                                      \
        }                                                                                      \
      }                                                                                        \
      __builtin_amdgcn_sched_barrier(0);                                                       \
    }                                                                                          \
    wait_vmcnt<(TNBUF - 2) * TLOADS>();                                                        \
    __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) */                                       \
    __builtin_amdgcn_s_barrier();                                                              \
  } while (0)

  // prologue: stages 0 .. TNBUF-1 in flight; 0 and 1 landed and published;
  // stage 0's fragments in registers and its slot released
#pragma unroll
  for (int st = 0; st < TNBUF; ++st) {
#pragma unroll
    for (int i = 0; i < TA_INS; ++i) T8_DMA_A(i, st, st);
#pragma unroll
    for (int i = 0; i < TB_INS; ++i) T8_DMA_B(i, st, st);
  }
  wait_vmcnt<(TNBUF - 2) * TLOADS>();
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < FM; ++i) T8_AREAD(fa0, i, 0);
#pragma unroll
  for (int j = 0; j < FN; ++j) T8_BREAD(fb0, j, 0);
  __builtin_amdgcn_s_waitcnt(0xC07F); /* lgkmcnt(0) */
  __builtin_amdgcn_s_barrier();
  // unrolled by 10 = ring depth x register parity (slots and buffers
  // compile-time); accumulators pinned to AGPRs at each iteration
#define T8_STEPR(R)                                                                            \
  do {                                                                                         \
    if constexpr ((R) % 2 == 0) T8_STEP((R), fa0, fb0, fa1, fb1);                              \
    else T8_STEP((R), fa1, fb1, fa0, fb0);                                                     \
  } while (0)
  int kt = 0;
  for (; kt + 10 <= nk; kt += 10) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+a"(acc[i][j]));
    T8_STEPR(0); T8_STEPR(1); T8_STEPR(2); T8_STEPR(3); T8_STEPR(4);
    T8_STEPR(5); T8_STEPR(6); T8_STEPR(7); T8_STEPR(8); T8_STEPR(9);
  }
  const int left = nk - kt;   // 0 .. 9
  if (left > 0) { T8_STEPR(0);
  if (left > 1) { T8_STEPR(1);
  if (left > 2) { T8_STEPR(2);
  if (left > 3) { T8_STEPR(3);
  if (left > 4) { T8_STEPR(4);
  if (left > 5) { T8_STEPR(5);
  if (left > 6) { T8_STEPR(6);
  if (left > 7) { T8_STEPR(7);
  if (left > 8) { T8_STEPR(8); } } } } } } } } }
  wait_vmcnt<0>();
#undef T8_STEPR
#undef T8_AREAD
#undef T8_BREAD
#undef T8_DMA_A
#undef T8_DMA_B
#undef T8_STEP

  // ---- epilogue.  Column scales first, the row tables through LDS, then the
  // tile through LDS so that global memory sees 16-byte row chunks.
  const int lcol = lane & 31;
  float csc[FN];
  {
    const float* sB = GATEUP ? (shared ? p.sB_shared : p.sB + static_cast<int64_t>(g) * 2 * NH)
                             : (MODE == MODE_DOWN_ROUTED ? p.sB + static_cast<int64_t>(g) * NH : p.sB_shared);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int jj = GATEUP ? j % (FN / 2) : j;
      const int col = n0 + wn * (BNH / 2) + jj * 32 + lcol;
      csc[j] = col < NH ? sB[(GATEUP && j >= FN / 2 ? NH : 0) + col] : 0.0f;
    }
  }
  typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
  typedef __attribute__((address_space(3))) float lds_f32;
  typedef __attribute__((address_space(3))) int lds_i32;
  __syncthreads();
  reinterpret_cast<lds_f32*>(As)[tid] = row_scale;
  reinterpret_cast<lds_i32*>(As)[BM + tid] = row_out;
  reinterpret_cast<lds_u32*>(As)[2 * BM + tid] = 0u;
  __syncthreads();
  constexpr int TABB = 12 * BM;           // the three row tables
  lds_u8* const stage = As + TABB;
  // tile row of accumulator element e of fragment row i: wm 128 + 32 i +
  // 8 (e / 4) + 4 kh + e % 4
  const int wrow = wm * 128 + 4 * kh;
  if constexpr (GATEUP) {
    // h tile [256][128] fp32 (row pitch HP) and each row's max |h|: over this
    // lane's two columns, over the 16 lanes of its DPP row (DPP), then over
    // the two DPP rows and two waves that share the tile row (LDS atomic max
    // on the bit patterns of non-negative floats); then rows to global memory
    // in 24 bits (the max is that of the fp32 values) and one atomic per row.
    // Columns past NH hold h = 0.
    constexpr int HP = BNH * 4 + 16;
    static_assert(TABB + BM * HP <= TNBUF * (TA_STAGE + TB_STAGE), "h staging fits the ring");
    uint32_t* const rmax = reinterpret_cast<uint32_t*>(smem) + 2 * BM;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float mx[4][4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int rt0 = wrow + 32 * i + 8 * b;
        const f32x4 sc = *(const lds_f32x4*)(As + 4 * rt0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float m = 0.f;
#pragma unroll
          for (int j = 0; j < FN / 2; ++j) {
            const float gv = acc[i][j][4 * b + q] * sc[q] * csc[j];
            const float uv = acc[i][j + FN / 2][4 * b + q] * sc[q] * csc[j + FN / 2];
            const float h = silu_f(gv) * uv;
            *(lds_f32*)(stage + (rt0 + q) * HP + (wn * (BNH / 2) + j * 32 + lcol) * 4) = h;
            m = fmaxf(m, fabsf(h));
          }
          mx[b][q] = row16_max(m);
        }
      }
      if ((lane & 15) == 15) {
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) atomicMax(rmax + wrow + 32 * i + 8 * b + q, __float_as_uint(mx[b][q]));
      }
    }
    __syncthreads();
    constexpr int CPR = BNH / 4;          // 32 chunks of 4 columns per row
    uint16_t* C = reinterpret_cast<uint16_t*>(shared ? p.C_shared : p.C);
    uint8_t* Clo = shared ? p.C_shared_lo : p.C_lo;
    uint32_t* amax = shared ? p.amax_shared : p.amax;
    if (m0 + tid < rows) atomicMax(&amax[row_base + m0 + tid], reinterpret_cast<const lds_u32*>(As)[2 * BM + tid]);
    // thread: chunk tid % 32 of rows tid / 32 + 8 u, 8 rows read before any
    // is stored; each chunk leaves in the 24-bit form (8 + 4 bytes)
    static_assert(CPR == 32, "a row's chunks are 32 consecutive threads");
    const int cc = tid & 31, col = n0 + cc * 4;
#pragma unroll
    for (int u0 = 0; u0 < BM / 8; u0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *(const lds_f32x4*)(stage + ((tid >> 5) + 8 * (u0 + u)) * HP + cc * 16);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = (tid >> 5) + 8 * (u0 + u);
        if (m0 + r < rows && col < NH) {
          const int64_t o = static_cast<int64_t>(row_base + m0 + r) * NH + col;
          store_h24(C + o, Clo + o, v[u]);
        }
      }
    }
  } else {
    // scaled fp32 tile in two passes of 128 rows (one per wave row), then
    // 16-byte chunks: shared down stores them; routed down adds the shared
    // expert's output.  Thread: chunk tid % 64 of pass rows tid / 64 + 4 u.
    // The routed down loads its 32 chunks of that output for the pass before
    // the pass's staging writes (unconditionally: the rows past the group
    // repeat its last token, a column past NH reads column 0; neither is
    // stored) and waits for them before the first store, as in the tiles
    // above.
    constexpr int FPB = BN * 4 + 16;
    constexpr int PR = BM / 2;
    static_assert(TABB + PR * FPB <= TNBUF * (TA_STAGE + TB_STAGE), "fp32 staging fits the ring");
    constexpr int CPR = BN / 4;
    constexpr int NPR = PR * CPR / 256;   // 32
    static_assert(CPR == 64 && (PR * CPR) % 256 == 0, "rows of 64 chunks, whole passes");
    const int cc = tid & 63, col = n0 + cc * 4;
    const lds_i32* const orows = reinterpret_cast<const lds_i32*>(As) + BM;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      f32x4 y[MODE == MODE_DOWN_ROUTED ? NPR : 1];
      if constexpr (MODE == MODE_DOWN_ROUTED) {
        const int ycol = col < NH ? col : 0;
#pragma unroll
        for (int u = 0; u < NPR; ++u) {
          y[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (p.Y) y[u] = *reinterpret_cast<const f32x4*>(p.Y + static_cast<int64_t>(orows[pass * PR + (tid >> 6) + 4 * u]) * NH + ycol);
        }
      }
      if (pass > 0) __syncthreads();      // the previous pass's chunks are read
      if (wm == pass) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int rt0 = wrow + 32 * i + 8 * b;
            const f32x4 sc = *(const lds_f32x4*)(As + 4 * rt0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int rp = rt0 + q - pass * PR;
#pragma unroll
              for (int j = 0; j < FN; ++j)
                *(lds_f32*)(stage + rp * FPB + (wn * (BN / 2) + j * 32 + lcol) * 4) = acc[i][j][4 * b + q] * sc[q] * csc[j];
            }
          }
        }
      }
      __syncthreads();
      wait_vmcnt<0>();
      if constexpr (MODE == MODE_DOWN_ROUTED) {
        if (p.out_bf16) {
#pragma unroll
          for (int u = 0; u < NPR; ++u) {
            const int r = (tid >> 6) + 4 * u, rt = pass * PR + r;
            if (m0 + rt >= rows || col >= NH) continue;
            const f32x4 v = *(const lds_f32x4*)(stage + r * FPB + cc * 16) + y[u];
            const uint32_t lo = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
            const uint32_t hi = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p.C) + static_cast<int64_t>(orows[rt]) * NH + col) =
                make_uint2(lo, hi);
          }
        } else {
#pragma unroll
          for (int u = 0; u < NPR; ++u) {
            const int r = (tid >> 6) + 4 * u, rt = pass * PR + r;
            if (m0 + rt >= rows || col >= NH) continue;
            const f32x4 v = *(const lds_f32x4*)(stage + r * FPB + cc * 16) + y[u];
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C) + static_cast<int64_t>(orows[rt]) * NH + col) = v;
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < NPR; ++u) {
          const int r = (tid >> 6) + 4 * u, rt = pass * PR + r;
          if (m0 + rt >= rows || col >= NH) continue;
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C_shared) + static_cast<int64_t>(m0 + rt) * NH + col) =
              *(const lds_f32x4*)(stage + r * FPB + cc * 16);
        }
      }
    }
  }
}

template <int MODE, int BM>
hipError_t launch_f8(const GemmArgs& a0, int T, hipStream_t s, const int32_t* tiles_all) {
  GemmArgs a = a0;
  a.tiles = tiles_all + bm_index(BM) * (a.E + 2);
  constexpr int BNH = MODE == MODE_GATEUP ? BN / 2 : BN;
  const bool has_routed = a.group_lo < a.E;
  const bool has_shared = a.group_hi > a.E;
  int gm, nmax = a.N;
  if constexpr (MODE == MODE_DOWN_SHARED) {
    gm = (T + BM - 1) / BM;
  } else {
    const int Tr = T * (a.top_k > 1 ? a.top_k : 1);   // routed rows (slots)
    gm = (has_routed ? (Tr + BM - 1) / BM + a.E : 0) + (has_shared ? (T + BM - 1) / BM : 0);
    if (MODE == MODE_GATEUP) nmax = max(has_routed ? a.N : 0, has_shared ? a.N_shared : 0);
  }
  if (gm <= 0) return hipSuccess;
  const int gn = (nmax + BNH - 1) / BNH;
  a.n_tiles = gn;
  const int64_t nblk = (gn >= 8 && gn % 8 != 0 && gn % 4 == 0) ? 8 * static_cast<int64_t>((gm + 1) / 2) * (gn / 4)
                       : gn >= 8 ? 8 * static_cast<int64_t>(gm) * ((gn + 7) / 8)
                                 : static_cast<int64_t>(gm) * gn;
  if constexpr (BM == 256)
    hipLaunchKernelGGL((gemm_fp8_tall_kernel<MODE>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_fp8_kernel<MODE, BM>), dim3(static_cast<unsigned>(nblk)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(int mode, int bm, const GemmArgs& a, int T, hipStream_t s, const int32_t* tiles_all) {
  if (bm == 256) {
    switch (mode) {
      case MODE_GATEUP: return launch_f8<MODE_GATEUP, 256>(a, T, s, tiles_all);
      case MODE_DOWN_SHARED: return launch_f8<MODE_DOWN_SHARED, 256>(a, T, s, tiles_all);
      case MODE_DOWN_ROUTED: return launch_f8<MODE_DOWN_ROUTED, 256>(a, T, s, tiles_all);
    }
    return hipErrorInvalidValue;
  }
  if (bm == 160 && mode == MODE_GATEUP) return launch_f8<MODE_GATEUP, 160>(a, T, s, tiles_all);
  if (bm == 160 && mode == MODE_DOWN_ROUTED) return launch_f8<MODE_DOWN_ROUTED, 160>(a, T, s, tiles_all);
  if (bm != 128) return hipErrorInvalidValue;
  switch (mode) {
    case MODE_GATEUP: return launch_f8<MODE_GATEUP, 128>(a, T, s, tiles_all);
    case MODE_DOWN_SHARED: return launch_f8<MODE_DOWN_SHARED, 128>(a, T, s, tiles_all);
    case MODE_DOWN_ROUTED: return launch_f8<MODE_DOWN_ROUTED, 128>(a, T, s, tiles_all);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
