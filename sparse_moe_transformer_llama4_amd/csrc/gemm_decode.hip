// Weight-streaming grouped GEMMs for decode-sized token counts (gfx950):
// bf16 weights (also the routed tails of bf16 prefill and dense decode),
// and int8 / int4 weight codes (gemm_q8_kernel, further below).
//
// With a few tokens per expert the block is a weight stream: every touched
// expert's W_gate_up and W_down are read once from HBM and each weight is
// used by a handful of rows.  The kernels therefore optimise bytes in
// flight, not MFMA reuse:
//   * workgroup tile = (group, 16 or 32 rows, 128 weight columns; gate/up:
//     128 gate + the matching 128 up columns), grid (row tile, column tile)
//     with the row tile fastest: the workgroups running together read many
//     different weight matrices (measured faster than walking one matrix's
//     columns together);
//   * wave-level split-K: each of the 4 waves streams its own quarter of K
//     through a private 4-deep LDS ring fed by direct-to-LDS loads
//     (global_load_lds_dwordx4, weights with the non-temporal hint), so the
//     main loop needs no workgroup barrier -- each wave only waits for its
//     own DMA (vmcnt) -- and ~108 KB per CU are in flight against HBM
//     latency;
//   * down tiles keep 256-byte weight rows in LDS (16-byte chunk c of row r
//     at c ^ 2 (r & 3)), gate/up tiles 512-byte rows (c ^ 2 (r & 7)), so the
//     LDS transpose reads (ds_read_b64_tr_b16) hit disjoint banks;
//   * the activation rows of each stage travel through the same per-wave
//     DMA ring (1-2 KB per stage), so every load in the loop is ordered by
//     the explicit waits and none by compiler-inserted ones;
//   * MFMAs only for the 16-row fragments that hold valid rows;
//   * the four K-quarter partial sums are added through LDS once at the end,
//     followed by the same epilogues as the prefill kernels (SwiGLU with the
//     gate on routed rows; fp32 shared output; un-permute + combine).
#include <algorithm>

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
// The same with the non-temporal hint, for the weights: each weight byte is
// read once per call, and the streaming policy lifts the rate of these
// 128/256-byte row segments by ~8 % (measured: 5.6 -> 6.0 TB/s for the
// gate/up tiles' two 128-byte segments per row).
__device__ __forceinline__ void dma16_nt(const void* g, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds_base), "v"(g) : "memory", "m0");
}
// Scalar-base forms (the int8 / int4 tiles): `sbase` is wave-uniform (an
// SGPR pair) and each lane adds its own 32-bit byte offset, so advancing
// along K is a scalar add per stage and no lane computes a 64-bit address.
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_s_nt(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
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

// ---------------------------------------------------------------- gate/up
//
// Tile = 128 gate columns + the matching 128 up columns, i.e. two 256-byte
// segments per weight row (a streaming probe: 256-byte segments ~7 % faster
// than 128-byte ones when the workgroups fill whole rounds).  With 512-byte
// weight rows a stage holds 16 K rows (8 KB) and feeds the 16x16x16 MFMA, so
// the 4-deep per-wave ring still fits in 144 KB.  A launch over the shared
// group alone (group_lo == E) addresses its tiles directly, without the tile
// table, so it can run before the routing has finished.
constexpr int GBN = 256;               // weight columns per tile
constexpr int GBNH = GBN / 2;          // output columns per tile
constexpr int GBK = 16;                // K rows per stage
constexpr int GROWB = GBN * 2;         // bytes per weight row in LDS
constexpr int GWSTAGE = GBK * GROWB;   // 8 KB of weights per stage
constexpr int GINS = GWSTAGE / 1024;   // weight DMA instructions per stage per wave (8)
constexpr int GFN = GBN / 16;          // weight fragments (16 columns each)
constexpr int GSTAGE = GWSTAGE + 1024; // + 32 activation rows x 16 K values
constexpr int GPP = GBN + 16;          // floats per row of the partial-sum buffer (padded)

// B fragment of the 16x16x16 MFMA for columns col .. col+15: lane gets column
// col + lane%16, K rows 4 (lane/16) .. +3 of the stage.  The 16 lanes of a
// group address 4 rows x 4 columns each; the transposing read returns every
// lane its column's 4 values.  16-byte chunk c of row r sits at c ^ 2 (r & 7).
__device__ __forceinline__ s16x4 read_w_frag16(const lds_u8* st, int col, int lane) {
  const int s = lane & 15;
  const int r = 4 * (lane >> 4) + (s >> 2);
  const int lbyte = (col + 4 * (s & 3)) * 2;
  const int pbyte = ((lbyte >> 4) ^ (2 * (r & 7))) * 16 + (lbyte & 15);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(st + r * GROWB + pbyte));
}

template <int FMMAX>
__global__ __launch_bounds__(256, 1) void gemm_decode_gateup_kernel(GemmArgs p) {
  constexpr int DBM = 16 * FMMAX;              // rows per tile
  constexpr int DNBUF = 4;                     // per-wave ring depth
  constexpr int LOADS = GINS + 1;              // DMA instructions per stage per wave
  constexpr int PART = 4 * DBM * GPP * 4;      // the four waves' partial sums
  constexpr int RING = 4 * DNBUF * GSTAGE;
  constexpr int TAB = PART;                    // per-row gate scales
  constexpr int SMEM = RING > TAB + 4 * DBM ? RING : TAB + 4 * DBM;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, K = p.K;

  // ---- tile lookup (DBM-row tiles over groups group_lo .. group_hi - 1);
  // grid (row tile, column tile), or (column tile, row tile) for tail launches
  const int bi_m = p.tail_bm > 0 ? blockIdx.y : blockIdx.x;
  const int bi_n = p.tail_bm > 0 ? blockIdx.x : blockIdx.y;
  int g, m0;
  if (p.group_lo == E) {
    g = E;
    m0 = bi_m * DBM;
    if (m0 >= p.T) return;
  } else {
    const int mt = bi_m + p.tiles[p.group_lo];
    if (mt >= p.tiles[p.group_hi]) return;
    int lo = p.group_lo, hi = p.group_hi - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.tiles[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    g = lo;
    m0 = (mt - p.tiles[g]) * DBM;
  }
  const int rows = (g == E) ? p.T : p.offsets[g + 1] - p.offsets[g];
  // tail launches: the tile starts after the group's full tail_bm-row tiles
  if (p.tail_bm > 0 && g < E) m0 += (rows / p.tail_bm) * p.tail_bm;
  const bool shared = g == E;
  const int NH = shared ? p.N_shared : p.N;
  const int n0 = bi_n * GBNH;
  if (n0 >= NH) return;
  if (!shared && !MOE_DCHECK_TILE(p, g, m0, rows)) return;   // debug builds: the tile is in its group
  const int row_base = shared ? 0 : p.offsets[g];
  const int ldb = 2 * NH;
  const int nvalid = min(DBM, rows - m0);
  const int fm = (nvalid + 15) >> 4;           // fragments with valid rows (uniform)

  // the routed rows' gate scale, loaded now so its latency hides behind the loop
  float row_scale = 1.0f;
  if (tid < DBM && !shared) row_scale = p.gate[p.perm[row_base + min(m0 + tid, rows - 1)]];

  // ---- this wave's quarter of K
  // K split over gridDim.z (launches that write pre-activation partials)
  const int kz = K / static_cast<int>(gridDim.z);
  const int kq = kz >> 2;                      // multiple of GBK
  const int k0 = static_cast<int>(blockIdx.z) * kz + wave * kq;
  const int ns = kq / GBK;

  // weights: DMA instruction i fills K rows 2i, 2i+1 of the stage; lane ->
  // row 2i + lane/32, physical chunk lane%32 holding logical chunk
  // c = (lane%32) ^ 2 (row & 7); logical chunks 0..15 are the gate columns
  // n0 + 8c, 16..31 the up columns NH + n0 + 8 (c - 16)
  const uint16_t* wbase = reinterpret_cast<const uint16_t*>(shared ? p.B_shared : p.B) +
                          (shared ? 0 : static_cast<int64_t>(g) * K * ldb);
  int64_t w_off[GINS];
#pragma unroll
  for (int i = 0; i < GINS; ++i) {
    const int kr = 2 * i + (lane >> 5);
    const int c = (lane & 31) ^ (2 * (kr & 7));
    const int lc = (c & 15) * 8;
    const int gc = (c < 16 ? n0 : NH + n0) + lc;
    w_off[i] = static_cast<int64_t>(k0 + kr) * ldb + (n0 + lc < NH ? gc : 0);
  }
  const int64_t w_kstride = static_cast<int64_t>(GBK) * ldb;

  // activations: one DMA instruction per stage; lane -> tile row lane/2,
  // physical chunk lane%2 holding logical chunk (lane%2) ^ ((row >> 3) & 1)
  // (8 K values); rows past the group are clamped to its last row
  const uint16_t* abase = reinterpret_cast<const uint16_t*>(shared ? p.A_shared : p.A);
  int64_t a_off;
  {
    const int ar = lane >> 1;
    const int r = min(m0 + ar, rows - 1);
    const int arow = shared ? r : slot_token(p.perm[row_base + r], p.top_k);
    a_off = static_cast<int64_t>(arow) * K + k0 + (((lane & 1) ^ ((ar >> 3) & 1)) * 8);
  }

  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem)) +
                        __builtin_amdgcn_readfirstlane(wave) * (DNBUF * GSTAGE);
  const lds_u8* ring_p = (const lds_u8*)smem + wave * (DNBUF * GSTAGE);
  // A fragment f: row 16f + lane%16, K values 4 (lane/16) .. +3 = logical
  // chunk lane/32, bytes 8 ((lane/16) & 1) of it
  int a_rd[FMMAX];
#pragma unroll
  for (int f = 0; f < FMMAX; ++f) {
    const int r = 16 * f + (lane & 15);
    a_rd[f] = GWSTAGE + r * 32 + (((lane >> 5) ^ ((r >> 3) & 1)) << 4) + (((lane >> 4) & 1) << 3);
  }

  f32x4 acc[FMMAX][GFN];
#pragma unroll
  for (int f = 0; f < FMMAX; ++f)
#pragma unroll
    for (int j = 0; j < GFN; ++j) acc[f][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#define GU_ISSUE(st)                                                                           \
  do {                                                                                         \
    const int s_ = min((st), ns - 1);                                                          \
    const uint32_t b_ = ring + static_cast<uint32_t>(((st) % DNBUF) * GSTAGE);                 \
    _Pragma("unroll") for (int i = 0; i < GINS; ++i)                                           \
      dma16_nt(wbase + w_off[i] + s_ * w_kstride, b_ + i * 1024);                              \
    dma16(abase + a_off + s_ * GBK, b_ + GWSTAGE);                                             \
  } while (0)
  // Stage kt: its DMA is complete once only the later stages' DMAs remain.
#define GU_STEP(kt)                                                                            \
  do {                                                                                         \
    GU_ISSUE((kt) + DNBUF - 1);                                                                \
    wait_vmcnt<(DNBUF - 1) * LOADS>();                                                         \
    const lds_u8* st_ = ring_p + ((kt) % DNBUF) * GSTAGE;                                      \
    s16x4 wf[GFN], af[FMMAX];                                                                  \
    _Pragma("unroll") for (int j = 0; j < GFN; ++j)                                            \
      wf[j] = read_w_frag16(st_, (j < GFN / 2 ? 0 : GBNH) + (j % (GFN / 2)) * 16, lane);       \
    _Pragma("unroll") for (int f = 0; f < FMMAX; ++f)                                          \
      af[f] = *reinterpret_cast<const lds_s16x4*>(st_ + a_rd[f]);                              \
    _Pragma("unroll") for (int f = 0; f < FMMAX; ++f)                                          \
      if (f < fm)                                                                              \
        _Pragma("unroll") for (int j = 0; j < GFN; ++j)                                        \
          acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(af[f], wf[j], acc[f][j], 0, 0, 0); \
    /* this stage's slot is refilled DNBUF-1 steps later: reads must be done */                \
    __builtin_amdgcn_s_waitcnt(0xC07F);                                                        \
  } while (0)

#pragma unroll
  for (int st = 0; st < DNBUF - 1; ++st) GU_ISSUE(st);
  for (int kt = 0; kt < ns; ++kt) GU_STEP(kt);
  wait_vmcnt<0>();
#undef GU_ISSUE
#undef GU_STEP

  // ---- the four waves' partial sums through LDS ([row][GPP] fp32 each)
  __syncthreads();
  float* part = reinterpret_cast<float*>(smem);
  float* tab = reinterpret_cast<float*>(smem + TAB);
  const int lcol = lane & 15, rq = 4 * (lane >> 4);
#pragma unroll
  for (int f = 0; f < FMMAX; ++f) {
    if (f < fm) {
#pragma unroll
      for (int j = 0; j < GFN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          part[(wave * DBM + 16 * f + rq + q) * GPP + j * 16 + lcol] = acc[f][j][q];
    }
  }
  if (tid < DBM) tab[tid] = row_scale;
  __syncthreads();
  // thread -> quads of 4 consecutive columns of a row; sum in wave order
  constexpr int C4 = GBN / 4;
  constexpr int NQ = DBM * C4 / 256;
  f32x4 tq[NQ];
#pragma unroll
  for (int it = 0; it < NQ; ++it) {
    const int e = tid + 256 * it;
    const int r = e / C4, c = (e % C4) * 4;
    const f32x4* p0 = reinterpret_cast<const f32x4*>(part + r * GPP + c);
    constexpr int WS = DBM * GPP / 4;            // one wave's buffer in quads
    tq[it] = ((p0[0] + p0[WS]) + p0[2 * WS]) + p0[3 * WS];
  }
  if (p.gu_part) {
    // pre-activation partial of this K part: [z][row][2 NH] fp32, gate
    // columns at n0.., up columns at NH + n0.. (the SwiGLU runs after the
    // parts are summed)
    float* dst = p.gu_part + static_cast<int64_t>(blockIdx.z) * p.T * (2 * NH);
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = tid + 256 * it;
      const int r = e / C4, c = (e % C4) * 4;
      const int gcol = c < GBNH ? n0 + c : NH + n0 + (c - GBNH);
      if (r < nvalid && n0 + (c % GBNH) < NH)
        *reinterpret_cast<f32x4*>(dst + static_cast<int64_t>(row_base + m0 + r) * (2 * NH) + gcol) = tq[it];
    }
    return;
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < NQ; ++it) {
    const int e = tid + 256 * it;
    const int r = e / C4, c = (e % C4) * 4;
    *reinterpret_cast<f32x4*>(part + r * GPP + c) = tq[it];
  }
  __syncthreads();

  // ---- SwiGLU epilogue: h = SiLU(s acc_gate) * (s acc_up), s = the token's
  // gate on routed rows, 1 on shared rows; columns fastest
  constexpr int NIT = DBM * GBNH / 256;
  uint16_t* C = reinterpret_cast<uint16_t*>(shared ? p.C_shared : p.C);
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int e = tid + 256 * it;
    const int r = e / GBNH, c = e % GBNH;
    const int col = n0 + c;
    if (r >= nvalid || col >= NH) continue;
    const float sc = tab[r];
    const float gv = part[r * GPP + c] * sc;
    const float uv = part[r * GPP + GBNH + c] * sc;
    C[static_cast<int64_t>(row_base + m0 + r) * NH + col] = f32_to_bf16(silu_f(gv) * uv);
  }
}

// ---------------------------------------------------------------- down

template <int MODE, int FMMAX>
__global__ __launch_bounds__(256, 1) void gemm_decode_kernel(GemmArgs p) {
  static_assert(MODE == MODE_DOWN_SHARED || MODE == MODE_DOWN_ROUTED, "down modes only");
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

  // ---- tile lookup (DBM-row tiles); grid (row tile, column tile, K part),
  // or (column tile, row tile) for tail launches
  const int bi_m = p.tail_bm > 0 ? blockIdx.y : blockIdx.x;
  const int bi_n = p.tail_bm > 0 ? blockIdx.x : blockIdx.y;
  int g, m0, rows;
  if constexpr (MODE == MODE_DOWN_SHARED) {
    g = 0;
    m0 = bi_m * DBM;
    rows = T;
    if (m0 >= T) return;
  } else {
    const int mt = bi_m + p.tiles[p.group_lo];
    if (mt >= p.tiles[p.group_hi]) return;
    int lo = p.group_lo, hi = p.group_hi - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.tiles[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    g = lo;
    m0 = (mt - p.tiles[g]) * DBM;
    rows = p.offsets[g + 1] - p.offsets[g];
    if (p.tail_bm > 0) m0 += (rows / p.tail_bm) * p.tail_bm;   // tail launches
  }
  constexpr bool shared = MODE == MODE_DOWN_SHARED;
  const int NH = p.N;
  const int n0 = bi_n * DBN;
  if (n0 >= NH) return;
  if (!shared && !MOE_DCHECK_TILE(p, g, m0, rows)) return;   // debug builds: the tile is in its group
  const int row_base = shared ? 0 : p.offsets[g];
  const int ldb = NH;
  const int nvalid = min(DBM, rows - m0);
  const int fm = (nvalid + 15) >> 4;            // fragments with valid rows (uniform)

  // the routed down's output row (un-permutation), one tile row per thread,
  // loaded now so its latency hides behind the main loop
  int row_out = 0;
  if (MODE == MODE_DOWN_ROUTED && tid < DBM) row_out = p.perm[row_base + min(m0 + tid, rows - 1)];

  // ---- this block's K range (split over blockIdx.z for the shared down
  // GEMM, whose single M-tile would otherwise leave most CUs idle) and this
  // wave's quarter of it.  K is cut into 128-row units, part z taking units
  // [z U / nsplit, (z+1) U / nsplit): parts differ by one unit at most when
  // nsplit does not divide U
  const int nsplit = gridDim.z;
  const int units = K >> 7;
  const int u0 = static_cast<int>(blockIdx.z) * units / nsplit;
  const int u1 = (static_cast<int>(blockIdx.z) + 1) * units / nsplit;
  const int ns = u1 - u0;                       // DBK-row stages per wave
  const int kq = ns * DBK;
  const int k0 = u0 * 128 + wave * kq;

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
    w_off[i] = static_cast<int64_t>(k0 + kr) * ldb + (n0 + lc < NH ? n0 + lc : 0);
  }
  const int64_t w_kstride = static_cast<int64_t>(DBK) * ldb;

  // activations: DMA instruction f fills rows 16f .. 16f+15 (64 B each) of the
  // stage's activation block; lane -> row 16f + lane/4, slot lane%4, which
  // holds logical chunk slot ^ ((row >> 1) & 3) (conflict-free fragment reads)
  const uint16_t* abase = reinterpret_cast<const uint16_t*>(shared ? p.A_shared : p.A);
  int64_t a_off[FMMAX];
#pragma unroll
  for (int f = 0; f < FMMAX; ++f) {
    const int r = min(m0 + 16 * f + (lane >> 2), rows - 1);
    const int arow = row_base + r;
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
      dma16_nt(wbase + w_off[i] + s_ * w_kstride, b_ + i * 1024);                                 \
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
    _Pragma("unroll") for (int j = 0; j < FN; ++j)                                             \
      wf[j] = read_w_frag(st_, (lane >> 4) * 8, j * 16, lane);                                 \
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
  if (tid < DBM) reinterpret_cast<int*>(smem + PART)[tid] = row_out;
  __syncthreads();
  auto total = [&](int r, int c) -> float {
    return part[(0 * DBM + r) * DBN + c] + part[(1 * DBM + r) * DBN + c] + part[(2 * DBM + r) * DBN + c] +
           part[(3 * DBM + r) * DBN + c];
  };

  // ---- epilogue: thread -> (row, column) pairs, columns fastest.  Fixed
  // trip count, fully unrolled, every global load ahead of the stores (the
  // compiler must assume stores through C may alias the loaded arrays, so a
  // load between stores would wait a full round trip).
  constexpr int NIT = DBM * DBN / 256;
  {
    const int* ot = reinterpret_cast<const int*>(smem + PART);
    float y[NIT];
    if constexpr (MODE == MODE_DOWN_ROUTED) {
      // the shared expert's output, as y_parts K-split partials summed in order
      const int nparts = !p.Y ? 0 : p.y_parts > 1 ? p.y_parts : 1;
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
            const int r = e / DBN, col = n0 + e % DBN;
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
      const int r = e / DBN, c = e % DBN;
      const int col = n0 + c;
      if (r >= nvalid || col >= NH) continue;
      const int orow = (MODE == MODE_DOWN_ROUTED) ? ot[r] : m0 + r;
      const int64_t o = static_cast<int64_t>(orow) * NH + col;
      const float v = total(r, c);
      if constexpr (MODE == MODE_DOWN_SHARED) {
        reinterpret_cast<float*>(p.C_shared)[static_cast<int64_t>(blockIdx.z) * T * NH + o] = v;
      } else {
        const float yv = p.Y ? v + y[it] : v;
        if (p.out_bf16) reinterpret_cast<uint16_t*>(p.C)[o] = f32_to_bf16(yv);
        else reinterpret_cast<float*>(p.C)[o] = yv;
      }
    }
  }
}

// ---------------------------------------------------------------- int8 weights
//
// Weight-only int8 (codes q, one fp32 scale s per output column, weight =
// q * s) on the same weight-streaming design, for all three GEMMs:
//   * 256-byte weight rows per tile (down: 256 output columns; gate/up: 128
//     gate + the matching 128 up columns), 32 K rows = 8 KB per stage, the
//     same per-wave 4-deep ring and activation staging as the bf16 down
//     tiles; 16-byte chunk c of LDS row r sits at c ^ (r & 15);
//   * the 16x16x32 bf16 MFMA's B fragment comes from the 8-bit LDS transpose
//     read: each group of 16 lanes reads an 8-row x 16-column block (lane s
//     gives row s/2, columns 8 (s%2) .. +7) and lane s receives column s of
//     the 8 rows, i.e. its 8 K values;
//   * codes become bf16 exactly (|q| <= 127: at most 7 significant bits):
//     int8 -> fp32, upper half;
//   * the column scale multiplies the fp32 sums in the epilogue (exact
//     algebra: sum_k x_k q_kn s_n = s_n sum_k x_k q_kn).
// int4 (QB = 4): two codes per byte along K (byte (k/2, n) holds rows k, k+1
// of column n, the even row in the low nibble, two's complement), so the
// same 256-byte rows and transpose reads carry 64 K rows per stage: a lane's
// 8 bytes are 16 consecutive K values of its column, the B operands of two
// MFMA steps (K rows 16g .. 16g+7 and 16g+8 .. 16g+15 of lane group g), and
// the activation stage holds 64 K values per row, read as the matching
// contiguous 16-byte chunks 2g and 2g + 1.
constexpr int QBN = 256;               // weight bytes per tile row (int8: columns)
constexpr int QBK = 32;                // K rows per stage
constexpr int QWSTAGE = QBK * QBN;     // 8 KB of weights per stage
constexpr int QINS = QWSTAGE / 1024;   // weight DMA instructions per stage per wave (8)
constexpr int QFN = QBN / 16;          // weight fragments (16 columns each)
constexpr int QPP = QBN + 16;          // floats per row of the partial-sum buffer (padded)

typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// B fragment for tile columns col .. col+15 (col % 16 == 0): lane gets column
// col + lane%16, byte rows 8 (lane/16) .. +7 of the stage (int8: 8 codes;
// int4: 16 codes) ...
__device__ __forceinline__ i32x2 read_q_frag(const lds_u8* st, int col, int lane) {
  const int s = lane & 15;
  const int r = 8 * (lane >> 4) + (s >> 1);
  const int pbyte = (((col >> 4) ^ (r & 15)) << 4) + 8 * (s & 1);
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(st + r * QBN + pbyte));
}
// ... and as bf16 (exact: int8 -> fp32 -> upper half)
__device__ __forceinline__ bf16x8 q_to_bf16(i32x2 q) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int w = q[i >> 1];
    const int sh = 16 * (i & 1);
    const float lo = static_cast<float>(static_cast<int8_t>(w >> sh));
    const float hi = static_cast<float>(static_cast<int8_t>(w >> (sh + 8)));
    // the upper halves of both (one byte permute): lo's in bits 0..15, hi's above
    o[i] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  const u32x4 v = {o[0], o[1], o[2], o[3]};
  return __builtin_bit_cast(bf16x8, v);
}
// ... and, int4, the 8 codes of word w (K rows 0..7: byte j holds rows 2j
// (low nibble) and 2j + 1) as the bf16 values 136 + q, exactly, in the K
// order 0 2 4 6 1 3 5 7: flipping each nibble's top bit turns the
// two's-complement code q into u = q + 8 in 0..15, and the bf16 pattern
// 0x43 | u (high byte 0x43, low byte u) is 128 + u.  The even rows' nibbles,
// masked, are bytes 0..3 of one word and the odd rows' of another; a byte
// permute then pairs two of them with 0x43 bytes per output dword (eight
// operations for eight codes).  The A fragment is put in the same K order
// (a4_order); the kernel removes the offset 136 * sum_k x_k once per row
// after the K loop.
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4q;
__device__ __forceinline__ bf16x8 q4_to_bf16_off(int w) {
  // (mask, then flip each nibble's top bit: one three-input bit operation for
  // the even nibbles, a shift and one for the odd ones)
  const uint32_t b = static_cast<uint32_t>(w);
  const uint32_t ev = (b & 0x0F0F0F0Fu) ^ 0x08080808u, od = ((b >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
  constexpr uint32_t kHi = 0x43434343u;
  const u32x4q o = {__builtin_amdgcn_perm(kHi, ev, 0x04010400u), __builtin_amdgcn_perm(kHi, ev, 0x04030402u),
                    __builtin_amdgcn_perm(kHi, od, 0x04010400u), __builtin_amdgcn_perm(kHi, od, 0x04030402u)};
  return __builtin_bit_cast(bf16x8, o);
}
// A fragment of K rows 0..7 (in order, two per dword) -> K order 0 2 4 6
// 1 3 5 7: the low halves of dwords 0, 1, then 2, 3, then the high halves
__device__ __forceinline__ bf16x8 a4_order(bf16x8 a) {
  const u32x4q v = __builtin_bit_cast(u32x4q, a);
  const u32x4q r = {__builtin_amdgcn_perm(v[1], v[0], 0x05040100u), __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
                    __builtin_amdgcn_perm(v[1], v[0], 0x07060302u), __builtin_amdgcn_perm(v[3], v[2], 0x07060302u)};
  return __builtin_bit_cast(bf16x8, r);
}

template <int MODE, int FMMAX, int QB>
__global__ __launch_bounds__(256, 1) void gemm_q8_kernel(GemmArgs p) {
  static_assert(QB == 8 || (QB == 4 && FMMAX == 1), "int8 codes, or int4 codes on 16-row tiles");
  constexpr bool GU = MODE == MODE_GATEUP;
  constexpr int KPS = QB == 8 ? QBK : 2 * QBK;  // K rows per stage
  constexpr int DBM = 16 * FMMAX;               // rows per tile
  constexpr int AROW = KPS * 2;                 // activation bytes per row per stage (64 / 128)
  constexpr int AINS = 16 * AROW / 1024;        // activation DMA instructions per fragment (1 / 2)
  constexpr int ASTAGE = FMMAX * 16 * AROW;     // activation bytes per stage
  constexpr int STAGE = QWSTAGE + ASTAGE;
  constexpr int DNBUF = 4 * 4 * STAGE <= 160 * 1024 ? 4 : 3;   // per-wave ring depth within 160 KB
  constexpr int LOADS = QINS + FMMAX * AINS;    // DMA instructions per stage per wave
  constexpr int PART = 4 * DBM * QPP * 4;       // the four waves' partial sums
  constexpr int RING = 4 * DNBUF * STAGE;
  constexpr int TABS = 8 * DBM + (QB == 4 ? 4 * 5 * DBM : 0);   // per-row tables after PART (+ int4 row sums)
  constexpr int SMEM = RING > PART + TABS ? RING : PART + TABS;
  constexpr int OUTC = GU ? QBN / 2 : QBN;      // output columns per tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int E = p.E, T = p.T, K = p.K;

  // ---- tile lookup: grid (row tile, column tile, K part), or (column tile,
  // row tile) for tail launches.  Group E is the shared expert (GATEUP over
  // the shared group alone, DOWN_SHARED) addressed without the tile table.
  const int bi_m = p.tail_bm > 0 ? blockIdx.y : blockIdx.x;
  const int bi_n = p.tail_bm > 0 ? blockIdx.x : blockIdx.y;
  int g, m0;
  if (MODE == MODE_DOWN_SHARED || (GU && p.group_lo == E)) {
    g = E;
    m0 = bi_m * DBM;
    if (m0 >= T) return;
  } else {
    const int mt = bi_m + p.tiles[p.group_lo];
    if (mt >= p.tiles[p.group_hi]) return;
    int lo = p.group_lo, hi = p.group_hi - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.tiles[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    g = lo;
    m0 = (mt - p.tiles[g]) * DBM;
  }
  const bool shared = g == E;
  const int rows = shared ? T : p.offsets[g + 1] - p.offsets[g];
  if (p.tail_bm > 0 && !shared) m0 += (rows / p.tail_bm) * p.tail_bm;   // tail launches
  const int NH = (GU && shared) ? p.N_shared : p.N;   // output width of this GEMM
  const int n0 = bi_n * OUTC;
  if (n0 >= NH) return;
  if (!shared && !MOE_DCHECK_TILE(p, g, m0, rows)) return;   // debug builds: the tile is in its group
  const int row_base = shared ? 0 : p.offsets[g];
  const int ldb = GU ? 2 * NH : NH;                   // bytes per weight row
  const int nvalid = min(DBM, rows - m0);
  const int fm = (nvalid + 15) >> 4;                  // fragments with valid rows (uniform)

  // per-row values loaded now so their latency hides behind the main loop:
  // GATEUP routed rows: the token's gate; DOWN_ROUTED: the output row
  float row_scale = 1.0f;
  int row_out = 0;
  if (tid < DBM) {
    const int r = min(m0 + tid, rows - 1);
    if (GU && !shared) row_scale = p.gate[p.perm[row_base + r]];
    if (MODE == MODE_DOWN_ROUTED) row_out = p.perm[row_base + r];
  }

  // ---- this block's K range (DOWN_SHARED: split over blockIdx.z in units
  // of 4 stages) and this wave's quarter of it
  const int nsplit = gridDim.z;
  const int units = K / (4 * KPS);
  const int u0 = static_cast<int>(blockIdx.z) * units / nsplit;
  const int u1 = (static_cast<int>(blockIdx.z) + 1) * units / nsplit;
  const int ns = u1 - u0;                       // stages per wave
  const int k0 = u0 * 4 * KPS + __builtin_amdgcn_readfirstlane(wave) * ns * KPS;   // wave-uniform

  // weights: DMA instruction i fills K rows 4i .. 4i+3 of the stage; lane ->
  // row 4i + lane/16, physical chunk lane%16 holding logical chunk
  // c = (lane%16) ^ (row & 15) = 16 columns: down n0 + 16c; gate/up chunks
  // 0..7 the gate columns n0 + 16c, 8..15 the up columns NH + n0 + 16 (c-8)
  // (int4: byte rows are pairs of K rows)
  const int kb0 = QB == 8 ? k0 : k0 / 2;         // first byte row of this wave
  // scalar base: the group's weights from this wave's first byte row; lane
  // offsets within a stage (< QBK + 1 rows) stay in 32 bits
  const uint8_t* wbase = static_cast<const uint8_t*>(shared ? p.B_shared : p.B) +
                         (shared ? 0 : static_cast<int64_t>(g) * (QB == 8 ? K : K / 2) * ldb) +
                         static_cast<int64_t>(kb0) * ldb;
  uint32_t w_off[QINS];
#pragma unroll
  for (int i = 0; i < QINS; ++i) {
    const int kr = 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ (kr & 15);
    const int oc = GU ? n0 + 16 * (c & 7) : n0 + 16 * c;       // output column of the chunk
    const int gc = (GU && c >= 8) ? NH + oc : oc;              // weight column
    w_off[i] = static_cast<uint32_t>(kr * ldb + (oc < NH ? gc : 0));
  }
  const int64_t w_kstride = static_cast<int64_t>(QBK) * ldb;

  // activations, AROW bytes per row and stage.  int8: DMA instruction f
  // fills rows 16f .. 16f+15 (64 B each); lane -> row 16f + lane/4, slot
  // lane%4 holding logical chunk slot ^ ((row >> 1) & 3).  int4: instructions
  // 2f, 2f+1 fill rows 16f + 8i + lane/8 (128 B each), slot lane%8 holding
  // logical chunk slot ^ (row & 7).  GATEUP reads x (routed rows gathered
  // through perm), DOWN the h rows in group order.
  // (scalar base: the A matrix from this wave's first K column; lane byte
  // offsets row * 2K + 2 (chunk * 8), at most 64 * top_k rows)
  const uint8_t* abase = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(shared ? p.A_shared : p.A) + k0);
  uint32_t a_off[FMMAX * AINS];
#pragma unroll
  for (int f = 0; f < FMMAX; ++f)
#pragma unroll
    for (int i = 0; i < AINS; ++i) {
      const int tr = QB == 8 ? (lane >> 2) : 8 * i + (lane >> 3);     // row within the fragment
      const int slot = QB == 8 ? (lane & 3) : (lane & 7);
      const int lc = QB == 8 ? (slot ^ ((tr >> 1) & 3)) : (slot ^ (tr & 7));
      const int r = min(m0 + 16 * f + tr, rows - 1);
      const int arow = (GU && !shared) ? slot_token(p.perm[row_base + r], p.top_k) : row_base + r;
      a_off[f * AINS + i] = static_cast<uint32_t>((static_cast<int64_t>(arow) * K + lc * 8) * 2);
    }

  const uint32_t ring = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_u8*)smem)) +
                        __builtin_amdgcn_readfirstlane(wave) * (DNBUF * STAGE);
  const lds_u8* ring_p = (const lds_u8*)smem + wave * (DNBUF * STAGE);
  // A fragment of a step: row lane%16, K chunk lane/16 (int8) or chunk
  // 2 (lane/16) + step (int4), at its swizzled slot
  const int am = lane & 15, ag = lane >> 4;
  const int a_rd = QB == 8 ? QWSTAGE + am * 64 + ((ag ^ ((am >> 1) & 3)) << 4)
                           : QWSTAGE + am * 128 + (((2 * ag) ^ (am & 7)) << 4);
  const int a_rd1 = QWSTAGE + am * 128 + (((2 * ag + 1) ^ (am & 7)) << 4);   // int4 second step

  f32x4 acc[FMMAX][QFN];
#pragma unroll
  for (int f = 0; f < FMMAX; ++f)
#pragma unroll
    for (int j = 0; j < QFN; ++j) acc[f][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // int4: sum_k x[row][k] of this wave's K range, from one MFMA per step
  // against a fragment of ones (every column of the result is the row sum)
  f32x4 accx = f32x4{0.f, 0.f, 0.f, 0.f};
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4_t{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

#define Q8_ISSUE(st)                                                                           \
  do {                                                                                         \
    const int s_ = min((st), ns - 1);                                                          \
    const uint32_t b_ = ring + static_cast<uint32_t>(((st) % DNBUF) * STAGE);                  \
    const uint8_t* const wst_ = wbase + s_ * w_kstride;                                        \
    const uint8_t* const ast_ = abase + s_ * (KPS * 2);                                        \
    _Pragma("unroll") for (int i = 0; i < QINS; ++i)                                           \
      dma16_s_nt(wst_, w_off[i], b_ + i * 1024);                                               \
    _Pragma("unroll") for (int f = 0; f < FMMAX * AINS; ++f)                                   \
      dma16_s(ast_, a_off[f], b_ + QWSTAGE + f * 1024);                                        \
  } while (0)
#define Q8_STEP(kt)                                                                            \
  do {                                                                                         \
    Q8_ISSUE((kt) + DNBUF - 1);                                                                \
    wait_vmcnt<(DNBUF - 1) * LOADS>();                                                         \
    const lds_u8* st_ = ring_p + ((kt) % DNBUF) * STAGE;                                       \
    /* every LDS read of the stage in flight before the first use */                         \
    i32x2 wq[QFN];                                                                             \
    bf16x8 af[FMMAX], af1[FMMAX];                                                              \
    _Pragma("unroll") for (int j = 0; j < QFN; ++j) wq[j] = read_q_frag(st_, j * 16, lane);    \
    _Pragma("unroll") for (int f = 0; f < FMMAX; ++f) {                                        \
      af[f] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(st_ + a_rd + f * 16 * AROW); \
      if constexpr (QB == 4)                                                                   \
        af1[f] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(st_ + a_rd1 + f * 16 * AROW); \
    }                                                                                          \
    if constexpr (QB == 8) {                                                                   \
      bf16x8 wf[QFN];                                                                          \
      _Pragma("unroll") for (int j = 0; j < QFN; ++j) wf[j] = q_to_bf16(wq[j]);                \
      _Pragma("unroll") for (int f = 0; f < FMMAX; ++f)                                        \
        if (f < fm)                                                                            \
          _Pragma("unroll") for (int j = 0; j < QFN; ++j)                                      \
            acc[f][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[f], wf[j], acc[f][j], 0, 0, 0); \
    } else {                                                                                   \
      /* codes converted per fragment (transient registers), 16-row tiles */                  \
      af[0] = a4_order(af[0]);                                                                 \
      af1[0] = a4_order(af1[0]);                                                               \
      accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0], ones, accx, 0, 0, 0);              \
      accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af1[0], ones, accx, 0, 0, 0);             \
      /* one fragment at a time: converted just before its two MFMAs (the    */                \
      /* scheduler would otherwise convert all 32 words first and keep them) */                \
      _Pragma("unroll") for (int j = 0; j < QFN; ++j) {                                        \
        const bf16x8 w0 = q4_to_bf16_off(wq[j][0]), w1 = q4_to_bf16_off(wq[j][1]);             \
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0], w0, acc[0][j], 0, 0, 0);    \
        acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af1[0], w1, acc[0][j], 0, 0, 0);   \
        __builtin_amdgcn_sched_barrier(0);                                                     \
      }                                                                                        \
    }                                                                                          \
    /* this stage's slot is refilled DNBUF-1 steps later: reads must be done */                \
    __builtin_amdgcn_s_waitcnt(0xC07F);                                                        \
  } while (0)

#pragma unroll
  for (int st = 0; st < DNBUF - 1; ++st) Q8_ISSUE(st);
  for (int kt = 0; kt < ns; ++kt) Q8_STEP(kt);
  wait_vmcnt<0>();
#undef Q8_ISSUE
#undef Q8_STEP

  // ---- the four K-quarter partial sums through LDS ([row][QPP] fp32 per wave)
  __syncthreads();
  float* part = reinterpret_cast<float*>(smem);
  const int lcol = lane & 15, rq = 4 * (lane >> 4);
#pragma unroll
  for (int f = 0; f < FMMAX; ++f) {
    if (f < fm) {
#pragma unroll
      for (int j = 0; j < QFN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          part[(wave * DBM + 16 * f + rq + q) * QPP + j * 16 + lcol] = acc[f][j][q];
    }
  }
  float* tab = reinterpret_cast<float*>(smem + PART);          // [DBM] gate scales
  int* ot = reinterpret_cast<int*>(smem + PART + 4 * DBM);     // [DBM] output rows
  float* xw = reinterpret_cast<float*>(smem + PART + 8 * DBM); // int4: [4 waves][DBM] row sums, then [DBM] total
  if (tid < DBM) {
    tab[tid] = row_scale;
    ot[tid] = row_out;
  }
  if constexpr (QB == 4) {
    if (lcol == 0 && fm > 0)
#pragma unroll
      for (int q = 0; q < 4; ++q) xw[wave * DBM + rq + q] = accx[q];
    __syncthreads();
    if (tid < DBM) xw[4 * DBM + tid] = 136.0f * (((xw[tid] + xw[DBM + tid]) + xw[2 * DBM + tid]) + xw[3 * DBM + tid]);
  }
  __syncthreads();
  // the K-quarter sums in wave order (int4: less the code offset 136 sum_k x_k)
  auto total = [&](int r, int c) -> float {
    const float v = ((part[(0 * DBM + r) * QPP + c] + part[(1 * DBM + r) * QPP + c]) + part[(2 * DBM + r) * QPP + c]) +
                    part[(3 * DBM + r) * QPP + c];
    if constexpr (QB == 4) return v - xw[4 * DBM + r];
    return v;
  };
  const float* sbase = shared ? p.sB_shared : p.sB + static_cast<int64_t>(g) * ldb;

  if constexpr (GU) {
    // SwiGLU: h = SiLU(s_g acc_g t) * (s_u acc_u t), t = the token's gate on
    // routed rows (1 on shared rows); thread -> one output column, rows in turn
    const int c = tid % OUTC;
    const int col = n0 + c;
    const float sg = col < NH ? sbase[col] : 0.f;
    const float su = col < NH ? sbase[NH + col] : 0.f;
    uint16_t* C = static_cast<uint16_t*>(shared ? p.C_shared : p.C);
    constexpr int NIT = DBM * OUTC / 256;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = (tid + 256 * it) / OUTC;
      if (r >= nvalid || col >= NH) continue;
      const float t = tab[r];
      const float gv = total(r, c) * sg * t;
      const float uv = total(r, c + OUTC) * su * t;
      C[static_cast<int64_t>(row_base + m0 + r) * NH + col] = f32_to_bf16(silu_f(gv) * uv);
    }
  } else {
    // down: thread -> one output column (tile column tid), rows in turn
    const int c = tid;
    const int col = n0 + c;
    const float sc = col < NH ? sbase[col] : 0.f;
    constexpr int NIT = DBM;
    if constexpr (MODE == MODE_DOWN_SHARED) {
      float* Cs = static_cast<float*>(p.C_shared) + static_cast<int64_t>(blockIdx.z) * T * NH;
#pragma unroll 4
      for (int r = 0; r < NIT; ++r)
        if (r < nvalid && col < NH) Cs[static_cast<int64_t>(m0 + r) * NH + col] = total(r, c) * sc;
    } else {
      // the shared expert's output, y_parts K-split partials summed in order
      const int nparts = !p.Y ? 0 : p.y_parts > 1 ? p.y_parts : 1;
      const int64_t pstride = static_cast<int64_t>(T) * NH;
#pragma unroll 4
      for (int r = 0; r < NIT; ++r) {
        if (r >= nvalid || col >= NH) continue;
        const int64_t o = static_cast<int64_t>(ot[r]) * NH + col;
        float y = 0.f;
        for (int q = 0; q < nparts; ++q) y += p.Y[q * pstride + o];
        const float v = nparts ? total(r, c) * sc + y : total(r, c) * sc;
        if (p.out_bf16) static_cast<uint16_t*>(p.C)[o] = f32_to_bf16(v);
        else static_cast<float*>(p.C)[o] = v;
      }
    }
  }
}

template <int MODE, int FMMAX, int QB>
hipError_t launch_q8(const GemmArgs& a0, int T, hipStream_t s, const int32_t* tiles_all) {
  constexpr int DBM = 16 * FMMAX;
  GemmArgs a = a0;
  a.tiles = tiles_all + bm_index(DBM) * (a.E + 2);
  const int mt_tok = (T + DBM - 1) / DBM;
  const bool shared_only = MODE == MODE_DOWN_SHARED || (MODE == MODE_GATEUP && a.group_lo == a.E);
  if (MODE == MODE_GATEUP && !shared_only && a.group_hi > a.E) return hipErrorInvalidValue;   // one kind per launch
  const int mt_r = (T * (a.top_k > 1 ? a.top_k : 1) + DBM - 1) / DBM;   // routed rows are slots
  const int gm = shared_only ? mt_tok : mt_r + a.E;
  const int NH = (MODE == MODE_GATEUP && shared_only) ? a.N_shared : a.N;
  const int gn = (NH + (MODE == MODE_GATEUP ? QBN / 2 : QBN) - 1) / (MODE == MODE_GATEUP ? QBN / 2 : QBN);
  if (gm <= 0 || gn <= 0) return hipSuccess;
  const int ks = (MODE == MODE_DOWN_SHARED && a.ksplit > 1) ? a.ksplit : 1;
  constexpr int unit = QB == 8 ? 128 : 256;   // K rows of 4 waves' stages
  if (a.K % unit != 0 || a.K / unit < ks || NH % 16 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_q8_kernel<MODE, FMMAX, QB>), dim3(gm, gn, ks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int MODE, int FMMAX>
hipError_t launch_dec(const GemmArgs& a0, int T, hipStream_t s, const int32_t* tiles_all) {
  constexpr int DBM = 16 * FMMAX;
  GemmArgs a = a0;
  a.tiles = tiles_all + bm_index(DBM) * (a.E + 2);
  const int mt_tok = (T + DBM - 1) / DBM;
  const int mt_r = (T * (a.top_k > 1 ? a.top_k : 1) + DBM - 1) / DBM;   // routed rows are slots
  const int gm = MODE == MODE_DOWN_SHARED ? mt_tok : mt_r + a.E;
  if (gm <= 0) return hipSuccess;
  const int gn = (a.N + DBN - 1) / DBN;
  const int ks = (MODE == MODE_DOWN_SHARED && a.ksplit > 1) ? a.ksplit : 1;
  if (a.K % 128 != 0 || a.K / 128 < ks) return hipErrorInvalidValue;   // >= one 128-row unit per part
  hipLaunchKernelGGL((gemm_decode_kernel<MODE, FMMAX>), dim3(gm, gn, ks), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int FMMAX>
hipError_t launch_dec_gateup(const GemmArgs& a0, int T, hipStream_t s, const int32_t* tiles_all) {
  constexpr int DBM = 16 * FMMAX;
  GemmArgs a = a0;
  a.tiles = tiles_all + bm_index(DBM) * (a.E + 2);
  const bool has_routed = a.group_lo < a.E;
  const bool has_shared = a.group_hi > a.E;
  const int mt_tok = (T + DBM - 1) / DBM;
  const int mt_r = (T * (a.top_k > 1 ? a.top_k : 1) + DBM - 1) / DBM;   // routed rows are slots
  const int gm = (has_routed ? mt_r + a.E : 0) + (has_shared ? mt_tok : 0);
  const int nmax = std::max(has_routed ? a.N : 0, has_shared ? a.N_shared : 0);
  const int gn = (nmax + GBNH - 1) / GBNH;
  if (gm <= 0 || gn <= 0) return hipSuccess;
  // partial mode (gu_part): K split over ksplit workgroups, no SwiGLU (and
  // no gate scale) here: the shared group alone
  if (a.gu_part && has_routed) return hipErrorInvalidValue;
  const int ks = (a.gu_part && a.ksplit > 1) ? a.ksplit : 1;
  if (a.K % (4 * GBK * ks) != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_decode_gateup_kernel<FMMAX>), dim3(gm, gn, ks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int K) { return K % 128 == 0 && K >= 128; }

hipError_t launch_gemm_decode_tail(int mode, const GemmArgs& a0, int bm_main, hipStream_t s,
                                   const int32_t* tiles_all) {
  static_assert(kTailRows == 32, "tails are single 32-row tiles");
  GemmArgs a = a0;
  // bm_main == 0: the groups of at most kTailRows rows (class table), whole
  a.tiles = tiles_all + (bm_main > 0 ? table_tail(bm_main) : table_class(kTailRows)) * (a.E + 2);
  a.tail_bm = bm_main > 0 ? bm_main : (1 << 30);
  a.group_lo = 0;
  a.group_hi = a.E;
  // one tail tile per group at most.  Grid (column tile, row tile), column
  // tile fastest: a group's workgroups spread over the 8 XCDs (ids go
  // round-robin) whichever groups have tails, and run together on adjacent
  // segments of the same weight rows, which the group's main tiles also read
  const int gm = a.E;
  if (gm <= 0 || a.N <= 0) return hipSuccess;
  if (mode == MODE_GATEUP) {
    if (a.K % (4 * GBK) != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_decode_gateup_kernel<2>), dim3((a.N + GBNH - 1) / GBNH, gm), dim3(256), 0, s, a);
  } else if (mode == MODE_DOWN_ROUTED) {
    if (a.K % 128 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_decode_kernel<MODE_DOWN_ROUTED, 2>), dim3((a.N + DBN - 1) / DBN, gm, 1), dim3(256), 0,
                       s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// rows32: 32-row tiles (for groups that may exceed 16 rows), else 16-row tiles.
hipError_t launch_gemm_decode(int mode, bool rows32, const GemmArgs& a, int T, hipStream_t s,
                              const int32_t* tiles_all) {
  if (a.w_int8) {
    if (a.gu_part || (a.w_int8 != 8 && a.w_int8 != 4)) return hipErrorInvalidValue;
    const bool q4 = a.w_int8 == 4;
#define Q8_DISPATCH(FM)                                                                        \
    switch (mode) {                                                                            \
      case MODE_GATEUP:                                                                        \
        return q4 ? launch_q8<MODE_GATEUP, 1, 4>(a, T, s, tiles_all) : launch_q8<MODE_GATEUP, FM, 8>(a, T, s, tiles_all); \
      case MODE_DOWN_SHARED:                                                                   \
        return q4 ? launch_q8<MODE_DOWN_SHARED, 1, 4>(a, T, s, tiles_all)                      \
                  : launch_q8<MODE_DOWN_SHARED, FM, 8>(a, T, s, tiles_all);                    \
      case MODE_DOWN_ROUTED:                                                                   \
        return q4 ? launch_q8<MODE_DOWN_ROUTED, 1, 4>(a, T, s, tiles_all)                      \
                  : launch_q8<MODE_DOWN_ROUTED, FM, 8>(a, T, s, tiles_all);                    \
    }
    // int4 takes 16-row tiles only: a 32-row int4 tile needs more registers
    // than a wave has (its spills cost more than re-streaming the weights of
    // the few groups with more than 16 rows)
    if (rows32 && !q4) { Q8_DISPATCH(2) } else { Q8_DISPATCH(1) }
#undef Q8_DISPATCH
    return hipErrorInvalidValue;
  }
  if (rows32) {
    switch (mode) {
      case MODE_GATEUP: return launch_dec_gateup<2>(a, T, s, tiles_all);
      case MODE_DOWN_SHARED: return launch_dec<MODE_DOWN_SHARED, 2>(a, T, s, tiles_all);
      case MODE_DOWN_ROUTED: return launch_dec<MODE_DOWN_ROUTED, 2>(a, T, s, tiles_all);
    }
  } else {
    switch (mode) {
      case MODE_GATEUP: return launch_dec_gateup<1>(a, T, s, tiles_all);
      case MODE_DOWN_SHARED: return launch_dec<MODE_DOWN_SHARED, 1>(a, T, s, tiles_all);
      case MODE_DOWN_ROUTED: return launch_dec<MODE_DOWN_ROUTED, 1>(a, T, s, tiles_all);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
