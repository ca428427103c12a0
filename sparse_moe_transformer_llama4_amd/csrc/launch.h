// Kernel argument blocks and host-side launchers (internal to libmoe355).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Debug builds (-DMOE_DEBUG): device-side checks of the structure a kernel
// derives addresses from (routing indices, group offsets, tile tables).  A
// failed check sets bit `bit` of *flags (a word of the workspace the host
// reads after the call) and the caller then skips the work it guards, so a
// broken invariant becomes an error code instead of an out-of-bounds access.
// Release builds compile every check to `true`.
enum DebugBit {
  kDbgIdx = 0,      // an expert index outside [0, E)
  kDbgOffsets = 1,  // offsets / counts inconsistent (offsets[0] != 0, decreasing, offsets[E] != T k)
  kDbgPerm = 2,     // perm entry outside [0, T k), in another expert's group, or out of slot order
  kDbgTiles = 3,    // a tile table not starting at 0 or decreasing
  kDbgTile = 4,     // a GEMM tile outside its group's rows
};
#ifdef MOE_DEBUG
__device__ __forceinline__ bool dbg_check(uint32_t* flags, bool ok, int bit) {
  if (!ok && flags) atomicOr(flags, 1u << bit);
  return ok;
}
#define MOE_DCHECK(flags, cond, bit) ::moe::dbg_check((flags), (cond), (bit))
#else
__host__ __device__ constexpr bool dbg_pass() { return true; }
#define MOE_DCHECK(flags, cond, bit) ::moe::dbg_pass()
#endif

struct RouterArgs {
  const void* x;      // [T][d] x dtype
  const void* wr;     // [d][E] x dtype
  const float* bias;  // [E] or nullptr
  int T, d, E;
  int32_t* idx;       // [T * k]: slot t*k + j = the token's j-th pick
  float* gate;        // [T * k]
  int32_t* hist;      // [nblocks][E] picks (slots) per block of kRouteTokens tokens
  int k;              // experts per token, 1 .. kMaxTopK
};

// Largest number of experts per token.
constexpr int kMaxTopK = 8;

// The token a routing slot belongs to (slot = token * k + rank).
__host__ __device__ inline int slot_token(int slot, int k) { return k > 1 ? slot / k : slot; }

struct ScanArgs {
  int32_t* hist;  // [nblocks][E], replaced by per-block bases
  int nblocks, E, T;
  int32_t* counts;   // [E]
  int32_t* offsets;  // [E + 1]
  int32_t* tiles;    // [kNumTables][E + 2]
};

enum GemmMode : int {
  MODE_GATEUP = 0,       // groups 0..E-1 routed (+ group E = shared): h = SiLU(g*acc_gate) * (g*acc_up)
  MODE_DOWN_SHARED = 1,  // y_s = h_s W_down_shared (fp32)
  MODE_DOWN_ROUTED = 2   // out[perm[r]] = h_r[r] W_down[e] + y_s[perm[r]]
};

struct GemmArgs {
  const void* A;         // routed A: x / x codes (GATEUP, gathered through perm) or h_r (DOWN)
  const void* A_shared;  // shared A: x / x codes (GATEUP) or h_s (DOWN_SHARED)
  const void* B;         // routed weights [E][K][Nb]
  const void* B_shared;  // shared weights [K][Nb]
  const float* sB;       // e4m3: routed column scales [E][Nb]
  const float* sB_shared;
  const float* sA;       // e4m3: per-row scale of A (x scale by token, or h scale by row)
  const float* sA_shared;
  int K;
  int N;                 // GATEUP: routed half width f; DOWN: d
  int N_shared;          // GATEUP: shared half width fs; DOWN_ROUTED over groups .. E: fs (must equal K)
  int T, E;
  const int32_t* offsets;
  const int32_t* perm;
  const int32_t* tiles;  // tile table row for this launch's BM ([E + 2])
  const float* gate;     // [T] by token
  void* C;               // GATEUP: h_r [T][f]; DOWN_ROUTED: out [T][d]; DOWN_SHARED: y_s
  void* C_shared;        // GATEUP: h_s [T][fs]
  uint8_t* C_lo;         // e4m3 GATEUP: h is stored in 24 bits (each fp32 pattern rounded at bit 8), bits
  uint8_t* C_shared_lo;  // 31..16 in C (uint16) and bits 15..8 here (one byte per element, same indexing)
  const float* Y;        // DOWN_ROUTED: y_s [T][d]
  uint32_t* amax;        // e4m3 GATEUP: per-row max |h| bits (routed rows)
  uint32_t* amax_shared;
  int out_bf16;          // DOWN_ROUTED: output dtype bf16 (else fp32)
  int group_lo, group_hi;  // groups [lo, hi) handled by this launch (group E = shared expert)
  int n_tiles;             // N-tiles per M-tile of this launch (set by the launcher)
  int ksplit;              // decode DOWN_SHARED (and GATEUP with gu_part): K split over blocks; partial s at
                           // C_shared + s*T*N (0 = 1).  DOWN_SHARED: parts take K/128-row units in turn, not
                           // necessarily equal counts (ksplit <= K/128); GATEUP: ksplit must divide K/64
  int y_parts;             // decode DOWN_ROUTED: Y holds this many partials, summed in order (0 = 1)
  int tail_bm;             // weight-streaming tail launches: rows of the groups' full main tiles (0 = none)
  int top_k;               // experts per token (0 / 1 = one): routed rows are slots, the routed gate/up
                           // reads x row slot_token(perm[.], top_k), grids cover T * top_k routed rows
  float* gu_part;          // weight-streaming GATEUP: write fp32 pre-activation partials [ksplit][T][2 N] here
                           // instead of h (K split over ksplit workgroups; null = normal epilogue)
  int w_int8;              // weight-streaming kernels: 8 = B / B_shared hold int8 codes, 4 = int4 codes packed two
                           // per byte along K (low nibble = even row), sB / sB_shared their fp32 column scales
                           // (a GATEUP launch covers the routed groups or the shared one, not both); 0 = none
  uint32_t* dbg;           // debug builds: the check flags (MOE_DCHECK); unused otherwise
};

// A tile (group g, first row m0 of the group's `rows`) lies inside its
// group: the check every grouped GEMM makes after its tile lookup in debug
// builds (group E, the shared expert, has T rows and no offsets).
#define MOE_DCHECK_TILE(p, g, m0, rows)                                                                 \
  MOE_DCHECK((p).dbg,                                                                                   \
             (g) >= 0 && (g) <= (p).E && (m0) >= 0 && (m0) < (rows) &&                                  \
                 ((g) == (p).E || ((p).offsets[g] >= 0 && (p).offsets[g] + (rows) <= (p).offsets[(p).E])), \
             kDbgTile)

// Router in two launches: partial logits over K slices of d (the slice count
// grows for few tokens so the GPU fills), then a fixed-order sum + top-1 +
// gate + histogram.  `part` holds router_splits(T, d) * T * E floats.
int router_splits(int T, int d, int x_dtype);
hipError_t launch_router(const RouterArgs& a, int x_dtype, float* part, hipStream_t s);
// T <= 64: partial logits, then one workgroup does top-1, gate, counts,
// offsets, tile tables and the stable permutation.
hipError_t launch_route_small(const RouterArgs& a, int x_dtype, float* part, int32_t* counts, int32_t* offsets,
                              int32_t* tiles, int32_t* perm, hipStream_t s);
hipError_t launch_scan(const ScanArgs& a, hipStream_t s);
hipError_t launch_perm(const int32_t* idx, const int32_t* base, const int32_t* offsets, int T, int E, int k,
                       int32_t* perm, hipStream_t s);
// The fixed-order finish of launch_router over `nsplit` partial logit slices
// (used with nsplit = 1 when the logits come from the prefill GEMM).
hipError_t launch_router_finish(const RouterArgs& a, int nsplit, const float* part, hipStream_t s);
// Per-token e4m3 codes and scales of bf16 x; with zero_a /
// zero_b also zero_a[t] = 0 and zero_b[t * kb + j] = 0 for j < kb.
hipError_t launch_quant_x(const uint16_t* x, int T, int d, uint8_t* xq, float* sx, hipStream_t s,
                          uint32_t* zero_a = nullptr, uint32_t* zero_b = nullptr, int kb = 0);
// RMSNorm of x's rows into xn (x's dtype, DT_BF16 or DT_F32); with xq / sx
// (bf16 only) also xn's per-token e4m3 codes and scales.
hipError_t launch_rmsnorm(int x_dtype, const void* x, const void* w, int T, int d, float eps, void* xn,
                          uint8_t* xq, float* sx, hipStream_t s);
// The RMSNorm fused with the router GEMM (bf16 x, d a multiple of 128 up to
// 5120, 1 <= E <= 128): packs W_router into wr_pack (norm_route_pack_bytes),
// then writes xn (and, with xq / sx non-null, xn's e4m3 codes and per-token
// scales) and the fp32 logits [T][E] without the bias.  With w == nullptr
// there is no norm: x's own e4m3 codes and scales (xq, sx required) and its
// logits, xn unused.
bool norm_route_supported(int x_dtype, int d, int E);
size_t norm_route_pack_bytes(int d, int E);
hipError_t launch_norm_route(const void* x, const void* w, int T, int d, int E, float eps, const void* wr,
                             void* wr_pack, void* xn, uint8_t* xq, float* sx, float* logits, hipStream_t s);
// T <= 64 with the logits [T][E] already computed: top-k, gate, counts,
// offsets, tile tables and the permutation in one workgroup.
hipError_t launch_route_small_finish(const RouterArgs& a, const float* logits, int32_t* counts, int32_t* offsets,
                                     int32_t* tiles, int32_t* perm, hipStream_t s);
hipError_t launch_quant_h(const uint16_t* h, const uint8_t* h_lo, const uint32_t* amax, int rows, int n,
                          uint8_t* hq, float* sh, hipStream_t s);
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
// Debug builds: check every routing invariant the GEMMs rely on (expert
// indices, offsets against counts, perm grouped by expert in slot order,
// tile tables non-decreasing from 0) and record failures in *flags; then, if
// any flag is set, zero the tile tables so that no grouped GEMM tile runs on
// the broken routing.  S = T * k routed slots; tables: kNumTables rows of
// E + 2 entries.
hipError_t launch_validate_routing(const int32_t* idx, const int32_t* counts, const int32_t* offsets,
                                   const int32_t* perm, int32_t* tiles, int S, int E, uint32_t* flags,
                                   hipStream_t s);
// Debug builds, tests of the check path: overwrite perm[0] with perm[S - 1]
// (an in-range slot in the wrong place) before the validation runs.
hipError_t launch_debug_break_perm(int32_t* perm, int S, hipStream_t s);
// out = r + y[0] + y[1] + ... + y[parts-1] element by element, in that order
// (n fp32 values per array, n % 4 == 0; r may be null), stored as bf16 when
// out_bf16: the combine of the two down GEMMs when they run unordered, and the
// sum of a dense layer's K-split partials.
hipError_t launch_combine(const float* r, const float* y, int parts, void* out, int64_t n, int out_bf16,
                          hipStream_t s);
// out[t] = y[t] (+ its partials in order) + r[t*k] + ... + r[t*k + k - 1] (fp32; r: [T*k][d] slot rows)
hipError_t launch_combine_topk(const float* r, int k, const float* y, int parts, void* out, int T, int d,
                               int out_bf16, hipStream_t s);
// h[t][c] = bf16(SiLU(g) * u), g = sum over the parts of gu[q][t][c], u of
// gu[q][t][N + c], in order (parts of a K-split gate/up GEMM; N % 4 == 0).
hipError_t launch_swiglu_parts(const float* gu, int parts, int T, int N, uint16_t* h, hipStream_t s);

// Grouped GEMM launch.  `grid_m` is an upper bound of M tiles; surplus
// workgroups exit after reading the tile table.
hipError_t launch_gemm(int mode, int w_dtype, const GemmArgs& a, int grid_m_tokens, hipStream_t s,
                       const int32_t* tiles_all);

// bf16 prefill tiling (BM in {64, 128, 256} rows x 256 weight columns).
bool bf16_v2_supported(int K, int N, int N_shared);
hipError_t launch_gemm_bf16_v2(int mode, int bm, const GemmArgs& a, int T, hipStream_t s,
                               const int32_t* tiles_all);
// The 256-row tiles of launch_gemm_bf16_v2 (separate unit: AGPR-form MFMAs).
hipError_t launch_gemm_bf16_tall(int mode, const GemmArgs& a, int T, hipStream_t s, const int32_t* tiles_all);

// fp8 prefill tiling (bm x 256 tiles, K 128 per stage; K multiple of 128):
// bm = 128, or 160 for MODE_GATEUP and MODE_DOWN_ROUTED.
hipError_t launch_gemm_fp8(int mode, int bm, const GemmArgs& a, int T, hipStream_t s, const int32_t* tiles_all);

// bf16 weight-streaming tiling for decode-sized T (16- or 32-row tiles, K
// split over the 4 waves; K must be a multiple of 128).  Gate/up tiles are 128
// gate + 128 up columns, down tiles 128 columns.  A gate/up or shared down
// launch over the shared group alone does not read the routing tables.
bool decode_supported(int K);
hipError_t launch_gemm_decode(int mode, bool rows32, const GemmArgs& a, int T, hipStream_t s,
                              const int32_t* tiles_all);
// The tails of the routed groups for main tiles of bm_main rows (table
// table_tail(bm_main): one 32-row tile per group, starting after the group's
// full bm_main-row tiles) on the weight-streaming tiles: MODE_GATEUP (SwiGLU
// epilogue) or MODE_DOWN_ROUTED (un-permute + combine with the y_parts shared
// partials).  The rest is left to launches over table_main(bm_main).
// bm_main == 0 takes the groups of at most 32 rows whole (table_class(32)).
hipError_t launch_gemm_decode_tail(int mode, const GemmArgs& a, int bm_main, hipStream_t s,
                                   const int32_t* tiles_all);

}  // namespace moe
