// Host side of libmoe355: the C ABI declared in include/moe.h.
// Validation happens before any enqueue; the launch sequence is
//   router -> scan -> permutation -> grouped gate/up GEMM (+ shared) ->
//   [e4m3: quantise h] -> shared down GEMM -> routed down GEMM + combine,
// on the caller's stream, with no host synchronisation.  Decode-sized bf16
// calls run the shared expert's two GEMMs on a side stream forked from and
// joined back into the caller's stream.
#include <algorithm>
#include <atomic>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "common.h"
#include "launch.h"
#include "moe.h"

using namespace moe;

// Side stream of one device for the decode schedule, with its fork / join
// events (no timing).  Created on first use, default priority.
struct AuxStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;  // side stream starts after / main stream resumes after
  hipEvent_t routed = nullptr;                // routing done (main stream)
  hipEvent_t shared = nullptr;                // shared expert's output done (side stream)
  hipEvent_t gateup = nullptr;                // routed main gate/up tiles done (main stream)
};
constexpr int kMaxDevices = 16;

struct moe_plan_s {
  moe_config cfg;
  int last_hip_error;
  std::mutex mu;               // guards aux and each fork / join enqueue sequence
  AuxStream aux[kMaxDevices];  // by device id
};

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-launch events of moe_forward_traced: while a traced call is enqueued
// on this thread, every launch below is bracketed by two events recorded on
// the stream the launch goes to.  Null (no tracing) for every other call.
struct Trace {
  hipEvent_t* ev;          // [2 * cap]
  moe_launch_record* rec;  // [cap]
  int cap, n;
  hipStream_t caller;
  hipError_t err;
};
thread_local Trace* g_trace = nullptr;

void trace_begin(const char* name, int tile_rows, int groups, int part, hipStream_t s) {
  Trace* t = g_trace;
  if (!t) return;
  if (t->n >= t->cap) {
    if (t->err == hipSuccess) t->err = hipErrorInvalidValue;
    return;
  }
  t->rec[t->n] = moe_launch_record{name, s != t->caller ? 1 : 0, tile_rows, groups, part};
  const hipError_t e = hipEventRecord(t->ev[2 * t->n], s);
  if (e != hipSuccess && t->err == hipSuccess) t->err = e;
}

hipError_t trace_end(hipStream_t s, hipError_t call) {
  Trace* t = g_trace;
  if (!t || t->n >= t->cap) return call;
  const hipError_t e = hipEventRecord(t->ev[2 * t->n + 1], s);
  ++t->n;
  return call != hipSuccess ? call : e;
}

// groups: 0 routed, 1 shared, 2 both, -1 not a GEMM; part: 0 all rows,
// 1 the main tiles (tails left out), 2 the tails alone
#define TRACED(name, rows, groups, part, s, call) \
  (trace_begin((name), (rows), (groups), (part), (s)), trace_end((s), (call)))

bool config_dtypes_ok(const moe_config& c) {
  if (c.x_dtype == MOE_F32 && c.w_dtype == MOE_F32 && c.out_dtype == MOE_F32) return true;
  if (c.x_dtype == MOE_BF16 && c.w_dtype == MOE_BF16 && (c.out_dtype == MOE_F32 || c.out_dtype == MOE_BF16))
    return true;
  if (c.x_dtype == MOE_BF16 && c.w_dtype == MOE_E4M3 && c.out_dtype == MOE_BF16) return true;
  if (c.x_dtype == MOE_BF16 && (c.w_dtype == MOE_INT8 || c.w_dtype == MOE_INT4) &&
      (c.out_dtype == MOE_F32 || c.out_dtype == MOE_BF16))
    return true;
  return false;
}

bool scaled_weights(const moe_config& c) {
  return c.w_dtype == MOE_E4M3 || c.w_dtype == MOE_INT8 || c.w_dtype == MOE_INT4;
}
bool int_weights(const moe_config& c) { return c.w_dtype == MOE_INT8 || c.w_dtype == MOE_INT4; }

// int4: 4 waves x 64 K rows per stage of the weight-streaming tiles
int k_multiple(const moe_config& c) { return c.w_dtype == MOE_INT4 ? 256 : scaled_weights(c) ? 128 : 64; }

constexpr int64_t kDecodeTokensMax = 64;
// Token count from which the bf16 prefill tiling is used.
constexpr int64_t kPrefillTokens = 256;

// Decode-sized calls split the shared down GEMM over K (its single M-tile
// would leave most CUs idle): the number of partial shared outputs, summed in
// order by the routed down GEMM.  1 for every other path.
int decode_y_parts(const moe_config& c, int64_t T) {
  if (T > kDecodeTokensMax || (c.w_dtype != MOE_BF16 && !int_weights(c))) return 1;
  const int unit = c.w_dtype == MOE_INT4 ? 256 : 128;   // K rows per part at least (4 waves' stages)
  for (int s = 8; s > 1; s >>= 1)
    if (c.f_shared % (unit * s) == 0) return s;
  return 1;
}

// The weight-streaming decode tiling serves bf16 calls of at most 64 tokens
// and every int8 call (a plan with int8 weights takes at most 64 tokens).
bool use_decode(const moe_config& c, int64_t T) {
  return (c.w_dtype == MOE_BF16 || int_weights(c)) && T > 0 && T <= kDecodeTokensMax &&
         decode_supported(c.d) && decode_supported(c.f) && decode_supported(c.f_shared);
}

// A dense layer's gate/up GEMM at decode sizes has one row tile per 128
// output columns, too few workgroups for the GPU: its K is split into this
// many parts (at most 4, until there are >= 256 workgroups), whose fp32
// pre-activation partials are summed before the SwiGLU.  1 otherwise.
int dense_gateup_parts(const moe_config& c, int64_t T) {
  if (c.n_experts != 0 || T < 1 || T > kDecodeTokensMax) return 1;
  const int64_t wg = ((T + 31) / 32) * (c.f_shared / 128);
  int ks = 1;
  while (ks < 4 && wg * ks < 256 && c.d % (128 * ks) == 0) ks *= 2;
  return ks;
}

// The same layer's down GEMM (the shared group alone, d / 128 column tiles
// per 32-row tile): K parts for about one workgroup per CU, 1..8.
int dense_down_parts(const moe_config& c, int64_t T) {
  if (c.n_experts != 0 || T < 1 || T > kDecodeTokensMax) return 1;
  const int64_t wg = ((T + 31) / 32) * ((c.d + 127) / 128);
  const int64_t ks = std::min<int64_t>({8, std::max<int64_t>(1, 256 / wg), c.f_shared / 128});
  return static_cast<int>(ks);
}

// The RMSNorm runs inside the router kernel (one read of x for both) when
// the block has a router of at most 32 experts and the fused kernel takes the
// shape; with e4m3 weights and no norm the same kernel quantises x while it
// computes the logits (again one read of x).  Every 16 rows of the fused
// kernel read the whole router weight from L2: at 128 experts (1.3 MB at
// d = 5120) that traffic made it slower than the stand-alone norm and router
// GEMM (measured on the Maverick-shaped fp8 layer: 0.43 against 0.18 ms with
// the norm, 0.18 against 0.13 ms without).
bool fused_norm_route(const moe_config& c) {
  return (c.has_norm || c.w_dtype == MOE_E4M3) && c.n_experts > 0 && c.n_experts <= 32 &&
         norm_route_supported(c.x_dtype, c.d, c.n_experts);
}

WsLayout layout_for(const moe_config& c, int64_t T) {
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t E = static_cast<size_t>(c.n_experts);
  const size_t t = static_cast<size_t>(T);
  const size_t nb = (t + kRouteTokens - 1) / kRouteTokens;
  const bool fp8 = c.w_dtype == MOE_E4M3;
  // h: fp32 for fp32 weights, else bf16; e4m3: 24 bits in two planes (the
  // upper 16 bits of the fp32 value here, the next 8 in h_r_lo / h_s_lo)
  const size_t hsz = c.w_dtype == MOE_F32 ? 4 : 2;
  const size_t ts = t * static_cast<size_t>(c.top_k > 1 ? c.top_k : 1);   // routing slots (routed rows)
  L.idx = take(ts * 4);
  L.gate = take(ts * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(ts * 4);
  L.hist = take(nb * E * 4);
  L.logits = take(static_cast<size_t>(router_splits(static_cast<int>(T), c.d, c.x_dtype)) * t * E * 4);
  L.tiles = take(kNumTables * (E + 2) * 4);
  L.h_r = take(ts * c.f * hsz);
  L.h_s = take(t * c.f_shared * hsz);
  L.y_s = take(t * c.d * 4 * static_cast<size_t>(std::max(decode_y_parts(c, T), dense_down_parts(c, T))));
  if (c.top_k > 1) L.r_out = take(ts * c.d * 4);   // routed output by slot, summed per token by the combine
  else if (c.w_dtype == MOE_BF16 && T >= kPrefillTokens) L.r_out = take(t * c.d * 4);
  if (dense_gateup_parts(c, T) > 1)
    L.gu_part = take(static_cast<size_t>(dense_gateup_parts(c, T)) * t * 2 * c.f_shared * 4);
  if (c.has_norm) L.x_n = take(t * c.d * (c.x_dtype == MOE_F32 ? 4 : 2));
  if (fused_norm_route(c)) L.wr_pack = take(norm_route_pack_bytes(c.d, c.n_experts));
  if (fp8) {
    L.h_r_lo = take(ts * c.f);
    L.h_s_lo = take(t * c.f_shared);
    L.hq_r = take(ts * c.f);
    L.hq_s = take(t * c.f_shared);
    L.sh_r = take(ts * 4);
    L.sh_s = take(t * 4);
    L.amax_r = take(ts * 4);
    L.amax_s = take(t * 4);
    L.xq = take(t * c.d);
    L.sx = take(t * 4);
  }
  L.dbg = take(4);
  L.total = off;
  return L;
}

moe_status hip_fail(moe_plan_t p, hipError_t e) {
  p->last_hip_error = static_cast<int>(e);
  return MOE_ERR_HIP;
}

moe_status check_common(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, void* ws,
                        size_t ws_bytes) {
  if (!plan || !w) return MOE_ERR_INVALID_ARGUMENT;
  const moe_config& c = plan->cfg;
  if (T < 0 || T > c.max_tokens) return MOE_ERR_SHAPE;
  if (T > 0 && (!x || !aligned16(x))) return MOE_ERR_INVALID_ARGUMENT;
  if (c.n_experts > 0 && (!w->w_router || !aligned16(w->w_router))) return MOE_ERR_INVALID_ARGUMENT;
  if (c.has_router_bias && (!w->router_bias || !aligned16(w->router_bias))) return MOE_ERR_INVALID_ARGUMENT;
  if (c.has_norm && (!w->norm_weight || !aligned16(w->norm_weight))) return MOE_ERR_INVALID_ARGUMENT;
  if (layout_for(c, T).total > ws_bytes) return MOE_ERR_WORKSPACE;
  if (T > 0 && (!ws || !aligned16(ws))) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

moe_status check_expert_weights(const moe_config& c, const moe_weights* w) {
  const void* req[] = {w->ws_gate_up, w->ws_down, w->w_gate_up, w->w_down};
  for (int i = 0; i < (c.n_experts > 0 ? 4 : 2); ++i)    // a dense layer has no routed experts
    if (!req[i] || !aligned16(req[i])) return MOE_ERR_INVALID_ARGUMENT;
  if (scaled_weights(c)) {
    const void* sc[] = {w->s_gate_up, w->s_down, w->ss_gate_up, w->ss_down};
    for (const void* p : sc)
      if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  }
  return MOE_OK;
}

moe_status check_routing(const moe_routing* r) {
  const void* ps[] = {r->expert_idx, r->gate, r->counts, r->offsets, r->perm};
  for (const void* p : ps)
    if (!p || !aligned16(p)) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

// Pointers of the routing record: the caller's, or workspace-backed.
struct Route {
  int32_t *idx, *counts, *offsets, *perm, *hist, *tiles;
  float *gate, *logits;
  bool logits_ready;   // logits [T][E] (no bias) already written by the fused RMSNorm + router kernel
  uint32_t* dbg;       // the debug builds' check flags (workspace)
};

Route route_ptrs(uint8_t* ws, const WsLayout& L, const moe_routing* r) {
  Route o;
  o.idx = r ? r->expert_idx : reinterpret_cast<int32_t*>(ws + L.idx);
  o.gate = r ? r->gate : reinterpret_cast<float*>(ws + L.gate);
  o.counts = r ? r->counts : reinterpret_cast<int32_t*>(ws + L.counts);
  o.offsets = r ? r->offsets : reinterpret_cast<int32_t*>(ws + L.offsets);
  o.perm = r ? r->perm : reinterpret_cast<int32_t*>(ws + L.perm);
  o.hist = reinterpret_cast<int32_t*>(ws + L.hist);
  o.tiles = reinterpret_cast<int32_t*>(ws + L.tiles);
  o.logits = reinterpret_cast<float*>(ws + L.logits);
  o.logits_ready = false;
  o.dbg = reinterpret_cast<uint32_t*>(ws + L.dbg);
  return o;
}


// Tile height for the routed groups: 256 rows when the mean group holds at
// least 192 tokens, else 128 (a taller tile reuses each weight tile for more
// rows; a shorter one wastes fewer MFMA rows on ragged group tails).  64-row
// tiles lost to 128-row ones even at 64 tokens per expert with skewed routing.
int routed_tile_rows(int64_t T, int E) {
  const int64_t mean = T / E;
  return mean >= 192 ? 256 : 128;
}

// e4m3 tile height of the gate/up and routed down GEMMs: 160 rows when the
// mean routed group holds 96..136 rows (one 160-row tile then takes nearly
// every group whole, where 128-row tiles add a second, nearly empty tile to
// each group above 128 rows), else 128.
int fp8_routed_rows(int64_t Tr, int E) {
  const int64_t mean = E > 0 ? Tr / E : 0;
  return mean >= 96 && mean <= 136 ? 160 : 128;
}

// Tile height for a down GEMM (N = d columns in 256-wide tiles) over `rows`
// tokens in `groups` groups: 256-row tiles when they still give at least
// ~1.5 rounds of workgroups over the GPU's 256 CUs, else 128 (fewer idle CUs
// in the last round outweigh the lower per-tile efficiency).  Measured on the
// Scout- and Maverick-shaped prefill layers.
int down_tile_rows(int64_t rows, int groups, int d, int bm_max) {
  const int64_t ntile = (d + 255) / 256;
  const int64_t t256 = ((rows + 255) / 256 + (groups > 1 ? groups / 2 : 0)) * ntile;
  if (bm_max >= 256 && t256 >= 384) return 256;
  return bm_max >= 128 ? 128 : bm_max;
}

// Debug builds (-DMOE_DEBUG) check the routing on the device before any
// grouped GEMM reads it (launch_validate_routing: on a failure the tile
// tables are zeroed, so no GEMM tile runs) and the GEMMs check each tile
// against its group; every call clears the flag word first and, at its end,
// waits for its stream and returns MOE_ERR_CHECK if a check failed.  With
// MOE_DEBUG_BREAK_PERM=1 in the environment a debug build first moves one
// in-range slot of perm to a wrong position (for tests of that path).
// Release builds do none of this.
#ifdef MOE_DEBUG
constexpr bool kDebugBuild = true;
#else
constexpr bool kDebugBuild = false;
#endif
std::atomic<uint32_t> g_debug_flags{0};   // flags of the last call that failed a check

hipError_t debug_validate_route(const moe_config& c, int T, const Route& R, hipStream_t s) {
  if (!kDebugBuild || T <= 0) return hipSuccess;
  const int S = T * c.top_k;
  const char* brk = std::getenv("MOE_DEBUG_BREAK_PERM");
  hipError_t e = hipSuccess;
  if (brk && brk[0] == '1') e = launch_debug_break_perm(R.perm, S, s);
  if (e == hipSuccess) e = launch_validate_routing(R.idx, R.counts, R.offsets, R.perm, R.tiles, S, c.n_experts, R.dbg, s);
  return e;
}

// (flags == nullptr: a call without tokens, whose workspace may be null)
hipError_t debug_begin(uint32_t* flags, hipStream_t s) {
  return kDebugBuild && flags ? launch_fill_u32(flags, 1, 0u, s) : hipSuccess;
}

moe_status debug_end(moe_plan_t plan, moe_status st, const uint32_t* flags, hipStream_t s) {
  if (!kDebugBuild || !flags || st != MOE_OK) return st;
  uint32_t v = 0;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(&v, flags, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(plan, e);
  if (v == 0u) return MOE_OK;
  g_debug_flags.store(v);
  return MOE_ERR_CHECK;
}

// Router + scan + permutation.
hipError_t enqueue_route(const moe_config& c, const void* x, int T, const moe_weights* w, const Route& R,
                         hipStream_t s) {
  hipError_t e;
  RouterArgs ra{x, w->w_router, c.has_router_bias ? w->router_bias : nullptr, T, c.d, c.n_experts,
                R.idx, R.gate, R.hist, c.top_k};
  if (T > 0 && T <= kRouteTokens) {
    e = R.logits_ready
            ? TRACED("route_small", 0, -1, 0, s,
                     launch_route_small_finish(ra, R.logits, R.counts, R.offsets, R.tiles, R.perm, s))
            : TRACED("route_small", 0, -1, 0, s,
                     launch_route_small(ra, c.x_dtype, R.logits, R.counts, R.offsets, R.tiles, R.perm, s));
    return e != hipSuccess ? e : debug_validate_route(c, T, R, s);
  }
  // Prefill-sized bf16 calls with E a multiple of 64: the logits x·W_router
  // come from the pipelined bf16 GEMM (its fp32 [T][N] mode), then the
  // fixed-order finish; otherwise the dedicated router kernels.
  const bool gemm_router = c.x_dtype == MOE_BF16 && T >= kPrefillTokens && c.n_experts % 64 == 0 &&
                           bf16_v2_supported(c.d, c.n_experts, c.n_experts) &&
                           static_cast<int64_t>(T) * c.d * 2 < (int64_t{1} << 31);
  if (T > 0 && R.logits_ready) {
    if ((e = TRACED("router_finish", 0, -1, 0, s, launch_router_finish(ra, 1, R.logits, s))) != hipSuccess) return e;
  } else if (T > 0 && gemm_router) {
    GemmArgs g{};
    g.A_shared = x;
    g.B_shared = w->w_router;
    g.K = c.d;
    g.N = c.n_experts;
    g.N_shared = c.n_experts;
    g.T = T;
    g.E = c.n_experts;
    g.C_shared = R.logits;
    g.group_lo = c.n_experts;
    g.group_hi = c.n_experts + 1;
    g.dbg = R.dbg;
    if ((e = TRACED("router_gemm", 64, -1, 0, s, launch_gemm_bf16_v2(MODE_DOWN_SHARED, 64, g, T, s, R.tiles))) != hipSuccess)
      return e;
    if ((e = TRACED("router_finish", 0, -1, 0, s, launch_router_finish(ra, 1, R.logits, s))) != hipSuccess) return e;
  } else if (T > 0) {
    if ((e = TRACED("router", 0, -1, 0, s, launch_router(ra, c.x_dtype, R.logits, s))) != hipSuccess) return e;
  }
  ScanArgs sa{R.hist, (T + kRouteTokens - 1) / kRouteTokens, c.n_experts, T, R.counts, R.offsets, R.tiles};
  if ((e = TRACED("scan", 0, -1, 0, s, launch_scan(sa, s))) != hipSuccess) return e;
  if (T > 0 && (e = TRACED("perm", 0, -1, 0, s, launch_perm(R.idx, R.hist, R.offsets, T, c.n_experts, c.top_k, R.perm, s))) !=
                   hipSuccess)
    return e;
  return debug_validate_route(c, T, R, s);
}

GemmArgs gateup_args(const moe_config& c, const moe_weights* w, uint8_t* ws, const WsLayout& L, const Route& R,
                     const void* a_x, float* sx, uint32_t* amax_r, uint32_t* amax_s, int T) {
  const bool fp8 = scaled_weights(c);
  GemmArgs g{};
  g.w_int8 = c.w_dtype == MOE_INT8 ? 8 : c.w_dtype == MOE_INT4 ? 4 : 0;
  g.top_k = c.top_k;
  g.A = a_x;
  g.A_shared = a_x;
  g.B = w->w_gate_up;
  g.B_shared = w->ws_gate_up;
  g.sB = fp8 ? w->s_gate_up : nullptr;
  g.sB_shared = fp8 ? w->ss_gate_up : nullptr;
  g.sA = sx;
  g.sA_shared = sx;
  g.K = c.d;
  g.N = c.f;
  g.N_shared = c.f_shared;
  g.T = T;
  g.E = c.n_experts;
  g.offsets = R.offsets;
  g.dbg = R.dbg;
  g.perm = R.perm;
  g.gate = R.gate;
  g.C = ws + L.h_r;
  g.C_shared = ws + L.h_s;
  if (fp8) {
    g.C_lo = ws + L.h_r_lo;
    g.C_shared_lo = ws + L.h_s_lo;
  }
  g.amax = amax_r;
  g.amax_shared = amax_s;
  return g;
}

GemmArgs down_shared_args(const moe_config& c, const moe_weights* w, uint8_t* ws, const WsLayout& L,
                          const Route& R, const void* h_s, const float* sh_s, int T, int ksplit) {
  const bool fp8 = scaled_weights(c);
  GemmArgs g{};
  g.w_int8 = c.w_dtype == MOE_INT8 ? 8 : c.w_dtype == MOE_INT4 ? 4 : 0;
  g.A_shared = h_s;
  g.B_shared = w->ws_down;
  g.sB_shared = fp8 ? w->ss_down : nullptr;
  g.sA_shared = sh_s;
  g.K = c.f_shared;
  g.N = c.d;
  g.T = T;
  g.E = c.n_experts;
  g.offsets = R.offsets;
  g.dbg = R.dbg;
  g.C_shared = reinterpret_cast<float*>(ws + L.y_s);
  g.ksplit = ksplit;
  g.group_lo = c.n_experts;
  g.group_hi = c.n_experts + 1;
  return g;
}

GemmArgs down_routed_args(const moe_config& c, const moe_weights* w, uint8_t* ws, const WsLayout& L,
                          const Route& R, const void* h_r, const float* sh_r, void* out, int T, int y_parts) {
  const bool fp8 = scaled_weights(c);
  GemmArgs g{};
  g.w_int8 = c.w_dtype == MOE_INT8 ? 8 : c.w_dtype == MOE_INT4 ? 4 : 0;
  g.A = h_r;
  g.B = w->w_down;
  g.sB = fp8 ? w->s_down : nullptr;
  g.sA = sh_r;
  g.K = c.f;
  g.N = c.d;
  g.T = T;
  g.E = c.n_experts;
  g.offsets = R.offsets;
  g.dbg = R.dbg;
  g.perm = R.perm;
  g.C = out;
  g.Y = reinterpret_cast<const float*>(ws + L.y_s);
  g.y_parts = y_parts;
  g.out_bf16 = c.out_dtype == MOE_BF16;
  g.group_lo = 0;
  g.group_hi = c.n_experts;
  g.top_k = c.top_k;
  if (c.top_k > 1) {
    // k picks per token: one fp32 row per slot, summed per token by
    // finish_topk (one writer per row, no atomics)
    g.C = ws + L.r_out;
    g.Y = nullptr;
    g.out_bf16 = 0;
  }
  return g;
}

// k > 1: out[t] = y_s[t] (its `parts` partials in order) + the token's k slot
// rows of r_out, in pick order.  Nothing to do for k = 1 (the routed down
// epilogue or the combine has written out).
hipError_t finish_topk(const moe_config& c, uint8_t* ws, const WsLayout& L, int T, int parts, void* out,
                       hipStream_t s) {
  if (c.top_k <= 1) return hipSuccess;
  return TRACED("combine_topk", 0, -1, 0, s,
                launch_combine_topk(reinterpret_cast<const float*>(ws + L.r_out), c.top_k,
                                    reinterpret_cast<const float*>(ws + L.y_s), parts, out, T, c.d,
                                    c.out_dtype == MOE_BF16, s));
}

// The plan's side stream of the calling device (created on first use), or
// null when the caller's stream belongs to another device than the current
// one.  Called with plan->mu held.
const AuxStream* aux_for(moe_plan_t plan, hipStream_t stream, hipError_t* err) {
  *err = hipSuccess;
  int cur = 0;
  hipDevice_t sdev = 0;
  if ((*err = hipGetDevice(&cur)) != hipSuccess) return nullptr;
  if ((*err = hipStreamGetDevice(stream, &sdev)) != hipSuccess) return nullptr;
  if (sdev != cur || cur < 0 || cur >= kMaxDevices) return nullptr;
  AuxStream& a = plan->aux[cur];
  if (!a.stream) {
    hipStream_t st = nullptr;
    hipEvent_t ev[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
    if ((*err = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return nullptr;
    for (hipEvent_t& x : ev) {
      if ((*err = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) {
        for (hipEvent_t y : ev)
          if (y) (void)hipEventDestroy(y);
        (void)hipStreamDestroy(st);
        return nullptr;
      }
    }
    a.stream = st;
    a.fork = ev[0];
    a.join = ev[1];
    a.routed = ev[2];
    a.shared = ev[3];
    a.gateup = ev[4];
  }
  return &a;
}

// Decode-sized bf16 schedule with the shared expert on a side stream: the
// shared gate/up and down GEMMs depend on x alone, so they run while the
// routing and the routed gate/up proceed on `stream`; the routed down GEMM,
// which adds the shared output, waits for them.  Same kernels and arguments
// as the serial schedule, hence the same results.
hipError_t enqueue_decode_overlapped(const moe_config& c, const void* x, int T, const moe_weights* w, void* out,
                                     uint8_t* ws, const WsLayout& L, const Route& R, const AuxStream& aux,
                                     hipStream_t stream) {
  hipError_t e;
  const int ys = decode_y_parts(c, T);
  if ((e = hipEventRecord(aux.fork, stream)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(aux.stream, aux.fork, 0)) != hipSuccess) return e;
  GemmArgs g1 = gateup_args(c, w, ws, L, R, x, nullptr, nullptr, nullptr, T);
  g1.group_lo = c.n_experts;
  g1.group_hi = c.n_experts + 1;
  if ((e = TRACED("gateup", 32, 1, 0, aux.stream, launch_gemm_decode(MODE_GATEUP, true, g1, T, aux.stream, R.tiles))) !=
      hipSuccess)
    return e;
  const GemmArgs g2 = down_shared_args(c, w, ws, L, R, ws + L.h_s, nullptr, T, ys);
  if ((e = TRACED("down_shared", 32, 1, 0, aux.stream,
                  launch_gemm_decode(MODE_DOWN_SHARED, true, g2, T, aux.stream, R.tiles))) != hipSuccess)
    return e;
  if ((e = hipEventRecord(aux.join, aux.stream)) != hipSuccess) return e;

  if ((e = enqueue_route(c, x, T, w, R, stream)) != hipSuccess) return e;
  g1.group_lo = 0;
  g1.group_hi = c.n_experts;
  if ((e = TRACED("gateup", 32, 0, 0, stream, launch_gemm_decode(MODE_GATEUP, true, g1, T, stream, R.tiles))) != hipSuccess)
    return e;
  if ((e = hipStreamWaitEvent(stream, aux.join, 0)) != hipSuccess) return e;
  const GemmArgs g3 = down_routed_args(c, w, ws, L, R, ws + L.h_r, nullptr, out, T, ys);
  if ((e = TRACED("down_routed", 16, 0, 0, stream, launch_gemm_decode(MODE_DOWN_ROUTED, false, g3, T, stream, R.tiles))) !=
      hipSuccess)
    return e;
  return finish_topk(c, ws, L, T, ys, out, stream);
}

// bf16 prefill over the class tables (see enqueue_bf16_prefill).  With a
// side stream:
//   side: shared gate/up -> shared down (into y_s) -> (shared done) ->
//         [routing done] -> gate/up and down of the groups of <= 32 rows
//         (into r_out) -> (join)
//   main: routing -> gate/up of the 33..128-row groups (128-row tiles) and of
//         the larger ones (256-row tiles) -> their down GEMMs (into r_out) ->
//         [join] -> combine out = r_out + y_s
// Each group's rows are written (h_r, r_out) by launches of one stream only.
// Without a side stream the same GEMMs run in stage order on `stream`, the
// routed down epilogues adding y_s themselves.
hipError_t enqueue_bf16_prefill_classes(const moe_config& c, int T, const moe_weights* w, void* out, uint8_t* ws,
                                        const WsLayout& L, const Route& R, const GemmArgs& g1, const GemmArgs& gs,
                                        const GemmArgs& g2, const GemmArgs& g3, const AuxStream* aux,
                                        hipStream_t stream, hipEvent_t* ev) {
  hipError_t e;
  const int E = c.n_experts;
  const int32_t* tiles_class = R.tiles + 3 * kNumBM * (E + 2);   // the class tables, indexed by tile height
  const int bm_sd = down_tile_rows(T, 1, c.d, 256);
  auto gateup_small = [&](hipStream_t s) {
    return TRACED("gateup", 32, 0, 3, s, launch_gemm_decode_tail(MODE_GATEUP, g1, 0, s, R.tiles));
  };
  auto gateup_mid_big = [&](hipStream_t s) {
    hipError_t r = TRACED("gateup", 128, 0, 3, s, launch_gemm_bf16_v2(MODE_GATEUP, 128, g1, T, s, tiles_class));
    if (r == hipSuccess) r = TRACED("gateup", 256, 0, 3, s, launch_gemm_bf16_v2(MODE_GATEUP, 256, g1, T, s, tiles_class));
    return r;
  };
  auto down_small = [&](const GemmArgs& g, const char* name, hipStream_t s) {
    return TRACED(name, 32, 0, 3, s, launch_gemm_decode_tail(MODE_DOWN_ROUTED, g, 0, s, R.tiles));
  };
  auto down_mid_big = [&](const GemmArgs& g, const char* name, hipStream_t s) {
    hipError_t r = TRACED(name, 128, 0, 3, s, launch_gemm_bf16_v2(MODE_DOWN_ROUTED, 128, g, T, s, tiles_class));
    if (r == hipSuccess) r = TRACED(name, 256, 0, 3, s, launch_gemm_bf16_v2(MODE_DOWN_ROUTED, 256, g, T, s, tiles_class));
    return r;
  };
  if (aux) {
    const hipStream_t a = aux->stream;
    GemmArgs g3r = g3;   // routed rows into r_out (fp32, token order); the combine adds y_s
    g3r.C = ws + L.r_out;
    g3r.Y = nullptr;
    g3r.out_bf16 = 0;
    if ((e = hipEventRecord(aux->fork, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(a, aux->fork, 0)) != hipSuccess) return e;
    if ((e = TRACED("gateup", 256, 1, 0, a, launch_gemm_bf16_v2(MODE_GATEUP, 256, gs, T, a, R.tiles))) != hipSuccess)
      return e;
    if ((e = TRACED("down_shared", bm_sd, 1, 0, a, launch_gemm_bf16_v2(MODE_DOWN_SHARED, bm_sd, g2, T, a, R.tiles))) !=
        hipSuccess)
      return e;
    if ((e = hipEventRecord(aux->shared, a)) != hipSuccess) return e;
    if ((e = enqueue_route(c, g1.A, T, w, R, stream)) != hipSuccess) return e;
    if ((e = hipEventRecord(aux->routed, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(a, aux->routed, 0)) != hipSuccess) return e;
    if ((e = gateup_small(a)) != hipSuccess || (e = down_small(g3r, "down_routed_r", a)) != hipSuccess) return e;
    if ((e = hipEventRecord(aux->join, a)) != hipSuccess) return e;
    if ((e = gateup_mid_big(stream)) != hipSuccess || (e = down_mid_big(g3r, "down_routed_r", stream)) != hipSuccess)
      return e;
    if ((e = hipStreamWaitEvent(stream, aux->join, 0)) != hipSuccess) return e;
    if (c.top_k > 1) return finish_topk(c, ws, L, T, 1, out, stream);
    return TRACED("combine", 0, -1, 0, stream,
                  launch_combine(reinterpret_cast<const float*>(ws + L.r_out), reinterpret_cast<const float*>(ws + L.y_s),
                                 1, out, static_cast<int64_t>(T) * c.d, c.out_dtype == MOE_BF16, stream));
  }
  auto mark = [&](int i) -> hipError_t { return ev && ev[i] ? hipEventRecord(ev[i], stream) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess) return e;
  if ((e = enqueue_route(c, g1.A, T, w, R, stream)) != hipSuccess) return e;
  if ((e = mark(1)) != hipSuccess) return e;
  if ((e = gateup_small(stream)) != hipSuccess || (e = gateup_mid_big(stream)) != hipSuccess) return e;
  if ((e = TRACED("gateup", 256, 1, 0, stream, launch_gemm_bf16_v2(MODE_GATEUP, 256, gs, T, stream, R.tiles))) !=
      hipSuccess)
    return e;
  if ((e = mark(2)) != hipSuccess) return e;
  if ((e = TRACED("down_shared", bm_sd, 1, 0, stream, launch_gemm_bf16_v2(MODE_DOWN_SHARED, bm_sd, g2, T, stream,
                                                                           R.tiles))) != hipSuccess)
    return e;
  if ((e = mark(3)) != hipSuccess) return e;
  if ((e = down_small(g3, "down_routed", stream)) != hipSuccess || (e = down_mid_big(g3, "down_routed", stream)) != hipSuccess)
    return e;
  if ((e = finish_topk(c, ws, L, T, 1, out, stream)) != hipSuccess) return e;
  return mark(4);
}

// bf16 prefill.  Routed groups: main tiles of bm_r rows (gate/up) and bm_d
// rows (down) on the MFMA kernels over table_main; the tails (the 1..32 rows
// past a group's last full main tile, or all of a group of at most 32
// tokens) on the 32-row weight-streaming tiles over table_tail.  With a side
// stream:
//   side: shared gate/up -> (h_s done) -> [routing done] -> tail gate/up ->
//         [main gate/up done, only when bm_d < bm_r] -> tail down (into
//         r_out) -> (join)
//   main: routing -> routed main gate/up -> [h_s done] -> one down launch:
//         routed main tiles (into r_out) + shared tiles (into y_s) ->
//         [join] -> combine out = r_out + y_s
// The shared expert depends on x alone and the tails are weight streams;
// both overlap the MFMA-bound main tiles, and neither down GEMM waits for
// the other.  Without a side stream (the stage-timed variant) the same GEMMs
// run in stage order on `stream`, the routed down epilogue adding y_s itself
// (the same fp32 addition as the combine's).
hipError_t enqueue_bf16_prefill(const moe_config& c, const void* x, int T, const moe_weights* w, void* out,
                                uint8_t* ws, const WsLayout& L, const Route& R, const AuxStream* aux,
                                hipStream_t stream, hipEvent_t* ev) {
  hipError_t e;
  const int E = c.n_experts;
  const int64_t Tr = static_cast<int64_t>(T) * c.top_k;   // routed rows (slots)
  const int bm_r = routed_tile_rows(Tr, E);
  const int bm_d = down_tile_rows(Tr, E, c.d, bm_r);
  const int bm_sd = down_tile_rows(T, 1, c.d, 256);
  const bool tails = decode_supported(c.d) && decode_supported(c.f);
  const int32_t* tiles_main = tails ? R.tiles + kNumBM * (E + 2) : R.tiles;
  GemmArgs g1 = gateup_args(c, w, ws, L, R, x, nullptr, nullptr, nullptr, T);
  GemmArgs gs = g1;
  gs.group_lo = E;
  gs.group_hi = E + 1;
  g1.group_lo = 0;
  g1.group_hi = E;
  const GemmArgs g2 = down_shared_args(c, w, ws, L, R, ws + L.h_s, nullptr, T, 1);
  const GemmArgs g3 = down_routed_args(c, w, ws, L, R, ws + L.h_r, nullptr, out, T, 1);
  // Groups averaging under 192 rows (the Maverick-shaped layer: 13..647 rows
  // over 128 experts) stream nearly all their weights from HBM; each group
  // then takes one tile height by its size (the class tables), so that its
  // weights are read by one set of tiles: 1..32 rows on the weight-streaming
  // tiles, 33..128 rows on one 128-row tile, more on 256-row tiles.  (With
  // the main / tail split a group of 129..160 rows read its weights twice.)
  if (tails && bm_r == 128) return enqueue_bf16_prefill_classes(c, T, w, out, ws, L, R, g1, gs, g2, g3, aux, stream, ev);

  if (aux) {
    const hipStream_t a = aux->stream;
    // the routed down GEMMs store their sums (fp32, token order) in r_out and
    // the combine adds the shared output at the end.  The main tiles of the
    // routed groups and the shared group's tiles (group E, into y_s) form one
    // down launch
    GemmArgs g3r = g3;
    g3r.C = ws + L.r_out;
    g3r.Y = nullptr;
    g3r.out_bf16 = 0;
    // (when both take 256-row tiles and one K, f == f_shared; else the
    // shared down GEMM runs in 256-row tiles on the side stream after the
    // shared gate/up: in a 128-row launch it lost more than the merge gains)
    const bool merge_down = c.f == c.f_shared && bm_d == 256;
    GemmArgs g3m = g3r;
    if (merge_down) {
      g3m.A_shared = ws + L.h_s;
      g3m.B_shared = w->ws_down;
      g3m.C_shared = ws + L.y_s;
      g3m.N_shared = c.f_shared;
      g3m.group_hi = E + 1;
    }
    if ((e = hipEventRecord(aux->fork, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(a, aux->fork, 0)) != hipSuccess) return e;
    if ((e = TRACED("gateup", 256, 1, 0, a, launch_gemm_bf16_v2(MODE_GATEUP, 256, gs, T, a, R.tiles))) != hipSuccess) return e;
    if (!merge_down &&
        (e = TRACED("down_shared", 256, 1, 0, a, launch_gemm_bf16_v2(MODE_DOWN_SHARED, 256, g2, T, a, R.tiles))) != hipSuccess)
      return e;
    if ((e = hipEventRecord(aux->shared, a)) != hipSuccess) return e;
    if ((e = enqueue_route(c, x, T, w, R, stream)) != hipSuccess) return e;
    if (tails) {
      if ((e = hipEventRecord(aux->routed, stream)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(a, aux->routed, 0)) != hipSuccess) return e;
      if ((e = TRACED("gateup", bm_r, 0, 2, a, launch_gemm_decode_tail(MODE_GATEUP, g1, bm_r, a, R.tiles))) != hipSuccess)
        return e;
    }
    if ((e = TRACED("gateup", bm_r, 0, tails ? 1 : 0, stream,
                    launch_gemm_bf16_v2(MODE_GATEUP, bm_r, g1, T, stream, tiles_main))) != hipSuccess)
      return e;
    if (tails) {
      // With bm_d < bm_r the down tails are not the gate/up tails: a group
      // of n rows with n % bm_r in bm_d+1 .. bm_d+32 has its last n % bm_d
      // rows of h_r written by a main gate/up tile on `stream`, so the tail
      // down GEMM waits for the main gate/up launch.  With bm_d == bm_r the
      // down tails read exactly the rows the tail gate/up wrote on this side
      // stream.  (bm_d <= bm_r always; for bm_r = 256, bm_d = 128 the gate/up
      // tails are a subset of the down tails, so the main down tiles never
      // read a row the side stream writes.)
      if (bm_d != bm_r) {
        if ((e = hipEventRecord(aux->gateup, stream)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(a, aux->gateup, 0)) != hipSuccess) return e;
      }
      if ((e = TRACED("down_routed_r", bm_d, 0, 2, a, launch_gemm_decode_tail(MODE_DOWN_ROUTED, g3r, bm_d, a, R.tiles))) !=
          hipSuccess)
        return e;
    }
    if ((e = hipEventRecord(aux->join, a)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(stream, aux->shared, 0)) != hipSuccess) return e;
    if ((e = TRACED("down_routed_r", bm_d, merge_down ? 2 : 0, tails ? 1 : 0, stream,
                    launch_gemm_bf16_v2(MODE_DOWN_ROUTED, bm_d, g3m, T, stream, tiles_main))) != hipSuccess)
      return e;
    if ((e = hipStreamWaitEvent(stream, aux->join, 0)) != hipSuccess) return e;
    if (c.top_k > 1) return finish_topk(c, ws, L, T, 1, out, stream);
    return TRACED("combine", 0, -1, 0, stream,
                  launch_combine(reinterpret_cast<const float*>(ws + L.r_out), reinterpret_cast<const float*>(ws + L.y_s),
                                 1, out, static_cast<int64_t>(T) * c.d, c.out_dtype == MOE_BF16, stream));
  }

  auto mark = [&](int i) -> hipError_t { return ev && ev[i] ? hipEventRecord(ev[i], stream) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess) return e;
  if ((e = enqueue_route(c, x, T, w, R, stream)) != hipSuccess) return e;
  if ((e = mark(1)) != hipSuccess) return e;
  if (tails && (e = TRACED("gateup", bm_r, 0, 2, stream, launch_gemm_decode_tail(MODE_GATEUP, g1, bm_r, stream, R.tiles))) !=
                   hipSuccess)
    return e;
  if ((e = TRACED("gateup", bm_r, 0, tails ? 1 : 0, stream,
                  launch_gemm_bf16_v2(MODE_GATEUP, bm_r, g1, T, stream, tiles_main))) != hipSuccess)
    return e;
  if ((e = TRACED("gateup", 256, 1, 0, stream, launch_gemm_bf16_v2(MODE_GATEUP, 256, gs, T, stream, R.tiles))) != hipSuccess)
    return e;
  if ((e = mark(2)) != hipSuccess) return e;
  if ((e = TRACED("down_shared", bm_sd, 1, 0, stream, launch_gemm_bf16_v2(MODE_DOWN_SHARED, bm_sd, g2, T, stream, R.tiles))) !=
      hipSuccess)
    return e;
  if ((e = mark(3)) != hipSuccess) return e;
  if (tails && (e = TRACED("down_routed", bm_d, 0, 2, stream, launch_gemm_decode_tail(MODE_DOWN_ROUTED, g3, bm_d, stream, R.tiles))) !=
                   hipSuccess)
    return e;
  if ((e = TRACED("down_routed", bm_d, 0, tails ? 1 : 0, stream,
                  launch_gemm_bf16_v2(MODE_DOWN_ROUTED, bm_d, g3, T, stream, tiles_main))) != hipSuccess)
    return e;
  if ((e = finish_topk(c, ws, L, T, 1, out, stream)) != hipSuccess) return e;
  return mark(4);
}

// e4m3 prefill (T >= 256).  The routed groups' gate/up and down GEMMs take
// bm_r-row tiles (160 when the mean group holds 96..136 rows, so one tile
// takes a group whole; else 128): they stream each expert's weights once
// from HBM.  The shared expert's gate/up and down GEMMs are MFMA-bound and
// take the 256 x 256 tiles.  h is quantised per row to e4m3 between the two
// GEMMs of each expert (from the 24-bit h the gate/up epilogue stores, with
// the scale from the max of the fp32 values it gathered), and the routed down
// epilogue adds the shared output.
// With a side stream the shared expert's three launches run there, next to
// the routed gate/up:
//   side: [fork] shared gate/up -> quantise h_s -> shared down -> (done)
//   main: routed gate/up -> quantise h_r -> [done] -> routed down
// Without one (the stage-timed variant) the same launches run in stage
// order on `stream`; the results are the same bit for bit.
hipError_t enqueue_fp8_prefill(const moe_config& c, const moe_weights* w, void* out, uint8_t* ws, const WsLayout& L,
                               const Route& R, const void* xq, float* sx, uint32_t* amax_r, uint32_t* amax_s, int T,
                               const AuxStream* aux, hipStream_t stream, hipEvent_t* ev, bool shared_only = false,
                               bool shared_enqueued = false) {
  hipError_t e;
  auto mark = [&](int i) -> hipError_t { return ev && ev[i] ? hipEventRecord(ev[i], stream) : hipSuccess; };
  const int E = c.n_experts;
  const int bm_r = fp8_routed_rows(static_cast<int64_t>(T) * c.top_k, E);
  GemmArgs g1 = gateup_args(c, w, ws, L, R, xq, sx, amax_r, amax_s, T);
  GemmArgs gs = g1;
  gs.group_lo = E;
  gs.group_hi = E + 1;
  g1.group_lo = 0;
  g1.group_hi = E;
  float* sh_r = reinterpret_cast<float*>(ws + L.sh_r);
  float* sh_s = reinterpret_cast<float*>(ws + L.sh_s);
  const GemmArgs g2 = down_shared_args(c, w, ws, L, R, ws + L.hq_s, sh_s, T, 1);
  const GemmArgs g3 = down_routed_args(c, w, ws, L, R, ws + L.hq_r, sh_r, out, T, 1);
  auto routed_gateup = [&](hipStream_t s) {
    return TRACED("gateup", bm_r, 0, 0, s, launch_gemm_fp8(MODE_GATEUP, bm_r, g1, T, s, R.tiles));
  };
  auto shared_gateup = [&](hipStream_t s) {
    return TRACED("gateup", 256, 1, 0, s, launch_gemm_fp8(MODE_GATEUP, 256, gs, T, s, R.tiles));
  };
  auto quant_r = [&](hipStream_t s) {
    return TRACED("quant_h", 0, 0, 0, s,
                  launch_quant_h(reinterpret_cast<const uint16_t*>(ws + L.h_r), ws + L.h_r_lo, amax_r, T * c.top_k, c.f, ws + L.hq_r,
                                 sh_r, s));
  };
  auto quant_s = [&](hipStream_t s) {
    return TRACED("quant_h", 0, 1, 0, s,
                  launch_quant_h(reinterpret_cast<const uint16_t*>(ws + L.h_s), ws + L.h_s_lo, amax_s, T, c.f_shared, ws + L.hq_s, sh_s,
                                 s));
  };
  auto shared_down = [&](hipStream_t s) {
    return TRACED("down_shared", 256, 1, 0, s, launch_gemm_fp8(MODE_DOWN_SHARED, 256, g2, T, s, R.tiles));
  };
  auto routed_down = [&](hipStream_t s) {
    return TRACED("down_routed", bm_r, 0, 0, s, launch_gemm_fp8(MODE_DOWN_ROUTED, bm_r, g3, T, s, R.tiles));
  };
  if (aux) {
    const hipStream_t a = aux->stream;
    if (!shared_enqueued) {
      if ((e = hipEventRecord(aux->fork, stream)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(a, aux->fork, 0)) != hipSuccess) return e;
      if ((e = shared_gateup(a)) != hipSuccess || (e = quant_s(a)) != hipSuccess || (e = shared_down(a)) != hipSuccess)
        return e;
      if ((e = hipEventRecord(aux->shared, a)) != hipSuccess) return e;
    }
    if (shared_only) return hipSuccess;
    if ((e = routed_gateup(stream)) != hipSuccess || (e = quant_r(stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(stream, aux->shared, 0)) != hipSuccess) return e;
    if ((e = routed_down(stream)) != hipSuccess) return e;
    return finish_topk(c, ws, L, T, 1, out, stream);
  }
  if ((e = routed_gateup(stream)) != hipSuccess || (e = shared_gateup(stream)) != hipSuccess) return e;
  if ((e = mark(2)) != hipSuccess) return e;
  if ((e = quant_r(stream)) != hipSuccess || (e = quant_s(stream)) != hipSuccess || (e = shared_down(stream)) != hipSuccess)
    return e;
  if ((e = mark(3)) != hipSuccess) return e;
  if ((e = routed_down(stream)) != hipSuccess) return e;
  if ((e = finish_topk(c, ws, L, T, 1, out, stream)) != hipSuccess) return e;
  return mark(4);
}

// A dense layer (n_experts == 0; llm-architectures-explained "Llama 4
// Maverick", table "Every architecture field": every other layer's FFN is a
// gated MLP of width d_ff = 16384): out = SwiGLU_s(x), the shared group
// alone, with no routing.  Up to 64 tokens on the weight-streaming tiles
// (both GEMMs split over K, their partials summed in order), else on the
// prefill tiles; both address the shared group without tile tables.
hipError_t enqueue_dense(const moe_config& c, const void* x, int T, const moe_weights* w, void* out, uint8_t* ws,
                         const WsLayout& L, const Route& R, hipStream_t stream, hipEvent_t* ev) {
  hipError_t e;
  auto mark = [&](int i) -> hipError_t { return ev && ev[i] ? hipEventRecord(ev[i], stream) : hipSuccess; };
  if ((e = mark(0)) != hipSuccess || (e = mark(1)) != hipSuccess) return e;   // no routing stage
  if (T == 0) {
    for (int i = 2; i <= MOE_NUM_STAGES; ++i)
      if ((e = mark(i)) != hipSuccess) return e;
    return hipSuccess;
  }
  const bool small = T <= kDecodeTokensMax;
  GemmArgs g1 = gateup_args(c, w, ws, L, R, x, nullptr, nullptr, nullptr, T);
  g1.group_lo = 0;   // == E: the shared group alone
  g1.group_hi = 1;
  const int gp = dense_gateup_parts(c, T);
  if (gp > 1) {      // K-split gate/up partials, then the SwiGLU over their sum
    g1.gu_part = reinterpret_cast<float*>(ws + L.gu_part);
    g1.ksplit = gp;
  }
  e = small ? TRACED("gateup", 32, 1, 0, stream, launch_gemm_decode(MODE_GATEUP, true, g1, T, stream, R.tiles))
            : TRACED("gateup", 256, 1, 0, stream, launch_gemm_bf16_v2(MODE_GATEUP, 256, g1, T, stream, R.tiles));
  if (e == hipSuccess && gp > 1)
    e = TRACED("swiglu_parts", 0, -1, 0, stream,
               launch_swiglu_parts(reinterpret_cast<const float*>(ws + L.gu_part), gp, T, c.f_shared,
                                   reinterpret_cast<uint16_t*>(ws + L.h_s), stream));
  if (e != hipSuccess || (e = mark(2)) != hipSuccess) return e;
  const int parts = small ? dense_down_parts(c, T) : 1;
  GemmArgs g2 = down_shared_args(c, w, ws, L, R, ws + L.h_s, nullptr, T, parts);
  const bool direct = !small && c.out_dtype == MOE_F32;   // fp32 output straight from the GEMM
  if (direct) g2.C_shared = out;
  // prefill down tiles of 128 rows: on the Maverick-shaped layer (T = 8192,
  // d = 5120) 1280 of them fill 5 rounds of the 256 CUs where 640 256-row
  // tiles fill 2.5 (measured 1.55 -> 1.39 ms; 128-row gate/up tiles lost)
  e = small ? TRACED("down_shared", 32, 1, 0, stream, launch_gemm_decode(MODE_DOWN_SHARED, true, g2, T, stream, R.tiles))
            : TRACED("down_shared", 128, 1, 0, stream,
                     launch_gemm_bf16_v2(MODE_DOWN_SHARED, 128, g2, T, stream, R.tiles));
  if (e != hipSuccess || (e = mark(3)) != hipSuccess) return e;
  if (!direct &&
      (e = TRACED("combine", 0, -1, 0, stream,
                  launch_combine(nullptr, reinterpret_cast<const float*>(ws + L.y_s), parts, out,
                                 static_cast<int64_t>(T) * c.d, c.out_dtype == MOE_BF16, stream))) != hipSuccess)
    return e;
  return mark(4);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_SHAPE: return "token count out of range";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    case MOE_ERR_CHECK: return "device-side check failed (debug build)";
  }
  return "unknown status";
}

const char* moe_version(void) { return kDebugBuild ? "moe355 2 gfx950 debug" : "moe355 2 gfx950"; }

int32_t moe_debug_flags(int32_t clear) {
  if (!kDebugBuild) return -1;
  return static_cast<int32_t>(clear ? g_debug_flags.exchange(0u) : g_debug_flags.load());
}

moe_status moe_plan(const moe_config* cfg, moe_plan_t* out) {
  if (!out) return MOE_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (!cfg || cfg->abi_version != MOE_ABI_VERSION) return MOE_ERR_INVALID_ARGUMENT;
  const moe_config& c = *cfg;
  if (c.top_k < 1 || c.top_k > kMaxTopK || (c.n_experts > 0 && c.top_k > c.n_experts) ||
      (c.n_experts == 0 && c.top_k != 1))
    return MOE_ERR_UNSUPPORTED;
  if (c.n_experts < 0 || c.n_experts > 256) return MOE_ERR_UNSUPPORTED;
  if (!config_dtypes_ok(c)) return MOE_ERR_UNSUPPORTED;
  if (c.has_router_bias != 0 && c.has_router_bias != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c.has_norm != 0 && c.has_norm != 1) return MOE_ERR_INVALID_ARGUMENT;
  if (c.has_norm && !(c.norm_eps >= 0.0f && c.norm_eps <= 3.4e38f)) return MOE_ERR_INVALID_ARGUMENT;
  if (c.max_tokens < 1 || c.max_tokens > (int64_t{1} << 30)) return MOE_ERR_SHAPE;
  if (c.max_tokens * c.top_k >= (int64_t{1} << 31)) return MOE_ERR_SHAPE;   // routing slots are int32
  if (c.n_experts == 0) {
    // a dense layer: the shared gated MLP alone, bf16 weights, widths that
    // the weight-streaming and prefill tilings both take
    if (c.x_dtype != MOE_BF16 || c.w_dtype != MOE_BF16 || c.has_router_bias || c.f != 0) return MOE_ERR_UNSUPPORTED;
    if (c.d <= 0 || c.f_shared <= 0 || c.d % 128 || c.f_shared % 128) return MOE_ERR_UNSUPPORTED;
    if (c.max_tokens * std::max(c.d, c.f_shared) * 2 >= (int64_t{1} << 31)) return MOE_ERR_SHAPE;
  } else {
    const int km = k_multiple(c);
    if (c.d <= 0 || c.f <= 0 || c.f_shared <= 0 || c.d % km || c.f % km || c.f_shared % km)
      return MOE_ERR_UNSUPPORTED;
    // int8 / int4 weights are decode formats: the weight-streaming tiles only
    if (int_weights(c) && c.max_tokens > kDecodeTokensMax) return MOE_ERR_SHAPE;
  }
  moe_plan_s* p = new (std::nothrow) moe_plan_s;
  if (!p) return MOE_ERR_INVALID_ARGUMENT;
  p->cfg = c;
  p->last_hip_error = 0;
  *out = p;
  return MOE_OK;
}

void moe_plan_destroy(moe_plan_t plan) {
  if (!plan) return;
  for (AuxStream& a : plan->aux) {
    for (hipEvent_t ev : {a.fork, a.join, a.routed, a.shared, a.gateup})
      if (ev) (void)hipEventDestroy(ev);
    if (a.stream) (void)hipStreamDestroy(a.stream);
  }
  delete plan;
}

int moe_last_hip_error(moe_plan_t plan) { return plan ? plan->last_hip_error : 0; }

moe_status moe_workspace_size(moe_plan_t plan, int64_t T, size_t* bytes) {
  if (!plan || !bytes) return MOE_ERR_INVALID_ARGUMENT;
  if (T < 0 || T > plan->cfg.max_tokens) return MOE_ERR_SHAPE;
  *bytes = layout_for(plan->cfg, T).total;
  return MOE_OK;
}

moe_status moe_route(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, moe_routing* out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  moe_status st = check_common(plan, x, T, w, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  if (plan->cfg.n_experts == 0) return MOE_ERR_UNSUPPORTED;   // a dense layer routes nothing
  if (!out) return MOE_ERR_INVALID_ARGUMENT;
  if ((st = check_routing(out)) != MOE_OK) return st;
  const WsLayout L = layout_for(plan->cfg, T);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  Route R = route_ptrs(ws, L, out);
  uint32_t* const dbg = T > 0 ? R.dbg : nullptr;
  hipError_t e = debug_begin(dbg, stream);
  const moe_config& c = plan->cfg;
  // (routing alone needs no e4m3 codes: the fused kernel only with the norm)
  if (e != hipSuccess) {
  } else if (c.has_norm && fused_norm_route(c)) {
    e = TRACED("norm_route", 0, -1, 0, stream,
               launch_norm_route(x, w->norm_weight, static_cast<int>(T), c.d, c.n_experts, c.norm_eps, w->w_router,
                                 ws + L.wr_pack, ws + L.x_n, nullptr, nullptr, R.logits, stream));
    x = ws + L.x_n;
    R.logits_ready = T > 0;
  } else if (c.has_norm) {
    e = TRACED("rmsnorm", 0, -1, 0, stream,
               launch_rmsnorm(c.x_dtype, x, w->norm_weight, static_cast<int>(T), c.d, c.norm_eps, ws + L.x_n,
                              nullptr, nullptr, stream));
    x = ws + L.x_n;
  }
  if (e == hipSuccess) e = enqueue_route(plan->cfg, x, static_cast<int>(T), w, R, stream);
  return debug_end(plan, e == hipSuccess ? MOE_OK : hip_fail(plan, e), dbg, stream);
}

static moe_status forward_enqueue(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, void* out,
                                  uint8_t* ws, const WsLayout& L, Route R, hipStream_t stream, hipEvent_t* ev,
                                  bool serial);

static moe_status forward_impl(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, void* out,
                               moe_routing* routing_out, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, hipEvent_t* ev, bool serial = false) {
  moe_status st = check_common(plan, x, T, w, workspace, workspace_bytes);
  if (st != MOE_OK) return st;
  const moe_config& c = plan->cfg;
  if ((st = check_expert_weights(c, w)) != MOE_OK) return st;
  if (T > 0 && (!out || !aligned16(out))) return MOE_ERR_INVALID_ARGUMENT;
  if (routing_out && c.n_experts == 0) return MOE_ERR_INVALID_ARGUMENT;   // a dense layer routes nothing
  if (routing_out && (st = check_routing(routing_out)) != MOE_OK) return st;

  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const WsLayout L = layout_for(c, T);
  const Route R = route_ptrs(ws, L, routing_out);
  uint32_t* const dbg = T > 0 ? R.dbg : nullptr;
  const hipError_t e = debug_begin(dbg, stream);
  if (e != hipSuccess) return hip_fail(plan, e);
  return debug_end(plan, forward_enqueue(plan, x, T, w, out, ws, L, R, stream, ev, serial), dbg, stream);
}

// The schedules of one forward call (arguments already checked).
static moe_status forward_enqueue(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, void* out,
                                  uint8_t* ws, const WsLayout& L, Route R, hipStream_t stream, hipEvent_t* ev,
                                  bool serial) {
  const moe_config& c = plan->cfg;
  const int Ti = static_cast<int>(T);
  const bool fp8 = c.w_dtype == MOE_E4M3;

  // the RMSNorm runs first, inside the routing stage of the timed variant
  // (its events[0] is recorded here and the schedules below skip theirs);
  // for e4m3 weights it also writes x's e4m3 codes and scales.  When the
  // block has a router and the shape allows, the norm and the router GEMM
  // are one kernel (x read once; the routing stage then starts from the
  // logits)
  hipEvent_t evn[MOE_NUM_STAGES + 1];
  if ((c.has_norm || fused_norm_route(c)) && T > 0) {
    if (ev) {
      hipError_t e0 = hipEventRecord(ev[0], stream);
      if (e0 != hipSuccess) return hip_fail(plan, e0);
      evn[0] = nullptr;
      for (int i = 1; i <= MOE_NUM_STAGES; ++i) evn[i] = ev[i];
      ev = evn;
    }
    uint8_t* xq = fp8 ? ws + L.xq : nullptr;
    float* sx = fp8 ? reinterpret_cast<float*>(ws + L.sx) : nullptr;
    const hipError_t en =
        fused_norm_route(c)
            ? TRACED(c.has_norm ? "norm_route" : "route_quant", 0, -1, 0, stream,
                     launch_norm_route(x, c.has_norm ? w->norm_weight : nullptr, Ti, c.d, c.n_experts, c.norm_eps,
                                       w->w_router, ws + L.wr_pack, c.has_norm ? ws + L.x_n : nullptr, xq, sx,
                                       R.logits, stream))
            : TRACED("rmsnorm", 0, -1, 0, stream,
                     launch_rmsnorm(c.x_dtype, x, w->norm_weight, Ti, c.d, c.norm_eps, ws + L.x_n, xq, sx, stream));
    if (en != hipSuccess) return hip_fail(plan, en);
    if (c.has_norm) x = ws + L.x_n;
    R.logits_ready = fused_norm_route(c);
  }
  if (c.n_experts == 0) {
    const hipError_t e = enqueue_dense(c, x, Ti, w, out, ws, L, R, stream, ev);
    return e == hipSuccess ? MOE_OK : hip_fail(plan, e);
  }
  const bool dec = use_decode(c, T);
  // the prefill kernels address activations with 32-bit byte offsets
  const int64_t kmax = std::max(std::max(c.d, c.f), c.f_shared);
  const bool offsets32 = T * c.top_k * kmax * 2 < (int64_t{1} << 31);   // routed rows: T k slots
  const bool v2 = c.w_dtype == MOE_BF16 && T >= kPrefillTokens && offsets32 && bf16_v2_supported(c.d, c.f, c.f_shared) &&
                  bf16_v2_supported(c.f, c.d, c.d) && bf16_v2_supported(c.f_shared, c.d, c.d);
  const bool f8 = fp8 && T >= kPrefillTokens && offsets32;
  hipError_t e;

  // decode-sized and bf16 prefill calls use the plan's side stream (not the
  // stage-timed variant or a serial call, which keep every stage on `stream`)
  std::unique_lock<std::mutex> lock(plan->mu, std::defer_lock);
  const AuxStream* aux = nullptr;
  if (!ev && !serial && T > 0 && (dec || v2 || f8)) {
    lock.lock();
    aux = aux_for(plan, stream, &e);
    if (e != hipSuccess) return hip_fail(plan, e);
  }
  if (dec && aux) {
    e = enqueue_decode_overlapped(c, x, Ti, w, out, ws, L, R, *aux, stream);
    return e == hipSuccess ? MOE_OK : hip_fail(plan, e);
  }
  if (v2) {
    e = enqueue_bf16_prefill(c, x, Ti, w, out, ws, L, R, aux, stream, ev);
    return e == hipSuccess ? MOE_OK : hip_fail(plan, e);
  }
  auto mark = [&](int i) -> hipError_t { return ev && ev[i] ? hipEventRecord(ev[i], stream) : hipSuccess; };
  // e4m3 prefill on two streams, x quantised by its own kernel: the shared
  // expert reads only x's codes, so its launches (which address the shared
  // group without tile tables) go to the side stream before the routing
  if (f8 && aux && !c.has_norm && !R.logits_ready) {
    uint8_t* xq = ws + L.xq;
    float* sx = reinterpret_cast<float*>(ws + L.sx);
    uint32_t* amax_r = reinterpret_cast<uint32_t*>(ws + L.amax_r);
    uint32_t* amax_s = reinterpret_cast<uint32_t*>(ws + L.amax_s);
    if ((e = TRACED("quant_x", 0, -1, 0, stream,
                    launch_quant_x(static_cast<const uint16_t*>(x), Ti, c.d, xq, sx, stream, amax_s, amax_r,
                                   c.top_k))) != hipSuccess ||
        (e = enqueue_fp8_prefill(c, w, out, ws, L, R, xq, sx, amax_r, amax_s, Ti, aux, stream, nullptr, true)) !=
            hipSuccess ||
        (e = enqueue_route(c, x, Ti, w, R, stream)) != hipSuccess ||
        (e = enqueue_fp8_prefill(c, w, out, ws, L, R, xq, sx, amax_r, amax_s, Ti, aux, stream, nullptr, false, true)) !=
            hipSuccess)
      return hip_fail(plan, e);
    return MOE_OK;
  }
  if ((e = mark(0)) != hipSuccess) return hip_fail(plan, e);
  e = enqueue_route(c, x, Ti, w, R, stream);
  if (e != hipSuccess) return hip_fail(plan, e);
  if (T == 0) {
    for (int i = 1; i <= MOE_NUM_STAGES; ++i)
      if ((e = mark(i)) != hipSuccess) return hip_fail(plan, e);
    return MOE_OK;
  }

  const void* a_x = x;
  float* sx = nullptr;
  uint32_t *amax_r = nullptr, *amax_s = nullptr;
  if (fp8) {
    uint8_t* xq = ws + L.xq;
    sx = reinterpret_cast<float*>(ws + L.sx);
    if (!c.has_norm && !R.logits_ready && (e = TRACED("quant_x", 0, -1, 0, stream,
                                   launch_quant_x(static_cast<const uint16_t*>(x), Ti, c.d, xq, sx, stream))) != hipSuccess)
      return hip_fail(plan, e);
    a_x = xq;
    amax_r = reinterpret_cast<uint32_t*>(ws + L.amax_r);
    amax_s = reinterpret_cast<uint32_t*>(ws + L.amax_s);
    if ((e = TRACED("fill", 0, -1, 0, stream, launch_fill_u32(amax_r, T * c.top_k, 0u, stream))) != hipSuccess)   // slot rows
      return hip_fail(plan, e);
    if ((e = TRACED("fill", 0, -1, 0, stream, launch_fill_u32(amax_s, T, 0u, stream))) != hipSuccess) return hip_fail(plan, e);
  }
  if ((e = mark(1)) != hipSuccess) return hip_fail(plan, e);
  if (f8) {
    e = enqueue_fp8_prefill(c, w, out, ws, L, R, a_x, sx, amax_r, amax_s, Ti, aux, stream, ev);
    return e == hipSuccess ? MOE_OK : hip_fail(plan, e);
  }

  // gate/up (routed groups + shared group) with the SwiGLU epilogue
  GemmArgs g1 = gateup_args(c, w, ws, L, R, a_x, sx, amax_r, amax_s, Ti);
  if (dec && int_weights(c)) {
    // int8 / int4 tiles: the routed groups, then the shared expert
    g1.group_lo = 0;
    g1.group_hi = c.n_experts;
    if ((e = TRACED("gateup", 32, 0, 0, stream, launch_gemm_decode(MODE_GATEUP, true, g1, Ti, stream, R.tiles))) != hipSuccess)
      return hip_fail(plan, e);
    g1.group_lo = c.n_experts;
    g1.group_hi = c.n_experts + 1;
    if ((e = TRACED("gateup", 32, 1, 0, stream, launch_gemm_decode(MODE_GATEUP, true, g1, Ti, stream, R.tiles))) != hipSuccess)
      return hip_fail(plan, e);
  } else if (dec) {
    // routed groups and the shared expert in one launch of 32-row tiles
    g1.group_lo = 0;
    g1.group_hi = c.n_experts + 1;
    if ((e = TRACED("gateup", 32, 2, 0, stream, launch_gemm_decode(MODE_GATEUP, true, g1, Ti, stream, R.tiles))) != hipSuccess)
      return hip_fail(plan, e);
  } else {
    g1.group_lo = 0;
    g1.group_hi = c.n_experts + 1;
    if ((e = TRACED("gateup", 0, 2, 0, stream, launch_gemm(MODE_GATEUP, c.w_dtype, g1, Ti, stream, R.tiles))) != hipSuccess)
      return hip_fail(plan, e);
  }
  if ((e = mark(2)) != hipSuccess) return hip_fail(plan, e);

  const void* h_r = ws + L.h_r;
  const void* h_s = ws + L.h_s;
  float *sh_r = nullptr, *sh_s = nullptr;
  if (fp8) {
    sh_r = reinterpret_cast<float*>(ws + L.sh_r);
    sh_s = reinterpret_cast<float*>(ws + L.sh_s);
    if ((e = TRACED("quant_h", 0, 0, 0, stream,
                    launch_quant_h(reinterpret_cast<const uint16_t*>(ws + L.h_r), ws + L.h_r_lo, amax_r, Ti * c.top_k, c.f, ws + L.hq_r,
                                   sh_r, stream))) != hipSuccess)
      return hip_fail(plan, e);
    if ((e = TRACED("quant_h", 0, 1, 0, stream,
                    launch_quant_h(reinterpret_cast<const uint16_t*>(ws + L.h_s), ws + L.h_s_lo, amax_s, Ti, c.f_shared, ws + L.hq_s,
                                   sh_s, stream))) != hipSuccess)
      return hip_fail(plan, e);
    h_r = ws + L.hq_r;
    h_s = ws + L.hq_s;
  }

  const int ys = dec ? decode_y_parts(c, T) : 1;
  const GemmArgs g2 = down_shared_args(c, w, ws, L, R, h_s, sh_s, Ti, ys);
  e = dec ? TRACED("down_shared", 32, 1, 0, stream, launch_gemm_decode(MODE_DOWN_SHARED, true, g2, Ti, stream, R.tiles))
          : TRACED("down_shared", 0, 1, 0, stream, launch_gemm(MODE_DOWN_SHARED, c.w_dtype, g2, Ti, stream, R.tiles));
  if (e != hipSuccess) return hip_fail(plan, e);
  if ((e = mark(3)) != hipSuccess) return hip_fail(plan, e);

  const GemmArgs g3 = down_routed_args(c, w, ws, L, R, h_r, sh_r, out, Ti, ys);
  e = dec ? TRACED("down_routed", 16, 0, 0, stream, launch_gemm_decode(MODE_DOWN_ROUTED, false, g3, Ti, stream, R.tiles))
          : TRACED("down_routed", 0, 0, 0, stream, launch_gemm(MODE_DOWN_ROUTED, c.w_dtype, g3, Ti, stream, R.tiles));
  if (e != hipSuccess) return hip_fail(plan, e);
  if ((e = finish_topk(c, ws, L, Ti, ys, out, stream)) != hipSuccess) return hip_fail(plan, e);
  if ((e = mark(4)) != hipSuccess) return hip_fail(plan, e);
  return MOE_OK;
}

moe_status moe_forward(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, void* out,
                       moe_routing* routing_out, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  return forward_impl(plan, x, T, w, out, routing_out, workspace, workspace_bytes, stream, nullptr);
}

moe_status moe_forward_timed(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, void* out,
                             moe_routing* routing_out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, hipEvent_t* events) {
  if (!events) return MOE_ERR_INVALID_ARGUMENT;
  return forward_impl(plan, x, T, w, out, routing_out, workspace, workspace_bytes, stream, events);
}

}  // extern "C"

// Device scratch of moe_forward_noalloc: one copy per GPU, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (in host
// code the name is a host-side stand-in, not a device address): each
// device's address comes from hipGetSymbolAddress once, with that device
// current, and only that address is used.
static __device__ __align__(256) uint8_t scratch[MOE_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

extern "C" {

moe_status moe_forward_noalloc(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, void* out,
                               moe_routing* routing_out, hipStream_t stream) {
  if (!plan) return MOE_ERR_INVALID_ARGUMENT;
  if (T < 0 || T > plan->cfg.max_tokens) return MOE_ERR_SHAPE;
  const size_t need = layout_for(plan->cfg, T).total;
  if (need > MOE_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(plan, e);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      e = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_scratch_ptr[dev] = nullptr;
        return hip_fail(plan, e);
      }
    }
    ptr = g_scratch_ptr[dev];
  }
  // serial schedule on `stream` alone: no side stream to create
  return forward_impl(plan, x, T, w, out, routing_out, ptr, MOE_SCRATCH_BYTES, stream, nullptr, true);
}

moe_status moe_forward_traced(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, void* out,
                              moe_routing* routing_out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, hipEvent_t* events, int32_t max_launches,
                              moe_launch_record* launches, int32_t* n_launches) {
  if (!events || !launches || !n_launches || max_launches < MOE_MAX_LAUNCHES) return MOE_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 2 * max_launches; ++i)
    if (!events[i]) return MOE_ERR_INVALID_ARGUMENT;
  Trace t{events, launches, max_launches, 0, stream, hipSuccess};
  g_trace = &t;
  moe_status st = forward_impl(plan, x, T, w, out, routing_out, workspace, workspace_bytes, stream, nullptr);
  g_trace = nullptr;
  *n_launches = t.n;
  if (st == MOE_OK && t.err != hipSuccess) st = hip_fail(plan, t.err);
  return st;
}

}  // extern "C"
