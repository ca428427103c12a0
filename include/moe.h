/*
 * moe.h -- C ABI of the Llama 4 mixture-of-experts feed-forward block on
 * AMD Instinct MI355X (gfx950).
 *
 * The block (KerasFormers "Llama 4", section "What is unusual about the
 * block"; superteams.ai "Llama 4", section "Mixture of Experts: Why Total
 * and Active Parameters Diverge"; llm-architectures-explained "Llama 4
 * Maverick", table "Every architecture field"):
 *
 *   logit[t,e] = sum_j x[t,j] * W_router[j,e] (+ bias[e])      one logit per expert
 *   e*(t)      = lowest index among the maxima of logit[t,:]    top-1 (argmax)
 *   g(t)       = 1 / (1 + exp(-logit[t,e*]))                    sigmoid gate on the input
 *   routed(t)  = SwiGLU_{e*}(g(t) * x[t])                       gated MLP of width f
 *   shared(t)  = SwiGLU_s(x[t])                                 shared gated MLP of width f_shared
 *   out[t]     = shared(t) + routed(t)                          the other experts contribute nothing
 *   SwiGLU_W(u) = (SiLU(u Wg) * (u Wu)) Wd,  SiLU(z) = z / (1 + exp(-z)),
 *                Wg / Wu = columns [0,f) / [f,2f) of W_gate_up.
 *
 * With top_k = k > 1 (torchtune llama4_decoder, Parameters:
 * experts_per_token; Llama 4 itself routes one expert per token) the token's
 * k largest logits are its picks e_0..e_{k-1}, best first, the lower index
 * first among equal logits; pick j is routing slot t*k + j with gate
 * g_j = 1 / (1 + exp(-logit[t,e_j])), and
 *   out[t] = shared(t) + sum_j SwiGLU_{e_j}(g_j * x[t]).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer (HBM) owned by the caller;
 *     the library never allocates, frees or keeps device memory.  Scratch
 *     space is the caller's workspace, sized by moe_workspace_size.
 *   - All work is enqueued asynchronously on `stream` (hipStream_t; NULL =
 *     the default stream).  No host synchronisation, no device-to-host copy.
 *     moe_forward also uses a side stream for decode-sized calls (T <= 64)
 *     with bf16, int8 or int4 weights and for prefill-sized calls (T >= 256)
 *     with bf16 or e4m3 weights.  The plan
 *     creates it for the current device on first use (non-blocking, default
 *     priority): it waits for `stream` before its first kernel and `stream`
 *     waits for it before the call's last kernel, so for the caller the whole
 *     call is still ordered in `stream` (and it can be captured into a HIP
 *     graph from `stream`).  If `stream` belongs to another device than the
 *     current one, the call runs on `stream` alone.
 *   - Arguments, shapes, alignment and workspace size are checked on the
 *     host BEFORE anything is enqueued; a failed check enqueues nothing.
 *   - Row-major layouts throughout.  Pointers must be 16-byte aligned.
 *   - Inputs must be finite; NaN / Inf inputs are outside the contract.
 *   - A plan may be shared by threads and streams (its side streams are
 *     created and used under a lock); concurrent calls need distinct
 *     workspaces.  Calls on one plan captured into a HIP graph must not
 *     overlap in time with uncaptured calls on the same plan.
 */
#ifndef MOE355_MOE_H
#define MOE355_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = -1, /* null / misaligned pointer, missing fp8 scale, bad abi_version */
  MOE_ERR_UNSUPPORTED = -2,      /* top_k outside [1, min(E, 8)], d / f / f_shared not multiples of 64 (128 for
                                    E4M3 and INT8 weights), E outside [1,256], dtype
                                    combination not implemented */
  MOE_ERR_SHAPE = -3,            /* T < 0 or T > max_tokens */
  MOE_ERR_WORKSPACE = -4,        /* workspace smaller than moe_workspace_size */
  MOE_ERR_HIP = -5,              /* a HIP launch failed; see moe_last_hip_error */
  MOE_ERR_CHECK = -6             /* debug builds only: a device-side check failed; see moe_debug_flags */
} moe_status;

typedef enum moe_dtype {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_E4M3 = 2, /* OCP 8-bit float E4M3 "fn": max 448, no infinities; stored as uint8 codes */
  MOE_INT8 = 3, /* signed 8-bit integer weight codes (-127..127), with fp32 scales */
  MOE_INT4 = 4  /* signed 4-bit weight codes (-7..7), two per byte along K, with fp32 scales */
} moe_dtype;

/*
 * Block configuration (KerasFormers "Llama 4", Llama4Model arguments
 * embed_dim / mlp_dim / num_experts / num_experts_per_tok; torchtune
 * llama4_decoder parameters num_experts, experts_per_token,
 * use_shared_expert).  Supported dtype triples (x, w, out):
 *   F32 / F32 / F32      fp32 everywhere, fp32 MFMA
 *   BF16 / BF16 / F32    bf16 MFMA, fp32 accumulate, h rounded to bf16, fp32 output
 *   BF16 / BF16 / BF16   as above with the output rounded to bf16
 *   BF16 / E4M3 / BF16   router in bf16; x and h quantised to e4m3 per token;
 *                        e4m3 weights with one fp32 scale per output column
 *   BF16 / INT8 / F32 or BF16
 *                        weight-only int8 for decode (superteams.ai "Llama 4",
 *                        section "The Llama 4 Herd"; aibase model card "Llama 4
 *                        Maverick 17B 128E Instruct FP8", section
 *                        "Quantization": Scout runs on one GPU with
 *                        weights quantised to int4 on the fly; int8 halves
 *                        the bytes a decode step streams): expert and
 *                        shared weights as int8 codes
 *                        with one fp32 scale per output column, dequantised
 *                        in the weight-streaming GEMMs, bf16 activations and
 *                        MFMA, h rounded to bf16; max_tokens <= 64
 *                        (MOE_ERR_SHAPE otherwise), E >= 1
 *   BF16 / INT4 / F32 or BF16
 *                        the same with int4 codes: a [K, N] matrix is stored
 *                        as [K/2, N] bytes, byte (i, n) = code(2i, n) in the
 *                        low nibble, code(2i+1, n) in the high one (two's
 *                        complement); d, f, f_shared multiples of 256
 *
 * n_experts == 0 configures a dense layer (llm-architectures-explained
 * "Llama 4 Maverick", table "Every architecture field": the layers between
 * the MoE layers have a plain gated MLP of width d_ff = 16384): out =
 * SwiGLU_s(x) with the shared weights and f_shared = d_ff, no router, no
 * routed experts.  It takes BF16 / BF16 / {F32, BF16}, f == 0, no router
 * bias, d and f_shared multiples of 128, and max_tokens * max(d, f_shared)
 * * 2 < 2^31; anything else is MOE_ERR_UNSUPPORTED (MOE_ERR_SHAPE for
 * max_tokens).  The router and routed-expert pointers may then be NULL,
 * moe_route returns MOE_ERR_UNSUPPORTED and moe_forward's routing_out must
 * be NULL (MOE_ERR_INVALID_ARGUMENT otherwise).
 *
 * has_norm == 1 puts the RMSNorm that precedes the feed-forward block
 * (llm-architectures-explained "Llama 4 Maverick", table "Every
 * architecture field": RMSNorm before the MLP; KerasFormers "Llama 4",
 * Llama4Model argument norm_eps) in front of every entry point that reads x:
 *   xn[t, j] = x[t, j] / sqrt(mean_j x[t, j]^2 + norm_eps) * norm_weight[j],
 * computed in fp32 and rounded to x_dtype; routing and both experts then
 * read xn in place of x (x itself is not modified).  Any config may have it.
 */
typedef struct moe_config {
  int32_t abi_version;     /* MOE_ABI_VERSION */
  int32_t d;               /* model width, multiple of 64 (128 for E4M3 / INT8 weights) */
  int32_t n_experts;       /* E, 1..256; 0 = a dense layer (see below) */
  int32_t f;               /* routed expert width, multiple of 64 (128 for E4M3 / INT8); 0 when E == 0 */
  int32_t f_shared;        /* shared expert width, multiple of 64 (128 for E4M3 / INT8) */
  int32_t top_k;           /* experts per token, 1..min(E, 8) (1 for a dense layer) */
  int32_t x_dtype;         /* moe_dtype of x and W_router */
  int32_t w_dtype;         /* moe_dtype of the expert and shared weights */
  int32_t out_dtype;       /* moe_dtype of out */
  int32_t has_router_bias; /* 0 / 1 */
  int64_t max_tokens;      /* largest T accepted by this plan, 1..2^30, max_tokens * top_k < 2^31 */
  int32_t has_norm;        /* 0 / 1: the block starts with the RMSNorm below */
  float norm_eps;          /* RMSNorm epsilon (1e-5 in Llama 4), finite and >= 0; read when has_norm */
} moe_config;

typedef struct moe_plan_s* moe_plan_t;

/*
 * Weights: all resident in device memory (KerasFormers "Llama 4": all
 * experts stay resident).  Scale pointers are required when w_dtype is
 * E4M3 or INT8 and ignored otherwise: one fp32 scale per output column n of
 * the [K, N] matrix, value = code * scale[n].
 */
typedef struct moe_weights {
  const void* w_router;     /* [d, E]         x_dtype */
  const float* router_bias; /* [E] fp32, or NULL when has_router_bias == 0 */
  const void* w_gate_up;    /* [E, d, 2f]     columns [0,f) feed SiLU, [f,2f) the linear branch */
  const float* s_gate_up;   /* [E, 2f] */
  const void* w_down;       /* [E, f, d] */
  const float* s_down;      /* [E, d] */
  const void* ws_gate_up;   /* [d, 2 f_shared] shared expert */
  const float* ss_gate_up;  /* [2 f_shared] */
  const void* ws_down;      /* [f_shared, d] */
  const float* ss_down;     /* [d] */
  const void* norm_weight;  /* [d] x_dtype RMSNorm gain, or NULL when has_norm == 0 */
} moe_weights;

/*
 * Routing record (device buffers owned by the caller), over the T * top_k
 * routing slots (slot t * k + j = token t's j-th pick; slot = token for k = 1):
 *   expert_idx[s] = the slot's expert;  gate[s] = its gate (fp32, from the
 *   fp32 logit);  counts[e] = #slots routed to e;  offsets[0] = 0,
 *   offsets[e+1] = offsets[e] + counts[e];
 *   perm[offsets[e] + r] = the r-th smallest slot routed to e
 *   (a stable grouping of slots by expert).
 */
typedef struct moe_routing {
  int32_t* expert_idx; /* [T * top_k] */
  float* gate;         /* [T * top_k] */
  int32_t* counts;     /* [E] */
  int32_t* offsets;    /* [E + 1] */
  int32_t* perm;       /* [T * top_k] */
} moe_routing;

/* Validate `cfg` and create a host-side plan (no device call is made; the
 * side stream of the decode schedule is created by the first call that uses it).
 * Returns MOE_ERR_UNSUPPORTED / MOE_ERR_INVALID_ARGUMENT for bad configs; *out
 * is set to NULL on failure. */
moe_status moe_plan(const moe_config* cfg, moe_plan_t* out);

/* Release a plan and the side streams and events it created (NULL is
 * ignored).  Does not touch device memory; work already enqueued completes. */
void moe_plan_destroy(moe_plan_t plan);

/* Bytes of device workspace moe_route / moe_forward need for T tokens. */
moe_status moe_workspace_size(moe_plan_t plan, int64_t T, size_t* bytes);

/*
 * Router, top-1 (top-k), gate and the stable expert grouping only (superteams.ai
 * "Llama 4", routing sketch: one logit per expert, argmax).  Fills every
 * pointer of *out.  T == 0 zeroes counts and offsets and enqueues nothing else.
 */
moe_status moe_route(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w,
                     moe_routing* out, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/*
 * The whole block: out[T, d] (out_dtype) = shared(x) + routed(x).
 * x: [T, d] x_dtype.  routing_out may be NULL; when given, the routing
 * record is written there as by moe_route.  Each output row is written
 * exactly once (no atomics), so results are deterministic.
 */
moe_status moe_forward(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w,
                       void* out, moe_routing* routing_out, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

/*
 * moe_forward with stage timing: records events[0..MOE_NUM_STAGES] on
 * `stream` at the stage boundaries
 *   [0] routing (RMSNorm if configured, router GEMM, top-k, gate, scan, permutation;
 *       e4m3: x quantisation)
 *   [1] grouped gate/up GEMM with the SwiGLU epilogue (routed groups + shared)
 *   [2] shared-expert down GEMM (e4m3: preceded by h quantisation)
 *   [3] routed down GEMM with un-permute + combine
 * so hipEventElapsedTime(events[i], events[i+1]) is the duration of stage i.
 * The stages run one after another on `stream` alone (no side stream), so a
 * decode-sized timed call can take longer than moe_forward.  Events are
 * created by the caller; everything else is as moe_forward.
 */
#define MOE_NUM_STAGES 4
moe_status moe_forward_timed(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w,
                             void* out, moe_routing* routing_out, void* workspace,
                             size_t workspace_bytes, hipStream_t stream, hipEvent_t* events);

/*
 * moe_forward with per-launch timing, for measuring each kernel inside the
 * schedule moe_forward runs (side stream included).  Every kernel launch of
 * the call is bracketed by events[2 i] and events[2 i + 1], recorded on the
 * stream that launch goes to, so hipEventElapsedTime(events[2 i],
 * events[2 i + 1]) is launch i's duration; launches[i] describes it and
 * *n_launches receives the count.  The events are created by the caller
 * (2 * max_launches of them); max_launches must be at least
 * MOE_MAX_LAUNCHES (MOE_ERR_INVALID_ARGUMENT otherwise, before anything is
 * enqueued).  The extra events are the only difference from moe_forward:
 * same kernels, arguments, streams and results.
 */
#define MOE_MAX_LAUNCHES 32
typedef struct moe_launch_record {
  const char* kernel;  /* static name: "gateup", "down_shared", "down_routed" (un-permute + add the shared output),
                          "down_routed_r" (routed rows into the fp32 workspace), "router", "router_gemm",
                          "router_finish", "route_small", "scan", "perm", "rmsnorm", "quant_x", "quant_h",
                          "fill", "combine", "combine_topk", "swiglu_parts" */
  int32_t side_stream; /* 1: the plan's side stream; 0: the caller's stream */
  int32_t tile_rows;   /* rows per tile of a GEMM launch (0 otherwise) */
  int32_t groups;      /* GEMMs and quant_h: 0 routed groups, 1 shared expert, 2 both; -1 otherwise */
  int32_t part;        /* routed GEMMs: 0 all rows; 1 the main tiles (a group's last 1..32 rows past its last
                          full tile_rows tile are left out); 2 those last rows alone; 3 the groups whose size
                          class is tile_rows (1..32 rows: 32, 33..128: 128, more: 256), whole */
} moe_launch_record;
moe_status moe_forward_traced(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, void* out,
                              moe_routing* routing_out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, hipEvent_t* events, int32_t max_launches,
                              moe_launch_record* launches, int32_t* n_launches);

/*
 * moe_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same block, with no workspace argument.  Its scratch space is a device
 * array of MOE_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; calls whose workspace (moe_workspace_size) exceeds it return
 * MOE_ERR_WORKSPACE before anything is enqueued -- with d = 5120 and
 * f = f_shared = 8192 that admits decode-sized calls (T <= 64).  The call
 * runs every stage on `stream` alone (no side stream), in the stage order of
 * moe_forward_timed, so its results equal moe_forward's bit for bit.  It calls
 * no hipMalloc / hipFree; the first call on a device looks up that device's
 * scratch address once (hipGetSymbolAddress).  Every call on one GPU shares
 * that GPU's scratch array, which keeps the last call's contents (nothing
 * relies on its initial contents): calls that overlap in time on one GPU
 * (two streams, two threads, two plans) race.
 */
#define MOE_SCRATCH_BYTES (32u << 20)
moe_status moe_forward_noalloc(moe_plan_t plan, const void* x, int64_t T, const moe_weights* w, void* out,
                               moe_routing* routing_out, hipStream_t stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status s);

/* hipError_t value behind the last MOE_ERR_HIP returned for this plan (0 if none). */
int moe_last_hip_error(moe_plan_t plan);

/* Library identity, e.g. "moe355 2 gfx950". */
const char* moe_version(void);

/*
 * Debug builds (libmoe355_debug.so, compiled with -DMOE_DEBUG) check on the
 * device, before any grouped GEMM uses them, the invariants of the routing
 * (expert indices in [0, E), group offsets consistent with the counts, perm
 * holding every slot once, grouped by expert in slot order, tile tables
 * non-decreasing from 0), and in every grouped GEMM that its tile lies inside
 * its group.  A failed check skips the work it guards (no out-of-bounds
 * access follows) and the call, which in debug builds waits for its stream
 * before returning, returns MOE_ERR_CHECK.  This returns the check bits of
 * the last call that failed (bit 0 expert index, 1 offsets / counts, 2 perm,
 * 3 tile tables, 4 a GEMM tile outside its group), then clears them when
 * `clear` is non-zero; release builds return -1 and make no device call.
 * Not for graph capture (the debug calls synchronise).
 */
int32_t moe_debug_flags(int32_t clear);

#ifdef __cplusplus
}
#endif
#endif /* MOE355_MOE_H */
