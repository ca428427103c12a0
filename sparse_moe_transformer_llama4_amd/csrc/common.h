// Internal definitions shared by the HIP translation units of libmoe355.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA matrix cores, 160 KiB LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

// Tile heights the device-side scheduler publishes tile tables for: 16, 32,
// 64, 128, 256, and 160 (the e4m3 gate/up tiles for groups of ~100..160 rows).
constexpr int kNumBM = 6;
__host__ __device__ constexpr int bm_of(int i) { return i < 5 ? 16 << i : 160; }
__host__ __device__ constexpr int bm_index(int bm) {
  return bm == 16 ? 0 : bm == 32 ? 1 : bm == 64 ? 2 : bm == 128 ? 3 : bm == 256 ? 4 : 5;
}

// Tile tables published by the routing stage, each [E + 2] int32 (entry g =
// first tile of group g, group E = the shared expert, entry E + 1 = total):
//   table_all(bm):  every group in bm-row tiles;
//   table_main(bm): the routed groups' bm-row tiles without their tails (and
//                   the shared group): a group whose last bm-row tile would
//                   hold only 1..kTailRows rows gets floor(n / bm) tiles;
//   table_tail(bm): those tails, one kTailRows-row tile each (rows
//                   bm * floor(n / bm) .. n - 1; no shared group).
// A group of 1..kTailRows tokens is all tail.  Tails are weight streams: they
// take the 32-row weight-streaming tiles while the MFMA tiles do the rest.
//   table_class(bm): every routed group in one tile height chosen by its size
//                   (class_tiles below), so that each group's weights are
//                   streamed by one set of tiles: groups of 1..kTailRows rows
//                   in the kTailRows table (weight-streaming tiles, row 0),
//                   kTailRows+1..128 rows in the 128 table (one tile),
//                   larger groups in the 256 table; no shared group.
constexpr int kTailRows = 32;
constexpr int kNumTables = 4 * kNumBM;
__host__ __device__ constexpr int table_all(int bm) { return bm_index(bm); }
__host__ __device__ constexpr int table_main(int bm) { return kNumBM + bm_index(bm); }
__host__ __device__ constexpr int table_tail(int bm) { return 2 * kNumBM + bm_index(bm); }
__host__ __device__ constexpr int table_class(int bm) { return 3 * kNumBM + bm_index(bm); }
__host__ __device__ constexpr int class_tiles(int n, int bm) {
  return n <= 0 ? 0
         : n <= kTailRows ? (bm == kTailRows ? 1 : 0)
         : n <= 128       ? (bm == 128 ? 1 : 0)
                          : (bm == 256 ? (n + 255) / 256 : 0);
}

// Tokens handled by one router workgroup (4 waves x 16 tokens).
constexpr int kRouteTokens = 64;

enum Dtype : int { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2 };

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

// ------------------------------------------------------------------ scalars

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two floats -> two OCP e4m3fn codes (low byte = a), round to nearest even,
// with gfx950's conversion instruction (its fp8 format is OCP E4M3, bias 7,
// largest finite 448).  Inputs are clamped to +-448 first, so values past
// the largest finite code saturate to it instead of becoming NaN.  On every
// float of magnitude below 448 + 256 ulps, and for both signs, the
// instruction gives the codes that the format definition does (4
// significant bits, subnormal quantum 2^-9, ties to even): an exhaustive
// comparison against an integer implementation of that definition found no
// difference.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  return e4m3x2(a, b) | (e4m3x2(c, d) << 16);
}

// fp64 -> fp32 rounded to odd (truncate, then set the last bit if inexact):
// a later RNE to bf16 (8 significant bits <= 24 - 2) is then correctly
// rounded from the fp64 value.
__device__ __forceinline__ float f64_to_f32_odd(double y) {
  const float f = __double2float_rz(y);
  return static_cast<double>(f) == y ? f : __uint_as_float(__float_as_uint(f) | 1u);
}

__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + __expf(-z)); }
// SiLU z / (1 + e^-z) with the hardware reciprocal (v_rcp_f32, 1 ulp) in
// place of the IEEE divide sequence: about 5 VALU instructions per element
// instead of 15, in epilogues during which the matrix pipe idles.
__device__ __forceinline__ float silu_f(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// ------------------------------------------------------------------ workspace

// Byte offsets of the scratch buffers inside the caller's workspace.  All
// offsets are multiples of 256.  Sizes depend on T (tokens) and the plan.
struct WsLayout {
  size_t idx, gate, counts, offsets, perm;  // routing record (used when the caller passes none)
  size_t hist;                              // int32 [nblocks_route][E] -> per-block bases
  size_t logits;                            // fp32 [router splits][T][E] partial router logits
  size_t tiles;                             // int32 [kNumTables][E + 2] tile tables
  size_t h_r, h_s;                          // SwiGLU outputs (bf16 / f32; e4m3: bits 31..16 of fp32 h)
  size_t h_r_lo, h_s_lo;                    // e4m3 only: bits 15..8 of fp32 h, one byte per element
  size_t hq_r, hq_s;                        // e4m3 codes of h (e4m3 only)
  size_t sh_r, sh_s;                        // per-row fp32 scales of h (e4m3 only)
  size_t amax_r, amax_s;                    // per-row max |h| as uint bits (e4m3 only)
  size_t y_s;                               // fp32 [T][d] shared-expert output
  size_t r_out;                             // fp32 [T][d] routed output before the combine (bf16 prefill)
  size_t gu_part;                           // fp32 [parts][T][2 fs] gate/up partials (dense decode)
  size_t x_n;                               // x's rows after the RMSNorm (x dtype), when the block has one
  size_t wr_pack;                           // W_router packed into MFMA B fragments (RMSNorm fused with the router)
  size_t xq, sx;                            // e4m3 x codes [T][d] and fp32 scales [T] (e4m3 only)
  size_t dbg;                               // uint32 check flags (debug builds; allocated in every build)
  size_t total;
};

}  // namespace moe
