// common.hpp -- shared definitions of the gfx950 kernels and the host-side
// validation of the C ABI (include/fp4gemv.h).
//
// Nothing in here is shared with the CPU oracle: the oracle decodes E2M1, E4M3
// and E8M0 from their closed forms in double precision, while the kernels use the
// gfx950 conversion instructions (v_cvt_scalef32_pk_bf16_fp4, v_cvt_f32_fp8,
// v_cvt_scalef32_pk_bf16_fp8) and FP32 dot products (v_dot2_f32_bf16).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/fp4gemv.h"

namespace fp4g {

// ---- packed layout (see fp4g_packed_bytes in the header) ---------------------
constexpr int kRowsPerGroup = 64;   // one row per lane of a wave64
constexpr int kChunkK = 256;        // columns per tile
constexpr int kPieceK = 32;         // columns per 16-byte code load of one lane
constexpr int kPiecesNv = 8;        // NVFP4/MXFP4: 8 x 16 B code loads per tile and lane
constexpr int kSlotsFp8 = 16;       // FP8: 16 x 16 B code loads per tile and lane
constexpr int kHalfFp8 = 8;         // kernels stream an FP8 tile as two 8 KiB halves
constexpr int kTileNv = 9216;       // 8 KiB codes + 64 x 16 B E4M3 scales
constexpr int kTileMx = 8704;       // 8 KiB codes + 64 x 8 B E8M0 scales
constexpr int kTileF8 = 16384;      // 16 KiB codes (row scales follow all tiles)
constexpr int kCodeBytes = 8192;
constexpr int kMaxM = 8;       // vectors per call: VALU kernels, MoE, FP8 rows
constexpr int kMaxMWide = 16;  // NVFP4/MXFP4 products on the matrix-core kernel
constexpr int kWavesPerWg = 4;
constexpr int kThreads = 256;
__host__ __device__ inline int tile_bytes(uint32_t fmt) {
  return fmt == FP4G_NVFP4 ? kTileNv : fmt == FP4G_MXFP4 ? kTileMx : kTileF8;
}
__host__ __device__ inline int64_t row_groups(int64_t d_out) { return (d_out + 63) / 64; }
__host__ __device__ inline int64_t chunks(int64_t d_in) { return (d_in + 255) / 256; }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---- device helpers ---------------------------------------------------------

__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld_stream2(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2, v); }

// E4M3FN code of t >= 0 (finite), round to nearest even, saturating at 448
// (the load-time quantisers and the 8-bit activation staging).
__device__ __forceinline__ uint32_t e4m3_rne_pos(float t) {
  if (t >= 448.0f) return 126u;
  if (t < 0.015625f) return (uint32_t)rintf(t * 512.0f);  // m x 2^-9; m = 8 is code 8 = 2^-6
  const int E = (int)((__float_as_uint(t) >> 23) & 0xffu) - 127;  // floor(log2 t), t normal
  const float m = rintf((__builtin_amdgcn_ldexpf(t, -E) - 1.0f) * 8.0f);  // exact up to the rounding
  return (uint32_t)(((E + 7) << 3) + (int)m);  // m = 8 carries into the exponent
}

// Two E2M1 codes (byte SEL of dw: bits 0-3 -> .x, bits 4-7 -> .y) to exact bf16.
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_bf16(uint32_t dw) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(dw, 1.0f, SEL);
}
// Two E4M3FN codes (bytes 0,1 or 2,3 of dw) to exact bf16.
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_bf16(uint32_t dw) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(dw, 1.0f, HI);
}
// One E4M3FN code (byte SEL of dw) to FP32 (exact).
template <int SEL>
__device__ __forceinline__ float e4m3_f32(uint32_t dw) {
  return __builtin_amdgcn_cvt_f32_fp8((int)dw, SEL);
}
// acc + w.x*x.x + w.y*x.y, products exact in FP32.
__device__ __forceinline__ float dot2(bf16x2 w, uint32_t x2, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(w, as_bf16x2(x2), acc, false);
}

// FP32 -> bf16 bit pattern, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ---- arg-max keys (MoE routing, LM-head greedy pick) -------------------------------
// Pick order of (value, index) as one 64-bit key: the logit mapped to an unsigned integer of the
// same order (sign bit flipped for positive values, all bits for negative ones)
// in the high word, the complement of the expert index in the low word.  A
// larger key is a larger logit, or an equal logit with a lower index (zeros of
// either sign are equal).  Key 0 is below every logit's key and marks "none".
__device__ __forceinline__ uint64_t pick_key(float v, int e) {
  const uint32_t b = __float_as_uint(v == 0.0f ? 0.0f : v);  // -0 ranks as +0
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t ord = (uint32_t)(k >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}
__device__ __forceinline__ int key_index(uint64_t k) { return (int)(0xffffffffu - (uint32_t)k); }

// One DPP step of the wave maximum: each lane takes the larger of its key and
// the key `CTRL` names (key 0 where the source lane does not exist).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t k) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)k, CTRL, ROW_MASK, 0xf, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(k >> 32), CTRL, ROW_MASK, 0xf, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > k ? o : k;
}

// Maximum key over the 64 lanes, uniform: row_shr 1, 2, 4, 8 leave each 16-lane
// row's maximum in its lane 15; row_bcast 15 and 31 carry it up to lane 63.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  k = dpp_max_step<0x111, 0xf>(k);  // row_shr:1
  k = dpp_max_step<0x112, 0xf>(k);  // row_shr:2
  k = dpp_max_step<0x114, 0xf>(k);  // row_shr:4
  k = dpp_max_step<0x118, 0xf>(k);  // row_shr:8
  k = dpp_max_step<0x142, 0xa>(k);  // row_bcast:15 into rows 1 and 3
  k = dpp_max_step<0x143, 0xc>(k);  // row_bcast:31 into rows 2 and 3
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)k, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(k >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Sum of lanes 0..7 (the others must hold 0), uniform: row_shr 1, 2, 4 add
// pairs, then pairs of pairs, so lane 7 holds ((e7+e6)+(e5+e4))+((e3+e2)+(e1+e0)).
__device__ __forceinline__ float wave_sum8(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, false));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 7));
}

// ---- host-side validation helpers -----------------------------------------------
inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

uint64_t packed_bytes_of(uint32_t format, int64_t d_out, int64_t d_in);

// Checks a weight descriptor: pointer, tag, shape, alignment, size, scale.
fp4g_status check_weight(const fp4g_weight* w, bool want_fp4);

// Workspace bytes of moe_route_gemv (0 for invalid arguments).
uint64_t moe_ws_bytes(const fp4g_moe* mo, int M);
uint64_t moe_slot_bytes(const fp4g_moe* mo);  // the part of that workspace that must start zero

}  // namespace fp4g
