// quant.hip -- load-time quantisers: fp4g_quantize (bf16 matrix -> NVFP4, MXFP4
// or FP8-row codes and scales in the logical layout fp4g_pack takes).
//
// NVFP4 (mdjawad.com DGX Spark feed, section "Fewer bytes per weight: NVFP4"):
// every block of 16 consecutive weights gets a scale that maps its largest
// magnitude to 6, stored as E4M3; one FP32 scale per tensor brings the block
// scales into E4M3's range.  Taken here: s_T = amax(W) / (6 * 448);
// block code = E4M3_RNE(amax_b / (6 s_T)); element = E2M1_RNE(w / (s_b s_T)).
// MXFP4: the smallest power of two 2^e with amax_b / 2^e <= 6 (E8M0 code
// e + 127); FP8 rows: s_row = amax_row / 448.  Rounding is to nearest, ties to
// the even code, saturating; zero magnitudes get the positive-zero code.  s_T
// and s_row are the FP32 values nearest to their quotients (IEEE division);
// every code is then the grid value nearest to the EXACT quotient: a first
// guess from the FP32 quotient (at most one code off) is corrected by the sign
// of fma(-mid * k, s, a) = a - mid * k * s rounded once, whose sign is exact.
#include <algorithm>

#include "common.hpp"

namespace fp4g {
namespace {

// E4M3FN code (0..126) to its value.
__device__ __forceinline__ float e4m3_val(uint32_t c) {
  const int e = (int)(c >> 3), m = (int)(c & 7u);
  return e == 0 ? __builtin_amdgcn_ldexpf((float)m, -9) : __builtin_amdgcn_ldexpf(8.0f + (float)m, e - 10);
}

// E2M1 code of q: the nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6 by magnitude (ties to
// the even code, larger magnitudes saturate to 6), sign in bit 3 unless zero.
__device__ __forceinline__ uint32_t e2m1_rne(float q) {
  const float a = fabsf(q);
  uint32_t c;
  if (a <= 0.25f) c = 0;
  else if (a < 0.75f) c = 1;
  else if (a <= 1.25f) c = 2;
  else if (a < 1.75f) c = 3;
  else if (a <= 2.5f) c = 4;
  else if (a < 3.5f) c = 5;
  else if (a <= 5.0f) c = 6;
  else c = 7;
  return (q < 0.0f && c != 0) ? (c | 8u) : c;
}

__device__ __forceinline__ float bf16_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Midpoint between the magnitudes of codes c and c + 1 (exact in FP32).
__device__ __forceinline__ float e2m1_mid(uint32_t c) {
  constexpr float kMid[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
  return kMid[c];
}
__device__ __forceinline__ float e4m3_mid(uint32_t c) { return (e4m3_val(c) + e4m3_val(c + 1)) * 0.5f; }

// The code nearest to the exact quotient a / (k s) (a >= 0, k s > 0), given a
// guess c at most one code away: the sign of a - mid * k * s decides each
// neighbouring midpoint exactly (mid * k is exact in FP32: at most 5 + 4
// significant bits; the fma rounds once, which keeps the sign).  At a midpoint
// the even code wins; cmax saturates.
template <class Mid>
__device__ __forceinline__ uint32_t exact_code(uint32_t c, uint32_t cmax, float a, float k, float s, Mid mid) {
  if (c < cmax) {
    const float r = __builtin_fmaf(-(mid(c) * k), s, a);
    if (r > 0.0f || (r == 0.0f && ((c + 1) & 1u) == 0)) return c + 1;
  }
  if (c > 0) {
    const float r = __builtin_fmaf(-(mid(c - 1) * k), s, a);
    if (r < 0.0f || (r == 0.0f && ((c - 1) & 1u) == 0)) return c - 1;
  }
  return c;
}

// Largest |w| of the tensor as the bit pattern of a non-negative bf16 (ordered
// like the value), into *amax (zeroed by k_zero_u32 first).
__global__ void k_zero_u32(unsigned* p) {
  if (threadIdx.x == 0) *p = 0u;
}
__global__ __launch_bounds__(256) void k_amax_bf16(const uint16_t* w, int64_t n, unsigned* amax) {
  unsigned m = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    m = max(m, (unsigned)(w[i] & 0x7fffu));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (unsigned)__shfl_xor((int)m, off, 64));
  if ((threadIdx.x & 63) == 0) atomicMax(amax, m);
}

// One thread per block of BLK weights (NVFP4: 16, MXFP4: 32).
template <uint32_t FMT>
__global__ __launch_bounds__(256) void k_quant_fp4(const uint16_t* w, int d_out, int d_in, const unsigned* amax_t,
                                                   uint8_t* codes, uint8_t* scales, float* tensor_scale) {
  constexpr int BLK = FMT == FP4G_NVFP4 ? 16 : 32;
  const int nb = d_in / BLK;
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float s_t = 1.0f, six_st = 6.0f;
  if constexpr (FMT == FP4G_NVFP4) {
    const float a = bf16_f32((uint16_t)*amax_t);
    s_t = a > 0.0f ? a / 2688.0f : 1.0f;
    six_st = 6.0f * s_t;
    if (b == 0 && tensor_scale) *tensor_scale = s_t;
  } else {
    if (b == 0 && tensor_scale) *tensor_scale = 1.0f;
  }
  if (b >= (int64_t)d_out * nb) return;
  const int64_t r = b / nb, k0 = (b % nb) * BLK;
  const uint16_t* src = w + r * d_in + k0;
  float v[BLK];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < BLK; ++k) {
    v[k] = bf16_f32(src[k]);
    amax = fmaxf(amax, fabsf(v[k]));
  }
  uint32_t el[BLK];
  if constexpr (FMT == FP4G_NVFP4) {
    const uint32_t sc = exact_code(e4m3_rne_pos(amax / six_st), 126u, amax, 6.0f, s_t, e4m3_mid);
    scales[b] = (uint8_t)sc;
    const float sb = e4m3_val(sc);
    const float den = sb * s_t;
#pragma unroll
    for (int k = 0; k < BLK; ++k) {
      const uint32_t c = exact_code(e2m1_rne(fabsf(v[k]) / den), 7u, fabsf(v[k]), sb, s_t, e2m1_mid);
      el[k] = sb > 0.0f ? ((v[k] < 0.0f && c != 0) ? (c | 8u) : c) : 0u;
    }
  } else {
    int code = 127;
    if (amax > 0.0f) {
      int ex;
      const float mant = frexpf(amax, &ex);  // amax = mant 2^ex, mant in [0.5, 1)
      // amax <= 6 * 2^e  <=>  e >= ex - 2 when 2 mant <= 1.5, else e >= ex - 1
      const int e = (mant <= 0.75f) ? ex - 3 : ex - 2;
      code = min(max(e + 127, 0), 254);
    }
    scales[b] = (uint8_t)code;
#pragma unroll
    for (int k = 0; k < BLK; ++k) el[k] = e2m1_rne(__builtin_amdgcn_ldexpf(v[k], 127 - code));
  }
  uint8_t* dst = codes + (r * d_in + k0) / 2;
#pragma unroll
  for (int k = 0; k < BLK; k += 2) dst[k / 2] = (uint8_t)(el[k] | (el[k + 1] << 4));
}

// One wave per row.
__global__ __launch_bounds__(256) void k_quant_fp8(const uint16_t* w, int d_out, int d_in, uint8_t* codes,
                                                   float* row_scale, float* tensor_scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0 && tensor_scale) *tensor_scale = 1.0f;
  if (r >= d_out) return;
  const uint16_t* src = w + r * d_in;
  float amax = 0.0f;
  for (int k = lane; k < d_in; k += 64) amax = fmaxf(amax, fabsf(bf16_f32(src[k])));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
  if (lane == 0) row_scale[r] = s;
  for (int k = lane; k < d_in; k += 64) {
    const float v = bf16_f32(src[k]);
    const uint32_t c = exact_code(e4m3_rne_pos(fabsf(v) / s), 126u, fabsf(v), 1.0f, s, e4m3_mid);
    codes[r * d_in + k] = (uint8_t)((v < 0.0f && c != 0) ? (c | 0x80u) : c);
  }
}

}  // namespace
}  // namespace fp4g

using namespace fp4g;

extern "C" int32_t fp4g_quantize(uint32_t format, int32_t d_out, int32_t d_in, const uint16_t* w, void* codes,
                                 void* scales, float* tensor_scale, void* ws, uint64_t ws_bytes, void* stream) {
  if (format != FP4G_NVFP4 && format != FP4G_MXFP4 && format != FP4G_FP8_ROW) return FP4G_E_FORMAT;
  if (!w || !codes || !scales) return FP4G_E_NULL;
  if (d_out < 1 || d_in < 32 || d_in % 32) return FP4G_E_SHAPE;
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 16) || (tensor_scale && !aligned(tensor_scale, 4)))
    return FP4G_E_ALIGN;
  const bool nv = format == FP4G_NVFP4;
  if (nv && !ws) return FP4G_E_NULL;
  if (nv && ws_bytes < 256) return FP4G_E_WORKSPACE;
  const size_t wb = (size_t)d_out * d_in * 2;
  const size_t cb = format == FP4G_FP8_ROW ? (size_t)d_out * d_in : (size_t)d_out * d_in / 2;
  const size_t sb = format == FP4G_FP8_ROW ? (size_t)d_out * 4 : (size_t)d_out * d_in / (nv ? 16 : 32);
  const void* outs[4] = {codes, scales, tensor_scale, nv ? ws : nullptr};
  const size_t ob[4] = {cb, sb, tensor_scale ? 4u : 0u, nv ? 256u : 0u};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], ob[i], w, wb)) return FP4G_E_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], ob[i], outs[j], ob[j])) return FP4G_E_ALIAS;
  }
  hipStream_t s = (hipStream_t)stream;
  if (format == FP4G_FP8_ROW) {
    k_quant_fp8<<<(unsigned)((d_out + 3) / 4), 256, 0, s>>>(w, d_out, d_in, (uint8_t*)codes, (float*)scales,
                                                            tensor_scale);
  } else {
    const int64_t blocks = (int64_t)d_out * (d_in / (nv ? 16 : 32));
    const unsigned grid = (unsigned)((blocks + 255) / 256);
    unsigned* amax = (unsigned*)ws;
    if (nv) {
      k_zero_u32<<<1, 64, 0, s>>>(amax);
      const int64_t n = (int64_t)d_out * d_in;
      const unsigned g = (unsigned)std::min<int64_t>((n + 255) / 256, 4096);
      k_amax_bf16<<<g, 256, 0, s>>>(w, n, amax);
      k_quant_fp4<FP4G_NVFP4><<<grid, 256, 0, s>>>(w, d_out, d_in, amax, (uint8_t*)codes, (uint8_t*)scales,
                                                    tensor_scale);
    } else {
      k_quant_fp4<FP4G_MXFP4><<<grid, 256, 0, s>>>(w, d_out, d_in, nullptr, (uint8_t*)codes, (uint8_t*)scales,
                                                    tensor_scale);
    }
  }
  return hipGetLastError() == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}
