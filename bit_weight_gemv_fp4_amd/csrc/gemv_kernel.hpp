// gemv_kernel.hpp -- the decode GEMV kernel template for gfx950 (included by the
// per-format translation units gemv_nvfp4.hip, gemv_mxfp4.hip, gemv_fp8.hip).
//
// The product y = W x streams every weight byte once at 16/b flop per byte (4 for
// NVFP4, 2 for FP8: mdjawad.com DGX Spark feed, "Decode speed is bytes divided by
// bandwidth"), so the kernels are built around HBM streaming, not arithmetic:
//
//  * Work item = one tile column range of one 64-row group.  Lane l of a wave owns
//    row 64g + l and keeps its M dot products in registers for the whole K range,
//    so the hot loop has no cross-lane traffic.  Every wave-wide load reads a
//    contiguous 1 KiB slice of the packed tile (nontemporal, 16 B per lane).
//  * x is the same for every lane: it is read with scalar loads into SGPRs and fed
//    to v_dot2_f32_bf16 as the scalar operand.
//  * E2M1 pairs become exact bf16 pairs with one v_cvt_scalef32_pk_bf16_fp4 (scale
//    1.0); v_dot2_f32_bf16 multiplies them by x exactly and accumulates in FP32.
//    The E4M3 block scale (v_cvt_f32_fp8) multiplies each 16-weight block sum once
//    (NVFP4); the E8M0 scale is applied by ldexp to each 32-weight block (MXFP4);
//    FP8 rows convert with v_cvt_scalef32_pk_bf16_fp8 and take the row scale in
//    the epilogue.
//  * Split-K: a row group's chunks are divided over S workgroups of four waves so
//    that there are enough waves to keep all 256 CUs streaming.  The four waves of
//    a workgroup reduce through LDS in a fixed order; across workgroups, partial
//    sums go to the workspace and the last workgroup to arrive (device-scope
//    counter) adds them in split order and runs the epilogue.  Results are
//    therefore deterministic.
#pragma once
#include "common.hpp"

namespace fp4g {


enum { EPI_STORE = 0, EPI_SILU = 1 };

struct GemvParams {
  const uint8_t* w[2];     // packed images (tiles) of up to two matrices of one shape
  float tscale[2];         // NVFP4 tensor scales (1.0 otherwise)
  const uint16_t* x;       // bf16 [M][d_in]
  float* y;                // EPI_STORE: f32 [M][d_out]
  uint16_t* h;             // EPI_SILU: bf16 [M][d_out]
  float* part;             // split-K partial sums [S][NMAT][M][R*64]
  unsigned* counters;      // [R] arrival counters (zero between calls)
  int d_out, d_in, R, C;
  int S;                   // workgroups per row group
  int wg_chunks;           // chunks per workgroup (the last one may get fewer)
};

template <uint32_t FMT>
struct Frag;
template <>
struct Frag<FP4G_NVFP4> {
  u32x4 q[kPiecesNv];
  u32x4 s;
};
template <>
struct Frag<FP4G_MXFP4> {
  u32x4 q[kPiecesNv];
  u32x2 s;
};
template <>
struct Frag<FP4G_FP8_ROW> {
  u32x4 q[kSlotsFp8];
};

template <uint32_t FMT>
__device__ __forceinline__ void load_frag(Frag<FMT>& f, const uint8_t* tile, int lane) {
  if constexpr (FMT == FP4G_FP8_ROW) {
#pragma unroll
    for (int j = 0; j < kSlotsFp8; ++j) f.q[j] = ld_stream(tile + j * 1024 + lane * 16);
  } else {
#pragma unroll
    for (int j = 0; j < kPiecesNv; ++j) f.q[j] = ld_stream(tile + j * 1024 + lane * 16);
    if constexpr (FMT == FP4G_NVFP4)
      f.s = ld_stream(tile + kCodeBytes + lane * 16);
    else
      f.s = ld_stream2(tile + kCodeBytes + lane * 8);
  }
}

// Accumulate one tile (columns 256c .. 256c+255, or its first `npieces` 32-column
// pieces when FULL is false) of one matrix into acc[0..M).  xc points at the bf16
// pairs of column 256c of token 0; token m is xc + m * xstride (in u32 units).
template <uint32_t FMT, int M, bool FULL>
__device__ __forceinline__ void tile_dot(const Frag<FMT>& f, const uint32_t* __restrict__ xc, int xstride,
                                         int npieces, float (&acc)[M]) {
  if constexpr (FMT == FP4G_FP8_ROW) {
#pragma unroll
    for (int j = 0; j < kSlotsFp8; ++j) {
      if (!FULL && j >= 2 * npieces) continue;
      bf16x2 w[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        w[2 * d] = e4m3x2_bf16<false>(f.q[j][d]);
        w[2 * d + 1] = e4m3x2_bf16<true>(f.q[j][d]);
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint32_t* xm = xc + m * xstride + j * 8;
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          p0 = dot2(w[i], xm[i], p0);
          p1 = dot2(w[i + 1], xm[i + 1], p1);
        }
        acc[m] += p0 + p1;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPiecesNv; ++j) {
      if (!FULL && j >= npieces) continue;
      // 32 weights: dwords 0,1 = block 0 (16 weights), dwords 2,3 = block 1
      bf16x2 w[16];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        w[4 * d + 0] = e2m1x2_bf16<0>(f.q[j][d]);
        w[4 * d + 1] = e2m1x2_bf16<1>(f.q[j][d]);
        w[4 * d + 2] = e2m1x2_bf16<2>(f.q[j][d]);
        w[4 * d + 3] = e2m1x2_bf16<3>(f.q[j][d]);
      }
      if constexpr (FMT == FP4G_NVFP4) {
        // scale bytes 2j, 2j+1 of the lane's 16: dword j/2, bytes 2(j&1), 2(j&1)+1
        const uint32_t sdw = f.s[j >> 1];
        const float s0 = (j & 1) ? e4m3_f32<2>(sdw) : e4m3_f32<0>(sdw);
        const float s1 = (j & 1) ? e4m3_f32<3>(sdw) : e4m3_f32<1>(sdw);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const uint32_t* xm = xc + m * xstride + j * 16;
          float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            p0 = dot2(w[i], xm[i], p0);
            p1 = dot2(w[8 + i], xm[8 + i], p1);
          }
          acc[m] = __builtin_fmaf(p0, s0, acc[m]);
          acc[m] = __builtin_fmaf(p1, s1, acc[m]);
        }
      } else {
        // one E8M0 scale per 32 weights: byte j of the lane's 8
        const int e = (int)((f.s[j >> 2] >> (8 * (j & 3))) & 0xffu);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const uint32_t* xm = xc + m * xstride + j * 16;
          float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            p0 = dot2(w[i], xm[i], p0);
            p1 = dot2(w[8 + i], xm[8 + i], p1);
          }
          acc[m] += __builtin_amdgcn_ldexpf(p0 + p1, e - 127);
        }
      }
    }
  }
}

// Epilogue for one row of one 64-row group, given the full dot products v.
template <uint32_t FMT, int M, int NMAT, int EPI>
__device__ __forceinline__ void finish_row(const GemvParams& p, int row, const float (&v)[NMAT * M]) {
  if (row >= p.d_out) return;
  if constexpr (EPI == EPI_STORE) {
    float sc = p.tscale[0];
    if constexpr (FMT == FP4G_FP8_ROW) {
      const float* rs = reinterpret_cast<const float*>(p.w[0] + (int64_t)p.R * p.C * kTileF8);
      sc = rs[row];
    }
#pragma unroll
    for (int m = 0; m < M; ++m) p.y[(int64_t)m * p.d_out + row] = v[m] * sc;
  } else {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const float g = v[m] * p.tscale[0];
      const float u = v[M + m] * p.tscale[1];
      p.h[(int64_t)m * p.d_out + row] = f32_to_bf16_rne(silu_f32(g) * u);
    }
  }
}

template <uint32_t FMT, int M, int NMAT, int EPI>
__global__ __launch_bounds__(kThreads) void k_gemv(GemvParams p) {
  constexpr int NA = NMAT * M;
  constexpr int TILE = FMT == FP4G_NVFP4 ? kTileNv : FMT == FP4G_MXFP4 ? kTileMx : kTileF8;
  __shared__ float red[kWavesPerWg][NA][64];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int g = uniform(blockIdx.x / p.S);
  const int s = uniform(blockIdx.x % p.S);
  const int wg_c0 = s * p.wg_chunks;
  const int wg_c1 = min(p.C, wg_c0 + p.wg_chunks);
  const int per_wave = (wg_c1 - wg_c0 + kWavesPerWg - 1) / kWavesPerWg;
  const int c0 = min(wg_c1, wg_c0 + wave * per_wave);
  const int c1 = min(wg_c1, c0 + per_wave);

  float acc[NMAT][M];
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[a][m] = 0.0f;

  const uint32_t* __restrict__ x32 = reinterpret_cast<const uint32_t*>(p.x);
  const int xstride = p.d_in / 2;
  const int full_chunks = p.d_in / kChunkK;  // chunks with all 8 pieces present
  const int tail_pieces = (p.d_in % kChunkK) / kPieceK;

  // Items are (chunk, matrix) pairs visited chunk-major.  Two register fragments
  // alternate: the tile of item it+1 is in flight while item it is consumed.
  const int n_items = (c1 - c0) * NMAT;
  const int64_t tile0 = (int64_t)g * p.C;
  auto item_tile = [&](int it) { return p.w[it % NMAT] + (tile0 + c0 + it / NMAT) * TILE; };
  auto consume = [&](const Frag<FMT>& f, int it) {
    const int c = c0 + it / NMAT;
    const uint32_t* xc = x32 + (int64_t)c * (kChunkK / 2);
    float part[M];
#pragma unroll
    for (int m = 0; m < M; ++m) part[m] = 0.0f;
    if (c < full_chunks)
      tile_dot<FMT, M, true>(f, xc, xstride, kPiecesNv, part);
    else
      tile_dot<FMT, M, false>(f, xc, xstride, tail_pieces, part);
    if (NMAT == 1 || it % NMAT == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[0][m] += part[m];
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[NMAT - 1][m] += part[m];
    }
  };
  if (n_items > 0) {
    // The loop body always has both fragments' loads in flight, so the wait before
    // each consume is a fixed "all but the newest fragment" count; the last one
    // or two items are peeled off.
    Frag<FMT> fa, fb;
    load_frag<FMT>(fa, item_tile(0), lane);
    int it = 0;
    for (; it + 2 < n_items; it += 2) {
      load_frag<FMT>(fb, item_tile(it + 1), lane);
      consume(fa, it);
      load_frag<FMT>(fa, item_tile(it + 2), lane);
      consume(fb, it + 1);
    }
    if (it + 1 < n_items) {
      load_frag<FMT>(fb, item_tile(it + 1), lane);
      consume(fa, it);
      consume(fb, it + 1);
    } else {
      consume(fa, it);
    }
  }

#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int m = 0; m < M; ++m) red[wave][a * M + m][lane] = acc[a][m];
  __syncthreads();
  if (wave != 0) return;

  float v[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) v[i] = ((red[0][i][lane] + red[1][i][lane]) + red[2][i][lane]) + red[3][i][lane];

  const int row = g * 64 + lane;
  if (p.S == 1) {
    finish_row<FMT, M, NMAT, EPI>(p, row, v);
    return;
  }
  // split-K hand-off: publish partials, count arrivals, the last one finishes
  const int64_t rpad = (int64_t)p.R * 64;
#pragma unroll
  for (int i = 0; i < NA; ++i) publish_partial(p.part + ((int64_t)s * NA + i) * rpad + row, v[i]);
  if (!arrive_last(p.counters + g, (unsigned)(p.S - 1))) return;
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    float t = 0.0f;
    for (int q = 0; q < p.S; ++q) t += collect_partial(p.part + ((int64_t)q * NA + i) * rpad + row);
    v[i] = t;
  }
  finish_row<FMT, M, NMAT, EPI>(p, row, v);
  reset_counter(p.counters + g);
}

template <uint32_t FMT, int NMAT, int EPI>
hipError_t launch_m(int M, const GemvParams& p, unsigned grid, hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM) \
  case MM:            \
    k_gemv<FMT, MM, NMAT, EPI><<<grid, kThreads, 0, s>>>(p); \
    break;
    FP4G_CASE(1) FP4G_CASE(2) FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---- launch planning -----------------------------------------------------------
struct Plan {
  int S;          // workgroups per row group
  int wg_chunks;  // chunks per workgroup
};

// Enough waves to cover HBM latency on all 256 CUs (about eight per CU), with at
// least one chunk per wave; chunks are spread evenly over the S workgroups.
inline Plan plan_for(int64_t R, int64_t C, int nmat) {
  (void)nmat;
  const int64_t target_waves = 2048;
  int64_t q = (R * C) / target_waves;  // chunks per wave
  if (q < 1) q = 1;
  if (R > kMaxCounters) return Plan{1, (int)C};  // (S > 1 needs R < 512 anyway)
  int64_t S = (C + kWavesPerWg * q - 1) / (kWavesPerWg * q);
  if (S < 1) S = 1;
  const int64_t wg_chunks = (C + S - 1) / S;
  S = (C + wg_chunks - 1) / wg_chunks;
  return Plan{(int)S, (int)wg_chunks};
}

inline uint64_t align256(uint64_t b) { return (b + 255) & ~uint64_t(255); }

inline uint64_t gemv_ws_bytes(int64_t R, int64_t C, int nmat, int M) {
  const Plan pl = plan_for(R, C, nmat);
  if (pl.S == 1) return 0;
  return kCounterBytes + (uint64_t)pl.S * nmat * M * R * 64 * 4;
}

}  // namespace fp4g
