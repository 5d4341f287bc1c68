// gemv_mfma.hpp -- the matrix-core variant of the decode product for M = 1..8
// vectors (the verify step of speculative decoding scores K+1 positions against
// the same weights: feed, section "MTP: the drafter inside the checkpoint").
//
// Same packed tiles, same work split and same split-K exchange tree as the VALU
// kernel (gemv_kernel.hpp); only the arithmetic differs.  The VALU kernel issues
// one v_dot2 per weight pair and token, so its issue rate falls short of HBM
// from M = 4 on.  Here the products run on v_mfma_f32_16x16x32_bf16:
//
//  * A operand = weights, as loaded: lane i holds 32 columns of row i of the
//    64-row group, so the A row of lane i is i % 16 and its K group is i / 16.
//    The four K groups therefore carry four different weight rows.
//  * B operand = a block-diagonal spread of the input: column c of B belongs to
//    token c / 4 and K group c % 4, and is nonzero only in that K group.  Then
//    D[r][c] = sum over 8 columns of W[16 (c % 4) + r][k] x_{c/4}[k]: every dot
//    product lands in its own output element, four tokens per instruction (two
//    instructions for M = 5..8).  Three quarters of each B are zeros; the matrix
//    cores still have about 5x the rate needed.
//  * E2M1 -> bf16 is exact (v_cvt_scalef32_pk_bf16_fp4), products are exact in
//    FP32.  One block (16 columns NVFP4, 32 MXFP4) is summed by chained MFMAs into
//    a fresh accumulator, then scaled once per row on the VALU: lane i's outputs
//    are rows 16 (i % 4) + 4 (i / 16) + 0..3 of token (i / 4) % 4, so it loads
//    those four rows' block scales.  Tiles stream as two halves (4 code slots
//    and their scales) to keep the double-buffered fragments in 48 VGPRs.
//  * The input columns of a workgroup's chunk range are staged in LDS (zero past
//    d_in), with a 512-byte zero area that the off-diagonal lanes read.
#pragma once
#include "gemv_kernel.hpp"

namespace fp4g {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaXBytes = 40960;  // LDS for the staged input of one workgroup (with the
                                    // 16 KiB reduction buffer: under 64 KiB)
constexpr int kZeroBytes = 512;     // one chunk row of zeros

// A fragment is half a tile: code slots 4h .. 4h+3 of lane i's row, and the
// block scales of those slots for the lane's four output rows srow .. srow+3.
template <uint32_t FMT>
struct MFrag;
template <>
struct MFrag<FP4G_NVFP4> {
  u32x4 q[4];
  u32x2 s[4];  // row srow + v: E4M3 scales of blocks 8h .. 8h+7
};
template <>
struct MFrag<FP4G_MXFP4> {
  u32x4 q[4];
  uint32_t s[4];  // row srow + v: E8M0 scales of blocks 4h .. 4h+3
};

__device__ __forceinline__ uint32_t ld_stream1(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

template <uint32_t FMT>
__device__ __forceinline__ void load_mfrag(MFrag<FMT>& f, const uint8_t* tile, int half, int lane, int srow) {
#pragma unroll
  for (int j = 0; j < 4; ++j) f.q[j] = ld_stream(tile + (4 * half + j) * 1024 + lane * 16);
  if constexpr (FMT == FP4G_NVFP4) {
#pragma unroll
    for (int v = 0; v < 4; ++v) f.s[v] = ld_stream2(tile + kCodeBytes + (srow + v) * 16 + half * 8);
  } else {
#pragma unroll
    for (int v = 0; v < 4; ++v) f.s[v] = ld_stream1(tile + kCodeBytes + (srow + v) * 8 + half * 4);
  }
}

// Eight E2M1 codes (one dword: columns 8d .. 8d+7 of the lane's 32) as bf16.
__device__ __forceinline__ bf16x8 e2m1x8_bf16(uint32_t dw) {
  const bf16x2 p0 = e2m1x2_bf16<0>(dw), p1 = e2m1x2_bf16<1>(dw);
  const bf16x2 p2 = e2m1x2_bf16<2>(dw), p3 = e2m1x2_bf16<3>(dw);
  return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const uint8_t* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

template <uint32_t FMT, int M, int NMAT, int EPI>
__global__ __launch_bounds__(kThreads) void k_gemv_mfma(GemvParams p) {
  constexpr int NSET = (M + 3) / 4;  // MFMA column sets of four tokens
  constexpr int NV = NMAT * NSET * 4;
  constexpr int TILE = FMT == FP4G_NVFP4 ? kTileNv : kTileMx;
  __shared__ float red[kWavesPerWg][NV][64];
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // [M][wg_chunks * 512] bf16, then zeros

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int gt = uniform(blockIdx.x / p.S);
  const int s = uniform(blockIdx.x % p.S);
  const int mem = NMAT == 1 ? member_of(p, gt) : 0;
  const int g = gt - p.gbase[mem];
  const uint8_t* w0 = p.w[mem];
  const uint8_t* w1 = NMAT == 2 ? p.w[1] : w0;
  const int wg_c0 = s * p.wg_chunks;
  const int wg_c1 = min(p.C, wg_c0 + p.wg_chunks);
  const int per_wave = (wg_c1 - wg_c0 + kWavesPerWg - 1) / kWavesPerWg;
  const int c0 = min(wg_c1, wg_c0 + wave * per_wave);
  const int c1 = min(wg_c1, c0 + per_wave);
  const int srow = 16 * (lane & 3) + 4 * (lane >> 4);  // first of the lane's four output rows
  const int tok = (lane >> 2) & 3;                     // the lane's token within a set
  const int64_t tile0 = (int64_t)g * p.C;
  // items (chunk, half, matrix), matrix fastest: with NMAT = 2 the even items
  // are gate, the odd ones up
  auto item_tile = [&](int it) { return (it % NMAT ? w1 : w0) + (tile0 + c0 + it / (2 * NMAT)) * TILE; };
  auto item_half = [&](int it) { return (it / NMAT) & 1; };

  // first fragment in flight before the input is staged
  const int n_items = (c1 - c0) * 2 * NMAT;
  MFrag<FMT> fa, fb;
  if (n_items > 0) load_mfrag<FMT>(fa, item_tile(0), item_half(0), lane, srow);

  // stage x[m][256 wg_c0 ..) for m < M (zero past d_in), then the zero area; all
  // loads are issued before the first LDS store
  const int tstride = p.wg_chunks * 512;  // bytes per token row in LDS
  {
    constexpr int kMaxPieces = kMfmaXBytes / 16 / kThreads;
    const int per_tok = p.wg_chunks * 32;  // 16-byte pieces per token
    const int pieces = M * per_tok;
    u32x4 v[kMaxPieces];
#pragma unroll
    for (int k = 0; k < kMaxPieces; ++k) {
      const int idx = threadIdx.x + k * kThreads;
      v[k] = u32x4{0u, 0u, 0u, 0u};
      const int m = idx / per_tok, r = idx - m * per_tok;
      const int col = wg_c0 * kChunkK + r * 8;
      if (idx < pieces && col < p.d_in) v[k] = *reinterpret_cast<const u32x4*>(p.x + (int64_t)m * p.d_in + col);
    }
#pragma unroll
    for (int k = 0; k < kMaxPieces; ++k) {
      const int idx = threadIdx.x + k * kThreads;
      if (idx < pieces) {
        const int m = idx / per_tok, r = idx - m * per_tok;
        *reinterpret_cast<u32x4*>(xs + m * tstride + r * 16) = v[k];
      }
    }
    if (threadIdx.x < kZeroBytes / 16)
      *reinterpret_cast<u32x4*>(xs + M * tstride + threadIdx.x * 16) = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  // B operand addresses: a lane is on the diagonal when its column's K group
  // (lane % 4) is its own K group (lane / 16)
  const bool diag = (lane & 3) == (lane >> 4);
  int boff[NSET];
  bool bval[NSET];
#pragma unroll
  for (int q = 0; q < NSET; ++q) {
    bval[q] = diag && (4 * q + tok < M);
    boff[q] = bval[q] ? (4 * q + tok) * tstride : M * tstride;
  }

  f32x4 acc[NMAT][NSET];
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int q = 0; q < NSET; ++q) acc[a][q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // items alternate matrices (NMAT = 2), so fragment fa always holds matrix 0
  // and fb the last one: each call names its accumulators statically
  auto consume = [&](const MFrag<FMT>& f, int it, f32x4(&ac)[NSET]) {
    const int cc = c0 + it / (2 * NMAT) - wg_c0;  // chunk within the staged range
    const int half = item_half(it);
    int bb[NSET];
#pragma unroll
    for (int q = 0; q < NSET; ++q) bb[q] = boff[q] + (bval[q] ? cc * 512 : 0);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = 4 * half + jj;  // slot within the chunk
      if constexpr (FMT == FP4G_NVFP4) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // 16-column blocks 2j, 2j+1 = dwords 2h, 2h+1
          const bf16x8 a0 = e2m1x8_bf16(f.q[jj][2 * h]);
          const bf16x8 a1 = e2m1x8_bf16(f.q[jj][2 * h + 1]);
          const int lb = 2 * jj + h;  // block within the half: dword lb/4, byte lb%4 of s[v]
          float sc[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t sdw = f.s[v][lb >> 2];
            sc[v] = (lb & 3) == 0 ? e4m3_f32<0>(sdw) : (lb & 3) == 1 ? e4m3_f32<1>(sdw)
                  : (lb & 3) == 2 ? e4m3_f32<2>(sdw) : e4m3_f32<3>(sdw);
          }
#pragma unroll
          for (int q = 0; q < NSET; ++q) {
            const int off = bb[q] + (32 * j + 16 * h) * 2;
            f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, lds_bf16x8(xs, off), f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                              0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, lds_bf16x8(xs, off + 16), t, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) ac[q][v] = __builtin_fmaf(t[v], sc[v], ac[q][v]);
          }
        }
      } else {
        // one 32-column block per slot: byte jj of s[v]
        int e[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) e[v] = (int)((f.s[v] >> (8 * jj)) & 0xffu) - 127;
        bf16x8 av[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) av[d] = e2m1x8_bf16(f.q[jj][d]);
#pragma unroll
        for (int q = 0; q < NSET; ++q) {
          const int off = bb[q] + 32 * j * 2;
          f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[0], lds_bf16x8(xs, off), f32x4{0.0f, 0.0f, 0.0f, 0.0f},
                                                            0, 0, 0);
#pragma unroll
          for (int d = 1; d < 4; ++d)
            t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[d], lds_bf16x8(xs, off + 16 * d), t, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) ac[q][v] += __builtin_amdgcn_ldexpf(t[v], e[v]);
        }
      }
      // keep each slot's LDS reads and conversions next to its MFMAs (hoisting
      // them across slots costs registers, then spills)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (n_items > 0) {
    int it = 0;
    for (; it + 2 < n_items; it += 2) {
      load_mfrag<FMT>(fb, item_tile(it + 1), item_half(it + 1), lane, srow);
      consume(fa, it, acc[0]);
      load_mfrag<FMT>(fa, item_tile(it + 2), item_half(it + 2), lane, srow);
      consume(fb, it + 1, acc[NMAT - 1]);
    }
    if (it + 1 < n_items) {
      load_mfrag<FMT>(fb, item_tile(it + 1), item_half(it + 1), lane, srow);
      consume(fa, it, acc[0]);
      consume(fb, it + 1, acc[NMAT - 1]);
    } else {
      consume(fa, it, acc[0]);
    }
  }

#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int q = 0; q < NSET; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][(a * NSET + q) * 4 + v][lane] = acc[a][q][v];
  __syncthreads();
  if (wave != 0) return;

  float val[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) val[i] = ((red[0][i][lane] + red[1][i][lane]) + red[2][i][lane]) + red[3][i][lane];

  // units: EPI_STORE rows (srow + 2w, srow + 2w + 1) of set q; EPI_SILU (gate,
  // up) of row srow + v of set q
  constexpr int NU = EPI == EPI_SILU ? 4 * NSET : 2 * NSET;
  float ua[NU], ub[NU];
  bool live[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if constexpr (EPI == EPI_SILU) {
      ua[u] = val[u];
      ub[u] = val[NSET * 4 + u];
    } else {
      ua[u] = val[2 * u];
      ub[u] = val[2 * u + 1];
    }
    live[u] = true;
  }
  exchange_tree<NU>(p.slots, (int64_t)p.gbase[p.n] * 64, (int64_t)gt * 64 + lane, p.S, s, ua, ub, live);

  const int d_out = p.d_out[mem];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (!live[u]) continue;
    if constexpr (EPI == EPI_SILU) {
      const int q = u / 4, v = u % 4;
      const int m = 4 * q + tok, row = g * 64 + srow + v;
      if (m < M && row < d_out) {
        const float gv = ua[u] * p.tscale[0], uv = ub[u] * p.tscale[1];
        p.h[(int64_t)m * d_out + row] = f32_to_bf16_rne(silu_f32(gv) * uv);
      }
    } else {
      const int q = u / 2, w = u % 2;
      const int m = 4 * q + tok, row = g * 64 + srow + 2 * w;
      if (m < M) {
        float* y = p.y[mem] + (int64_t)m * d_out;
        if (row < d_out) y[row] = ua[u] * p.tscale[mem];
        if (row + 1 < d_out) y[row + 1] = ub[u] * p.tscale[mem];
      }
    }
  }
}

// ---- launch planning for the MFMA kernel ------------------------------------------
// The VALU plan, with S raised where needed so that a workgroup's staged input
// (M rows of its chunk range) fits the LDS budget.
inline Plan plan_mfma(int64_t R, int64_t C, int nmat, int M) {
  (void)nmat;
  Plan pl = plan_nw4(R, C);
  const int64_t max_chunks = kMfmaXBytes / (M * 512);
  if (pl.wg_chunks > max_chunks) {
    int64_t S = (C + max_chunks - 1) / max_chunks;
    const int64_t wg_chunks = (C + S - 1) / S;
    S = (C + wg_chunks - 1) / wg_chunks;
    pl = Plan{(int)S, (int)wg_chunks, kWavesPerWg};
  }
  return pl;
}

inline size_t mfma_lds_bytes(const Plan& pl, int M) { return (size_t)M * pl.wg_chunks * 512 + kZeroBytes; }

// Exchange units per lane: the larger of the two kernels' needs.
inline int64_t exchange_units_any(int nmat, int M) {
  const int64_t nset = (M + 3) / 4;
  const int64_t mf = nmat == 2 ? 4 * nset : 2 * nset;
  const int64_t vu = exchange_units(nmat, M);
  return mf > vu ? mf : vu;
}

// Workspace for either kernel (the caller may choose the path per call).
inline uint64_t gemv_ws_bytes_any(int64_t R_total, int64_t C, int nmat, int M) {
  const Plan a = plan_for(R_total, C, nmat, M), b = plan_mfma(R_total, C, nmat, M);
  const int64_t nodes = tree_nodes(a.S) > tree_nodes(b.S) ? tree_nodes(a.S) : tree_nodes(b.S);
  return (uint64_t)nodes * exchange_units_any(nmat, M) * R_total * 64 * 8;
}

template <uint32_t FMT, int NMAT, int EPI>
hipError_t launch_mfma(int M, const GemvParams& p, unsigned grid, size_t lds, hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM)                                                       \
  case MM:                                                                  \
    k_gemv_mfma<FMT, MM, NMAT, EPI><<<grid, kThreads, lds, s>>>(p); \
    break;
    FP4G_CASE(1) FP4G_CASE(2) FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fp4g
