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
//    a workgroup reduce through LDS in a fixed order; across workgroups the sums
//    meet in a binary tree of device-scope atomic exchanges (one round trip per
//    level, no counters, no fences).  Each pair sum is commutative and the tree
//    shape is fixed, so results are deterministic.
//  * Grouped launch: up to four matrices of one format and input width (the Q, K
//    and V projections of a layer) share one launch; each row group knows its
//    member from the group's row-group offsets.
#pragma once
#include <initializer_list>

#include "common.hpp"

namespace fp4g {


// EPI_ARGMAX: products as EPI_STORE (logits written only when y[0] is set), plus
// each vector's largest logit and its row (ties to the lower row) over the launch.
enum { EPI_STORE = 0, EPI_SILU = 1, EPI_ARGMAX = 2 };
constexpr int kArgSlots = 64;  // spread slots of the launch-wide maximum

constexpr int kMaxGroup = 4;  // matrices sharing one input in one launch

struct GemvParams {
  // NMAT == 1: n members (matrices sharing x), each with its own output;
  // NMAT == 2: one gate/up pair (w[0], w[1]) of one shape, fused epilogue.
  const uint8_t* w[kMaxGroup];
  float tscale[kMaxGroup];
  float* y[kMaxGroup];        // EPI_STORE: f32 [M][d_out[i]]
  int d_out[kMaxGroup];
  int gbase[kMaxGroup + 1];   // first global 64-row group of member i; gbase[n] = all groups
  int n;
  const uint16_t* x;          // bf16 [M][d_in]
  uint16_t* h;                // EPI_SILU: bf16 [M][d_out[0]]
  unsigned long long* slots;  // split-K exchange slots, zero between calls
  const float* rs[kMaxGroup];  // FP8 rows: member i's row scales (EPI_SILU: gate, up)
  unsigned long long* amax;   // EPI_ARGMAX: [kArgSlots][kMaxMWide] keys, zero between calls
  int32_t* top_idx;           // EPI_ARGMAX: [M] row of the largest logit (+ row_base)
  float* top_val;             // EPI_ARGMAX: [M] the largest logit
  int row_base;               // EPI_ARGMAX: added to the reported row
  int d_in, C;
  int S;                      // workgroups per row group
  int wg_chunks;              // chunks per workgroup (the last ones may get fewer)
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
struct Frag<FP4G_FP8_ROW> {  // half a tile: slots 0-7 or 8-15
  u32x4 q[kHalfFp8];
};

template <uint32_t FMT>
__device__ __forceinline__ void load_frag(Frag<FMT>& f, const uint8_t* tile, int lane) {
  if constexpr (FMT == FP4G_FP8_ROW) {  // `tile` is the half's first byte
#pragma unroll
    for (int j = 0; j < kHalfFp8; ++j) f.q[j] = ld_stream(tile + j * 1024 + lane * 16);
  } else {
#pragma unroll
    for (int j = 0; j < kPiecesNv; ++j) f.q[j] = ld_stream(tile + j * 1024 + lane * 16);
    if constexpr (FMT == FP4G_NVFP4)
      f.s = ld_stream(tile + kCodeBytes + lane * 16);
    else
      f.s = ld_stream2(tile + kCodeBytes + lane * 8);
  }
}

// One 32-column piece j of an NVFP4/MXFP4 tile against x values xv[m][0..15]
// (bf16 pairs of the piece's columns, per vector).
template <uint32_t FMT, int M>
__device__ __forceinline__ void piece_dot(const Frag<FMT>& f, int j, const uint32_t (&xv)[M][16], float (&acc)[M]) {
  bf16x2 w[16];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    w[4 * d + 0] = e2m1x2_bf16<0>(f.q[j][d]);
    w[4 * d + 1] = e2m1x2_bf16<1>(f.q[j][d]);
    w[4 * d + 2] = e2m1x2_bf16<2>(f.q[j][d]);
    w[4 * d + 3] = e2m1x2_bf16<3>(f.q[j][d]);
  }
  if constexpr (FMT == FP4G_NVFP4) {
    const uint32_t sdw = f.s[j >> 1];
    const float s0 = (j & 1) ? e4m3_f32<2>(sdw) : e4m3_f32<0>(sdw);
    const float s1 = (j & 1) ? e4m3_f32<3>(sdw) : e4m3_f32<1>(sdw);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p0 = dot2(w[i], xv[m][i], p0);
        p1 = dot2(w[8 + i], xv[m][8 + i], p1);
      }
      acc[m] = __builtin_fmaf(p0, s0, acc[m]);
      acc[m] = __builtin_fmaf(p1, s1, acc[m]);
    }
  } else {
    const int e = (int)((f.s[j >> 2] >> (8 * (j & 3))) & 0xffu);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p0 = dot2(w[i], xv[m][i], p0);
        p1 = dot2(w[8 + i], xv[m][8 + i], p1);
      }
      acc[m] += __builtin_amdgcn_ldexpf(p0 + p1, e - 127);
    }
  }
}

// Accumulate one tile (columns 256c .. 256c+255, or its first `npieces` 32-column
// pieces when FULL is false) of one matrix into acc[0..M).  xc points at the bf16
// pairs of column 256c of token 0; token m is xc + m * xstride (in u32 units).
// FP8: one half tile (128 columns; its first `npieces` 16-column slots when FULL
// is false), xc at the half's first column.
template <uint32_t FMT, int M, bool FULL>
__device__ __forceinline__ void tile_dot(const Frag<FMT>& f, const uint32_t* __restrict__ xc, int xstride,
                                         int npieces, float (&acc)[M]) {
  if constexpr (FMT == FP4G_FP8_ROW) {
    // x of up to XV vectors is read together (scalar loads, one wait per group)
    constexpr int XV = M < 4 ? M : 4;
#pragma unroll
    for (int j = 0; j < kHalfFp8; ++j) {
      if (!FULL && j >= npieces) continue;
      bf16x2 w[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        w[2 * d] = e4m3x2_bf16<false>(f.q[j][d]);
        w[2 * d + 1] = e4m3x2_bf16<true>(f.q[j][d]);
      }
#pragma unroll
      for (int m0 = 0; m0 < M; m0 += XV) {
        uint32_t xv[XV][8];
#pragma unroll
        for (int mm = 0; mm < XV; ++mm)
#pragma unroll
          for (int i = 0; i < 8; ++i) xv[mm][i] = m0 + mm < M ? xc[(m0 + mm) * xstride + j * 8 + i] : 0u;
#pragma unroll
        for (int mm = 0; mm < XV; ++mm) {
          if (m0 + mm >= M) continue;
          float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            p0 = dot2(w[i], xv[mm][i], p0);
            p1 = dot2(w[i + 1], xv[mm][i + 1], p1);
          }
          acc[m0 + mm] += p0 + p1;
        }
      }
    }
  } else if constexpr (FULL) {
    // x is read with scalar loads, which may return out of order, so each use
    // waits for all of them: read the x of XG pieces together and wait once per
    // group (a wait per piece put eight round trips in every tile)
    constexpr int XG = M >= 4 ? 1 : 4 / M;
#pragma unroll
    for (int j0 = 0; j0 < kPiecesNv; j0 += XG) {
      uint32_t xv[XG][M][16];
#pragma unroll
      for (int jj = 0; jj < XG; ++jj)
#pragma unroll
        for (int m = 0; m < M; ++m)
#pragma unroll
          for (int i = 0; i < 16; ++i) xv[jj][m][i] = xc[m * xstride + (j0 + jj) * 16 + i];
#pragma unroll
      for (int jj = 0; jj < XG; ++jj) piece_dot<FMT, M>(f, j0 + jj, xv[jj], acc);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPiecesNv; ++j) {
      if (j >= npieces) continue;
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

// Double-buffered stream over n_items tiles: the tile of item it+1 is in flight
// while item it is consumed.  The loop body always has both fragments' loads in
// flight, so the wait before each consume is a fixed "all but the newest
// fragment" count (loads complete in order); the last one or two items are
// peeled off so that no load is conditional.  tile_of(it) is the tile address of
// item it, eat(fragment, it) consumes it.
template <uint32_t FMT, class TileOf, class Eat>
__device__ __forceinline__ void stream_items(int n_items, int lane, TileOf tile_of, Eat eat) {
  if (n_items <= 0) return;
  Frag<FMT> fa, fb;
  load_frag<FMT>(fa, tile_of(0), lane);
  int it = 0;
  for (; it + 2 < n_items; it += 2) {
    load_frag<FMT>(fb, tile_of(it + 1), lane);
    eat(fa, it);
    load_frag<FMT>(fa, tile_of(it + 2), lane);
    eat(fb, it + 1);
  }
  if (it + 1 < n_items) {
    load_frag<FMT>(fb, tile_of(it + 1), lane);
    eat(fa, it);
    eat(fb, it + 1);
  } else {
    eat(fa, it);
  }
}

// Split-K results travel as 64-bit units: EPI_STORE packs the values of tokens
// 2u and 2u+1, EPI_SILU the (gate, up) pair of token u.  Encoding: low word =
// bits(a) + 1, high word = bits(b), so that 0 (a zero-filled slot) never
// encodes a value (that would need bits(a) = 0xFFFFFFFF, a NaN arithmetic never
// produces).
__device__ __forceinline__ unsigned long long enc_unit(float a, float b) {
  return (unsigned long long)(__float_as_uint(a) + 1u) | ((unsigned long long)__float_as_uint(b) << 32);
}
__device__ __forceinline__ void dec_unit(unsigned long long v, float& a, float& b) {
  a = __uint_as_float((uint32_t)v - 1u);
  b = __uint_as_float((uint32_t)(v >> 32));
}

// Split-K across workgroups: a binary tree of exchanges over the S workgroups
// of a row group.  At each level the two subtrees of a node swap their sums into
// the node's slot; the first to arrive deposits, the second receives the first's
// sum in the same round trip, adds (a + b == b + a, so the result does not
// depend on who is second) and carries on; an unpaired last node passes up.  One
// device-scope atomic round trip per level; slots are left zero.  Units still
// live afterwards hold the full sums.  Slot of (node, unit, lane_slot):
// slots[(node * NU + unit) * unit_stride + lane_slot].
template <int NU>
__device__ __forceinline__ void exchange_tree(unsigned long long* __restrict__ slots, int64_t unit_stride,
                                              int64_t lane_slot, int S, int s, float (&ua)[NU], float (&ub)[NU],
                                              bool (&live)[NU]) {
  int node_off = 0, n = S, idx = s;
  while (n > 1) {
    if ((idx ^ 1) < n) {
      unsigned long long* base = slots + ((int64_t)(node_off + (idx >> 1)) * NU) * unit_stride + lane_slot;
      unsigned long long old[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u)
        old[u] = live[u] ? __hip_atomic_exchange(base + u * unit_stride, enc_unit(ua[u], ub[u]), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                         : 0ull;
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        if (!live[u]) continue;
        if (old[u] == 0ull) {
          live[u] = false;  // deposited: the partner carries the pair sum on
        } else {
          float oa, ob;
          dec_unit(old[u], oa, ob);
          ua[u] = oa + ua[u];
          ub[u] = ob + ub[u];
          __hip_atomic_store(base + u * unit_stride, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    node_off += n >> 1;
    n = (n + 1) >> 1;
    idx >>= 1;
  }
}

// Row group of a grouped launch: member index and its local row group.
__device__ __forceinline__ int member_of(const GemvParams& p, int gt) {
  int mem = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < p.n && gt >= p.gbase[i]) mem = i;
  return mem;
}

// Epilogue for unit u of one row of member `mem` (row local to that member).
template <uint32_t FMT, int M, int NMAT, int EPI>
__device__ __forceinline__ void finish_unit(const GemvParams& p, int mem, int row, int u, float a, float b) {
  if (row >= p.d_out[mem]) return;
  if constexpr (EPI == EPI_STORE || EPI == EPI_ARGMAX) {
    const float sc = FMT == FP4G_FP8_ROW ? p.rs[mem][row] : p.tscale[mem];
    const int m0 = 2 * u;
    if (EPI == EPI_STORE || p.y[0]) {
      p.y[mem][(int64_t)m0 * p.d_out[mem] + row] = a * sc;
      if (m0 + 1 < M) p.y[mem][(int64_t)(m0 + 1) * p.d_out[mem] + row] = b * sc;
    }
  } else {
    const float g = a * (FMT == FP4G_FP8_ROW ? p.rs[0][row] : p.tscale[0]);
    const float v = b * (FMT == FP4G_FP8_ROW ? p.rs[1][row] : p.tscale[1]);
    p.h[(int64_t)u * p.d_out[0] + row] = f32_to_bf16_rne(silu_f32(g) * v);
  }
}

// Greedy pick over the launch (wave 0 of every workgroup, after the split-K
// tree).  The surviving lanes' logits become pick keys (the same float as the
// logit written, ties to the lower row); each vector's wave maximum goes into one
// of kArgSlots slots with a device-scope atomic max that nobody waits for.
// k_argmax_finish, launched next on the same stream, reads the slots, writes
// (row, value) per vector and leaves the slots at zero.
template <uint32_t FMT, int M, int NU>
__device__ __forceinline__ void argmax_epilogue(const GemvParams& p, int row, int lane, const float (&ua)[NU],
                                                const float (&ub)[NU], const bool (&live)[NU]) {
  const bool valid = row < p.d_out[0];
  const float sc = valid ? (FMT == FP4G_FP8_ROW ? p.rs[0][row] : p.tscale[0]) : 0.0f;
  uint64_t key[M];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const bool ok = live[u] && valid;
    key[2 * u] = ok ? pick_key(ua[u] * sc, p.row_base + row) : 0ull;
    if (2 * u + 1 < M) key[2 * u + 1] = ok ? pick_key(ub[u] * sc, p.row_base + row) : 0ull;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) key[m] = wave_max_key(key[m]);
  unsigned long long* slot = p.amax + (int64_t)(blockIdx.x % kArgSlots) * kMaxMWide;
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < M; ++m)
      if (key[m]) __hip_atomic_fetch_max(slot + m, (unsigned long long)key[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <uint32_t FMT, int M, int NMAT, int EPI, int NW>
__global__ __launch_bounds__(NW * 64) void k_gemv(GemvParams p) {
  constexpr int NA = NMAT * M;
  constexpr int TILE = FMT == FP4G_NVFP4 ? kTileNv : FMT == FP4G_MXFP4 ? kTileMx : kTileF8;
  __shared__ float red[NW][NA][64];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int gt = uniform(blockIdx.x / p.S);  // global row group
  const int s = uniform(blockIdx.x % p.S);
  const int mem = NMAT == 1 ? member_of(p, gt) : 0;
  const int g = gt - p.gbase[mem];
  const uint8_t* w0 = p.w[mem];
  const uint8_t* w1 = NMAT == 2 ? p.w[1] : w0;
  const int wg_c0 = s * p.wg_chunks;
  const int wg_c1 = min(p.C, wg_c0 + p.wg_chunks);
  // the workgroup's chunks split as evenly as possible over its NW waves
  const int c0 = wg_c0 + (wave * (wg_c1 - wg_c0)) / NW;
  const int c1 = wg_c0 + ((wave + 1) * (wg_c1 - wg_c0)) / NW;

  float acc[NMAT][M];
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[a][m] = 0.0f;

  const uint32_t* __restrict__ x32 = reinterpret_cast<const uint32_t*>(p.x);
  const int xstride = p.d_in / 2;
  const int full_chunks = p.d_in / kChunkK;  // chunks with all 8 pieces present
  const int tail_pieces = (p.d_in % kChunkK) / kPieceK;

  // Items are (chunk, half, matrix) visited chunk-major, matrix fastest; an FP8
  // tile is streamed as two halves, an NVFP4/MXFP4 tile whole.
  constexpr bool F8 = FMT == FP4G_FP8_ROW;
  constexpr int HALVES = F8 ? 2 : 1;
  constexpr int PER = HALVES * NMAT;  // items per chunk
  const int n_items = (c1 - c0) * PER;
  const int64_t tile0 = (int64_t)g * p.C;
  auto item_tile = [&](int it) {
    const uint8_t* t = (it % NMAT ? w1 : w0) + (tile0 + c0 + it / PER) * TILE;
    return F8 ? t + ((it / NMAT) % HALVES) * (kHalfFp8 * 1024) : t;
  };
  auto consume = [&](const Frag<FMT>& f, int it) {
    const int c = c0 + it / PER;
    const int half = F8 ? (it / NMAT) % HALVES : 0;
    const uint32_t* xc = x32 + (int64_t)c * (kChunkK / 2) + half * (kHalfFp8 * 8);
    float part[M];
#pragma unroll
    for (int m = 0; m < M; ++m) part[m] = 0.0f;
    if (c < full_chunks) {
      tile_dot<FMT, M, true>(f, xc, xstride, kPiecesNv, part);
    } else if constexpr (F8) {
      const int slots = min(max(2 * tail_pieces - kHalfFp8 * half, 0), kHalfFp8);
      tile_dot<FMT, M, false>(f, xc, xstride, slots, part);
    } else {
      tile_dot<FMT, M, false>(f, xc, xstride, tail_pieces, part);
    }
    if constexpr (NMAT == 1) {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[0][m] += part[m];
    } else {
      // branch-free (item it belongs to matrix it % 2): the compiler merges two
      // branches into a store through a chosen pointer, which keeps the
      // accumulators in private memory
      const bool up = it % NMAT != 0;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        acc[0][m] += up ? 0.0f : part[m];
        acc[1][m] += up ? part[m] : 0.0f;
      }
    }
  };
  stream_items<FMT>(n_items, lane, item_tile, consume);

#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int m = 0; m < M; ++m) red[wave][a * M + m][lane] = acc[a][m];
  __syncthreads();
  if (wave != 0) return;

  float v[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    float t = red[0][i][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += red[w][i][lane];
    v[i] = t;
  }

  // units: EPI_STORE (v[2u], v[2u+1]); EPI_SILU (gate v[u], up v[M+u])
  constexpr int NU = EPI == EPI_SILU ? M : (M + 1) / 2;
  float ua[NU], ub[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if constexpr (EPI == EPI_SILU) {
      ua[u] = v[u];
      ub[u] = v[M + u];
    } else {
      ua[u] = v[2 * u];
      ub[u] = 2 * u + 1 < M ? v[2 * u + 1] : 0.0f;
    }
  }
  const int row = g * 64 + lane;
  bool live[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) live[u] = true;
  exchange_tree<NU>(p.slots, (int64_t)p.gbase[p.n] * 64, (int64_t)gt * 64 + lane, p.S, s, ua, ub, live);
#pragma unroll
  for (int u = 0; u < NU; ++u)
    if (live[u]) finish_unit<FMT, M, NMAT, EPI>(p, mem, row, u, ua[u], ub[u]);
  if constexpr (EPI == EPI_ARGMAX) argmax_epilogue<FMT, M, NU>(p, row, lane, ua, ub, live);
}

template <uint32_t FMT, int M, int NMAT, int EPI>
hipError_t launch_nw(int nw, const GemvParams& p, unsigned grid, hipStream_t s) {
  switch (nw) {
    case 4: k_gemv<FMT, M, NMAT, EPI, 4><<<grid, 256, 0, s>>>(p); break;
    case 8: k_gemv<FMT, M, NMAT, EPI, 8><<<grid, 512, 0, s>>>(p); break;
    case 16:
      if constexpr (NMAT == 1 ? M <= 5 : M <= 3) {  // where plan_for offers 16 waves
        k_gemv<FMT, M, NMAT, EPI, 16><<<grid, 1024, 0, s>>>(p);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <uint32_t FMT, int NMAT, int EPI>
hipError_t launch_m(int M, int nw, const GemvParams& p, unsigned grid, hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM) \
  case MM:            \
    return launch_nw<FMT, MM, NMAT, EPI>(nw, p, grid, s);
    FP4G_CASE(1) FP4G_CASE(2) FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
#undef FP4G_CASE
    default: break;
  }
  // FP8 rows have no matrix-core kernel: their plain products and greedy pick
  // take verify blocks of 9..16 vectors on this one (one read of the matrix)
  if constexpr (FMT == FP4G_FP8_ROW && NMAT == 1) {
    switch (M) {
#define FP4G_CASE(MM) \
  case MM:            \
    return launch_nw<FMT, MM, NMAT, EPI>(nw, p, grid, s);
      FP4G_CASE(9) FP4G_CASE(10) FP4G_CASE(11) FP4G_CASE(12) FP4G_CASE(13) FP4G_CASE(14) FP4G_CASE(15) FP4G_CASE(16)
#undef FP4G_CASE
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

// ---- launch planning -----------------------------------------------------------
struct Plan {
  int S;          // workgroups per row group
  int wg_chunks;  // chunks per workgroup
  int nw;         // waves per workgroup
};

// Four-wave workgroups: enough waves to cover HBM latency on all 256 CUs (about
// eight per CU), with at least one chunk per wave; chunks spread evenly over the
// S workgroups.  (The MoE and matrix-core kernels use this split.)
inline Plan plan_nw4(int64_t R, int64_t C, int64_t target_waves = 2048) {
  int64_t q = (R * C) / target_waves;  // chunks per wave
  if (q < 1) q = 1;
  int64_t S = (C + kWavesPerWg * q - 1) / (kWavesPerWg * q);
  if (S < 1) S = 1;
  const int64_t wg_chunks = (C + S - 1) / S;
  S = (C + wg_chunks - 1) / wg_chunks;
  return Plan{(int)S, (int)wg_chunks, kWavesPerWg};
}

inline int tree_depth(int64_t S) {
  int d = 0;
  for (int64_t n = S; n > 1; n = (n + 1) / 2) ++d;
  return d;
}

// VALU kernel: 4, 8 or 16 waves per workgroup and S workgroups per row group.
// Workgroups go round-robin to the 256 CUs, so the busiest CU gets ceil(WGs /
// 256) of them while the average CU needs WGs / 256: the plan minimises that
// imbalance, times 1 + 3% per level of the split-K tree (one device-scope round
// trip each), times 1 + 15% per extra round of waves beyond what the CUs hold at
// once (16 waves per CU while the kernel needs at most 128 VGPRs: NMAT * M up to
// 5 for plain products, M up to 3 fused; 12 above), times 1 + half the excess of
// the busiest wave of a workgroup over its average (ceil(chunks / waves) against
// chunks / waves: a workgroup ends with its slowest wave, and a per-wave timeline
// showed the short waves idle for up to half the launch).  No more than a
// quarter of a workgroup's waves may be left without a chunk; ties go to more
// waves.  (The weights are fitted to timings of the dense-model shapes on
// MI355X: the balance term moved the fused 17408x5120 gate/up from 4 to 5
// workgroups of 4 waves per row group and a 16384-row one from one 16-wave to
// one 4-wave workgroup per row group.)  A kernel with more registers passes its
// own waves_per_cu.
constexpr int kCUs = 256;
inline Plan plan_for(int64_t R, int64_t C, int nmat, int M, int waves_per_cu = 0) {
  if (waves_per_cu == 0) waves_per_cu = (nmat == 1 ? M <= 5 : M <= 3) ? 16 : 12;
  Plan best = plan_nw4(R, C);
  double best_cost = 1e30;
  int64_t best_waves = 0;
  for (int nw : {4, 8, 16}) {
    if (nw > waves_per_cu) continue;
    for (int64_t S0 = 1; S0 <= C; ++S0) {
      const int64_t wg_chunks = (C + S0 - 1) / S0;
      const int64_t S = (C + wg_chunks - 1) / wg_chunks;
      if (S != S0) continue;              // each S once
      if (4 * wg_chunks < 3 * nw) break;  // more than a quarter of the waves idle
      const int64_t wgs = R * S, waves = wgs * nw;
      const double imbalance = (double)((wgs + kCUs - 1) / kCUs) * kCUs / (double)wgs;
      const double rounds = (double)waves / ((double)kCUs * waves_per_cu);
      const double intra = (double)((wg_chunks + nw - 1) / nw) * nw / (double)wg_chunks;
      const double cost = imbalance * (1.0 + 0.03 * tree_depth(S)) * (1.0 + 0.15 * (rounds > 1.0 ? rounds - 1.0 : 0.0)) *
                          (1.0 + 0.5 * (intra - 1.0));
      if (cost < best_cost - 1e-9 || (cost < best_cost + 1e-9 && waves > best_waves)) {
        best = Plan{(int)S, (int)wg_chunks, nw};
        best_cost = cost;
        best_waves = waves;
      }
    }
  }
  // Plain products of 2..5 vectors whose plan fits the CUs in one round take 16
  // waves where the cost above picks 8: the uneven chunks per wave it charges
  // for matter less than hiding the M-fold VALU work (measured, 5120x17408 down
  // projection: 14.1 -> 13.4 us at M = 2, 17.7 -> 15.9 at 3, 19.8 -> 18.0 at 4;
  // the 5120x5120 product unchanged; at M = 1 the two are level)
  if (nmat == 1 && M >= 2 && M <= 5 && best.nw == 8 && R * best.S * 16 <= (int64_t)kCUs * 16) best.nw = 16;
  return best;
}

// Small products (a few thousand tiles, such as the experts a token picked) are
// bound by the chain of round trips in each wave, not by bandwidth: this plan
// minimises the rounds of workgroups times the chunks each wave streams in
// turn, plus half a chunk per level of the split-K tree, plus half the missing
// fraction when fewer workgroups than CUs leave some CUs idle (the last tiles'
// compute then piles up on the busy ones); among equals the fewest waves.  nws
// lists the workgroup sizes the kernel is built for.
inline Plan plan_latency(int64_t R, int64_t C, int waves_per_cu, std::initializer_list<int> nws) {
  Plan best = plan_nw4(R, C);
  double best_cost = 1e30;
  int64_t best_waves = 0;
  for (int nw : nws) {
    if (nw > waves_per_cu) continue;
    for (int64_t S0 = 1; S0 <= C; ++S0) {
      const int64_t wg_chunks = (C + S0 - 1) / S0;
      const int64_t S = (C + wg_chunks - 1) / wg_chunks;
      if (S != S0) continue;
      const int64_t waves = R * S * nw;
      const int64_t per_round = (int64_t)kCUs * (waves_per_cu / nw) * nw;
      const int64_t rounds = (waves + per_round - 1) / per_round;
      const int64_t per_wave = (wg_chunks + nw - 1) / nw;
      const double idle = R * S < kCUs ? (double)kCUs / (double)(R * S) - 1.0 : 0.0;
      const double cost = (double)(rounds * per_wave) + 0.5 * tree_depth(S) + 0.5 * idle;
      if (cost < best_cost - 1e-9 || (cost < best_cost + 1e-9 && waves < best_waves)) {
        best = Plan{(int)S, (int)wg_chunks, nw};
        best_cost = cost;
        best_waves = waves;
      }
    }
  }
  return best;
}

inline uint64_t align256(uint64_t b) { return (b + 255) & ~uint64_t(255); }

// Pair nodes of the split-K exchange tree over S leaves (S - 1 when S is a power
// of two; an unpaired node passes up without one).
inline int64_t tree_nodes(int64_t S) {
  int64_t t = 0;
  for (int64_t n = S; n > 1; n = (n + 1) / 2) t += n / 2;
  return t;
}

// Units per row: EPI_SILU exchanges (gate, up) per token, EPI_STORE two tokens.
inline int64_t exchange_units(int nmat, int M) { return nmat == 2 ? M : (M + 1) / 2; }

// Exchange slots: tree nodes x units x all rows of all members, 8 bytes each.
inline uint64_t gemv_ws_bytes(int64_t R_total, int64_t C, int nmat, int M) {
  const Plan pl = plan_for(R_total, C, nmat, M);
  if (pl.S == 1) return 0;
  return (uint64_t)tree_nodes(pl.S) * exchange_units(nmat, M) * R_total * 64 * 8;
}

}  // namespace fp4g
