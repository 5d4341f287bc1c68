// gemv_mfma.hpp -- the matrix-core variant of the decode product for M = 1..16
// vectors (the verify step of speculative decoding scores K+1 positions against
// the same weights: feed, sections "MTP: the drafter inside the checkpoint" and
// "More tokens per weight read", where blocks of up to 10 drafts are verified).
//
// Same packed tiles, same work split and same split-K exchange tree as the VALU
// kernel (gemv_kernel.hpp); only the arithmetic differs.  The VALU kernel issues
// one v_dot2 per weight pair and vector, so its issue rate falls short of HBM
// from M = 4 on.  Here the products run on v_mfma_f32_16x16x32_bf16 with the
// input as the A operand (16 rows: vectors) and the weights as the B operand
// (16 columns: weight rows), so one instruction covers 16 weight rows x 32
// columns for up to 16 vectors:
//
//  * B operand: the MFMA wants lane i to hold 8 consecutive columns (K group
//    i / 16) of weight row i % 16, while the packed layout gives lane l all 32
//    columns of one 1 KiB slot for row l.  A 4 x 4 transpose of dwords between
//    the four 16-lane groups (two v_permlane32_swap and two v_permlane16_swap)
//    turns the slot into four B operands, one per 16-row block of the 64-row
//    group.  E2M1 -> bf16 is exact (v_cvt_scalef32_pk_bf16_fp4 with scale 1).
//  * A operand: lane i reads 8 input columns of vector i % 16 (K group i / 16)
//    from the LDS staging of the workgroup's input range; lanes with no vector
//    read a zero area.
//  * Block scales are applied in FP32 to each MFMA result, per weight row.  An
//    MXFP4 block is one slot (32 columns): one MFMA per 16-row block.  An NVFP4
//    block is half a slot: with M <= 8 the A rows 0..7 carry the vectors over
//    the slot's first 16 columns and rows 8..15 over the last 16 (zeros in the
//    other half), so one MFMA still gives both blocks' sums separately; with
//    M > 8 each block takes its own MFMA.
//  * A work item is kMfmaSlots code slots of one tile (half of it) and their
//    scales, double-buffered; the NVFP4 gate/up forms up to 8 vectors take
//    whole tiles instead (MTile).  The reduction across waves reuses the input's
//    LDS area, so a workgroup holds no more LDS than its staged input.
#pragma once
#include <type_traits>

#include "gemv_kernel.hpp"
#include "moe_route.hpp"

namespace fp4g {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaXBytes = 40960;  // LDS for the staged input of one workgroup
constexpr int kZeroBytes = 512;     // one chunk row of zeros
// Each vector's staged row is padded by 64 bytes: rows then start 16 banks apart
// (64 banks of 4 bytes), so the lanes that read the same columns of different
// vectors (an A operand) hit different banks instead of one.
constexpr int kXPad = 64;
constexpr int kMfmaRedOwn = 0;      // values per lane up to which the reduction has its own LDS

constexpr int kMfmaSlots = 4;  // code slots per work item (half a tile: fewer registers, more waves)

// A fragment: code slots SL h .. SL h + SL - 1 of lane l's row (as stored), and
// the block scales of those slots for the rows 16 r + (l % 16), r < 4, whose
// sums the lane computes (one byte per block, SW dwords per row).
template <uint32_t FMT>
struct MFrag {
  static constexpr int SL = kMfmaSlots;
  static constexpr int SW = FMT == FP4G_NVFP4 ? SL / 2 : SL / 4;
  u32x4 q[SL];
  uint32_t s[4][SW];
};

__device__ __forceinline__ uint32_t ld_stream1(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

template <uint32_t FMT>
__device__ __forceinline__ void load_mfrag(MFrag<FMT>& f, const uint8_t* tile, int half, int lane) {
  constexpr int SL = MFrag<FMT>::SL, SW = MFrag<FMT>::SW;
  const int c = lane & 15;
#pragma unroll
  for (int j = 0; j < SL; ++j) f.q[j] = ld_stream(tile + (SL * half + j) * 1024 + lane * 16);
  constexpr int rowb = FMT == FP4G_NVFP4 ? 16 : 8;  // scale bytes per row and tile
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint8_t* sp = tile + kCodeBytes + (16 * r + c) * rowb + half * SW * 4;
    if constexpr (SW == 4) {
      const u32x4 v = ld_stream(sp);
      f.s[r][0] = v[0], f.s[r][1] = v[1], f.s[r][2] = v[2], f.s[r][3] = v[3];
    } else if constexpr (SW == 2) {
      const u32x2 v = ld_stream2(sp);
      f.s[r][0] = v[0], f.s[r][1] = v[1];
    } else {
      f.s[r][0] = ld_stream1(sp);
    }
  }
}

// A whole tile, for the NVFP4 gate/up forms up to kMaxM vectors: its eight code
// slots and the lane's own row of block scales as stored (one 16-byte load per
// lane, as the VALU kernel reads them; 8 bytes for MXFP4).  The scales reach
// the lanes that apply them (rows 16 r + l % 16) through LDS when the tile is
// consumed, into s, laid out as MFrag's.  Against half tiles with four scale
// loads each (whose 128-byte scale lines both halves of a tile fetch), this
// took the 17408x5120 gate/up pair from 30.7 to 27.0 us at M = 4, at three
// waves per SIMD (144 registers); the plain products keep half tiles (no gain
// on the down projection).
template <uint32_t FMT>
struct MTile {
  static constexpr int SL = 8;
  static constexpr int SW = FMT == FP4G_NVFP4 ? 4 : 2;
  u32x4 q[SL];
  uint32_t sr[SW];
  uint32_t s[4][SW];
};

template <uint32_t FMT>
__device__ __forceinline__ void load_mtile(MTile<FMT>& f, const uint8_t* tile, int lane) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.q[j] = ld_stream(tile + j * 1024 + lane * 16);
  if constexpr (FMT == FP4G_NVFP4) {
    const u32x4 v = ld_stream(tile + kCodeBytes + lane * 16);
    f.sr[0] = v[0], f.sr[1] = v[1], f.sr[2] = v[2], f.sr[3] = v[3];
  } else {
    const u32x2 v = ld_stream2(tile + kCodeBytes + lane * 8);
    f.sr[0] = v[0], f.sr[1] = v[1];
  }
}

// Eight E2M1 codes (one dword: 8 consecutive columns) as bf16.
__device__ __forceinline__ bf16x8 e2m1x8_bf16(uint32_t dw) {
  const bf16x2 p0 = e2m1x2_bf16<0>(dw), p1 = e2m1x2_bf16<1>(dw);
  const bf16x2 p2 = e2m1x2_bf16<2>(dw), p3 = e2m1x2_bf16<3>(dw);
  return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const uint8_t* base, int off) {
  return *reinterpret_cast<const bf16x8*>(base + off);
}

// Lane group g = l / 16 holds dword d of its rows in q[d]; afterwards lane group g
// holds, in q[r], dword g of the rows of lane group r (the same l % 16): the
// B operand of 16-row block r.
__device__ __forceinline__ void transpose_slot(u32x4& q) {
  const auto a = __builtin_amdgcn_permlane32_swap(q[0], q[2], false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(q[1], q[3], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  q = u32x4{c[0], c[1], d[0], d[1]};
}

// Sum of x over lane i and lane i +- 32 (both halves end with the sum).
__device__ __forceinline__ float add_halves(float x, int lane) {
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return x + __uint_as_float(lane < 32 ? t[1] : t[0]);
}

// Mixture-of-experts modes of this kernel.
//  MODE 1, gate/up: row group gt of the launch is (slot gt / rg, group gt % rg);
//    slot i multiplies expert route[1 + i] (-1: the shared expert), slots from
//    route[0] on do nothing, and h goes to slot i's rows of the workspace,
//    [slot][M][d_ff].
//  MODE 2, down: the K dimension runs over the union's slots, cd chunks each
//    (chunk v is chunk v % cd of slot v / cd's expert, its input that slot's h);
//    each chunk's products are weighted per token by coef[slot][token] (gate
//    weight x down tensor scale) before they add up, so the experts need no
//    combine step.  Chunks past the realised union do nothing.
struct MfmaMoe {
  const int32_t* route;  // [0] = slots in use, [1 + i] = expert of slot i (-1 = shared)
  uint64_t stride[2];    // bytes between experts: gate, up (p.w[0], p.w[1] = expert 0); down: [0]
  const uint8_t* sh[2];  // the shared expert's gate, up; down: [0]
  float sh_ts[2];        // and their tensor scales (gate/up)
  int rg;                // 64-row groups per expert (gate/up)
  uint16_t* hdbg;        // optional bf16 [M][k + shared][d_ff]: h per (token, pick)
  const int32_t* ids;    // [M][k] picked experts
  int k, nh;             // picks per token; k + shared
  const float* coef;     // down: [slot][M]
  const uint16_t* hbuf;  // down: bf16 [slot][M][d_ff]
  int cd, dff;           // down: chunks per slot; d_ff
  MoeParams rp;          // gate/up up to kMfmaMoeRouteM vectors: routing inputs and tables
};

// MoE gate/up forms that route the tokens themselves (one wave per token, each
// workgroup for itself; workgroup 0 also writes the routing tables for the down
// half), instead of reading a routing launch's tables: the launch and its two
// dependent table reads leave the layer's critical path.  Above four vectors a
// wave would route several tokens in turn: measured with routing in the
// workgroups up to eight vectors, layers at M = 5..8 were 0.6-1.9 us slower,
// so those keep the routing launch.
constexpr int kMfmaMoeRouteM = 4;

// Gate/up forms that stream whole tiles (MTile): NVFP4 up to kMaxM vectors.
// (MXFP4 keeps half tiles: its gate/up pair went from 28.4 to 30.0 us at M = 4
// with whole tiles, and the MoE layer with it.)
template <uint32_t FMT, int M, int NMAT>
constexpr bool mfma_whole_tiles() {
  return FMT == FP4G_NVFP4 && NMAT == 2 && M <= kMaxM;
}

// Waves per SIMD the register allocation aims for.  VGPRs and AGPRs share one
// file of 512 per lane, so four waves leave 128 registers: enough, without
// spills, for the plain forms up to 16 vectors and the half-tile gate/up forms
// up to 8 (measured 5-25% faster than at three waves).  Whole-tile gate/up,
// gate/up above 8 vectors and the MoE down would spill at that budget; three
// waves (170 registers) fit them.
template <uint32_t FMT, int M, int NMAT, int MODE>
constexpr int mfma_waves_per_eu() {
  return mfma_whole_tiles<FMT, M, NMAT>() || (NMAT == 2 && M > kMaxM) || MODE == 2 ? 3 : 4;
}

template <uint32_t FMT, int M, int NMAT, int EPI, int MODE = 0>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_eu<FMT, M, NMAT, MODE>())))
void k_gemv_mfma(GemvParams p, MfmaMoe q) {
  constexpr bool MOE = MODE == 1, MOED = MODE == 2;
  // NVFP4 with up to 8 vectors: both blocks of a slot in one MFMA (A rows 8..15
  // carry the second block); the outputs of lanes i and i + 32 then add up
  constexpr bool PACK2 = FMT == FP4G_NVFP4 && M <= 8;
  constexpr bool TWO = FMT == FP4G_NVFP4 && M > 8;  // one MFMA per NVFP4 block
  constexpr int NR = PACK2 ? 2 : 4;                  // 16-row blocks per lane at the end
  constexpr int NV = NMAT * NR * 4;                  // values per lane at the end
  constexpr int TILE = FMT == FP4G_NVFP4 ? kTileNv : kTileMx;
  // Cross-wave reduction buffer: its own array up to 16 values per lane, else
  // the staged-input area, reused once every wave has finished reading it.
  constexpr bool kRedInX = NV > kMfmaRedOwn;
  __shared__ float red_own[kRedInX ? 1 : kWavesPerWg][kRedInX ? 1 : NV][64];
  // NVFP4 gate/up up to kMaxM vectors streams whole tiles (MTile); their scales
  // pass through one row of 16 bytes per lane here
  constexpr bool WHOLE = mfma_whole_tiles<FMT, M, NMAT>();
  using Frag = std::conditional_t<WHOLE, MTile<FMT>, MFrag<FMT>>;
  __shared__ u32x4 sc_lds[WHOLE ? kWavesPerWg : 1][WHOLE ? 64 : 1];
  constexpr bool ROUTE = MOE && M <= kMfmaMoeRouteM;
  __shared__ RouteLds<ROUTE ? M : 1> rl;
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];  // [M][wg_chunks * 512 + kXPad] bf16, then zeros
  float(*red)[NV][64] = kRedInX ? reinterpret_cast<float(*)[NV][64]>(xs) : reinterpret_cast<float(*)[NV][64]>(red_own);

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int gt = uniform(blockIdx.x / p.S);
  const int s = uniform(blockIdx.x % p.S);
  const int mem = NMAT == 1 && !MOE ? member_of(p, gt) : 0;
  int g = gt - p.gbase[mem];
  const uint8_t* w0 = p.w[mem];
  const uint8_t* w1 = NMAT == 2 ? p.w[1] : w0;
  int slot = 0, expert = 0;
  if constexpr (MOE) {
    slot = uniform(gt / q.rg);
    g = gt - slot * q.rg;
    if constexpr (ROUTE) {
      route_tokens<M, kWavesPerWg>(q.rp, rl);
      if (blockIdx.x == 0) write_route_tables<M, kWavesPerWg>(q.rp, rl);
      if (slot >= rl.n_slots) return;  // past the realised union: no byte read
      expert = rl.uni[slot];
    } else {
      if (slot >= q.route[0]) return;
      expert = q.route[1 + slot];
    }
    w0 = expert >= 0 ? p.w[0] + (uint64_t)expert * q.stride[0] : q.sh[0];
    w1 = expert >= 0 ? p.w[1] + (uint64_t)expert * q.stride[1] : q.sh[1];
  }
  const int wg_c0 = s * p.wg_chunks;
  const int wg_c1 = min(p.C, wg_c0 + p.wg_chunks);
  const int per_wave = (wg_c1 - wg_c0 + kWavesPerWg - 1) / kWavesPerWg;
  int c0 = min(wg_c1, wg_c0 + wave * per_wave);
  int c1 = min(wg_c1, c0 + per_wave);
  int n_valid = p.C;  // chunks that carry data (down: those of the realised union)
  if constexpr (MOED) {
    n_valid = uniform(q.route[0]) * q.cd;
    c1 = min(c1, n_valid);
    c0 = min(c0, c1);
  }
  const int cl = lane & 15;   // A row / B column of the lane
  const int kg = lane >> 4;   // K group of the lane
  const int64_t tile0 = (int64_t)g * (MOED ? q.cd : p.C);
  // items (chunk, part, matrix), matrix fastest: with NMAT = 2 the even items
  // are gate, the odd ones up
  constexpr int SL = Frag::SL, PER = 8 / SL;  // parts per tile
  auto item_tile = [&](int it) {
    const int cv = c0 + it / (PER * NMAT);
    if constexpr (MOED) {
      const int sl = cv / q.cd, e = q.route[1 + sl];
      const uint8_t* base = e >= 0 ? p.w[0] + (uint64_t)e * q.stride[0] : q.sh[0];
      return base + (tile0 + (cv - sl * q.cd)) * TILE;
    }
    return (it % NMAT ? w1 : w0) + (tile0 + cv) * TILE;
  };
  auto item_half = [&](int it) { return (it / NMAT) % PER; };

  // first fragment in flight before the input is staged
  const int n_items = (c1 - c0) * PER * NMAT;
  Frag fa, fb;
  if (n_items > 0) {
    if constexpr (WHOLE) load_mtile<FMT>(fa, item_tile(0), lane);
    else load_mfrag<FMT>(fa, item_tile(0), item_half(0), lane);
  }

  // stage x[m][256 wg_c0 ..) for m < M (zero past d_in), then the zero area; all
  // loads are issued before the first LDS store
  const int tstride = p.wg_chunks * 512 + kXPad;  // bytes per vector in LDS
  {
    constexpr int kMaxPieces = kMfmaXBytes / 16 / kThreads;
    const int per_tok = p.wg_chunks * 32;  // 16-byte pieces per vector
    const int pieces = M * per_tok;
    u32x4 v[kMaxPieces];
#pragma unroll
    for (int k = 0; k < kMaxPieces; ++k) {
      const int idx = threadIdx.x + k * kThreads;
      v[k] = u32x4{0u, 0u, 0u, 0u};
      const int m = idx / per_tok, r = idx - m * per_tok;
      if constexpr (MOED) {
        // chunk cv of the union: columns of slot cv / cd's h (zero past d_ff and
        // past the union)
        const int cv = wg_c0 + r / 32, sl = cv / q.cd, col = (cv - sl * q.cd) * kChunkK + (r % 32) * 8;
        if (idx < pieces && cv < n_valid && col < q.dff)
          v[k] = *reinterpret_cast<const u32x4*>(q.hbuf + ((int64_t)sl * M + m) * q.dff + col);
      } else {
        const int col = wg_c0 * kChunkK + r * 8;
        if (idx < pieces && col < p.d_in) v[k] = *reinterpret_cast<const u32x4*>(p.x + (int64_t)m * p.d_in + col);
      }
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

  // A operand addresses (bytes into xs, before the chunk and slot offsets): the
  // lane's vector and K group, or the zero area.  Operand 0 is the only one
  // except for NVFP4 with M > 8 (operand 0: first block, operand 1: second).
  constexpr int NA = TWO ? 2 : 1;
  int aoff[NA];
  bool aval[NA];
  if constexpr (PACK2) {
    const int m = cl & 7;
    aval[0] = m < M && (kg >> 1) == (cl >> 3);
    aoff[0] = (aval[0] ? m * tstride : M * tstride) + kg * 16;
  } else if constexpr (TWO) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      aval[b] = cl < M && (kg >> 1) == b;
      aoff[b] = (aval[b] ? cl * tstride : M * tstride) + kg * 16;
    }
  } else {
    aval[0] = cl < M;
    aoff[0] = (aval[0] ? cl * tstride : M * tstride) + kg * 16;
  }

  f32x4 acc[NMAT][4];
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[a][r] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  auto consume = [&](Frag& f, int it, f32x4(&ac)[4]) {
    if constexpr (WHOLE) {
      // the tile's scales: each lane writes its own row, then reads the rows
      // 16 r + cl whose products it holds (one wave's area: the LDS keeps a
      // wave's accesses in order)
      if constexpr (FMT == FP4G_NVFP4)
        sc_lds[wave][lane] = u32x4{f.sr[0], f.sr[1], f.sr[2], f.sr[3]};
      else
        sc_lds[wave][lane] = u32x4{f.sr[0], f.sr[1], 0u, 0u};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const u32x4 v = sc_lds[wave][16 * r + cl];
#pragma unroll
        for (int w = 0; w < MTile<FMT>::SW; ++w) f.s[r][w] = v[w];
      }
    }
    const int cc = c0 + it / (PER * NMAT) - wg_c0;  // chunk within the staged range
    const int half = item_half(it);
    // weights of the lane's four vectors (MoE down: the chunk's slot's
    // coefficients; 1 otherwise, which the compiler folds away)
    float cf[4] = {1.0f, 1.0f, 1.0f, 1.0f};
    if constexpr (MOED) {
      const int sl = (cc + wg_c0) / q.cd;
      const int tb = PACK2 ? 4 * (kg & 1) : 4 * kg;
#pragma unroll
      for (int v = 0; v < 4; ++v) cf[v] = tb + v < M ? q.coef[sl * M + tb + v] : 0.0f;
    }
#pragma unroll
    for (int jj = 0; jj < SL; ++jj) {
      const int j = SL * half + jj;  // slot within the chunk
      bf16x8 xa[NA];
#pragma unroll
      for (int b = 0; b < NA; ++b) xa[b] = lds_bf16x8(xs, aoff[b] + (aval[b] ? cc * 512 : 0) + j * 64);
      transpose_slot(f.q[jj]);
      f32x4 d[NA][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bf16x8 bw = e2m1x8_bf16(f.q[jj][r]);
#pragma unroll
        for (int b = 0; b < NA; ++b)
          d[b][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[b], bw, f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (FMT == FP4G_NVFP4) {
          // blocks 2j (columns 0..15 of the slot) and 2j + 1 of row 16 r + cl:
          // bytes 2jj, 2jj + 1 of the item's scale bytes
          const uint32_t sdw = f.s[r][jj >> 1];
          const float s0 = (jj & 1) ? e4m3_f32<2>(sdw) : e4m3_f32<0>(sdw);
          const float s1 = (jj & 1) ? e4m3_f32<3>(sdw) : e4m3_f32<1>(sdw);
          if constexpr (PACK2) {
            const float sc = kg < 2 ? s0 : s1;  // output rows 0..7: first block, 8..15: second
#pragma unroll
            for (int v = 0; v < 4; ++v) ac[r][v] = __builtin_fmaf(d[0][r][v], sc * cf[v], ac[r][v]);
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              ac[r][v] = __builtin_fmaf(d[1][r][v], s1 * cf[v], __builtin_fmaf(d[0][r][v], s0 * cf[v], ac[r][v]));
          }
        } else {
          const int e = (int)((f.s[r][jj >> 2] >> (8 * (jj & 3))) & 0xffu) - 127;
#pragma unroll
          for (int v = 0; v < 4; ++v) ac[r][v] = __builtin_fmaf(__builtin_amdgcn_ldexpf(d[0][r][v], e), cf[v], ac[r][v]);
        }
      }
      // keep each slot's LDS reads and conversions next to its MFMAs
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // items alternate matrices (NMAT = 2), so fragment fa always holds matrix 0
  // and fb the last one: each call names its accumulators statically
  if (n_items > 0) {
    int it = 0;
    for (; it + 2 < n_items; it += 2) {
      if constexpr (WHOLE) load_mtile<FMT>(fb, item_tile(it + 1), lane);
      else load_mfrag<FMT>(fb, item_tile(it + 1), item_half(it + 1), lane);
      consume(fa, it, acc[0]);
      if constexpr (WHOLE) load_mtile<FMT>(fa, item_tile(it + 2), lane);
      else load_mfrag<FMT>(fa, item_tile(it + 2), item_half(it + 2), lane);
      consume(fb, it + 1, acc[NMAT - 1]);
    }
    if (it + 1 < n_items) {
      if constexpr (WHOLE) load_mtile<FMT>(fb, item_tile(it + 1), lane);
      else load_mfrag<FMT>(fb, item_tile(it + 1), item_half(it + 1), lane);
      consume(fa, it, acc[0]);
      consume(fb, it + 1, acc[NMAT - 1]);
    } else {
      consume(fa, it, acc[0]);
    }
  }

  // The lane's values: val[(a * NR + rr) * 4 + v] is matrix a, weight row
  // 16 rb + cl with rb = rr (+ 2 in the upper half for PACK2), vector
  // 4 (kg % 2) + v (PACK2) or 4 kg + v.
  float val[NV];
#pragma unroll
  for (int a = 0; a < NMAT; ++a) {
    if constexpr (PACK2) {
      // lanes i and i + 32 hold the two blocks' sums of one (row, vector): add
      // them, then the lower half keeps row blocks 0, 1 and the upper 2, 3
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float lo = add_halves(acc[a][rr][v], lane), hi = add_halves(acc[a][rr + 2][v], lane);
          val[(a * NR + rr) * 4 + v] = lane < 32 ? lo : hi;
        }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int v = 0; v < 4; ++v) val[(a * NR + r) * 4 + v] = acc[a][r][v];
    }
  }

  if constexpr (kRedInX) __syncthreads();  // every wave is past its last read of xs
#pragma unroll
  for (int i = 0; i < NV; ++i) red[wave][i][lane] = val[i];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int i = 0; i < NV; ++i) val[i] = ((red[0][i][lane] + red[1][i][lane]) + red[2][i][lane]) + red[3][i][lane];

  const int vbase = PACK2 ? 4 * (kg & 1) : 4 * kg;  // the lane's first vector
  // units: EPI_SILU (gate, up) of (row block rr, vector vbase + v); EPI_STORE
  // vectors (vbase + 2w, vbase + 2w + 1) of row block rr
  constexpr int NU = EPI == EPI_SILU ? NR * 4 : NR * 2;
  float ua[NU], ub[NU];
  bool live[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if constexpr (EPI == EPI_SILU) {
      ua[u] = val[u];
      ub[u] = val[NR * 4 + u];
      live[u] = vbase + (u & 3) < M;
    } else {
      ua[u] = val[2 * u];
      ub[u] = val[2 * u + 1];
      live[u] = vbase + 2 * (u & 1) < M;
    }
  }
  exchange_tree<NU>(p.slots, (int64_t)p.gbase[p.n] * 64, (int64_t)gt * 64 + lane, p.S, s, ua, ub, live);

  const int d_out = p.d_out[mem];
  const int rb0 = PACK2 && lane >= 32 ? 2 : 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (!live[u]) continue;
    if constexpr (EPI == EPI_SILU) {
      const int rr = u / 4, v = u % 4;
      const int m = vbase + v, row = g * 64 + 16 * (rb0 + rr) + cl;
      if (m < M && row < d_out) {
        const float tg = MOE && expert < 0 ? q.sh_ts[0] : p.tscale[0];
        const float tu = MOE && expert < 0 ? q.sh_ts[1] : p.tscale[1];
        const uint16_t hv = f32_to_bf16_rne(silu_f32(ua[u] * tg) * (ub[u] * tu));
        p.h[((int64_t)slot * M + m) * d_out + row] = hv;
        if constexpr (MOE) {
          if (q.hdbg) {
            if (expert < 0) {
              q.hdbg[((int64_t)m * q.nh + q.k) * d_out + row] = hv;
            } else {
              for (int j = 0; j < q.k; ++j) {
                // the picks: this workgroup's own routing, or the routing launch's table
                const int id = ROUTE ? rl.ids[ROUTE ? m : 0][j] : q.ids[m * q.k + j];
                if (id == expert) q.hdbg[((int64_t)m * q.nh + j) * d_out + row] = hv;
              }
            }
          }
        }
      }
    } else {
      const int rr = u / 2, w = u % 2;
      const int m = vbase + 2 * w, row = g * 64 + 16 * (rb0 + rr) + cl;
      if (row < d_out) {
        float* y = p.y[mem] + row;
        if (m < M) y[(int64_t)m * d_out] = ua[u] * p.tscale[mem];
        if (m + 1 < M) y[(int64_t)(m + 1) * d_out] = ub[u] * p.tscale[mem];
      }
    }
  }
}

// ---- launch planning for the MFMA kernel ------------------------------------------
// Four-wave workgroups as plan_nw4 lays them out (twice the waves above 8
// vectors, where each slot takes two MFMAs per 16 rows), with S raised where
// needed so that a workgroup's staged input (M rows of its chunk range) fits
// the LDS budget.
inline Plan plan_mfma(int64_t R, int64_t C, int nmat, int M) {
  (void)nmat;
  Plan pl = plan_nw4(R, C, M > kMaxM ? 4096 : 2048);
  const int64_t max_chunks = kMfmaXBytes / (M * 512);
  if (pl.wg_chunks > max_chunks) {
    int64_t S = (C + max_chunks - 1) / max_chunks;
    const int64_t wg_chunks = (C + S - 1) / S;
    S = (C + wg_chunks - 1) / wg_chunks;
    pl = Plan{(int)S, (int)wg_chunks, kWavesPerWg};
  }
  return pl;
}

// Dynamic LDS of a launch: the staged input, or the reduction buffer where it
// lives there and is larger.
inline size_t mfma_lds_bytes(const Plan& pl, uint32_t fmt, int nmat, int M) {
  const size_t staged = (size_t)M * (pl.wg_chunks * 512 + kXPad) + kZeroBytes;
  const int nv = nmat * (fmt == FP4G_NVFP4 && M <= 8 ? 8 : 16);  // values per lane at the end
  const size_t red = nv > kMfmaRedOwn ? (size_t)kWavesPerWg * nv * 64 * 4 : 0;
  return staged > red ? staged : red;
}

// Exchange units per lane: the larger of the two kernels' needs (the MFMA
// kernel's for its widest case, either format).
inline int64_t exchange_units_any(int nmat, int M) {
  const int64_t mf = nmat == 2 ? 16 : 8;
  const int64_t vu = exchange_units(nmat, M);
  return mf > vu ? mf : vu;
}

// Workspace for either kernel (the caller may choose the path per call).
inline uint64_t gemv_ws_bytes_any(int64_t R_total, int64_t C, int nmat, int M) {
  const Plan b = plan_mfma(R_total, C, nmat, M);
  const Plan a = plan_for(R_total, C, nmat, M);  // wider FP4: matrix cores only; FP8 rows: VALU up to 16
  const int64_t nodes = tree_nodes(a.S) > tree_nodes(b.S) ? tree_nodes(a.S) : tree_nodes(b.S);
  return (uint64_t)nodes * exchange_units_any(nmat, M) * R_total * 64 * 8;
}

template <uint32_t FMT, int NMAT, int EPI>
hipError_t launch_mfma(int M, const GemvParams& p, unsigned grid, size_t lds, hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM)                                                       \
  case MM:                                                                  \
    k_gemv_mfma<FMT, MM, NMAT, EPI><<<grid, kThreads, lds, s>>>(p, MfmaMoe{}); \
    break;
    FP4G_CASE(1) FP4G_CASE(2) FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
    FP4G_CASE(9) FP4G_CASE(10) FP4G_CASE(11) FP4G_CASE(12) FP4G_CASE(13) FP4G_CASE(14) FP4G_CASE(15) FP4G_CASE(16)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The mixture-of-experts gate/up (MODE 1) and down (MODE 2) launches, M = 3..8.
template <uint32_t FMT>
hipError_t launch_mfma_moe(int M, const GemvParams& p, const MfmaMoe& q, unsigned grid, size_t lds, hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM)                                                                 \
  case MM:                                                                            \
    k_gemv_mfma<FMT, MM, 2, EPI_SILU, 1><<<grid, kThreads, lds, s>>>(p, q); \
    break;
    FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <uint32_t FMT>
hipError_t launch_mfma_moe_down(int M, const GemvParams& p, const MfmaMoe& q, unsigned grid, size_t lds,
                                hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM)                                                           \
  case MM:                                                                      \
    k_gemv_mfma<FMT, MM, 1, EPI_STORE, 2><<<grid, kThreads, lds, s>>>(p, q); \
    break;
    FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The same for verify blocks of 9..16 tokens (instantiated in a translation unit
// of their own).
template <uint32_t FMT>
hipError_t launch_mfma_moe_wide(int M, const GemvParams& p, const MfmaMoe& q, unsigned grid, size_t lds,
                                hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM)                                                       \
  case MM:                                                                  \
    k_gemv_mfma<FMT, MM, 2, EPI_SILU, 1><<<grid, kThreads, lds, s>>>(p, q); \
    break;
    FP4G_CASE(9) FP4G_CASE(10) FP4G_CASE(11) FP4G_CASE(12) FP4G_CASE(13) FP4G_CASE(14) FP4G_CASE(15) FP4G_CASE(16)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <uint32_t FMT>
hipError_t launch_mfma_moe_down_wide(int M, const GemvParams& p, const MfmaMoe& q, unsigned grid, size_t lds,
                                     hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM)                                                        \
  case MM:                                                                   \
    k_gemv_mfma<FMT, MM, 1, EPI_STORE, 2><<<grid, kThreads, lds, s>>>(p, q); \
    break;
    FP4G_CASE(9) FP4G_CASE(10) FP4G_CASE(11) FP4G_CASE(12) FP4G_CASE(13) FP4G_CASE(14) FP4G_CASE(15) FP4G_CASE(16)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fp4g
