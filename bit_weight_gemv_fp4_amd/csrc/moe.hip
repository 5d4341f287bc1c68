// moe.hip -- one mixture-of-experts layer at decode batch sizes (M = 1..16):
// moe_route_gemv.
//
// The Ling-3.0 MoE decode article (magicnetworld.com, sec. 3 and the sec. 4
// flowchart) routes each token to 8 of 512 experts plus a shared expert, reads
// only the chosen experts' weights and accumulates back to the hidden size; its
// sec. 8 notes that M tokens read the union of their experts.  Routing never
// leaves the device.  For M = 1, 2 two launches:
//
//  k_moe_up   Every workgroup first routes the M tokens itself (top-k of the
//             logits by a wave arg-max per pick, softmax over the k picked),
//             then takes the (slot, 64-row group, K split) its block index
//             names.  At M = 1 the slots are the picks in pick order, then the
//             shared expert, and a workgroup picks only as far as its own slot;
//             at M = 2 they are the union's experts in ascending id (ranked
//             lane-parallel), then the shared expert.  Workgroups past the
//             realised union exit before reading a byte, so only the union's
//             gate/up bytes stream.  The K splits of a (slot, row group) meet in
//             the split-K exchange tree, and the survivor writes
//             h = bf16(SiLU(gate x) * (up x)) for all M tokens to the workspace.
//             One workgroup also writes the routing tables: the slots' experts
//             and, per (slot, token), the gate weight times the down matrix's
//             tensor scale (0 for a token that did not pick the expert, 1 x
//             scale for the shared expert).
//  k_moe_down Each workgroup owns one 64-row group of the hidden size and a
//             share of the (slot, chunk) tiles of that row group over all the
//             union's experts.  Each tile's dot products with the slot's h are
//             weighted by the slot's coefficients and summed in registers, so the
//             experts need no combine step; the K shares meet in the exchange
//             tree, whose survivor writes Y.
//
// From M = 3 vectors on, the gate/up half runs on the matrix cores instead
// (gemv_mfma.hpp).  Up to 4 vectors its workgroups route the tokens themselves
// (one wave per token, the union through an LDS bitmap; workgroup 0 writes the
// tables); above that k_moe_route (one workgroup) routes once and writes the
// tables that the matrix-core product reads.  k_moe_down follows as above;
// from M = 5 on the down half also runs on the matrix-core kernel (its down
// mode).  Measured crossovers set the thresholds.
// Verify blocks of 9..16 tokens (feed, "DFlash2: drafting a block in one pass":
// 11 positions) take the same three launches, the routing workgroup with one
// wave per token.  With 8-bit activations (W4A8, fp4g_moe.act) every M takes
// the routing launch and the scaled FP4 x FP8 matrix-core kernel for both
// halves (gemv_a8.hpp), x and each h quantised to MXFP8 in its staging.
//
// The kernels use the tile loop, the split-K tree and the launch planner of the
// dense product (gemv_kernel.hpp, gemv_mfma.hpp).  Results are deterministic.
#include <algorithm>

#include "gemv_a8.hpp"

namespace fp4g {

// Matrix-core gate/up launchers, in gemv_mfma_moe.hip.
extern template hipError_t launch_mfma_moe<FP4G_NVFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                       hipStream_t);
extern template hipError_t launch_mfma_moe<FP4G_MXFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                       hipStream_t);
extern template hipError_t launch_mfma_moe_down<FP4G_NVFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                            hipStream_t);
extern template hipError_t launch_mfma_moe_down<FP4G_MXFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                            hipStream_t);
// W4A8 gate/up and down, in gemv_a8_moe.hip.
hipError_t launch_a8_moe_up_ext(int M, const GemvParams& p, const MfmaMoe& q, unsigned grid, size_t lds,
                                hipStream_t s);
hipError_t launch_a8_moe_down_ext(int M, const GemvParams& p, const MfmaMoe& q, unsigned grid, size_t lds,
                                  hipStream_t s);
// 9..16 tokens, in gemv_mfma_moe_wide.hip.
extern template hipError_t launch_mfma_moe_wide<FP4G_NVFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                            hipStream_t);
extern template hipError_t launch_mfma_moe_wide<FP4G_MXFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                            hipStream_t);
extern template hipError_t launch_mfma_moe_down_wide<FP4G_NVFP4>(int, const GemvParams&, const MfmaMoe&, unsigned,
                                                                 size_t, hipStream_t);
extern template hipError_t launch_mfma_moe_down_wide<FP4G_MXFP4>(int, const GemvParams&, const MfmaMoe&, unsigned,
                                                                 size_t, hipStream_t);

namespace {

constexpr int kMoeMfmaMinM = 3;    // gate/up on the matrix cores from this many vectors
constexpr int kMoeMfmaDnMinM = 5;  // down on the matrix cores from this many (measured crossover)
constexpr int kMoeMfmaUnits = 16;  // exchange units per lane of that kernel: fused epilogue (at most)
constexpr int kMoeMfmaUnitsDn = 8;  // and plain products (at most)

// k_moe_down (up to kMoeMfmaDnMinM - 1 vectors) holds the slot table in one
// register per lane
static_assert((kMoeMfmaDnMinM - 1) * kMaxTopK + 1 < 64, "slot table exceeds a wave");

// Routing alone (in front of the matrix-core gate/up): one workgroup, one wave
// per token (at least 4).
template <int M>
constexpr int route_waves() { return M > 4 ? M : 4; }
template <int M>
__global__ __launch_bounds__(route_waves<M>() * 64) void k_moe_route(MoeParams p) {
  __shared__ RouteLds<M> r;
  route_tokens<M, route_waves<M>()>(p, r);
  write_route_tables<M, route_waves<M>()>(p, r);
}

// Gate/up of unit `blk` = (slot, 64-row group, K split) of the union, after the
// workgroup routed the tokens into r.  BY_PICK: the slots are in pick order
// (one token), so slot j's intermediate is column j of H.
template <uint32_t FMT, int M, int NW, bool BY_PICK>
__device__ __forceinline__ void moe_up_unit(const MoeParams& p, const RouteLds<M>& r, int blk,
                                            float (&red)[NW][2 * M][64]) {
  constexpr int TILE = FMT == FP4G_NVFP4 ? kTileNv : kTileMx;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int per_slot = p.Rg * p.S_up;
  const int slot = uniform(blk / per_slot);
  if (slot >= r.n_slots) return;
  const int rem = blk % per_slot;
  const int g = uniform(rem / p.S_up), s = uniform(rem % p.S_up);
  const int e = r.uni[slot];
  const uint8_t* wg_ = e >= 0 ? p.gate + (uint64_t)e * p.sg : p.sh_gate;
  const uint8_t* wu_ = e >= 0 ? p.up + (uint64_t)e * p.su : p.sh_up;
  const float tsg = e >= 0 ? p.ts_gate : p.ts_sh_gate;
  const float tsu = e >= 0 ? p.ts_up : p.ts_sh_up;

  const int wg_c0 = s * p.wg_up, wg_c1 = min(p.Cg, wg_c0 + p.wg_up);
  const int c0 = wg_c0 + (wave * (wg_c1 - wg_c0)) / NW;
  const int c1 = wg_c0 + ((wave + 1) * (wg_c1 - wg_c0)) / NW;
  const uint32_t* __restrict__ x32 = reinterpret_cast<const uint32_t*>(p.x);
  const int xstride = p.hidden / 2;
  const int full_chunks = p.hidden / kChunkK, tail_pieces = (p.hidden % kChunkK) / kPieceK;
  const int64_t tile0 = (int64_t)g * p.Cg;

  float acc[2][M];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[a][m] = 0.0f;
  // items (chunk, matrix) chunk-major: even items gate, odd items up
  auto tile_of = [&](int it) { return (it & 1 ? wu_ : wg_) + (tile0 + c0 + it / 2) * TILE; };
  auto eat = [&](const Frag<FMT>& f, int it) {
    const int c = c0 + it / 2;
    const uint32_t* xc = x32 + (int64_t)c * (kChunkK / 2);
    float part[M];
#pragma unroll
    for (int m = 0; m < M; ++m) part[m] = 0.0f;
    if (c < full_chunks)
      tile_dot<FMT, M, true>(f, xc, xstride, kPiecesNv, part);
    else
      tile_dot<FMT, M, false>(f, xc, xstride, tail_pieces, part);
    const bool up = (it & 1) != 0;  // branch-free, as in the dense kernel
#pragma unroll
    for (int m = 0; m < M; ++m) {
      acc[0][m] += up ? 0.0f : part[m];
      acc[1][m] += up ? part[m] : 0.0f;
    }
  };
  stream_items<FMT>((c1 - c0) * 2, lane, tile_of, eat);

#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int m = 0; m < M; ++m) red[wave][a * M + m][lane] = acc[a][m];
  __syncthreads();
  if (wave != 0) return;
  float ua[M], ub[M];
  bool live[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float tg = red[0][m][lane], tu = red[0][M + m][lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      tg += red[w][m][lane];
      tu += red[w][M + m][lane];
    }
    ua[m] = tg;
    ub[m] = tu;
    live[m] = true;
  }
  const int row = g * 64 + lane;
  exchange_tree<M>(p.x_up, (int64_t)p.n_slots_max * p.Rg * 64, ((int64_t)slot * p.Rg + g) * 64 + lane, p.S_up, s,
                   ua, ub, live);
  if (row < p.dff) {
    const int nh = p.K + p.has_shared;
#pragma unroll
    for (int m = 0; m < M; ++m) {
      if (!live[m]) continue;
      const uint16_t h = f32_to_bf16_rne(silu_f32(ua[m] * tsg) * (ub[m] * tsu));
      p.hbuf[((int64_t)slot * M + m) * p.dff + row] = h;
      if (p.hdbg) {
        if (BY_PICK) {
          p.hdbg[(int64_t)slot * p.dff + row] = h;  // slot j = pick j, the shared slot last
        } else if (e < 0) {
          p.hdbg[((int64_t)m * nh + p.K) * p.dff + row] = h;
        } else {
          for (int j = 0; j < p.K; ++j)
            if (r.ids[m][j] == e) p.hdbg[((int64_t)m * nh + j) * p.dff + row] = h;
        }
      }
    }
  }
}

template <uint32_t FMT, int M, int NW>
__global__ __launch_bounds__(NW * 64) void k_moe_up(MoeParams p) {
  __shared__ RouteLds<M> r;
  __shared__ float red[NW][2 * M][64];
  if constexpr (M == 1) {
    // slots in pick order: slot j needs the first j + 1 picks, the shared slot
    // none; the first unit of the last routed slot makes all K picks and writes
    // the tables
    const int per_slot = p.Rg * p.S_up;
    const int slot = uniform(blockIdx.x / per_slot);
    const bool tables = blockIdx.x == (p.K - 1) * per_slot;
    route_by_pick<M>(p, r, slot < p.K ? slot + 1 : 0, tables);
    if (tables) write_route_tables<M, NW>(p, r);
    moe_up_unit<FMT, M, NW, true>(p, r, blockIdx.x, red);
  } else {
    route_tokens<M, NW>(p, r);
    if (blockIdx.x == 0) write_route_tables<M, NW>(p, r);
    moe_up_unit<FMT, M, NW, false>(p, r, blockIdx.x, red);
  }
}

template <uint32_t FMT, int M, int NW>
__global__ __launch_bounds__(NW * 64) void k_moe_down(MoeParams p) {
  constexpr int TILE = FMT == FP4G_NVFP4 ? kTileNv : kTileMx;
  __shared__ float red[NW][M][64];
  const int lane = threadIdx.x & 63, wave = wave_id();
  // the slot table in one round trip: lane i holds route[i] (the slot count,
  // then the slots' experts)
  const int rt = lane <= p.n_slots_max ? p.route[lane] : 0;
  const int n_slots = __builtin_amdgcn_readfirstlane(rt);
  const int g = uniform(blockIdx.x / p.S_dn), s = uniform(blockIdx.x % p.S_dn);
  // this workgroup's share of the row group's (slot, chunk) tiles, then the wave's
  const int total = n_slots * p.Cd;
  const int w0 = (int)(((int64_t)s * total) / p.S_dn), w1 = (int)(((int64_t)(s + 1) * total) / p.S_dn);
  const int i0 = w0 + (wave * (w1 - w0)) / NW, i1 = w0 + ((wave + 1) * (w1 - w0)) / NW;
  const int xstride = p.dff / 2;
  const int full_chunks = p.dff / kChunkK, tail_pieces = (p.dff % kChunkK) / kPieceK;
  const int64_t tile0 = (int64_t)g * p.Cd;

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
  auto tile_of = [&](int it) {
    const int q = i0 + it, slot = q / p.Cd, c = q - slot * p.Cd;
    const int e = __builtin_amdgcn_readlane(rt, 1 + slot);
    const uint8_t* wd = e >= 0 ? p.down + (uint64_t)e * p.sd : p.sh_down;
    return wd + (tile0 + c) * TILE;
  };
  auto eat = [&](const Frag<FMT>& f, int it) {
    const int q = i0 + it, slot = q / p.Cd, c = q - slot * p.Cd;
    const uint32_t* xc =
        reinterpret_cast<const uint32_t*>(p.hbuf + (int64_t)slot * M * p.dff) + (int64_t)c * (kChunkK / 2);
    float part[M];
#pragma unroll
    for (int m = 0; m < M; ++m) part[m] = 0.0f;
    if (c < full_chunks)
      tile_dot<FMT, M, true>(f, xc, xstride, kPiecesNv, part);
    else
      tile_dot<FMT, M, false>(f, xc, xstride, tail_pieces, part);
#pragma unroll
    for (int m = 0; m < M; ++m) acc[m] = __builtin_fmaf(part[m], p.coef[slot * M + m], acc[m]);
  };
  stream_items<FMT>(i1 - i0, lane, tile_of, eat);

#pragma unroll
  for (int m = 0; m < M; ++m) red[wave][m][lane] = acc[m];
  __syncthreads();
  if (wave != 0) return;
  constexpr int NU = (M + 1) / 2;
  float ua[NU], ub[NU];
  bool live[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    float ta = red[0][2 * u][lane], tb = 2 * u + 1 < M ? red[0][2 * u + 1][lane] : 0.0f;
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      ta += red[w][2 * u][lane];
      if (2 * u + 1 < M) tb += red[w][2 * u + 1][lane];
    }
    ua[u] = ta;
    ub[u] = tb;
    live[u] = true;
  }
  exchange_tree<NU>(p.x_dn, (int64_t)p.Rd * 64, (int64_t)g * 64 + lane, p.S_dn, s, ua, ub, live);
  const int row = g * 64 + lane;
  if (row >= p.hidden) return;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (!live[u]) continue;
    p.y[(int64_t)(2 * u) * p.hidden + row] = ua[u];
    if (2 * u + 1 < M) p.y[(int64_t)(2 * u + 1) * p.hidden + row] = ub[u];
  }
}

// ---- host side ------------------------------------------------------------------
struct MoeLayout {
  int n_slots_max;
  int64_t Rg, Cg, Rd, Cd;
  Plan up, dn;
  uint32_t gate_fmt;
  uint64_t off_route, off_coef, off_hbuf, off_x_up, off_x_dn, total;
};

// Both kernels stream a few thousand tiles at most and are bound by each wave's
// chain of round trips (routing, loads, tree): latency plans.  k_moe_up holds
// two tiles in flight plus the routing state, up to 170 VGPRs (12 waves per CU:
// workgroups of 4, 8 or 12 waves; at M = 2 the 12-wave form spills a few
// registers and is still the fastest measured).  k_moe_down fits 16 waves per
// CU up to M = 5, like the dense kernel.
inline Plan plan_up(int64_t R, int64_t C, int M) { return plan_latency(R, C, 12, {4, 8, 12}); }
// Down projection on the VALU kernel.  At four vectors (the last count before
// the matrix cores take over) each tile costs four v_dot2 per weight pair, and
// spreading the tiles over every SIMD outweighs the tree: four-wave workgroups
// with one chunk per wave (C5 shapes, measured per layer with the gate/up plan
// below: 50.3 -> 48.1 us; the latency plan's 16-wave workgroups covered 160 of
// the 256 CUs).  Fewer vectors keep the latency plan (one chunk per wave was
// 0.8-1.2 us slower at one and two vectors, 2.3 us at three).
inline Plan plan_dn(int64_t R, int64_t C, int M) {
  if (M == 4) {
    const int64_t wg_chunks = 4, S = (C + wg_chunks - 1) / wg_chunks;
    return Plan{(int)S, (int)((C + S - 1) / S), 4};
  }
  return plan_latency(R, C, M <= 5 ? 16 : 12, {4, 8, 16});
}
// gate/up plan and exchange units per lane for M vectors (either kernel; the
// W4A8 path always runs on the matrix cores, planned like the bf16 ones).  On
// the matrix cores, once the union's row groups alone fill the CUs, K is not
// split unless the staged input needs it (no tree: C5 shapes, per layer, 55.6 ->
// 50.3 us at four vectors, 72.2 -> 70.6 at six, unchanged at three and eight;
// the W4A8 path keeps the shared plan).
inline Plan plan_gu(int64_t R, int64_t C, int M, bool a8) {
  if (!a8 && M >= kMoeMfmaMinM && R >= kCUs) {
    const int64_t max_chunks = kMfmaXBytes / (M * 512);
    const int64_t S = (C + max_chunks - 1) / max_chunks, wg_chunks = (C + S - 1) / S;
    return Plan{(int)((C + wg_chunks - 1) / wg_chunks), (int)wg_chunks, kWavesPerWg};
  }
  return a8 || M >= kMoeMfmaMinM ? plan_mfma(R, C, 2, M) : plan_up(R, C, M);
}
inline int units_gu(int M, bool a8) { return a8 || M >= kMoeMfmaMinM ? kMoeMfmaUnits : M; }
// down plan and units: C counts the union's slots x d_ff chunks
inline Plan plan_down(int64_t R, int64_t C, int M, bool a8) {
  if (!a8 && M == 8) {
    // matrix-core down at eight vectors: 8 chunks per workgroup instead of the
    // LDS-limited 10 (C5 shapes, three runs: 82.2 / 81.4 / 82.2 -> 78.2 / 78.7 /
    // 77.8 us per layer; the same count was slower at seven vectors)
    const int64_t wg_chunks = 8, S = (C + wg_chunks - 1) / wg_chunks;
    return Plan{(int)S, (int)((C + S - 1) / S), kWavesPerWg};
  }
  return a8 || M >= kMoeMfmaDnMinM ? plan_mfma(R, C, 1, M) : plan_dn(R, C, M);
}
inline int units_dn(int M, bool a8) { return a8 || M >= kMoeMfmaDnMinM ? kMoeMfmaUnitsDn : (M + 1) / 2; }


// Workspace: exchange slots first, sized for the largest need over M = 1..16
// (they must start zero-filled and every call leaves them zero), then the
// routing tables and h at an offset that does not depend on M: calls of any M on
// one layer shape can share a workspace without their tables ever landing in
// another call's slots.
int n_slots_for(const fp4g_moe* mo, int M) {
  return std::min(mo->num_experts, M * mo->top_k) + (mo->has_shared ? 1 : 0);
}

MoeLayout moe_layout(const fp4g_moe* mo, int M) {
  MoeLayout L{};
  L.n_slots_max = n_slots_for(mo, M);
  L.gate_fmt = mo->gate.format;
  L.Rg = row_groups(mo->d_ff);
  L.Cg = chunks(mo->hidden);
  L.Rd = row_groups(mo->hidden);
  L.Cd = chunks(mo->d_ff);
  const bool a8 = mo->act == FP4G_ACT_MXFP8;
  L.up = plan_gu(L.Rg * L.n_slots_max, L.Cg, M, a8);
  L.dn = plan_down(L.Rd, L.Cd * L.n_slots_max, M, a8);
  uint64_t slot_bytes = 0;  // the largest need of either activation format
  for (int m = 1; m <= kMaxMWide; ++m) {
    const int ns = n_slots_for(mo, m);
    for (bool q8 : {false, true}) {
      const Plan up = plan_gu(L.Rg * ns, L.Cg, m, q8), dn = plan_down(L.Rd, L.Cd * ns, m, q8);
      const uint64_t b = align256(8ull * tree_nodes(up.S) * units_gu(m, q8) * ns * L.Rg * 64) +
                         align256(8ull * tree_nodes(dn.S) * units_dn(m, q8) * L.Rd * 64);
      slot_bytes = std::max(slot_bytes, b);
    }
  }
  L.off_x_up = 0;
  L.off_x_dn = align256(8ull * tree_nodes(L.up.S) * units_gu(M, a8) * L.n_slots_max * L.Rg * 64);
  const int nsw = n_slots_for(mo, kMaxMWide);
  uint64_t o = slot_bytes;
  L.off_route = o;
  o = align256(o + 4ull * (1 + nsw));
  L.off_coef = o;
  o = align256(o + 4ull * nsw * kMaxMWide);
  L.off_hbuf = o;
  o = align256(o + 2ull * nsw * kMaxMWide * mo->d_ff);
  L.total = o;
  return L;
}

fp4g_status check_moe(const fp4g_moe* mo) {
  if (!mo) return FP4G_E_NULL;
  if (mo->num_experts < 1 || mo->num_experts > kMaxExperts || mo->top_k < 1 || mo->top_k > kMaxTopK ||
      mo->top_k > mo->num_experts || mo->hidden < 32 || mo->d_ff < 32 || (mo->has_shared != 0 && mo->has_shared != 1))
    return FP4G_E_SHAPE;
  if (mo->act != FP4G_ACT_BF16 && mo->act != FP4G_ACT_MXFP8) return FP4G_E_PATH;
  const fp4g_weight* ws[6] = {&mo->gate, &mo->up, &mo->down, &mo->sh_gate, &mo->sh_up, &mo->sh_down};
  const int nw = mo->has_shared ? 6 : 3;
  for (int i = 0; i < nw; ++i) {
    fp4g_status st = check_weight(ws[i], true);
    if (st != FP4G_OK) return st;
    if (ws[i]->format != mo->gate.format) return FP4G_E_FORMAT;
    const bool is_down = (i % 3) == 2;
    if (ws[i]->d_out != (is_down ? mo->hidden : mo->d_ff) || ws[i]->d_in != (is_down ? mo->d_ff : mo->hidden))
      return FP4G_E_SHAPE;
  }
  if (mo->act == FP4G_ACT_MXFP8 && mo->gate.format != FP4G_MXFP4) return FP4G_E_PATH;  // W4A8: MXFP4 experts
  const uint64_t pg = packed_bytes_of(mo->gate.format, mo->d_ff, mo->hidden);
  const uint64_t pd = packed_bytes_of(mo->gate.format, mo->hidden, mo->d_ff);
  if (mo->stride_gate < pg || mo->stride_up < pg || mo->stride_down < pd) return FP4G_E_SHAPE;
  if (mo->stride_gate % 256 || mo->stride_up % 256 || mo->stride_down % 256) return FP4G_E_ALIGN;
  // every routed expert must fit in the described buffers
  const uint64_t n1 = (uint64_t)(mo->num_experts - 1);
  if (mo->gate.packed_bytes < n1 * mo->stride_gate + pg || mo->up.packed_bytes < n1 * mo->stride_up + pg ||
      mo->down.packed_bytes < n1 * mo->stride_down + pd)
    return FP4G_E_SHAPE;
  return FP4G_OK;
}

// The matrix-core gate/up's view of the layer (used from kMoeMfmaMinM vectors on).
struct MoeMfma {
  GemvParams gp, gpd;  // gate/up, down
  MfmaMoe q, qd;
  size_t lds, lds_d;
};

template <uint32_t FMT, int M>
hipError_t launch_moe_m(const MoeParams& p, const MoeMfma& mf, const MoeLayout& L, unsigned grid_up,
                        unsigned grid_dn, hipStream_t s) {
  const Plan& up = L.up;
  const Plan& dn = L.dn;
  if constexpr (M >= kMoeMfmaMinM) {
    if constexpr (M > kMfmaMoeRouteM) {  // up to kMfmaMoeRouteM the gate/up workgroups route themselves
      k_moe_route<M><<<1, route_waves<M>() * 64, 0, s>>>(p);
      if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
    }
    const hipError_t eu = M > kMaxM ? launch_mfma_moe_wide<FMT>(M, mf.gp, mf.q, grid_up, mf.lds, s)
                                    : launch_mfma_moe<FMT>(M, mf.gp, mf.q, grid_up, mf.lds, s);
    if (eu != hipSuccess) return hipErrorLaunchFailure;
  } else {
    switch (up.nw) {
      case 4: k_moe_up<FMT, M, 4><<<grid_up, 256, 0, s>>>(p); break;
      case 8: k_moe_up<FMT, M, 8><<<grid_up, 512, 0, s>>>(p); break;
      case 12: k_moe_up<FMT, M, 12><<<grid_up, 768, 0, s>>>(p); break;
      default: return hipErrorInvalidValue;
    }
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  }
  if constexpr (M >= kMoeMfmaDnMinM) {
    return M > kMaxM ? launch_mfma_moe_down_wide<FMT>(M, mf.gpd, mf.qd, grid_dn, mf.lds_d, s)
                     : launch_mfma_moe_down<FMT>(M, mf.gpd, mf.qd, grid_dn, mf.lds_d, s);
  } else {
    switch (dn.nw) {
      case 4: k_moe_down<FMT, M, 4><<<grid_dn, 256, 0, s>>>(p); break;
      case 8: k_moe_down<FMT, M, 8><<<grid_dn, 512, 0, s>>>(p); break;
      case 16:
        if constexpr (M <= 5) {  // and for plain products up to M = 5
          k_moe_down<FMT, M, 16><<<grid_dn, 1024, 0, s>>>(p);
          break;
        }
        return hipErrorInvalidValue;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

// W4A8: routing once, then gate/up and down on the scaled FP4 x FP8 matrix cores.
template <int M>
hipError_t launch_moe_a8_m(const MoeParams& p, const MoeMfma& mf, unsigned grid_up, unsigned grid_dn, hipStream_t s) {
  k_moe_route<M><<<1, route_waves<M>() * 64, 0, s>>>(p);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  if (launch_a8_moe_up_ext(M, mf.gp, mf.q, grid_up, mf.lds, s) != hipSuccess) return hipErrorLaunchFailure;
  return launch_a8_moe_down_ext(M, mf.gpd, mf.qd, grid_dn, mf.lds_d, s);
}

hipError_t launch_moe_a8(int M, const MoeParams& p, const MoeMfma& mf, unsigned grid_up, unsigned grid_dn,
                         hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM) \
  case MM:            \
    return launch_moe_a8_m<MM>(p, mf, grid_up, grid_dn, s);
    FP4G_CASE(1) FP4G_CASE(2) FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
    FP4G_CASE(9) FP4G_CASE(10) FP4G_CASE(11) FP4G_CASE(12) FP4G_CASE(13) FP4G_CASE(14) FP4G_CASE(15) FP4G_CASE(16)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
}

template <uint32_t FMT>
hipError_t launch_moe(int M, const MoeParams& p, const MoeMfma& mf, const MoeLayout& L, unsigned grid_up,
                      unsigned grid_dn, hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM) \
  case MM:            \
    return launch_moe_m<FMT, MM>(p, mf, L, grid_up, grid_dn, s);
    FP4G_CASE(1) FP4G_CASE(2) FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
    FP4G_CASE(9) FP4G_CASE(10) FP4G_CASE(11) FP4G_CASE(12) FP4G_CASE(13) FP4G_CASE(14) FP4G_CASE(15) FP4G_CASE(16)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

uint64_t moe_ws_bytes(const fp4g_moe* mo, int M) {
  if (check_moe(mo) != FP4G_OK || M < 1 || M > kMaxMWide) return 0;
  return moe_layout(mo, M).total;
}

uint64_t moe_slot_bytes(const fp4g_moe* mo) {
  if (check_moe(mo) != FP4G_OK) return 0;
  return moe_layout(mo, 1).off_route;  // the tables follow the slots
}

namespace {

// One call's checked parameters: kernel arguments, plans and grids.
struct MoeCall {
  MoeParams p;
  MoeMfma mf;
  MoeLayout L;
  unsigned grid_up, grid_dn;
  bool a8;
};

// Host checks of moe_route_gemv and the set-up of its launches.
fp4g_status moe_prepare(const fp4g_moe* mo, const uint16_t* X, const float* logits, int32_t M, float* Y,
                        int32_t* topk_ids, float* topk_w, uint16_t* H, void* ws, uint64_t ws_bytes, MoeCall& c) {
  fp4g_status st = check_moe(mo);
  if (st != FP4G_OK) return st;
  if (!X || !logits || !Y || !topk_ids || !topk_w || !ws) return FP4G_E_NULL;
  if (M < 1 || M > kMaxMWide) return FP4G_E_SHAPE;
  if (!aligned(X, 16) || !aligned(logits, 16) || !aligned(Y, 16) || !aligned(topk_ids, 16) ||
      !aligned(topk_w, 16) || (H && !aligned(H, 16)))
    return FP4G_E_ALIGN;
  c.L = moe_layout(mo, M);
  const MoeLayout& L = c.L;
  if (ws_bytes < L.total) return FP4G_E_WORKSPACE;
  if (!aligned(ws, 256)) return FP4G_E_ALIGN;
  const int nh = mo->top_k + mo->has_shared;
  const size_t xb = (size_t)M * mo->hidden * 2, lb = (size_t)M * mo->num_experts * 4, yb = (size_t)M * mo->hidden * 4,
               ib = (size_t)M * mo->top_k * 4, hb = H ? (size_t)M * nh * mo->d_ff * 2 : 0;
  const void* outs[5] = {Y, topk_ids, topk_w, H, ws};
  const size_t outb[5] = {yb, ib, ib, hb, L.total};
  const void* ins[5] = {X, logits, mo->gate.packed, mo->up.packed, mo->down.packed};
  const size_t inb[5] = {xb, lb, mo->gate.packed_bytes, mo->up.packed_bytes, mo->down.packed_bytes};
  for (int i = 0; i < 5; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlap(outs[i], outb[i], ins[j], inb[j])) return FP4G_E_ALIAS;
    for (int j = i + 1; j < 5; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return FP4G_E_ALIAS;
    if (mo->has_shared &&
        (overlap(outs[i], outb[i], mo->sh_gate.packed, mo->sh_gate.packed_bytes) ||
         overlap(outs[i], outb[i], mo->sh_up.packed, mo->sh_up.packed_bytes) ||
         overlap(outs[i], outb[i], mo->sh_down.packed, mo->sh_down.packed_bytes)))
      return FP4G_E_ALIAS;
  }
  c.p = MoeParams{};
  MoeParams& p = c.p;
  p.gate = (const uint8_t*)mo->gate.packed;
  p.up = (const uint8_t*)mo->up.packed;
  p.down = (const uint8_t*)mo->down.packed;
  p.sg = mo->stride_gate;
  p.su = mo->stride_up;
  p.sd = mo->stride_down;
  p.ts_gate = mo->gate.tensor_scale;
  p.ts_up = mo->up.tensor_scale;
  p.ts_down = mo->down.tensor_scale;
  if (mo->has_shared) {
    p.sh_gate = (const uint8_t*)mo->sh_gate.packed;
    p.sh_up = (const uint8_t*)mo->sh_up.packed;
    p.sh_down = (const uint8_t*)mo->sh_down.packed;
    p.ts_sh_gate = mo->sh_gate.tensor_scale;
    p.ts_sh_up = mo->sh_up.tensor_scale;
    p.ts_sh_down = mo->sh_down.tensor_scale;
  }
  p.E = mo->num_experts;
  p.K = mo->top_k;
  p.hidden = mo->hidden;
  p.dff = mo->d_ff;
  p.has_shared = mo->has_shared;
  p.x = X;
  p.logits = logits;
  p.y = Y;
  p.topk_ids = topk_ids;
  p.topk_w = topk_w;
  p.hdbg = H;
  uint8_t* w = (uint8_t*)ws;
  p.route = (int*)(w + L.off_route);
  p.coef = (float*)(w + L.off_coef);
  p.hbuf = (uint16_t*)(w + L.off_hbuf);
  p.x_up = (unsigned long long*)(w + L.off_x_up);
  p.x_dn = (unsigned long long*)(w + L.off_x_dn);
  p.n_slots_max = L.n_slots_max;
  p.Rg = (int)L.Rg;
  p.Cg = (int)L.Cg;
  p.S_up = L.up.S;
  p.wg_up = L.up.wg_chunks;
  p.Rd = (int)L.Rd;
  p.Cd = (int)L.Cd;
  p.S_dn = L.dn.S;
  c.grid_up = (unsigned)(L.n_slots_max * L.Rg * L.up.S);
  c.grid_dn = (unsigned)(L.Rd * L.dn.S);
  const unsigned grid_up = c.grid_up;
  const bool a8 = c.a8 = mo->act == FP4G_ACT_MXFP8;
  c.mf = MoeMfma{};
  MoeMfma& mf = c.mf;
  if (a8 || M >= kMoeMfmaMinM) {
    GemvParams& gp = mf.gp;
    gp.n = 1;
    gp.w[0] = p.gate;
    gp.w[1] = p.up;
    gp.tscale[0] = p.ts_gate;
    gp.tscale[1] = p.ts_up;
    gp.d_out[0] = mo->d_ff;
    gp.gbase[0] = 0;
    gp.gbase[1] = (int)(L.n_slots_max * L.Rg);
    gp.x = X;
    gp.h = p.hbuf;
    gp.slots = p.x_up;
    gp.d_in = mo->hidden;
    gp.C = (int)L.Cg;
    gp.S = L.up.S;
    gp.wg_chunks = L.up.wg_chunks;
    MfmaMoe& q = mf.q;
    q.route = p.route;
    q.rp = p;
    q.stride[0] = p.sg;
    q.stride[1] = p.su;
    q.sh[0] = p.sh_gate;
    q.sh[1] = p.sh_up;
    q.sh_ts[0] = p.ts_sh_gate;
    q.sh_ts[1] = p.ts_sh_up;
    q.rg = (int)L.Rg;
    q.hdbg = H;
    q.ids = topk_ids;
    q.k = mo->top_k;
    q.nh = nh;
    mf.lds = a8 ? a8_lds_bytes(L.up, M, 2) : mfma_lds_bytes(L.up, mo->gate.format, 2, M);
    GemvParams& gd = mf.gpd;
    gd.n = 1;
    gd.w[0] = p.down;
    gd.tscale[0] = 1.0f;  // the coefficients carry the down tensor scales
    gd.y[0] = Y;
    gd.d_out[0] = mo->hidden;
    gd.gbase[0] = 0;
    gd.gbase[1] = (int)L.Rd;
    gd.slots = p.x_dn;
    gd.d_in = mo->d_ff;
    gd.C = (int)(L.Cd * L.n_slots_max);
    gd.S = L.dn.S;
    gd.wg_chunks = L.dn.wg_chunks;
    MfmaMoe& qd = mf.qd;
    qd.route = p.route;
    qd.stride[0] = p.sd;
    qd.sh[0] = p.sh_down;
    qd.coef = p.coef;
    qd.hbuf = p.hbuf;
    qd.cd = (int)L.Cd;
    qd.dff = mo->d_ff;
    mf.lds_d = a8 ? a8_lds_bytes(L.dn, M, 1) : mfma_lds_bytes(L.dn, mo->gate.format, 1, M);
  }
  return FP4G_OK;
}

hipError_t moe_launch(int M, const MoeCall& c, hipStream_t s) {
  if (c.a8) return launch_moe_a8(M, c.p, c.mf, c.grid_up, c.grid_dn, s);
  return c.L.gate_fmt == FP4G_NVFP4 ? launch_moe<FP4G_NVFP4>(M, c.p, c.mf, c.L, c.grid_up, c.grid_dn, s)
                                    : launch_moe<FP4G_MXFP4>(M, c.p, c.mf, c.L, c.grid_up, c.grid_dn, s);
}

}  // namespace
}  // namespace fp4g

using namespace fp4g;

extern "C" int32_t moe_route_gemv(const fp4g_moe* mo, const uint16_t* X, const float* logits, int32_t M, float* Y,
                                  int32_t* topk_ids, float* topk_w, uint16_t* H, void* ws, uint64_t ws_bytes,
                                  void* stream) {
  MoeCall c;
  const fp4g_status st = moe_prepare(mo, X, logits, M, Y, topk_ids, topk_w, H, ws, ws_bytes, c);
  if (st != FP4G_OK) return st;
  return moe_launch(M, c, (hipStream_t)stream) == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}
