// moe.hip -- one mixture-of-experts layer at decode batch sizes (M = 1..8):
// moe_route_gemv.
//
// The Ling-3.0 MoE decode article (magicnetworld.com, sec. 3 and the sec. 4
// flowchart) routes each token to 8 of 512 experts plus a shared expert, reads
// only the chosen experts' weights and accumulates back to the hidden size; its
// sec. 8 notes that M tokens read the union of their experts.  Two launches, and
// routing never leaves the device:
//
//  k_moe_up   Every workgroup first routes all M tokens itself (top-k of the
//             logits by a wave arg-max per pick, softmax over the k picked, the
//             sorted union of the picked experts via an LDS bitmap), then takes
//             the (slot, 64-row group, K split) its block index names.  Slots are
//             the union's experts in ascending id, then the shared expert.
//             Workgroups past the realised union exit before reading a byte, so
//             only the union's gate/up bytes stream.  The last workgroup of a
//             (slot, row group) writes h = bf16(SiLU(gate x) * (up x)) for all M
//             tokens to the workspace.  Workgroup 0 also writes the routing
//             tables.
//  k_moe_down Each (slot, 64-row group of the hidden size, K split) streams the
//             expert's down projection against its h, multiplies by the token's
//             gate weight (1 for the shared expert, 0 for tokens that did not pick
//             it), and the last of all slots' workgroups of a row group sums the
//             partial outputs in slot order into Y.
#include <algorithm>

#include "gemv_kernel.hpp"

namespace fp4g {
namespace {

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 8;

struct MoeParams {
  const uint8_t *gate, *up, *down;  // routed expert 0; expert e at + e * stride
  uint64_t sg, su, sd;
  const uint8_t *sh_gate, *sh_up, *sh_down;
  float ts_gate, ts_up, ts_down, ts_sh_gate, ts_sh_up, ts_sh_down;
  int E, K, hidden, dff, has_shared;
  const uint16_t* x;     // bf16 [M][hidden]
  const float* logits;   // f32 [M][E]
  float* y;              // f32 [M][hidden]
  int* topk_ids;         // [M][K]
  float* topk_w;         // [M][K]
  uint16_t* hdbg;        // optional bf16 [M][K + has_shared][dff]
  // workspace
  int* route;            // [0] = number of slots, [1 + i] = expert of slot i (-1 = shared)
  float* coef;           // [n_slots_max][M] gate weight of token m for slot i
  uint16_t* hbuf;        // bf16 [n_slots_max][M][dff]
  unsigned* cnt_up;      // [n_slots_max * Rg]
  float* part_up;        // [S_up][n_slots_max][2][M][Rg * 64]
  unsigned* cnt_dn;      // [Rd]
  float* part_dn;        // [n_slots_max][S_dn][M][Rd * 64]
  int n_slots_max;
  int Rg, Cg, S_up, wg_up;  // gate/up: d_ff rows, hidden columns
  int Rd, Cd, S_dn, wg_dn;  // down: hidden rows, d_ff columns
};

// Shared routing state of one workgroup.
template <int M>
struct RouteLds {
  int ids[M][kMaxTopK];
  float v[M][kMaxTopK];  // the picked logits
  float w[M][kMaxTopK];
  unsigned bits[kMaxExperts / 32];
  int uni[M * kMaxTopK + 1];
  int n_slots;
};

// (v, i) beats (bv, bi): larger value, or equal value and lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// All 256 threads: route the M tokens into `r` (ids, weights, sorted union).
template <int M>
__device__ void route_tokens(const MoeParams& p, RouteLds<M>& r) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int words = (p.E + 31) / 32;
  for (int i = threadIdx.x; i < words; i += kThreads) r.bits[i] = 0u;
  const int per_lane = (p.E + 63) / 64;  // <= 16
  for (int m = wave; m < M; m += kWavesPerWg) {
    const float* lg = p.logits + (int64_t)m * p.E;
    unsigned left = 0;  // bit t set: element lane + 64 t still available
    for (int t = 0; t < per_lane; ++t)
      if (lane + 64 * t < p.E) left |= 1u << t;
    for (int j = 0; j < p.K; ++j) {
      float bv = -__builtin_inff();
      int bi = 0x7fffffff;
      for (int t = 0; t < per_lane; ++t) {
        if (!((left >> t) & 1u)) continue;
        const int e = lane + 64 * t;
        const float v = lg[e];
        if (better(v, e, bv, bi)) {
          bv = v;
          bi = e;
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (better(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      if (bi != 0x7fffffff && (bi & 63) == lane) left &= ~(1u << (bi >> 6));
      if (lane == 0) {
        r.ids[m][j] = bi;
        r.v[m][j] = bv;
      }
    }
    if (lane == 0) {
      // picks are in descending order, so the first is the maximum
      float z = 0.0f;
      for (int j = 0; j < p.K; ++j) z += expf(r.v[m][j] - r.v[m][0]);
      for (int j = 0; j < p.K; ++j) r.w[m][j] = expf(r.v[m][j] - r.v[m][0]) / z;
    }
  }
  __syncthreads();
  if (threadIdx.x < M * p.K) {
    const int m = threadIdx.x / p.K, j = threadIdx.x % p.K;
    const int e = r.ids[m][j];
    atomicOr(&r.bits[e >> 5], 1u << (e & 31));
  }
  __syncthreads();
  if (wave == 0) {
    // ascending expert ids: exclusive scan of the words' popcounts over the lanes
    int base = 0;
    for (int w0 = 0; w0 < words; w0 += 64) {
      const unsigned word = (w0 + lane < words) ? r.bits[w0 + lane] : 0u;
      const int c = __popc(word);
      int incl = c;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
      }
      int pos = base + incl - c;
      unsigned wd = word;
      while (wd) {
        const int b = __ffs(wd) - 1;
        wd &= wd - 1;
        r.uni[pos++] = (w0 + lane) * 32 + b;
      }
      base += __shfl(incl, 63, 64);
    }
    if (lane == 0) {
      if (p.has_shared) r.uni[base] = -1;
      r.n_slots = base + (p.has_shared ? 1 : 0);
    }
  }
  __syncthreads();
}

template <int M>
__device__ __forceinline__ float coef_of(const RouteLds<M>& r, const MoeParams& p, int slot, int m) {
  const int e = r.uni[slot];
  if (e < 0) return 1.0f;
  float c = 0.0f;
  for (int j = 0; j < p.K; ++j)
    if (r.ids[m][j] == e) c = r.w[m][j];
  return c;
}

template <uint32_t FMT, int M>
__global__ __launch_bounds__(kThreads) void k_moe_up(MoeParams p) {
  constexpr int TILE = FMT == FP4G_NVFP4 ? kTileNv : kTileMx;
  constexpr int NA = 2 * M;
  __shared__ RouteLds<M> r;
  __shared__ float red[kWavesPerWg][NA][64];
  route_tokens<M>(p, r);

  const int lane = threadIdx.x & 63, wave = wave_id();
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < M * p.K; i += kThreads) {
      const int m = i / p.K, j = i % p.K;
      p.topk_ids[i] = r.ids[m][j];
      p.topk_w[i] = r.w[m][j];
    }
    for (int i = threadIdx.x; i < r.n_slots; i += kThreads) {
      p.route[1 + i] = r.uni[i];
      for (int m = 0; m < M; ++m) p.coef[i * M + m] = coef_of<M>(r, p, i, m);
    }
    if (threadIdx.x == 0) p.route[0] = r.n_slots;
  }

  const int per_slot = p.Rg * p.S_up;
  const int slot = uniform(blockIdx.x / per_slot);
  if (slot >= r.n_slots) return;
  const int rem = blockIdx.x % per_slot;
  const int g = uniform(rem / p.S_up), s = uniform(rem % p.S_up);
  const int e = r.uni[slot];
  const uint8_t* wg_ = e >= 0 ? p.gate + (uint64_t)e * p.sg : p.sh_gate;
  const uint8_t* wu_ = e >= 0 ? p.up + (uint64_t)e * p.su : p.sh_up;
  const float tsg = e >= 0 ? p.ts_gate : p.ts_sh_gate;
  const float tsu = e >= 0 ? p.ts_up : p.ts_sh_up;

  const int wg_c0 = s * p.wg_up, wg_c1 = min(p.Cg, wg_c0 + p.wg_up);
  const int per_wave = (wg_c1 - wg_c0 + kWavesPerWg - 1) / kWavesPerWg;
  const int c0 = min(wg_c1, wg_c0 + wave * per_wave), c1 = min(wg_c1, c0 + per_wave);
  const uint32_t* __restrict__ x32 = reinterpret_cast<const uint32_t*>(p.x);
  const int xstride = p.hidden / 2;
  const int full_chunks = p.hidden / kChunkK, tail_pieces = (p.hidden % kChunkK) / kPieceK;
  const int64_t tile0 = (int64_t)g * p.Cg;

  float acc[2][M];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[a][m] = 0.0f;
  for (int c = c0; c < c1; ++c) {
    Frag<FMT> fg, fu;
    load_frag<FMT>(fg, wg_ + (tile0 + c) * TILE, lane);
    load_frag<FMT>(fu, wu_ + (tile0 + c) * TILE, lane);
    const uint32_t* xc = x32 + (int64_t)c * (kChunkK / 2);
    if (c < full_chunks) {
      tile_dot<FMT, M, true>(fg, xc, xstride, kPiecesNv, acc[0]);
      tile_dot<FMT, M, true>(fu, xc, xstride, kPiecesNv, acc[1]);
    } else {
      tile_dot<FMT, M, false>(fg, xc, xstride, tail_pieces, acc[0]);
      tile_dot<FMT, M, false>(fu, xc, xstride, tail_pieces, acc[1]);
    }
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int m = 0; m < M; ++m) red[wave][a * M + m][lane] = acc[a][m];
  __syncthreads();
  if (wave != 0) return;
  float v[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) v[i] = ((red[0][i][lane] + red[1][i][lane]) + red[2][i][lane]) + red[3][i][lane];
  const int row = g * 64 + lane;
  if (p.S_up > 1) {
    const int64_t rpad = (int64_t)p.Rg * 64;
    float* base = p.part_up + ((int64_t)s * p.n_slots_max + slot) * NA * rpad;
#pragma unroll
    for (int i = 0; i < NA; ++i) publish_partial(base + i * rpad + row, v[i]);
    unsigned* cnt = p.cnt_up + slot * p.Rg + g;
    if (!arrive_last(cnt, (unsigned)(p.S_up - 1))) return;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      float t = 0.0f;
      for (int q = 0; q < p.S_up; ++q)
        t += collect_partial(p.part_up + (((int64_t)q * p.n_slots_max + slot) * NA + i) * rpad + row);
      v[i] = t;
    }
    reset_counter(cnt);
  }
  if (row >= p.dff) return;
  const int nh = p.K + p.has_shared;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint16_t h = f32_to_bf16_rne(silu_f32(v[m] * tsg) * (v[M + m] * tsu));
    p.hbuf[((int64_t)slot * M + m) * p.dff + row] = h;
    if (p.hdbg) {
      if (e < 0) {
        p.hdbg[((int64_t)m * nh + p.K) * p.dff + row] = h;
      } else {
        for (int j = 0; j < p.K; ++j)
          if (r.ids[m][j] == e) p.hdbg[((int64_t)m * nh + j) * p.dff + row] = h;
      }
    }
  }
}

template <uint32_t FMT, int M>
__global__ __launch_bounds__(kThreads) void k_moe_down(MoeParams p) {
  constexpr int TILE = FMT == FP4G_NVFP4 ? kTileNv : kTileMx;
  __shared__ float red[kWavesPerWg][M][64];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n_slots = uniform(p.route[0]);
  const int per_slot = p.Rd * p.S_dn;
  const int slot = uniform(blockIdx.x / per_slot);
  if (slot >= n_slots) return;
  const int rem = blockIdx.x % per_slot;
  const int g = uniform(rem / p.S_dn), s = uniform(rem % p.S_dn);
  const int e = uniform(p.route[1 + slot]);
  const uint8_t* wd = e >= 0 ? p.down + (uint64_t)e * p.sd : p.sh_down;
  const float tsd = e >= 0 ? p.ts_down : p.ts_sh_down;

  const int wg_c0 = s * p.wg_dn, wg_c1 = min(p.Cd, wg_c0 + p.wg_dn);
  const int per_wave = (wg_c1 - wg_c0 + kWavesPerWg - 1) / kWavesPerWg;
  const int c0 = min(wg_c1, wg_c0 + wave * per_wave), c1 = min(wg_c1, c0 + per_wave);
  const uint32_t* __restrict__ x32 = reinterpret_cast<const uint32_t*>(p.hbuf + (int64_t)slot * M * p.dff);
  const int xstride = p.dff / 2;
  const int full_chunks = p.dff / kChunkK, tail_pieces = (p.dff % kChunkK) / kPieceK;
  const int64_t tile0 = (int64_t)g * p.Cd;

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;
  for (int c = c0; c < c1; ++c) {
    Frag<FMT> f;
    load_frag<FMT>(f, wd + (tile0 + c) * TILE, lane);
    const uint32_t* xc = x32 + (int64_t)c * (kChunkK / 2);
    if (c < full_chunks)
      tile_dot<FMT, M, true>(f, xc, xstride, kPiecesNv, acc);
    else
      tile_dot<FMT, M, false>(f, xc, xstride, tail_pieces, acc);
  }
#pragma unroll
  for (int m = 0; m < M; ++m) red[wave][m][lane] = acc[m];
  __syncthreads();
  if (wave != 0) return;
  const int row = g * 64 + lane;
  const int64_t rpad = (int64_t)p.Rd * 64;
  float* base = p.part_dn + ((int64_t)slot * p.S_dn + s) * M * rpad;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float v = ((red[0][m][lane] + red[1][m][lane]) + red[2][m][lane]) + red[3][m][lane];
    publish_partial(base + m * rpad + row, v * tsd * p.coef[slot * M + m]);
  }
  if (!arrive_last(p.cnt_dn + g, (unsigned)(n_slots * p.S_dn - 1))) return;
  if (row < p.hidden) {
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float t = 0.0f;
      for (int q = 0; q < n_slots * p.S_dn; ++q) t += collect_partial(p.part_dn + ((int64_t)q * M + m) * rpad + row);
      p.y[(int64_t)m * p.hidden + row] = t;
    }
  }
  reset_counter(p.cnt_dn + g);
}

// ---- host side ------------------------------------------------------------------
struct MoeLayout {
  int n_slots_max;
  int64_t Rg, Cg, Rd, Cd;
  Plan up, dn;
  uint64_t off_route, off_coef, off_hbuf, off_cnt_up, off_part_up, off_cnt_dn, off_part_dn, total;
};

MoeLayout moe_layout(const fp4g_moe* mo, int M) {
  MoeLayout L{};
  L.n_slots_max = std::min(mo->num_experts, M * mo->top_k) + (mo->has_shared ? 1 : 0);
  L.Rg = row_groups(mo->d_ff);
  L.Cg = chunks(mo->hidden);
  L.Rd = row_groups(mo->hidden);
  L.Cd = chunks(mo->d_ff);
  L.up = plan_nw4(L.Rg * L.n_slots_max, L.Cg);
  L.dn = plan_nw4(L.Rd * L.n_slots_max, L.Cd);
  // counters first (the fixed region), then tables and partial sums
  L.off_cnt_up = 0;
  L.off_cnt_dn = 4ull * L.n_slots_max * L.Rg;
  uint64_t o = kCounterBytes;
  L.off_route = o;
  o = align256(o + 4ull * (1 + L.n_slots_max));
  L.off_coef = o;
  o = align256(o + 4ull * L.n_slots_max * M);
  L.off_hbuf = o;
  o = align256(o + 2ull * L.n_slots_max * M * mo->d_ff);
  L.off_part_up = o;
  o = align256(o + (L.up.S > 1 ? 4ull * L.up.S * L.n_slots_max * 2 * M * L.Rg * 64 : 0));
  L.off_part_dn = o;
  o = align256(o + 4ull * L.n_slots_max * L.dn.S * M * L.Rd * 64);
  L.total = o;
  return L;
}

fp4g_status check_moe_counters(const fp4g_moe* mo, int M) {
  const int64_t slots = std::min(mo->num_experts, M * mo->top_k) + (mo->has_shared ? 1 : 0);
  return slots * row_groups(mo->d_ff) + row_groups(mo->hidden) <= kMaxCounters ? FP4G_OK : FP4G_E_SHAPE;
}

fp4g_status check_moe(const fp4g_moe* mo) {
  if (!mo) return FP4G_E_NULL;
  if (mo->num_experts < 1 || mo->num_experts > kMaxExperts || mo->top_k < 1 || mo->top_k > kMaxTopK ||
      mo->top_k > mo->num_experts || mo->hidden < 32 || mo->d_ff < 32 || (mo->has_shared != 0 && mo->has_shared != 1))
    return FP4G_E_SHAPE;
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

template <uint32_t FMT>
hipError_t launch_moe(int M, const MoeParams& p, unsigned grid_up, unsigned grid_dn, hipStream_t s) {
  switch (M) {
#define FP4G_CASE(MM)                                           \
  case MM:                                                      \
    k_moe_up<FMT, MM><<<grid_up, kThreads, 0, s>>>(p);          \
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure; \
    k_moe_down<FMT, MM><<<grid_dn, kThreads, 0, s>>>(p);        \
    break;
    FP4G_CASE(1) FP4G_CASE(2) FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
#undef FP4G_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

uint64_t moe_ws_bytes(const fp4g_moe* mo, int M) {
  if (check_moe(mo) != FP4G_OK || M < 1 || M > kMaxM || check_moe_counters(mo, M) != FP4G_OK) return 0;
  return moe_layout(mo, M).total;
}

}  // namespace fp4g

using namespace fp4g;

extern "C" int32_t moe_route_gemv(const fp4g_moe* mo, const uint16_t* X, const float* logits, int32_t M, float* Y,
                                  int32_t* topk_ids, float* topk_w, uint16_t* H, void* ws, uint64_t ws_bytes,
                                  void* stream) {
  fp4g_status st = check_moe(mo);
  if (st != FP4G_OK) return st;
  if (!X || !logits || !Y || !topk_ids || !topk_w || !ws) return FP4G_E_NULL;
  if (M < 1 || M > kMaxM) return FP4G_E_SHAPE;
  if (check_moe_counters(mo, M) != FP4G_OK) return FP4G_E_SHAPE;
  if (!aligned(X, 16) || !aligned(logits, 16) || !aligned(Y, 16) || !aligned(topk_ids, 16) ||
      !aligned(topk_w, 16) || (H && !aligned(H, 16)))
    return FP4G_E_ALIGN;
  const MoeLayout L = moe_layout(mo, M);
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
  MoeParams p{};
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
  p.cnt_up = (unsigned*)(w + L.off_cnt_up);
  p.part_up = (float*)(w + L.off_part_up);
  p.cnt_dn = (unsigned*)(w + L.off_cnt_dn);
  p.part_dn = (float*)(w + L.off_part_dn);
  p.n_slots_max = L.n_slots_max;
  p.Rg = (int)L.Rg;
  p.Cg = (int)L.Cg;
  p.S_up = L.up.S;
  p.wg_up = L.up.wg_chunks;
  p.Rd = (int)L.Rd;
  p.Cd = (int)L.Cd;
  p.S_dn = L.dn.S;
  p.wg_dn = L.dn.wg_chunks;
  const unsigned grid_up = (unsigned)(L.n_slots_max * L.Rg * L.up.S);
  const unsigned grid_dn = (unsigned)(L.n_slots_max * L.Rd * L.dn.S);
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = mo->gate.format == FP4G_NVFP4 ? launch_moe<FP4G_NVFP4>(M, p, grid_up, grid_dn, s)
                                                     : launch_moe<FP4G_MXFP4>(M, p, grid_up, grid_dn, s);
  return e == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}
