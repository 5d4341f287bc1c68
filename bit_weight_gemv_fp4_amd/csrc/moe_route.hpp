// moe_route.hpp -- routing of decode tokens to their experts (the Ling-3.0 MoE
// decode article, sec. 3: each token takes the top-k of its router logits,
// weighted by a softmax over the k picked; sec. 8: M tokens read the union of
// their picks).  Shared by the MoE kernels (moe.hip) and by the matrix-core
// gate/up (gemv_mfma.hpp), which routes for itself at small M.
#pragma once
#include "common.hpp"

namespace fp4g {

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
  float* coef;           // [n_slots_max][M]: gate weight x down tensor scale
  uint16_t* hbuf;        // bf16 [n_slots_max][M][dff]
  unsigned long long* x_up;  // exchange slots of the gate/up splits (zero between calls)
  unsigned long long* x_dn;  // exchange slots of the down splits (zero between calls)
  int n_slots_max;
  int Rg, Cg, S_up, wg_up;  // gate/up: d_ff rows, hidden columns
  int Rd, Cd, S_dn;         // down: hidden rows, d_ff columns; S_dn shares of the tiles
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

// Compare-exchange for a descending order of 64-bit pick keys.
__device__ __forceinline__ void cas_desc(uint64_t& a, uint64_t& b) {
  const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
  a = hi;
  b = lo;
}

// The K picks of token m from its logits, one wave, E <= 512: each lane holds
// the pick keys of experts lane + 64 t (t < 8), sorted descending by a 19-
// comparator network, so the lane's best remaining key is always key[0].  A
// pick is the 64-bit wave maximum of the lanes' heads (DPP; keys are distinct,
// equal logits ordered by the lower expert index), and the lane holding it
// drops its head.  The loop has no branch: the shift is by selects, and lane j
// keeps pick j and writes it afterwards.  (A 32-bit maximum of the high words
// with a ballot for ties took 17% longer: the scalar round trips cost more
// than the second word saves.)
template <int M>
__device__ __forceinline__ void pick_sorted(const MoeParams& p, RouteLds<M>& r, int m, int lane, int npick,
                                            float& myv, float& v0) {
  const float* lg = p.logits + (int64_t)m * p.E;
  uint64_t k[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int e = lane + 64 * t;
    k[t] = e < p.E ? pick_key(lg[e], e) : 0ull;
  }
  cas_desc(k[0], k[2]); cas_desc(k[1], k[3]); cas_desc(k[4], k[6]); cas_desc(k[5], k[7]);
  cas_desc(k[0], k[4]); cas_desc(k[1], k[5]); cas_desc(k[2], k[6]); cas_desc(k[3], k[7]);
  cas_desc(k[0], k[1]); cas_desc(k[2], k[3]); cas_desc(k[4], k[5]); cas_desc(k[6], k[7]);
  cas_desc(k[2], k[4]); cas_desc(k[3], k[5]);
  cas_desc(k[1], k[4]); cas_desc(k[3], k[6]);
  cas_desc(k[1], k[2]); cas_desc(k[3], k[4]); cas_desc(k[5], k[6]);
  uint64_t mine = 0ull, first = 0ull;
  for (int j = 0; j < npick; ++j) {
    const uint64_t best = wave_max_key(k[0]);
    const bool won = k[0] == best;
#pragma unroll
    for (int t = 0; t < 7; ++t) k[t] = won ? k[t + 1] : k[t];
    k[7] = won ? 0ull : k[7];
    mine = lane == j ? best : mine;
    first = j == 0 ? best : first;
  }
  v0 = key_value(first);  // picks come in descending order
  if (lane < npick) {
    const float bv = key_value(mine);
    myv = bv;
    r.ids[m][lane] = key_index(mine);
    r.v[m][lane] = bv;
  }
}

// The same for up to 1024 experts (16 keys per lane): each pick takes the lane
// maximum over its keys, then the wave maximum, and clears the picked key.
template <int M>
__device__ __forceinline__ void pick_scan(const MoeParams& p, RouteLds<M>& r, int m, int lane, int npick,
                                          float& myv, float& v0) {
  const float* lg = p.logits + (int64_t)m * p.E;
  constexpr int kPer = kMaxExperts / 64;
  const int per_lane = (p.E + 63) / 64;
  uint64_t key[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int e = lane + 64 * t;
    key[t] = (t < per_lane && e < p.E) ? pick_key(lg[e], e) : 0ull;
  }
  for (int j = 0; j < npick; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int t = 1; t < kPer; ++t) best = key[t] > best ? key[t] : best;
    best = wave_max_key(best);
#pragma unroll
    for (int t = 0; t < kPer; ++t) key[t] = key[t] == best ? 0ull : key[t];
    const float bv = key_value(best);
    if (j == 0) v0 = bv;
    if (lane == j) myv = bv;
    if (lane == 0) {
      r.ids[m][j] = key_index(best);
      r.v[m][j] = bv;
    }
  }
}

// All NW * 64 threads: route the M tokens into `r` (ids, weights, sorted union).
// One wave per token picks and takes the softmax over its K picks; the union of
// the M x K picks, in ascending expert id, is ranked lane-parallel for one or
// two tokens (each pick's rank among the distinct smaller ids: two loops over
// the picks), else counted through a bitmap in LDS.
template <int M, int NW>
__device__ void route_tokens(const MoeParams& p, RouteLds<M>& r) {
  constexpr bool kByRank = M <= 2;  // measured: the rank loops cost ~45 ns per pick, the bitmap ~1 us in all
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int words = (p.E + 31) / 32;
  if constexpr (!kByRank)
    for (int i = threadIdx.x; i < words; i += NW * 64) r.bits[i] = 0u;
  for (int m = wave; m < M; m += NW) {
    float myv = 0.0f, v0 = 0.0f;  // lane j < K: the logit of pick j; the largest
    if (p.E <= 512)
      pick_sorted<M>(p, r, m, lane, p.K, myv, v0);
    else
      pick_scan<M>(p, r, m, lane, p.K, myv, v0);
    // softmax over the K picks, one pick per lane (lanes 0..7; K <= 8): the sum of
    // the exponentials by three DPP steps into lane 7
    const float ej = lane < p.K ? expf(myv - v0) : 0.0f;
    const float z = wave_sum8(ej);
    if (lane < p.K) r.w[m][lane] = ej / z;
  }
  __syncthreads();
  if constexpr (kByRank) {
    if (wave == 0) {
      const int n = M * p.K;
      const int id = lane < n ? r.ids[lane / p.K][lane % p.K] : 0x7fffffff;
      // the first pick of its expert (for M = 1 the picks are distinct already;
      // checked anyway, so that every slot below n_slots is written whatever
      // the picks hold)
      bool first = lane < n;
      for (int i = 0; i < n; ++i) {
        const int o = __builtin_amdgcn_readlane(id, i);
        first = first && !(i < lane && o == id);
      }
      const uint64_t fm = __ballot(first);
      int rank = 0;
      for (int i = 0; i < n; ++i) {
        const int o = __builtin_amdgcn_readlane(id, i);
        rank += (((fm >> i) & 1ull) != 0 && o < id) ? 1 : 0;
      }
      if (first) r.uni[rank] = id;
      const int nd = __popcll(fm);
      if (lane == 0) {
        if (p.has_shared) r.uni[nd] = -1;
        r.n_slots = nd + (p.has_shared ? 1 : 0);
      }
    }
  } else {
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
  }
  __syncthreads();
}

// One token's routing in pick order (k_moe_up at M = 1): slot j is the j-th
// pick (largest logit first), slot K the shared expert, so a gate/up unit of
// slot j needs only the first j + 1 picks and the shared slot none.  Wave 0
// makes `npick` picks; with `weights` (npick = K) it also takes the softmax.
template <int M>
__device__ void route_by_pick(const MoeParams& p, RouteLds<M>& r, int npick, bool weights) {
  const int lane = threadIdx.x & 63;
  if (wave_id() == 0 && npick > 0) {
    float myv = 0.0f, v0 = 0.0f;
    if (p.E <= 512)
      pick_sorted<M>(p, r, 0, lane, npick, myv, v0);
    else
      pick_scan<M>(p, r, 0, lane, npick, myv, v0);
    if (weights) {
      const float ej = lane < p.K ? expf(myv - v0) : 0.0f;
      const float z = wave_sum8(ej);
      if (lane < p.K) r.w[0][lane] = ej / z;
    }
    if (lane < npick) r.uni[lane] = r.ids[0][lane];
  }
  if (threadIdx.x == 0) {
    if (p.has_shared) r.uni[p.K] = -1;
    r.n_slots = p.K + (p.has_shared ? 1 : 0);
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

// The routing outputs and tables: top-k ids and weights, the slots' experts and
// their per-token coefficients (gate weight x down tensor scale), slot count.
template <int M, int NW>
__device__ void write_route_tables(const MoeParams& p, const RouteLds<M>& r) {
  for (int i = threadIdx.x; i < M * p.K; i += NW * 64) {
    const int m = i / p.K, j = i % p.K;
    p.topk_ids[i] = r.ids[m][j];
    p.topk_w[i] = r.w[m][j];
  }
  for (int i = threadIdx.x; i < r.n_slots; i += NW * 64) p.route[1 + i] = r.uni[i];
  for (int t = threadIdx.x; t < r.n_slots * M; t += NW * 64) {  // one (slot, token) per thread
    const int i = t / M, m = t - i * M;
    const float tsd = r.uni[i] >= 0 ? p.ts_down : p.ts_sh_down;
    p.coef[t] = coef_of<M>(r, p, i, m) * tsd;
  }
  if (threadIdx.x == 0) p.route[0] = r.n_slots;
}

}  // namespace fp4g
