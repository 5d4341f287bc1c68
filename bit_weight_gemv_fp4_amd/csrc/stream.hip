// stream.hip -- a whole decode step's chain of products in one launch:
// fp4g_stream_workspace_bytes, fp4g_stream_build, fp4_stream_run,
// fp4g_stream_error.
//
// Decoding one token reads every matrix of the model once, one after another
// (mdjawad.com DGX Spark feed, "Decode speed is bytes divided by bandwidth"), so
// a decode step is a chain of GEMVs whose only dependence is on activations,
// never on weights.  Launched one by one, every product pays a kernel boundary
// (ramp-up, the split-K tail, the compute of the last tiles, the next kernel's
// first-byte latency).  Here the whole chain is one launch:
//
//  * One workgroup per work unit (op, 64-row group, K split), units in op order:
//    the same units, tile loop, split-K exchange tree and epilogues as the
//    separate launches.
//  * A unit first puts its first weight tiles in flight, then waits until the
//    ops it depends on are complete, then stages its input range in LDS and
//    streams on.  Workgroups are dispatched in index order (per XCD), so the
//    units of the next op load their weights while the current op finishes --
//    HBM stays busy across the boundary -- and every wait is for ops whose
//    units were all dispatched earlier.
//  * Completion: the split-K survivor of each (lane, unit) reports it on one of
//    eight 64-bit sub-counters of the op (on separate cache lines) once its
//    output stores are complete; an op is complete when the reports reach
//    epoch x (its lane-units), epoch being the number of runs so far (a
//    one-thread kernel bumps it before each run, so counters never need a reset
//    and graph replays stay correct).
//  * Outputs and inputs that cross workgroups use device-scope stores and loads.
//  * Every wait is bounded: on time-out a sticky error flag is set and the unit
//    carries on (every unit still runs and reports); nothing spins forever.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "gemv_kernel.hpp"

namespace fp4g {
namespace {

constexpr uint32_t kStreamMagic = 0x53344732u;
constexpr int kSpinLimit = 1 << 15;   // polls (about 1-2 us each) before giving up
constexpr int kDoneLanes = 8;         // sub-counters per op
constexpr int kDoneStride = 16;       // u64 between sub-counters (128 B)
constexpr int kStreamXBytes = 32768;  // LDS for a unit's staged input
constexpr int kStreamNW = 4;          // waves per workgroup

enum { SK_GEMV = 0, SK_GATE_UP = 1 };

// One op as the kernel sees it (128 bytes, in the workspace).
struct StreamOp {
  const uint8_t* w0;  // packed matrix (gate for GATE_UP)
  const uint8_t* w1;  // packed up matrix (GATE_UP), else = w0
  const uint16_t* x;  // bf16 [M][d_in]
  void* out;          // f32 [M][d_out] or bf16 [M][d_out]
  const float* rs;    // FP8 row scales, else null
  float ts0, ts1;     // tensor scales
  int32_t fmt, kind, d_out, d_in;
  int32_t R, C, S, wg_chunks;
  int32_t wait_first, wait_op, unit_begin, nu;
  int64_t slot_off;   // exchange-slot words before this op's slots
  int64_t expect;     // lane-units this op's survivors report per run (R * 64 * nu)
  int32_t done_base;  // first of this op's sub-counters
  int32_t pad[3];
};
static_assert(sizeof(StreamOp) == 128, "StreamOp is 128 bytes");

struct StreamHdr {
  uint32_t magic;
  int32_t n_ops, n_units, M;
  int64_t off_ops, off_unit_op, off_done, off_slots;
  int32_t lds_bytes;
  int32_t pad0[19];
  uint64_t epoch;  // offset 128: runs so far
  int32_t pad1[30];
  int32_t err;     // offset 256: sticky error flag
  int32_t pad2[63];
};
static_assert(sizeof(StreamHdr) == 512, "StreamHdr is 512 bytes");

// Pointers read from the op table are generic; accesses through them are cast to
// the global address space so that they are issued as global (not FLAT)
// instructions, which count only in vmcnt.
#define FP4G_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ u32x4 ld_stream_g(const void* p) {
  return __builtin_nontemporal_load((const FP4G_GLOBAL u32x4*)p);
}
__device__ __forceinline__ u32x2 ld_stream2_g(const void* p) {
  return __builtin_nontemporal_load((const FP4G_GLOBAL u32x2*)p);
}
__device__ __forceinline__ uint64_t load_dev_u64(const void* p) {
  return __hip_atomic_load((const FP4G_GLOBAL uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_dev_i32(const int* p) {
  return __hip_atomic_load((const FP4G_GLOBAL int*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev_f32(void* p, float v) {
  __hip_atomic_store((FP4G_GLOBAL float*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev_u16(void* p, uint16_t v) {
  __hip_atomic_store((FP4G_GLOBAL uint16_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t uniform64(uint64_t v) {
  return ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
         __builtin_amdgcn_readfirstlane((uint32_t)v);
}

template <uint32_t FMT>
__device__ __forceinline__ void load_frag_g(Frag<FMT>& f, const uint8_t* tile, int lane) {
  if constexpr (FMT == FP4G_FP8_ROW) {  // a half tile
#pragma unroll
    for (int j = 0; j < kHalfFp8; ++j) f.q[j] = ld_stream_g(tile + j * 1024 + lane * 16);
  } else {
#pragma unroll
    for (int j = 0; j < kPiecesNv; ++j) f.q[j] = ld_stream_g(tile + j * 1024 + lane * 16);
    if constexpr (FMT == FP4G_NVFP4)
      f.s = ld_stream_g(tile + kCodeBytes + lane * 16);
    else
      f.s = ld_stream2_g(tile + kCodeBytes + lane * 8);
  }
}

// Wave 0: wait until ops first..last are complete in this run (bounded).
__device__ void wait_ops(StreamHdr* hdr, const StreamOp* ops, int first, int last, uint64_t epoch, int lane) {
  const uint8_t* done = reinterpret_cast<const uint8_t*>(hdr) + hdr->off_done;
  for (int j = first; j <= last; ++j) {
    const uint64_t target = epoch * (uint64_t)ops[j].expect;
    const int base = ops[j].done_base;
    for (int spins = 0;; ++spins) {
      uint64_t v = lane < kDoneLanes ? load_dev_u64(done + (int64_t)(base + lane) * kDoneStride * 8) : 0ull;
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      v += __shfl_xor(v, 4, 64);
      if (uniform64(v) >= target) break;
      if (spins >= kSpinLimit || load_dev_i32(&hdr->err) != 0) {
        if (lane == 0) __hip_atomic_store(&hdr->err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// One work unit of an op of format FMT (NMAT = 2: the fused gate/up pair).  FP8
// tiles stream as two 8 KiB halves, like in the separate kernel.
template <uint32_t FMT, int M, int NMAT>
__device__ __forceinline__ void run_unit(StreamHdr* hdr, const StreamOp* ops, const StreamOp& op, uint64_t epoch,
                                         float (*red)[2 * M][64], uint8_t* xs) {
  constexpr int NA = NMAT * M;
  constexpr int EPI = NMAT == 2 ? EPI_SILU : EPI_STORE;
  constexpr int TILE = FMT == FP4G_NVFP4 ? kTileNv : FMT == FP4G_MXFP4 ? kTileMx : kTileF8;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int local = uniform((int)blockIdx.x - op.unit_begin);
  const int g = local / op.S, s = local % op.S;
  const int wg_c0 = s * op.wg_chunks, wg_c1 = min(op.C, wg_c0 + op.wg_chunks);
  const int c0 = wg_c0 + (wave * (wg_c1 - wg_c0)) / kStreamNW;
  const int c1 = wg_c0 + ((wave + 1) * (wg_c1 - wg_c0)) / kStreamNW;
  const int64_t tile0 = (int64_t)g * op.C;
  const uint8_t* w0 = op.w0;
  const uint8_t* w1 = op.w1;
  // items: NVFP4/MXFP4 (chunk, matrix) chunk-major; FP8 (chunk, half)
  constexpr bool F8 = FMT == FP4G_FP8_ROW;
  constexpr int PER = F8 ? 2 : NMAT;  // items per chunk
  using FragT = Frag<FMT>;
  const int n_items = (c1 - c0) * PER;
  auto tile_of = [&](int it) {
    if constexpr (F8)
      return w0 + (tile0 + c0 + it / 2) * TILE + (it & 1) * (kHalfFp8 * 1024);
    else
      return (it % NMAT ? w1 : w0) + (tile0 + c0 + it / NMAT) * TILE;
  };
  auto load = [&](FragT& f, int it) { load_frag_g<FMT>(f, tile_of(it), lane); };

  // weights first: they do not depend on the ops this one waits for
  FragT fa, fb;
  if (n_items > 0) load(fa, 0);
  if (op.wait_op >= 0) {
    if (wave == 0) wait_ops(hdr, ops, op.wait_first, op.wait_op, epoch, lane);
    __syncthreads();
  }
  asm volatile("" ::: "memory");

  // the unit's input columns of all M vectors into LDS (device-scope loads, all
  // issued before the first LDS store)
  const int nck = wg_c1 - wg_c0;
  const int tstride = op.wg_chunks * 512;  // bytes per vector in LDS
  {
    constexpr int kMaxPieces = kStreamXBytes / 8 / (kStreamNW * 64);
    const int per_tok = nck * 64;  // 8-byte pieces per vector
    const int pieces = M * per_tok;
    uint64_t v[kMaxPieces];
#pragma unroll
    for (int k = 0; k < kMaxPieces; ++k) {
      const int idx = threadIdx.x + k * kStreamNW * 64;
      const int m = idx / per_tok, r = idx - m * per_tok;
      v[k] = idx < pieces ? load_dev_u64(op.x + (int64_t)m * op.d_in + wg_c0 * kChunkK + r * 4) : 0ull;
    }
#pragma unroll
    for (int k = 0; k < kMaxPieces; ++k) {
      const int idx = threadIdx.x + k * kStreamNW * 64;
      if (idx < pieces) {
        const int m = idx / per_tok, r = idx - m * per_tok;
        *reinterpret_cast<uint64_t*>(xs + m * tstride + r * 8) = v[k];
      }
    }
  }
  __syncthreads();

  float acc[NMAT][M];
#pragma unroll
  for (int a = 0; a < NMAT; ++a)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[a][m] = 0.0f;
  const uint32_t* xl = reinterpret_cast<const uint32_t*>(xs);
  const int xstride = tstride / 4;
  auto eat = [&](const FragT& f, int it) {
    // re-read x from LDS for every item: kept live across the gate and up items
    // of one chunk it would take 128 more VGPRs
    asm volatile("" ::: "memory");
    float part[M];
#pragma unroll
    for (int m = 0; m < M; ++m) part[m] = 0.0f;
    if constexpr (F8) {
      const uint32_t* xc = xl + (c0 + it / 2 - wg_c0) * (kChunkK / 2) + (it & 1) * (kHalfFp8 * 8);
      tile_dot<FMT, M, true>(f, xc, xstride, kHalfFp8, part);
    } else {
      const uint32_t* xc = xl + (c0 + it / NMAT - wg_c0) * (kChunkK / 2);
      tile_dot<FMT, M, true>(f, xc, xstride, kPiecesNv, part);
    }
    if (NMAT == 1 || it % NMAT == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[0][m] += part[m];
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[NMAT - 1][m] += part[m];
    }
  };
  // fa is already in flight; the rest as in the separate kernel
  if (n_items > 0) {
    int it = 0;
    for (; it + 2 < n_items; it += 2) {
      load(fb, it + 1);
      eat(fa, it);
      load(fa, it + 2);
      eat(fb, it + 1);
    }
    if (it + 1 < n_items) {
      load(fb, it + 1);
      eat(fa, it);
      eat(fb, it + 1);
    } else {
      eat(fa, it);
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
  for (int i = 0; i < NA; ++i) {
    float t = red[0][i][lane];
#pragma unroll
    for (int w = 1; w < kStreamNW; ++w) t += red[w][i][lane];
    v[i] = t;
  }
  constexpr int NU = EPI == EPI_SILU ? M : (M + 1) / 2;
  float ua[NU], ub[NU];
  bool live[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if constexpr (EPI == EPI_SILU) {
      ua[u] = v[u];
      ub[u] = v[M + u];
    } else {
      ua[u] = v[2 * u];
      ub[u] = 2 * u + 1 < M ? v[2 * u + 1] : 0.0f;
    }
    live[u] = true;
  }
  unsigned long long* slots =
      reinterpret_cast<unsigned long long*>(reinterpret_cast<uint8_t*>(hdr) + hdr->off_slots) + op.slot_off;
  exchange_tree<NU>(slots, (int64_t)op.R * 64, (int64_t)g * 64 + lane, op.S, s, ua, ub, live);

  const int row = g * 64 + lane;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    if (!live[u]) continue;
    if constexpr (EPI == EPI_SILU) {
      const float gv = ua[u] * op.ts0, uv = ub[u] * op.ts1;
      store_dev_u16(reinterpret_cast<uint16_t*>(op.out) + (int64_t)u * op.d_out + row,
                    f32_to_bf16_rne(silu_f32(gv) * uv));
    } else {
      const float sc = FMT == FP4G_FP8_ROW ? *(const FP4G_GLOBAL float*)(op.rs + row) : op.ts0;
      float* y = reinterpret_cast<float*>(op.out);
      store_dev_f32(y + (int64_t)(2 * u) * op.d_out + row, ua[u] * sc);
      if (2 * u + 1 < M) store_dev_f32(y + (int64_t)(2 * u + 1) * op.d_out + row, ub[u] * sc);
    }
  }
  // each (lane, unit) survives in exactly one workgroup: report the ones that
  // survived here once the stores above are complete
  int reports = 0;
#pragma unroll
  for (int u = 0; u < NU; ++u) reports += __builtin_popcountll(__ballot(live[u]));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0 && reports > 0) {
    uint8_t* done = reinterpret_cast<uint8_t*>(hdr) + hdr->off_done;
    uint64_t* c = reinterpret_cast<uint64_t*>(done) + (int64_t)(op.done_base + blockIdx.x % kDoneLanes) * kDoneStride;
    __hip_atomic_fetch_add(c, (uint64_t)reports, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int M>
__global__ __launch_bounds__(kStreamNW * 64) void k_stream(StreamHdr* hdr) {
  __shared__ float red[kStreamNW][2 * M][64];
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  const uint16_t* unit_op =
      reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(hdr) + hdr->off_unit_op);
  const StreamOp* ops = reinterpret_cast<const StreamOp*>(reinterpret_cast<const uint8_t*>(hdr) + hdr->off_ops);
  const int oi = uniform((int)unit_op[blockIdx.x]);
  const StreamOp& op = ops[oi];
  const uint64_t epoch = op.wait_op >= 0 ? uniform64(load_dev_u64(&hdr->epoch)) : 0ull;
  if (op.fmt == FP4G_NVFP4) {
    if (op.kind == SK_GATE_UP)
      run_unit<FP4G_NVFP4, M, 2>(hdr, ops, op, epoch, red, xs);
    else
      run_unit<FP4G_NVFP4, M, 1>(hdr, ops, op, epoch, red, xs);
  } else if (op.fmt == FP4G_MXFP4) {
    if (op.kind == SK_GATE_UP)
      run_unit<FP4G_MXFP4, M, 2>(hdr, ops, op, epoch, red, xs);
    else
      run_unit<FP4G_MXFP4, M, 1>(hdr, ops, op, epoch, red, xs);
  } else {
    run_unit<FP4G_FP8_ROW, M, 1>(hdr, ops, op, epoch, red, xs);
  }
}

// Runs so far: bumped once before each run (the same stream orders it).
__global__ void k_stream_epoch(StreamHdr* hdr) {
  if (threadIdx.x == 0) __hip_atomic_fetch_add(&hdr->epoch, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- host side ----------------------------------------------------------------------
// Splits of an op: the dense planner's cost for four-wave workgroups (a launch
// has one workgroup size), never more chunks per unit than the LDS staging of x
// holds at this M.
Plan plan_stream(int64_t R, int64_t C, int nmat, int M) {
  const int waves_per_cu = (nmat == 1 ? M <= 5 : M <= 3) ? 16 : 12;
  const int64_t max_chunks = kStreamXBytes / (M * 512);
  Plan best{(int)C, 1, kStreamNW};
  double best_cost = 1e30;
  for (int64_t S0 = 1; S0 <= C; ++S0) {
    const int64_t wg_chunks = (C + S0 - 1) / S0;
    const int64_t S = (C + wg_chunks - 1) / wg_chunks;
    if (S != S0 || wg_chunks > max_chunks) continue;
    if (4 * wg_chunks < 3 * kStreamNW) break;  // more than a quarter of the waves idle
    const int64_t wgs = R * S, waves = wgs * kStreamNW;
    const double imbalance = (double)((wgs + kCUs - 1) / kCUs) * kCUs / (double)wgs;
    const double rounds = (double)waves / ((double)kCUs * waves_per_cu);
    const double cost =
        imbalance * (1.0 + 0.03 * tree_depth(S)) * (1.0 + 0.15 * (rounds > 1.0 ? rounds - 1.0 : 0.0));
    if (cost < best_cost - 1e-9) {
      best = Plan{(int)S, (int)wg_chunks, kStreamNW};
      best_cost = cost;
    }
  }
  if (best_cost > 1e29) {  // short rows: as few splits as the LDS allows
    const int64_t wg_chunks = std::min<int64_t>(C, max_chunks);
    best = Plan{(int)((C + wg_chunks - 1) / wg_chunks), (int)wg_chunks, kStreamNW};
  }
  return best;
}

struct StreamLayout {
  uint64_t off_ops, off_unit_op, off_done, off_slots, total;
  int64_t n_units, slot_words;
  int lds_bytes;
};

fp4g_status layout_stream(const fp4g_stream_op* ops, int n, int M, StreamLayout& L, StreamOp* table) {
  if (!ops) return FP4G_E_NULL;
  if (n < 1 || n > 65535 || M < 1 || M > kMaxM) return FP4G_E_SHAPE;
  int64_t units = 0, slot_words = 0;
  int lds = 0;
  for (int i = 0; i < n; ++i) {
    const fp4g_stream_op& o = ops[i];
    if (!o.w || !o.x_dev || !o.out_dev) return FP4G_E_NULL;
    const bool gu = o.kind == FP4G_OP_GATE_UP;
    if (o.kind != FP4G_OP_GEMV && !gu && o.kind != FP4G_OP_LMHEAD) return FP4G_E_FORMAT;
    fp4g_status st = check_weight(o.w, o.kind != FP4G_OP_LMHEAD);
    if (st != FP4G_OK) return st;
    if (gu) {
      if (!o.w_up) return FP4G_E_NULL;
      st = check_weight(o.w_up, true);
      if (st != FP4G_OK) return st;
      if (o.w_up->format != o.w->format) return FP4G_E_FORMAT;
      if (o.w_up->d_out != o.w->d_out || o.w_up->d_in != o.w->d_in) return FP4G_E_SHAPE;
    }
    if (o.w->d_out % 64 || o.w->d_in % kChunkK) return FP4G_E_SHAPE;
    if (o.wait_op < -1 || o.wait_op >= i) return FP4G_E_SHAPE;
    const int wcount = o.wait_count < 1 ? 1 : o.wait_count;
    if (o.wait_op >= 0 && o.wait_op - wcount + 1 < 0) return FP4G_E_SHAPE;
    if (!aligned(o.x_dev, 16) || !aligned(o.out_dev, 256)) return FP4G_E_ALIGN;
    const int64_t R = row_groups(o.w->d_out), C = chunks(o.w->d_in);
    const int nmat = gu ? 2 : 1;
    const Plan pl = plan_stream(R, C, nmat, M);
    const int nu = gu ? M : (M + 1) / 2;
    lds = std::max(lds, M * pl.wg_chunks * 512);
    if (table) {
      StreamOp& t = table[i];
      memset(&t, 0, sizeof t);
      t.w0 = (const uint8_t*)o.w->packed;
      t.w1 = gu ? (const uint8_t*)o.w_up->packed : t.w0;
      t.x = o.x_dev;
      t.out = o.out_dev;
      t.rs = o.w->format == FP4G_FP8_ROW ? (const float*)((const uint8_t*)o.w->packed + R * C * kTileF8) : nullptr;
      t.ts0 = o.w->tensor_scale;
      t.ts1 = gu ? o.w_up->tensor_scale : 1.0f;
      t.fmt = (int32_t)o.w->format;
      t.kind = gu ? SK_GATE_UP : SK_GEMV;
      t.d_out = o.w->d_out;
      t.d_in = o.w->d_in;
      t.R = (int32_t)R;
      t.C = (int32_t)C;
      t.S = pl.S;
      t.wg_chunks = pl.wg_chunks;
      t.wait_op = o.wait_op;
      t.wait_first = o.wait_op >= 0 ? o.wait_op - wcount + 1 : -1;
      t.unit_begin = (int32_t)units;
      t.nu = nu;
      t.slot_off = slot_words;
      t.expect = R * 64 * nu;
      t.done_base = i * kDoneLanes;
    }
    units += R * pl.S;
    slot_words += tree_nodes(pl.S) * nu * R * 64;
    if (units > (int64_t)1 << 30) return FP4G_E_SHAPE;
  }
  L.n_units = units;
  L.slot_words = slot_words;
  L.lds_bytes = lds;
  uint64_t o = sizeof(StreamHdr);
  L.off_ops = o;
  o = align256(o + (uint64_t)n * sizeof(StreamOp));
  L.off_unit_op = o;
  o = align256(o + 2ull * units);
  L.off_done = o;
  o = align256(o + 8ull * n * kDoneLanes * kDoneStride);
  L.off_slots = o;
  o = align256(o + 8ull * slot_words);
  L.total = o;
  return FP4G_OK;
}

// Aliasing rules of a stream: outputs are disjoint from each other and from all
// weights; an op's input overlaps no output except those of the ops it waits for.
fp4g_status check_stream_aliases(const fp4g_stream_op* ops, int n, int M) {
  auto out_bytes = [&](const fp4g_stream_op& o) {
    return (size_t)M * o.w->d_out * (o.kind == FP4G_OP_GATE_UP ? 2 : 4);
  };
  for (int i = 0; i < n; ++i) {
    const size_t ob = out_bytes(ops[i]);
    for (int j = 0; j < n; ++j) {
      const fp4g_stream_op& b = ops[j];
      if (j != i && overlap(ops[i].out_dev, ob, b.out_dev, out_bytes(b))) return FP4G_E_ALIAS;
      if (overlap(ops[i].out_dev, ob, b.w->packed, b.w->packed_bytes)) return FP4G_E_ALIAS;
      if (b.w_up && overlap(ops[i].out_dev, ob, b.w_up->packed, b.w_up->packed_bytes)) return FP4G_E_ALIAS;
      const size_t xb = (size_t)M * b.w->d_in * 2;
      const int wc = b.wait_count < 1 ? 1 : b.wait_count;
      const bool waited_for = b.wait_op >= 0 && i <= b.wait_op && i > b.wait_op - wc;
      if (overlap(ops[i].out_dev, ob, b.x_dev, xb) && !waited_for) return FP4G_E_ALIAS;
    }
  }
  return FP4G_OK;
}

}  // namespace
}  // namespace fp4g

using namespace fp4g;

extern "C" {

uint64_t fp4g_stream_workspace_bytes(const fp4g_stream_op* ops, int32_t n_ops, int32_t M) {
  StreamLayout L{};
  if (layout_stream(ops, n_ops, M, L, nullptr) != FP4G_OK) return 0;
  return L.total;
}

int32_t fp4g_stream_build(const fp4g_stream_op* ops, int32_t n_ops, int32_t M, void* ws, uint64_t ws_bytes,
                          fp4g_stream_plan* plan, void* stream) {
  if (!ws || !plan) return FP4G_E_NULL;
  StreamLayout L{};
  fp4g_status st = layout_stream(ops, n_ops, M, L, nullptr);
  if (st != FP4G_OK) return st;
  if (ws_bytes < L.total) return FP4G_E_WORKSPACE;
  if (!aligned(ws, 256)) return FP4G_E_ALIGN;
  st = check_stream_aliases(ops, n_ops, M);
  if (st != FP4G_OK) return st;
  for (int i = 0; i < n_ops; ++i) {
    const size_t ob = (size_t)M * ops[i].w->d_out * (ops[i].kind == FP4G_OP_GATE_UP ? 2 : 4);
    if (overlap(ws, L.total, ops[i].out_dev, ob) ||
        overlap(ws, L.total, ops[i].x_dev, (size_t)M * ops[i].w->d_in * 2) ||
        overlap(ws, L.total, ops[i].w->packed, ops[i].w->packed_bytes))
      return FP4G_E_ALIAS;
  }
  // host image of header, op table and unit table; counters and slots zeroed
  const size_t img = L.off_done;
  uint8_t* h = (uint8_t*)calloc(1, img);
  if (!h) return FP4G_E_HIP;
  StreamHdr* hdr = (StreamHdr*)h;
  hdr->magic = kStreamMagic;
  hdr->n_ops = n_ops;
  hdr->n_units = (int32_t)L.n_units;
  hdr->M = M;
  hdr->off_ops = (int64_t)L.off_ops;
  hdr->off_unit_op = (int64_t)L.off_unit_op;
  hdr->off_done = (int64_t)L.off_done;
  hdr->off_slots = (int64_t)L.off_slots;
  hdr->lds_bytes = L.lds_bytes;
  StreamOp* table = (StreamOp*)(h + L.off_ops);
  layout_stream(ops, n_ops, M, L, table);
  uint16_t* uop = (uint16_t*)(h + L.off_unit_op);
  for (int i = 0; i < n_ops; ++i)
    for (int64_t u = 0; u < (int64_t)table[i].R * table[i].S; ++u) uop[table[i].unit_begin + u] = (uint16_t)i;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(ws, h, img, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemsetAsync((uint8_t*)ws + L.off_done, 0, L.total - L.off_done, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  free(h);
  if (e != hipSuccess) return FP4G_E_HIP;
  plan->magic = kStreamMagic;
  plan->M = M;
  plan->n_ops = n_ops;
  plan->n_items = (int32_t)L.n_units;
  plan->grid = (int32_t)L.n_units;
  plan->reserved = L.lds_bytes;
  plan->ws = ws;
  plan->ws_bytes = L.total;
  return FP4G_OK;
}

int32_t fp4_stream_run(const fp4g_stream_plan* plan, void* stream) {
  if (!plan || !plan->ws) return FP4G_E_NULL;
  if (plan->magic != kStreamMagic) return FP4G_E_FORMAT;
  if (plan->M < 1 || plan->M > kMaxM || plan->grid < 1 || plan->reserved < 0 || plan->reserved > kStreamXBytes)
    return FP4G_E_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  StreamHdr* hdr = (StreamHdr*)plan->ws;
  k_stream_epoch<<<1, 64, 0, s>>>(hdr);
  if (hipGetLastError() != hipSuccess) return FP4G_E_HIP;
  const size_t lds = (size_t)plan->reserved;
  switch (plan->M) {
#define FP4G_CASE(MM) \
  case MM:            \
    k_stream<MM><<<plan->grid, kStreamNW * 64, lds, s>>>(hdr); \
    break;
    FP4G_CASE(1) FP4G_CASE(2) FP4G_CASE(3) FP4G_CASE(4) FP4G_CASE(5) FP4G_CASE(6) FP4G_CASE(7) FP4G_CASE(8)
#undef FP4G_CASE
    default: return FP4G_E_SHAPE;
  }
  return hipGetLastError() == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}

int32_t fp4g_stream_error(const fp4g_stream_plan* plan, int32_t* err_host, void* stream) {
  if (!plan || !plan->ws || !err_host) return FP4G_E_NULL;
  if (plan->magic != kStreamMagic) return FP4G_E_FORMAT;
  hipStream_t s = (hipStream_t)stream;
  int32_t* err = &((StreamHdr*)plan->ws)->err;
  int32_t zero = 0;
  hipError_t e = hipMemcpyAsync(err_host, err, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess && *err_host != 0) e = hipMemcpy(err, &zero, 4, hipMemcpyHostToDevice);
  return e == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}

}  // extern "C"
