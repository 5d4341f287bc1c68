// stream.hip -- a whole decode step's chain of products in one persistent launch:
// fp4g_stream_workspace_bytes, fp4g_stream_build, fp4_stream_run,
// fp4g_stream_error.
//
// Decoding one token reads every matrix of the model once, one after another
// (mdjawad.com DGX Spark feed, "Decode speed is bytes divided by bandwidth"), so
// a decode step is a chain of GEMVs whose only dependence is on activations,
// never on weights.  Launching each product separately leaves HBM idle at every
// boundary (kernel ramp-up, the split-K tail and the next kernel's first-byte
// latency: about 5 us per matrix here).  This kernel keeps HBM busy across the
// boundaries:
//
//  * Work items are (op, 64-row group, K range) in op order; wave w of a grid of
//    G takes items w, w+G, w+2G, ...  An item only waits for items of earlier
//    ops, which every wave reaches first, so the chain progresses as long as the
//    grid is resident at once; the grid is sized from the kernel's occupancy.
//    (A global ticket would serialise: same-address device atomics cost about
//    11 ns each on this GPU.)
//  * Every wave streams a flat sequence of weight tiles across its items and
//    always has the next tile in flight, including the first tile of its next
//    item before that item's input vector is ready (weights do not depend on
//    activations).
//  * An op's input is read only after every row group of the op it waits on has
//    been finalised (device-scope done counters, eight per op on separate cache
//    lines so that finalisers do not queue on one address); outputs and partials
//    are written with device-scope stores.  Each buffer is written once per
//    launch and first read after it was written, so no cache holds a stale copy.
//  * Every wait is bounded: on time-out a sticky error flag is set and all waves
//    drain out; nothing can spin forever.
#include <algorithm>
#include <cstdlib>
#include <cstring>

#include "gemv_kernel.hpp"

namespace fp4g {
namespace {

constexpr uint32_t kStreamMagic = 0x53344731u;
constexpr int kSpinLimit = 1 << 20;  // polls of about 1 us each before giving up
constexpr int kDoneLanes = 8;        // sub-counters per op
constexpr int kDoneStride = 32;      // u32 between sub-counters (128 B)

enum { SK_GEMV = 0, SK_GATE_UP = 1 };

// One op as the kernel sees it (128 bytes, in the workspace).
struct StreamOp {
  const uint8_t* w0;    // packed matrix (gate for GATE_UP)
  const uint8_t* w1;    // packed up matrix (GATE_UP), else = w0
  const uint16_t* x;    // bf16 [M][d_in]
  void* out;            // f32 [M][d_out] or bf16 [M][d_out]
  const float* rs;      // FP8 row scales, else null
  float ts0, ts1;       // tensor scales
  int32_t fmt, kind, d_out, d_in;
  int32_t R, C, S, Q;   // row groups, chunks, splits, chunks per item
  int32_t wait_op;      // -1 or an earlier op
  int32_t item_begin, n_items, nmat;
  int32_t cnt_base;     // first arrival counter of this op
  int32_t halves;       // steps per chunk and matrix: 2 for FP8 (8 KiB halves), else 1
  int64_t part_off;     // float offset of this op's partial sums [S][nmat][M][R*64]
  int32_t wait_first;   // first op waited for (wait_first .. wait_op)
  int32_t pad[3];
};
static_assert(sizeof(StreamOp) == 128, "StreamOp is 128 bytes");

struct StreamHdr {
  uint32_t magic;
  int32_t n_ops, n_items, M, grid, total_cnt;
  int64_t off_ops, off_done, off_cnt, off_part;
  int32_t pad0[18];
  uint32_t unused;      // offset 128
  int32_t pad1[31];
  uint32_t exit_count;  // offset 256: waves that finished
  int32_t pad2[31];
  int32_t err;          // offset 384: sticky error flag
  int32_t pad3[31];
};
static_assert(sizeof(StreamHdr) == 512, "StreamHdr is 512 bytes");

typedef unsigned u32x8 __attribute__((ext_vector_type(8)));

// Scalar loads of read-only-after-ready data (the op table, an op's input once its
// producer is done).  Issued in program order with respect to every other
// memory access of the wave.
__device__ __forceinline__ const void* uptr(const void* p) {
  const uint64_t u = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ u32x8 sload8(const void* p) {
  u32x8 v;
  const void* q = uptr(p);
  asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(q) : "memory");
  return v;
}

// Pointers read from the op table are generic; accesses through them are cast to
// the global address space so that they are issued as global (not FLAT)
// instructions, which count only in vmcnt and leave scalar-load waits alone.
#define FP4G_GLOBAL __attribute__((address_space(1)))
__device__ __forceinline__ u32x4 ld_stream_g(const void* p) {
  return __builtin_nontemporal_load((const FP4G_GLOBAL u32x4*)p);
}
__device__ __forceinline__ void store_dev_f32(void* p, float v) {
  __hip_atomic_store((FP4G_GLOBAL float*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev_u32(void* p, uint32_t v) {
  __hip_atomic_store((FP4G_GLOBAL uint32_t*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_f32_g(const float* p) { return *(const FP4G_GLOBAL float*)p; }

__device__ __forceinline__ unsigned atomic_load_dev(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int atomic_load_dev(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A step: one 8 KiB slab of codes (a whole NVFP4/MXFP4 tile, or half an FP8
// tile) plus its scales.  Always nine 16-byte loads per lane, whatever the
// format, so that the wait counts of the pipeline are the same on every path.
struct StepFrag {
  u32x4 q[8];
  u32x4 s;
};

struct StepDesc {
  int op;        // -1: no step (end of the stream)
  int fmt;
  int g, s;      // row group, split
  int c;         // chunk
  int mat;       // 0 or 1 (up)
  int half;      // FP8 half tile
  int first, last;
  const uint8_t* slab;  // 8 KiB of codes for this step (tile + half * 8192)
  const uint8_t* tile;  // the tile (scales live at tile + 8192)
};

__device__ __forceinline__ void load_step(StepFrag& f, const StepDesc& d, int lane) {
  const int fmt = d.fmt;
#pragma unroll
  for (int j = 0; j < 8; ++j) f.q[j] = ld_stream_g(d.slab + j * 1024 + lane * 16);
  // ninth load: NVFP4 16 B of E4M3 scales; MXFP4 the 16-byte pair holding this
  // lane's 8 E8M0 scales; FP8 a repeat of the first slice (no scales in tiles)
  const uint8_t* sp = fmt == FP4G_NVFP4 ? d.tile + kCodeBytes + lane * 16
                      : fmt == FP4G_MXFP4 ? d.tile + kCodeBytes + (lane & ~1) * 8
                                          : d.slab + lane * 16;
  f.s = ld_stream_g(sp);
}

// acc[m] += the step's dot products, for one format known at compile time.
// xb: the bf16 pairs of column 256c of token 0 in LDS (the same address in every
// lane: broadcast reads); token stride xs u32.
template <uint32_t FMT, int M>
__device__ __forceinline__ void step_dot_fmt(const StepFrag& f, int half, int lane, const uint32_t* xb, int xs,
                                             float (&acc)[M]) {
  if constexpr (FMT == FP4G_FP8_ROW) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16x2 w[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        w[2 * d] = e4m3x2_bf16<false>(f.q[j][d]);
        w[2 * d + 1] = e4m3x2_bf16<true>(f.q[j][d]);
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x8 xv = *reinterpret_cast<const u32x8*>(xb + m * xs + half * 64 + j * 8);
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          p0 = dot2(w[i], xv[i], p0);
          p1 = dot2(w[i + 1], xv[i + 1], p1);
        }
        acc[m] += p0 + p1;
      }
    }
  } else {
    // MXFP4: this lane's 8 scale bytes are the low or high half of the 16 loaded
    const uint32_t mx_lo = (lane & 1) ? f.s[2] : f.s[0];
    const uint32_t mx_hi = (lane & 1) ? f.s[3] : f.s[1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16x2 w[16];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        w[4 * d + 0] = e2m1x2_bf16<0>(f.q[j][d]);
        w[4 * d + 1] = e2m1x2_bf16<1>(f.q[j][d]);
        w[4 * d + 2] = e2m1x2_bf16<2>(f.q[j][d]);
        w[4 * d + 3] = e2m1x2_bf16<3>(f.q[j][d]);
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x8 xa = *reinterpret_cast<const u32x8*>(xb + m * xs + j * 16);
        const u32x8 xc = *reinterpret_cast<const u32x8*>(xb + m * xs + j * 16 + 8);
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p0 = dot2(w[i], xa[i], p0);
          p1 = dot2(w[8 + i], xc[i], p1);
        }
        if constexpr (FMT == FP4G_NVFP4) {
          const uint32_t sdw = f.s[j >> 1];
          const float s0 = (j & 1) ? e4m3_f32<2>(sdw) : e4m3_f32<0>(sdw);
          const float s1 = (j & 1) ? e4m3_f32<3>(sdw) : e4m3_f32<1>(sdw);
          acc[m] = __builtin_fmaf(p0, s0, acc[m]);
          acc[m] = __builtin_fmaf(p1, s1, acc[m]);
        } else {
          const uint32_t sdw = (j < 4) ? mx_lo : mx_hi;
          const int e = (int)((sdw >> (8 * (j & 3))) & 0xffu);
          acc[m] += __builtin_amdgcn_ldexpf(p0 + p1, e - 127);
        }
      }
    }
  }
}

template <int M>
__device__ __forceinline__ void step_dot(const StepFrag& f, int fmt, int half, int lane, const uint32_t* xb, int xs,
                                         float (&acc)[M]) {
  if (fmt == FP4G_NVFP4)
    step_dot_fmt<FP4G_NVFP4, M>(f, half, lane, xb, xs, acc);
  else if (fmt == FP4G_MXFP4)
    step_dot_fmt<FP4G_MXFP4, M>(f, half, lane, xb, xs, acc);
  else
    step_dot_fmt<FP4G_FP8_ROW, M>(f, half, lane, xb, xs, acc);
}

// The fields of one op, loaded with scalar loads (never vector loads: those
// would wait behind the prefetched weight tile).
struct OpView {
  const uint8_t *w0, *w1;
  const uint16_t* x;
  void* out;
  const float* rs;
  float ts0, ts1;
  int fmt, kind, d_out, d_in, R, C, S, Q, wait_op, item_begin, n_items, nmat, cnt_base, halves;
  int64_t part_off;
  int wait_first;
};

__device__ __forceinline__ OpView load_op(const StreamOp* ops, int i) {
  const uint8_t* o = reinterpret_cast<const uint8_t*>(uptr(ops + i));
  const u32x8 a = sload8(o);
  const u32x8 b = sload8(o + 32);
  const u32x8 c = sload8(o + 64);
  const u32x8 d = sload8(o + 96);
  OpView v;
  v.w0 = (const uint8_t*)(((uint64_t)a[1] << 32) | a[0]);
  v.w1 = (const uint8_t*)(((uint64_t)a[3] << 32) | a[2]);
  v.x = (const uint16_t*)(((uint64_t)a[5] << 32) | a[4]);
  v.out = (void*)(((uint64_t)a[7] << 32) | a[6]);
  v.rs = (const float*)(((uint64_t)b[1] << 32) | b[0]);
  v.ts0 = __uint_as_float(b[2]);
  v.ts1 = __uint_as_float(b[3]);
  v.fmt = (int)b[4];
  v.kind = (int)b[5];
  v.d_out = (int)b[6];
  v.d_in = (int)b[7];
  v.R = (int)c[0];
  v.C = (int)c[1];
  v.S = (int)c[2];
  v.Q = (int)c[3];
  v.wait_op = (int)c[4];
  v.item_begin = (int)c[5];
  v.n_items = (int)c[6];
  v.nmat = (int)c[7];
  v.cnt_base = (int)d[0];
  v.halves = (int)d[1];
  v.part_off = (int64_t)(((uint64_t)d[3] << 32) | d[2]);
  v.wait_first = (int)d[4];
  return v;
}

// Walks the wave's flat sequence of steps across its items (w, w+G, ...).
struct Cursor {
  const StreamOp* ops;
  int n_items, stride;
  int opi;               // op of the current item
  int item;              // current item (>= n_items: end)
  int t, n_steps;        // step within the current item
  int g, s, c0;
  int fmt, nmat, halves, C;
  const uint8_t *w0, *w1;

  __device__ void decode() {
    if (item >= n_items) return;
    for (;;) {
      const uint8_t* o = reinterpret_cast<const uint8_t*>(uptr(ops + opi));
      const u32x8 c = sload8(o + 64);
      const int item_begin = (int)c[5], n = (int)c[6];
      if (item < item_begin + n) {
        const u32x8 a = sload8(o);
        const u32x8 b = sload8(o + 32);
        const u32x8 d = sload8(o + 96);
        const int S = (int)c[2], Q = (int)c[3];
        const int li = item - item_begin;
        g = li / S;
        s = li - g * S;
        c0 = s * Q;
        C = (int)c[1];
        const int c1 = min(C, c0 + Q);
        fmt = (int)b[4];
        nmat = (int)c[7];
        halves = (int)d[1];
        n_steps = (c1 - c0) * nmat * halves;
        w0 = (const uint8_t*)(((uint64_t)a[1] << 32) | a[0]);
        w1 = (const uint8_t*)(((uint64_t)a[3] << 32) | a[2]);
        t = 0;
        return;
      }
      ++opi;
    }
  }
  __device__ void init(const StreamOp* o, int n, int first, int grid) {
    ops = o;
    n_items = n;
    stride = grid;
    opi = 0;
    item = first;
    decode();
  }
  __device__ void stop() { item = n_items; }
  // Describe the current step (op = -1 past the end) and move to the next one.
  __device__ StepDesc step_and_advance(const uint8_t* fallback) {
    StepDesc d;
    if (item >= n_items) {
      d.op = -1;
      d.fmt = FP4G_FP8_ROW;
      d.slab = d.tile = fallback;
      d.g = d.s = d.c = d.mat = d.half = d.first = d.last = 0;
      return d;
    }
    const int per_chunk = nmat * halves;
    d.op = opi;
    d.fmt = fmt;
    d.g = g;
    d.s = s;
    d.c = c0 + t / per_chunk;
    const int r = t % per_chunk;
    d.mat = halves == 2 ? 0 : r;
    d.half = halves == 2 ? r : 0;
    d.first = t == 0;
    d.last = t == n_steps - 1;
    const int T = fmt == FP4G_NVFP4 ? kTileNv : fmt == FP4G_MXFP4 ? kTileMx : kTileF8;
    d.tile = (d.mat ? w1 : w0) + ((int64_t)g * C + d.c) * T;
    d.slab = d.tile + d.half * 8192;
    if (++t == n_steps) {
      item += stride;
      decode();
    }
    return d;
  }
};

template <int M>
__device__ __forceinline__ void finalize_row(const OpView& op, unsigned* done, int opi, int row, const float (&v)[2][M],
                                             int lane) {
  if (op.kind == SK_GATE_UP) {
    uint32_t* out = reinterpret_cast<uint32_t*>(op.out);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const uint32_t h = f32_to_bf16_rne(silu_f32(v[0][m] * op.ts0) * (v[1][m] * op.ts1));
      const uint32_t hn = __shfl_down(h, 1, 64);
      if ((lane & 1) == 0) store_dev_u32(out + ((int64_t)m * op.d_out + row) / 2, h | (hn << 16));
    }
  } else {
    float* out = reinterpret_cast<float*>(op.out);
    const float sc = op.rs ? load_f32_g(op.rs + row) : op.ts0;
#pragma unroll
    for (int m = 0; m < M; ++m) store_dev_f32(out + (int64_t)m * op.d_out + row, v[0][m] * sc);
  }
  // the outputs are complete before the op's done counter moves
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0)
    __hip_atomic_fetch_add(done + ((int64_t)opi * kDoneLanes + (row >> 6) % kDoneLanes) * kDoneStride, 1u,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int M>
__global__ __launch_bounds__(64) void k_stream(StreamHdr* hdr) {
  const int lane = threadIdx.x;
  const int n_items = hdr->n_items;
  const StreamOp* ops = reinterpret_cast<const StreamOp*>(reinterpret_cast<uint8_t*>(hdr) + hdr->off_ops);
  unsigned* done = reinterpret_cast<unsigned*>(reinterpret_cast<uint8_t*>(hdr) + hdr->off_done);
  unsigned* cnt = reinterpret_cast<unsigned*>(reinterpret_cast<uint8_t*>(hdr) + hdr->off_cnt);
  float* part = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(hdr) + hdr->off_part);
  const int grid = hdr->grid;
  const int n_ops = hdr->n_ops;
  const int total_cnt = hdr->total_cnt;
  const uint8_t* fallback = reinterpret_cast<const uint8_t*>(hdr);  // >= 16 KiB of workspace, read harmlessly

  // the x columns of the current item, M tokens x (Q chunks x 128 bf16 pairs)
  constexpr int kQ = M <= 2 ? 4 : M <= 4 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint32_t xs_lds[M * kQ * 128];
  Cursor cu;
  cu.init(ops, n_items, blockIdx.x, grid);
  int waited = -1;     // last op whose completion this wave has observed
  int item_c0 = 0;     // first chunk of the current item (x columns in LDS)
  int cached = -1;     // op whose fields are in `op`
  bool abort = false;
  float acc[2][M];
  OpView op;

  StepFrag fa, fb;
  StepDesc da = cu.step_and_advance(fallback);
  load_step(fa, da, lane);
  StepDesc db = cu.step_and_advance(da.slab);
  load_step(fb, db, lane);

  auto consume = [&](const StepFrag& f, const StepDesc& d) {
    if (d.op != cached) {
      op = load_op(ops, d.op);
      cached = d.op;
    }
    if (d.first) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[a][m] = 0.0f;
      const int w = op.wait_op;
      if (w >= 0 && w != waited && !abort) {
        for (int wi = op.wait_first; wi <= w && !abort; ++wi) {
          const uint8_t* wo = reinterpret_cast<const uint8_t*>(uptr(ops + wi));
          const unsigned need = (unsigned)sload8(wo + 64)[0];  // R of the awaited op
          int spins = 0;
          for (;;) {
            unsigned sum = 0;
            if (lane < kDoneLanes) sum = atomic_load_dev(done + ((int64_t)wi * kDoneLanes + lane) * kDoneStride);
#pragma unroll
            for (int off = 4; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
            if (__builtin_amdgcn_readfirstlane(sum) >= need) break;
            if (atomic_load_dev(&hdr->err) != 0 || ++spins > kSpinLimit) {
              abort = true;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
        }
        if (abort) {
          if (lane == 0) __hip_atomic_store(&hdr->err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          cu.stop();
        }
        waited = w;
      }
    }
    if (abort) return;
    if (d.first) {
      // stage this item's x columns (chunks c0 .. c0+nc-1 of every token) in LDS;
      // device-scope loads, issued once the producer of x is known to be done
      const int c0 = d.c;
      const int nc = min(op.Q, op.C - c0);
      const int per_tok = nc * 64;  // u64 per token
      const uint64_t* xg = reinterpret_cast<const uint64_t*>(op.x);
      uint64_t* xl = reinterpret_cast<uint64_t*>(xs_lds);
      for (int i = lane; i < M * per_tok; i += 64) {
        const int m = i / per_tok, k = i - m * per_tok;
        xl[m * (kQ * 64) + k] = __hip_atomic_load(
            (const FP4G_GLOBAL uint64_t*)(xg + (int64_t)m * (op.d_in / 4) + (int64_t)c0 * 64 + k), __ATOMIC_RELAXED,
            __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the LDS writes are done
      item_c0 = c0;
    }
    const uint32_t* xb = xs_lds + (d.c - item_c0) * 128;
    float pa[M];
#pragma unroll
    for (int m = 0; m < M; ++m) pa[m] = 0.0f;
    step_dot<M>(f, op.fmt, d.half, lane, xb, kQ * 128, pa);
    if (d.mat == 0) {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[0][m] += pa[m];
    } else {
#pragma unroll
      for (int m = 0; m < M; ++m) acc[1][m] += pa[m];
    }
    if (!d.last) return;
    const int row = d.g * 64 + lane;
    const int64_t rpad = (int64_t)op.R * 64;
    if (op.S == 1) {
      finalize_row<M>(op, done, d.op, row, acc, lane);
      return;
    }
    float* base = part + op.part_off + (int64_t)d.s * op.nmat * M * rpad;
#pragma unroll
    for (int a = 0; a < 2; ++a)
      if (a < op.nmat)
#pragma unroll
        for (int m = 0; m < M; ++m) publish_partial(base + (a * M + m) * rpad + row, acc[a][m]);
    unsigned* c = cnt + op.cnt_base + d.g;
    if (!arrive_last(c, (unsigned)(op.S - 1))) return;
    float v[2][M];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float tsum = 0.0f;
        if (a < op.nmat)
          for (int q = 0; q < op.S; ++q)
            tsum += collect_partial(part + op.part_off + (((int64_t)q * op.nmat + a) * M + m) * rpad + row);
        v[a][m] = tsum;
      }
    reset_counter(c);
    finalize_row<M>(op, done, d.op, row, v, lane);
  };

  // Two fragments alternate.  The loads are unconditional (past the end a wave
  // re-reads its last slab) so that the wait counts are the same on every path.
  while (da.op >= 0) {
    consume(fa, da);
    const StepDesc dn = cu.step_and_advance(db.slab);
    if (db.op < 0) break;
    da = dn;
    load_step(fa, da, lane);
    consume(fb, db);
    db = cu.step_and_advance(da.slab);
    load_step(fb, db, lane);
  }

  // the last wave to leave resets the counters for the next launch
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  unsigned prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(&hdr->exit_count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0, 64);
  if (prev != (unsigned)(grid - 1)) return;
  for (int i = lane; i < n_ops * kDoneLanes; i += 64)
    __hip_atomic_store(done + (int64_t)i * kDoneStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (atomic_load_dev(&hdr->err) != 0)
    for (int i = lane; i < total_cnt; i += 64)
      __hip_atomic_store(cnt + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (lane == 0) __hip_atomic_store(&hdr->exit_count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- host side ----------------------------------------------------------------------
// Chunks per item: enough items per op to give every wave of a full grid
// (256 CUs x 8 waves) about one, so that each op spreads over the whole GPU;
// never more chunks than the LDS staging of x holds at this M.
constexpr int64_t kTargetItems = 2048;
int max_chunks_per_item(int M) { return M <= 2 ? 4 : M <= 4 ? 2 : 1; }
int64_t chunks_per_item(int M, int64_t R, int64_t C) {
  int64_t S = (kTargetItems + R - 1) / R;
  if (S > C) S = C;
  int64_t Q = (C + S - 1) / S;
  const int64_t qmax = max_chunks_per_item(M);
  return Q < qmax ? Q : qmax;
}

struct StreamLayout {
  uint64_t off_ops, off_done, off_cnt, off_part, total;
  int64_t total_cnt, total_part, n_items;
};

fp4g_status layout_stream(const fp4g_stream_op* ops, int n, int M, StreamLayout& L, StreamOp* table) {
  if (!ops) return FP4G_E_NULL;
  if (n < 1 || n > (1 << 20) || M < 1 || M > kMaxM) return FP4G_E_SHAPE;
  int64_t cnt = 0, partf = 0, items = 0;
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
    const int64_t Q = chunks_per_item(M, R, C);
    const int64_t S = (C + Q - 1) / Q;
    const int nmat = gu ? 2 : 1;
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
      t.S = (int32_t)S;
      t.Q = (int32_t)Q;
      t.wait_op = o.wait_op;
      t.wait_first = o.wait_op >= 0 ? o.wait_op - wcount + 1 : -1;
      t.item_begin = (int32_t)items;
      t.n_items = (int32_t)(R * S);
      t.nmat = nmat;
      t.cnt_base = (int32_t)cnt;
      t.halves = o.w->format == FP4G_FP8_ROW ? 2 : 1;
      t.part_off = S > 1 ? partf : 0;
    }
    items += R * S;
    cnt += R;
    if (S > 1) partf += S * nmat * M * R * 64;
    if (items > (int64_t)1 << 30) return FP4G_E_SHAPE;
  }
  L.total_cnt = cnt;
  L.total_part = partf;
  L.n_items = items;
  uint64_t o = sizeof(StreamHdr);
  L.off_ops = o;
  o = align256(o + (uint64_t)n * sizeof(StreamOp));
  L.off_done = o;
  o = align256(o + 4ull * n * kDoneLanes * kDoneStride);
  L.off_cnt = o;
  o = align256(o + 4ull * cnt);
  L.off_part = o;
  o = align256(o + 4ull * partf);
  L.total = o < 16384 ? 16384 : o;  // the fallback slab of finished waves must be readable
  return FP4G_OK;
}

// Aliasing rules of a stream: outputs are disjoint from each other and from all
// weights; an op's input overlaps no output except that of the op it waits for.
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

const void* stream_kernel(int M) {
  switch (M) {
    case 1: return (const void*)&k_stream<1>;
    case 2: return (const void*)&k_stream<2>;
    case 3: return (const void*)&k_stream<3>;
    case 4: return (const void*)&k_stream<4>;
    case 5: return (const void*)&k_stream<5>;
    case 6: return (const void*)&k_stream<6>;
    case 7: return (const void*)&k_stream<7>;
    default: return (const void*)&k_stream<8>;
  }
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
    if (overlap(ws, L.total, ops[i].out_dev, ob) || overlap(ws, L.total, ops[i].x_dev, (size_t)M * ops[i].w->d_in * 2) ||
        overlap(ws, L.total, ops[i].w->packed, ops[i].w->packed_bytes))
      return FP4G_E_ALIAS;
  }
  // host image of header + op table, then one synchronous copy; counters zeroed
  const size_t img = L.off_done;
  uint8_t* h = (uint8_t*)calloc(1, img);
  if (!h) return FP4G_E_HIP;
  StreamHdr* hdr = (StreamHdr*)h;
  hdr->magic = kStreamMagic;
  hdr->n_ops = n_ops;
  hdr->n_items = (int32_t)L.n_items;
  hdr->M = M;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    free(h);
    return FP4G_E_HIP;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)stream_kernel(M), 64, 0) != hipSuccess ||
      per_cu < 1) {
    free(h);
    return FP4G_E_HIP;
  }
  // every workgroup must be resident at once (waits go to other workgroups)
  const int grid = cus * std::min(per_cu, 8);
  hdr->grid = grid;
  hdr->total_cnt = (int32_t)L.total_cnt;
  hdr->off_ops = (int64_t)L.off_ops;
  hdr->off_done = (int64_t)L.off_done;
  hdr->off_cnt = (int64_t)L.off_cnt;
  hdr->off_part = (int64_t)L.off_part;
  layout_stream(ops, n_ops, M, L, (StreamOp*)(h + L.off_ops));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(ws, h, img, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipMemsetAsync((uint8_t*)ws + L.off_done, 0, L.off_part - L.off_done, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  free(h);
  if (e != hipSuccess) return FP4G_E_HIP;
  plan->magic = kStreamMagic;
  plan->M = M;
  plan->n_ops = n_ops;
  plan->n_items = (int32_t)L.n_items;
  plan->grid = grid;
  plan->reserved = 0;
  plan->ws = ws;
  plan->ws_bytes = L.total;
  return FP4G_OK;
}

int32_t fp4_stream_run(const fp4g_stream_plan* plan, void* stream) {
  if (!plan || !plan->ws) return FP4G_E_NULL;
  if (plan->magic != kStreamMagic) return FP4G_E_FORMAT;
  if (plan->M < 1 || plan->M > kMaxM || plan->grid < 1) return FP4G_E_SHAPE;
  hipStream_t s = (hipStream_t)stream;
  StreamHdr* hdr = (StreamHdr*)plan->ws;
  switch (plan->M) {
#define FP4G_CASE(MM) \
  case MM:            \
    k_stream<MM><<<plan->grid, 64, 0, s>>>(hdr); \
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
