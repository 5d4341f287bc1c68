// gemv.hip -- launch planning, host-side validation and the product entry points
// fp4_gemv, fp4_skinny_gemm, fp4_gemv_grouped, fp4_gate_up_silu and
// fp8_lmhead_gemv.  The kernel itself is in gemv_kernel.hpp.
#include <mutex>

#include "gemv_a8.hpp"

namespace fp4g {

// Per-format launchers (gemv_kernel.hpp), instantiated in gemv_nvfp4.hip,
// gemv_mxfp4.hip, gemv_fp8.hip and gemv_fp8_silu.hip.
extern template hipError_t launch_m<FP4G_NVFP4, 1, EPI_STORE>(int, int, const GemvParams&, unsigned, hipStream_t);
extern template hipError_t launch_m<FP4G_NVFP4, 2, EPI_SILU>(int, int, const GemvParams&, unsigned, hipStream_t);
extern template hipError_t launch_m<FP4G_MXFP4, 1, EPI_STORE>(int, int, const GemvParams&, unsigned, hipStream_t);
extern template hipError_t launch_m<FP4G_MXFP4, 2, EPI_SILU>(int, int, const GemvParams&, unsigned, hipStream_t);
extern template hipError_t launch_m<FP4G_FP8_ROW, 1, EPI_STORE>(int, int, const GemvParams&, unsigned, hipStream_t);
extern template hipError_t launch_m<FP4G_FP8_ROW, 1, EPI_ARGMAX>(int, int, const GemvParams&, unsigned, hipStream_t);
extern template hipError_t launch_m<FP4G_FP8_ROW, 2, EPI_SILU>(int, int, const GemvParams&, unsigned, hipStream_t);
// W4A8 launchers (gemv_a8.hpp), in gemv_a8.hip: plain products and gate/up.
hipError_t launch_a8_ext(int M, const GemvParams& p, unsigned grid, size_t lds, hipStream_t s);
hipError_t launch_a8_silu_ext(int M, const GemvParams& p, unsigned grid, size_t lds, hipStream_t s);
// Matrix-core launchers (gemv_mfma.hpp), in gemv_mfma_nvfp4.hip and gemv_mfma_mxfp4.hip.
extern template hipError_t launch_mfma<FP4G_NVFP4, 1, EPI_STORE>(int, const GemvParams&, unsigned, size_t, hipStream_t);
extern template hipError_t launch_mfma<FP4G_NVFP4, 2, EPI_SILU>(int, const GemvParams&, unsigned, size_t, hipStream_t);
extern template hipError_t launch_mfma<FP4G_MXFP4, 1, EPI_STORE>(int, const GemvParams&, unsigned, size_t, hipStream_t);
extern template hipError_t launch_mfma<FP4G_MXFP4, 2, EPI_SILU>(int, const GemvParams&, unsigned, size_t, hipStream_t);

// AUTO takes the matrix cores from this many vectors on (below it the VALU
// kernel's dot products keep up with HBM).
constexpr int kMfmaMinM = 3;

// The kernel path a call runs: FP8 rows always take the VALU kernel.
static bool use_mfma(int32_t path, uint32_t format, int M) {
  if (format == FP4G_FP8_ROW) return false;
  if (path == FP4G_PATH_MFMA) return true;
  if (path == FP4G_PATH_VALU) return false;
  return M >= kMfmaMinM;
}

// A path the call can run: MFMA only for NVFP4/MXFP4; VALU up to kMaxM vectors
// for NVFP4/MXFP4 (their wider verify blocks run on the matrix cores alone) and
// up to kMaxMWide for FP8 rows (which have only the VALU kernel).
static bool valid_path(int32_t path, bool fp4, int M) {
  if (path == FP4G_PATH_AUTO) return true;
  if (path == FP4G_PATH_VALU) return M <= kMaxM || !fp4;
  return (path == FP4G_PATH_MFMA || path == FP4G_PATH_A8) && fp4;
}

// Workspace check shared by every entry point: NULL only when nothing is needed,
// large enough, 256-B aligned.
static fp4g_status check_ws(const void* ws, uint64_t ws_bytes, uint64_t need) {
  if (need && !ws) return FP4G_E_NULL;
  if (ws_bytes < need) return FP4G_E_WORKSPACE;
  if (need && !aligned(ws, 256)) return FP4G_E_ALIGN;
  return FP4G_OK;
}

// ---- the library's own scratch (fp4_skinny_gemm_noalloc) -----------------------
// A fixed device array that stands in for the caller's workspace, for callers
// that cannot allocate.  Each GPU the library runs on holds its own copy (at its
// own address) until the process ends; host code never uses the array's name as
// an address, only the pointer hipGetSymbolAddress returned for that device.
constexpr uint64_t kStaticScratchBytes = FP4G_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// The scratch array's device address on the device `stream` belongs to (looked up
// once per device, with that device current).
static fp4g_status static_scratch(void* stream, void** out) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FP4G_E_HIP;
  dev = cur;
  if (stream && hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return FP4G_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FP4G_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return FP4G_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return FP4G_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FP4G_OK;
}

// ---- workspace check ----------------------------------------------------------------
// One workgroup counts the non-zero 8-byte words of a region into a device word
// of the library's own (a region of a few MiB takes well under a millisecond).
static __device__ unsigned long long ws_check_total;
static void* g_check_ptr[kMaxDevices];

__global__ __launch_bounds__(1024) void k_count_nonzero(const unsigned long long* __restrict__ w, uint64_t n,
                                                        unsigned long long* out) {
  __shared__ unsigned long long part[16];
  unsigned long long c = 0;
  for (uint64_t i = threadIdx.x; i < n; i += 1024) c += w[i] != 0ull ? 1ull : 0ull;
  for (int off = 32; off > 0; off >>= 1) c += __shfl_down(c, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = c;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long t = 0;
    for (int i = 0; i < 16; ++i) t += part[i];
    *out = t;
  }
}

static fp4g_status check_total_ptr(void* stream, void** out) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return FP4G_E_HIP;
  dev = cur;
  if (stream && hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess) return FP4G_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FP4G_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_check_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return FP4G_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(ws_check_total));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return FP4G_E_HIP;
    g_check_ptr[dev] = p;
  }
  *out = g_check_ptr[dev];
  return FP4G_OK;
}

// Validation + launch of n products of one input (n = 1: fp4_gemv,
// fp4_skinny_gemm, fp8_lmhead_gemv).  Members share format and d_in.
// use_static: take the library's scratch array instead of (ws, ws_bytes).
static int32_t run_group(const fp4g_weight* const* W, int n, bool want_fp4, const uint16_t* X, int32_t M,
                         float* const* Y, int32_t path, void* ws, uint64_t ws_bytes, void* stream,
                         bool use_static = false) {
  if (n < 1 || n > kMaxGroup) return FP4G_E_SHAPE;
  for (int i = 0; i < n; ++i) {
    const fp4g_status st = check_weight(W[i], want_fp4);
    if (st != FP4G_OK) return st;
  }
  for (int i = 1; i < n; ++i) {
    if (W[i]->format != W[0]->format) return FP4G_E_FORMAT;
    if (W[i]->d_in != W[0]->d_in) return FP4G_E_SHAPE;
  }
  if (!X) return FP4G_E_NULL;
  for (int i = 0; i < n; ++i)
    if (!Y[i]) return FP4G_E_NULL;
  if (M < 1 || M > kMaxMWide) return FP4G_E_SHAPE;
  if (!aligned(X, 16)) return FP4G_E_ALIGN;
  for (int i = 0; i < n; ++i)
    if (!aligned(Y[i], 16)) return FP4G_E_ALIGN;
  int64_t R_total = 0;
  for (int i = 0; i < n; ++i) R_total += row_groups(W[i]->d_out);
  const int64_t C = chunks(W[0]->d_in);
  if (!valid_path(path, want_fp4, M)) return FP4G_E_PATH;
  const bool a8 = path == FP4G_PATH_A8;  // W4A8: MXFP4 weights only
  if (a8 && W[0]->format != FP4G_MXFP4) return FP4G_E_PATH;
  const bool mfma = a8 || use_mfma(path, W[0]->format, M);
  const uint64_t need = gemv_ws_bytes_any(R_total, C, 1, M);
  if (use_static) {  // every host check above is done; the first HIP call follows
    if (need > kStaticScratchBytes) return FP4G_E_WORKSPACE;
    const fp4g_status sst = static_scratch(stream, &ws);
    if (sst != FP4G_OK) return sst;
    ws_bytes = kStaticScratchBytes;
  }
  const fp4g_status wst = check_ws(ws, ws_bytes, need);
  if (wst != FP4G_OK) return wst;
  const size_t xbytes = (size_t)M * W[0]->d_in * 2;
  if (overlap(ws, need, X, xbytes)) return FP4G_E_ALIAS;
  for (int i = 0; i < n; ++i) {
    const size_t yb = (size_t)M * W[i]->d_out * 4;
    if (overlap(Y[i], yb, X, xbytes) || overlap(Y[i], yb, ws, need) || overlap(ws, need, W[i]->packed, W[i]->packed_bytes))
      return FP4G_E_ALIAS;
    for (int j = 0; j < n; ++j) {
      if (overlap(Y[i], yb, W[j]->packed, W[j]->packed_bytes)) return FP4G_E_ALIAS;
      if (j > i && overlap(Y[i], yb, Y[j], (size_t)M * W[j]->d_out * 4)) return FP4G_E_ALIAS;
    }
  }
  const Plan pl = mfma ? plan_mfma(R_total, C, 1, M) : plan_for(R_total, C, 1, M);
  GemvParams p{};
  p.n = n;
  int64_t gb = 0;
  for (int i = 0; i < n; ++i) {
    p.w[i] = (const uint8_t*)W[i]->packed;
    p.tscale[i] = W[i]->tensor_scale;
    p.y[i] = Y[i];
    p.d_out[i] = W[i]->d_out;
    p.gbase[i] = (int)gb;
    gb += row_groups(W[i]->d_out);
  }
  p.gbase[n] = (int)gb;
  if (W[0]->format == FP4G_FP8_ROW)  // row scales follow each member's tiles
    for (int i = 0; i < n; ++i)
      p.rs[i] = (const float*)((const uint8_t*)W[i]->packed + row_groups(W[i]->d_out) * C * kTileF8);
  p.x = X;
  p.slots = need ? (unsigned long long*)ws : nullptr;
  p.d_in = W[0]->d_in;
  p.C = (int)C;
  p.S = pl.S;
  p.wg_chunks = pl.wg_chunks;
  const unsigned grid = (unsigned)(R_total * pl.S);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (a8)
    e = launch_a8_ext(M, p, grid, a8_lds_bytes(pl, M, 1), s);
  else if (mfma)
    e = W[0]->format == FP4G_NVFP4 ? launch_mfma<FP4G_NVFP4, 1, EPI_STORE>(M, p, grid, mfma_lds_bytes(pl, W[0]->format, 1, M), s)
                                   : launch_mfma<FP4G_MXFP4, 1, EPI_STORE>(M, p, grid, mfma_lds_bytes(pl, W[0]->format, 1, M), s);
  else if (W[0]->format == FP4G_NVFP4)
    e = launch_m<FP4G_NVFP4, 1, EPI_STORE>(M, pl.nw, p, grid, s);
  else if (W[0]->format == FP4G_MXFP4)
    e = launch_m<FP4G_MXFP4, 1, EPI_STORE>(M, pl.nw, p, grid, s);
  else
    e = launch_m<FP4G_FP8_ROW, 1, EPI_STORE>(M, pl.nw, p, grid, s);
  return e == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}

static int32_t run_gemv(const fp4g_weight* W, bool want_fp4, const uint16_t* X, int32_t M, float* Y, int32_t path,
                        void* ws, uint64_t ws_bytes, void* stream) {
  if (!W) return FP4G_E_NULL;
  return run_group(&W, 1, want_fp4, X, M, &Y, path, ws, ws_bytes, stream);
}

// One wave: the pick of every vector from the slots, which it leaves at zero.
__global__ void k_argmax_finish(unsigned long long* amax, int M, int32_t* top_idx, float* top_val) {
  const int lane = threadIdx.x & 63;
  if (lane < M) {
    uint64_t best = 0;
    for (int j = 0; j < kArgSlots; ++j) {
      const uint64_t k = amax[(int64_t)j * kMaxMWide + lane];
      best = k > best ? k : best;
    }
    top_idx[lane] = key_index(best);
    top_val[lane] = key_value(best);
  }
  __syncthreads();
  for (int i = lane; i < kArgSlots * kMaxMWide; i += 64) amax[i] = 0ull;
}

// The greedy pick's slots (zero between calls).
static uint64_t argmax_ws_bytes() { return align256((uint64_t)kArgSlots * kMaxMWide * 8); }

static fp4g_status check_group(const fp4g_group* G) {
  if (!G) return FP4G_E_NULL;
  if (G->n < 1 || G->n > kMaxGroup) return FP4G_E_SHAPE;
  return FP4G_OK;
}

}  // namespace fp4g

using namespace fp4g;

extern "C" {

int32_t fp4_gemv(const fp4g_weight* W, const uint16_t* x, float* y, void* ws, uint64_t ws_bytes, void* stream) {
  return run_gemv(W, true, x, 1, y, FP4G_PATH_AUTO, ws, ws_bytes, stream);
}

int32_t fp4_skinny_gemm(const fp4g_weight* W, const uint16_t* X, int32_t M, float* Y, int32_t path, void* ws,
                        uint64_t ws_bytes, void* stream) {
  return run_gemv(W, true, X, M, Y, path, ws, ws_bytes, stream);
}

int32_t fp4_skinny_gemm_noalloc(const fp4g_weight* W, const uint16_t* X, int32_t M, float* Y, int32_t path,
                                void* stream) {
  if (!W) return FP4G_E_NULL;
  return run_group(&W, 1, true, X, M, &Y, path, nullptr, 0, stream, true);
}

int32_t fp4_gemv_grouped(const fp4g_group* G, const uint16_t* X, int32_t M, float* const* Y, int32_t path,
                         void* ws, uint64_t ws_bytes, void* stream) {
  const fp4g_status st = check_group(G);
  if (st != FP4G_OK) return st;
  if (!Y) return FP4G_E_NULL;
  const fp4g_weight* W[kMaxGroup];
  for (int i = 0; i < G->n; ++i) W[i] = &G->w[i];
  // NVFP4/MXFP4 members, or FP8 row-scaled ones (projections of a mixed layout)
  return run_group(W, G->n, G->w[0].format != FP4G_FP8_ROW, X, M, Y, path, ws, ws_bytes, stream);
}

int32_t fp8_lmhead_gemv(const fp4g_weight* W, const uint16_t* X, int32_t M, float* logits, void* ws,
                        uint64_t ws_bytes, void* stream) {
  return run_gemv(W, false, X, M, logits, FP4G_PATH_AUTO, ws, ws_bytes, stream);
}

int32_t fp8_lmhead_argmax(const fp4g_weight* W, const uint16_t* X, int32_t M, int32_t row_begin, int32_t n_rows,
                          float* logits, int32_t* top_idx, float* top_val, void* ws, uint64_t ws_bytes,
                          void* stream) {
  fp4g_status st = check_weight(W, false);
  if (st != FP4G_OK) return st;
  if (!X || !top_idx || !top_val) return FP4G_E_NULL;
  if (M < 1 || M > kMaxMWide) return FP4G_E_SHAPE;
  if (row_begin < 0 || row_begin % kRowsPerGroup || n_rows < 1 || (int64_t)row_begin + n_rows > W->d_out)
    return FP4G_E_SHAPE;
  if (!aligned(X, 16) || (logits && !aligned(logits, 16)) || !aligned(top_idx, 4) || !aligned(top_val, 4))
    return FP4G_E_ALIGN;
  const uint64_t need = argmax_ws_bytes();
  st = check_ws(ws, ws_bytes, need);
  if (st != FP4G_OK) return st;
  const int64_t R_all = row_groups(W->d_out), C = chunks(W->d_in), R = row_groups(n_rows);
  const size_t xbytes = (size_t)M * W->d_in * 2, lbytes = logits ? (size_t)M * n_rows * 4 : 0;
  const void* outs[4] = {logits, top_idx, top_val, ws};
  const size_t outb[4] = {lbytes, (size_t)M * 4, (size_t)M * 4, need};
  for (int i = 0; i < 4; ++i) {
    if (overlap(outs[i], outb[i], X, xbytes) || overlap(outs[i], outb[i], W->packed, W->packed_bytes))
      return FP4G_E_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return FP4G_E_ALIAS;
  }
  GemvParams p{};
  p.n = 1;
  // the rows [row_begin, row_begin + n_rows) as a matrix of their own: their
  // tiles are contiguous, their row scales sit after all the matrix's tiles
  const uint8_t* base = (const uint8_t*)W->packed;
  p.w[0] = base + (int64_t)(row_begin / kRowsPerGroup) * C * kTileF8;
  p.rs[0] = (const float*)(base + R_all * C * kTileF8) + row_begin;
  p.tscale[0] = 1.0f;
  p.y[0] = logits;
  p.d_out[0] = n_rows;
  p.gbase[0] = 0;
  p.gbase[1] = (int)R;
  p.x = X;
  p.slots = nullptr;
  p.amax = (unsigned long long*)ws;
  p.top_idx = top_idx;
  p.top_val = top_val;
  p.row_base = row_begin;
  p.d_in = W->d_in;
  p.C = (int)C;
  p.S = 1;  // whole rows per workgroup: no split-K tree
  p.wg_chunks = (int)C;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_m<FP4G_FP8_ROW, 1, EPI_ARGMAX>(M, 4, p, (unsigned)R, s);
  if (e != hipSuccess) return FP4G_E_HIP;
  k_argmax_finish<<<1, 64, 0, s>>>(p.amax, M, top_idx, top_val);
  return hipGetLastError() == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}

int32_t fp4_gate_up_silu(const fp4g_weight* Wg, const fp4g_weight* Wu, const uint16_t* X, int32_t M, uint16_t* H,
                         int32_t path, void* ws, uint64_t ws_bytes, void* stream) {
  // NVFP4/MXFP4 pairs, or FP8 row-scaled pairs (the FP8 MLPs of a mixed layout)
  const bool fp4 = Wg && Wg->format != FP4G_FP8_ROW;
  fp4g_status st = check_weight(Wg, fp4);
  if (st != FP4G_OK) return st;
  st = check_weight(Wu, fp4);
  if (st != FP4G_OK) return st;
  if (Wg->format != Wu->format) return FP4G_E_FORMAT;
  if (Wg->d_out != Wu->d_out || Wg->d_in != Wu->d_in) return FP4G_E_SHAPE;
  if (!X || !H) return FP4G_E_NULL;
  if (M < 1 || M > (fp4 ? kMaxMWide : kMaxM)) return FP4G_E_SHAPE;
  if (!valid_path(path, fp4, M)) return FP4G_E_PATH;
  const bool a8 = path == FP4G_PATH_A8;  // W4A8: MXFP4 weights only
  if (a8 && Wg->format != FP4G_MXFP4) return FP4G_E_PATH;
  if (!aligned(X, 16) || !aligned(H, 16)) return FP4G_E_ALIGN;
  const bool mfma = a8 || use_mfma(path, Wg->format, M);
  const int64_t R = row_groups(Wg->d_out), C = chunks(Wg->d_in);
  const uint64_t need = gemv_ws_bytes_any(R, C, 2, M);
  st = check_ws(ws, ws_bytes, need);
  if (st != FP4G_OK) return st;
  const size_t hbytes = (size_t)M * Wg->d_out * 2, xbytes = (size_t)M * Wg->d_in * 2;
  if (overlap(H, hbytes, X, xbytes) || overlap(H, hbytes, Wg->packed, Wg->packed_bytes) ||
      overlap(H, hbytes, Wu->packed, Wu->packed_bytes) || overlap(H, hbytes, ws, need) ||
      overlap(ws, need, X, xbytes) || overlap(ws, need, Wg->packed, Wg->packed_bytes) ||
      overlap(ws, need, Wu->packed, Wu->packed_bytes))
    return FP4G_E_ALIAS;
  const Plan pl = mfma ? plan_mfma(R, C, 2, M) : plan_for(R, C, 2, M);
  GemvParams p{};
  p.n = 1;
  p.w[0] = (const uint8_t*)Wg->packed;
  p.w[1] = (const uint8_t*)Wu->packed;
  p.tscale[0] = Wg->tensor_scale;
  p.tscale[1] = Wu->tensor_scale;
  p.d_out[0] = Wg->d_out;
  p.gbase[0] = 0;
  p.gbase[1] = (int)R;
  if (!fp4) {  // row scales follow each matrix's tiles
    p.rs[0] = (const float*)((const uint8_t*)Wg->packed + R * C * kTileF8);
    p.rs[1] = (const float*)((const uint8_t*)Wu->packed + R * C * kTileF8);
  }
  p.x = X;
  p.h = H;
  p.slots = need ? (unsigned long long*)ws : nullptr;
  p.d_in = Wg->d_in;
  p.C = (int)C;
  p.S = pl.S;
  p.wg_chunks = pl.wg_chunks;
  const unsigned grid = (unsigned)(R * pl.S);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (a8)
    e = launch_a8_silu_ext(M, p, grid, a8_lds_bytes(pl, M, 2), s);
  else if (mfma)
    e = Wg->format == FP4G_NVFP4 ? launch_mfma<FP4G_NVFP4, 2, EPI_SILU>(M, p, grid, mfma_lds_bytes(pl, Wg->format, 2, M), s)
                                 : launch_mfma<FP4G_MXFP4, 2, EPI_SILU>(M, p, grid, mfma_lds_bytes(pl, Wg->format, 2, M), s);
  else if (Wg->format == FP4G_NVFP4)
    e = launch_m<FP4G_NVFP4, 2, EPI_SILU>(M, pl.nw, p, grid, s);
  else if (Wg->format == FP4G_MXFP4)
    e = launch_m<FP4G_MXFP4, 2, EPI_SILU>(M, pl.nw, p, grid, s);
  else
    e = launch_m<FP4G_FP8_ROW, 2, EPI_SILU>(M, pl.nw, p, grid, s);
  return e == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}

int32_t fp4g_workspace_check(int32_t op, const void* desc, int32_t M, const void* ws, uint64_t ws_bytes,
                             uint64_t* nonzero, void* stream) {
  if (!desc || !ws || !nonzero) return FP4G_E_NULL;
  const uint64_t need = fp4g_workspace_bytes(op, desc, M);
  if (need == 0) return FP4G_E_SHAPE;
  if (ws_bytes < need) return FP4G_E_WORKSPACE;
  if (!aligned(ws, 256)) return FP4G_E_ALIGN;
  const uint64_t region = op == FP4G_OP_MOE ? moe_slot_bytes((const fp4g_moe*)desc) : need;
  void* total = nullptr;
  const fp4g_status st = check_total_ptr(stream, &total);
  if (st != FP4G_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  k_count_nonzero<<<1, 1024, 0, s>>>((const unsigned long long*)ws, region / 8, (unsigned long long*)total);
  if (hipGetLastError() != hipSuccess) return FP4G_E_HIP;
  if (hipMemcpyAsync(nonzero, total, sizeof(uint64_t), hipMemcpyDeviceToHost, s) != hipSuccess) return FP4G_E_HIP;
  return hipStreamSynchronize(s) == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}

uint64_t fp4g_workspace_bytes(int32_t op, const void* desc, int32_t M) {
  if (!desc || M < 1 || M > kMaxMWide) return 0;
  if (op == FP4G_OP_MOE) return moe_ws_bytes((const fp4g_moe*)desc, M);
  if (op == FP4G_OP_LMHEAD_ARGMAX) return check_weight((const fp4g_weight*)desc, false) == FP4G_OK ? argmax_ws_bytes() : 0;
  if (op == FP4G_OP_GROUPED) {
    const fp4g_group* G = (const fp4g_group*)desc;
    if (check_group(G) != FP4G_OK) return 0;
    const bool fp4 = G->w[0].format != FP4G_FP8_ROW;
    int64_t R = 0;
    for (int i = 0; i < G->n; ++i) {
      if (check_weight(&G->w[i], fp4) != FP4G_OK) return 0;
      if (G->w[i].format != G->w[0].format || G->w[i].d_in != G->w[0].d_in) return 0;
      R += row_groups(G->w[i].d_out);
    }
    return gemv_ws_bytes_any(R, chunks(G->w[0].d_in), 1, M);
  }
  const fp4g_weight* W = (const fp4g_weight*)desc;
  if (op != FP4G_OP_GEMV && op != FP4G_OP_GATE_UP && op != FP4G_OP_LMHEAD) return 0;
  // FP8 rows: the head (up to kMaxMWide vectors), or a gate/up pair of a mixed
  // layout (up to kMaxM)
  const bool fp4 = op == FP4G_OP_GEMV || (op == FP4G_OP_GATE_UP && W->format != FP4G_FP8_ROW);
  if (check_weight(W, fp4) != FP4G_OK) return 0;
  if (!fp4 && op == FP4G_OP_GATE_UP && M > kMaxM) return 0;
  return gemv_ws_bytes_any(row_groups(W->d_out), chunks(W->d_in), op == FP4G_OP_GATE_UP ? 2 : 1, M);
}

}  // extern "C"
