// gemv.hip -- launch planning, host-side validation and the product entry points
// fp4_gemv, fp4_skinny_gemm, fp4_gate_up_silu and fp8_lmhead_gemv.  The kernel
// itself is in gemv_kernel.hpp.
#include "gemv_kernel.hpp"

namespace fp4g {

// Per-format launchers (gemv_kernel.hpp), instantiated in gemv_nvfp4.hip,
// gemv_mxfp4.hip and gemv_fp8.hip.
extern template hipError_t launch_m<FP4G_NVFP4, 1, EPI_STORE>(int, const GemvParams&, unsigned, hipStream_t);
extern template hipError_t launch_m<FP4G_NVFP4, 2, EPI_SILU>(int, const GemvParams&, unsigned, hipStream_t);
extern template hipError_t launch_m<FP4G_MXFP4, 1, EPI_STORE>(int, const GemvParams&, unsigned, hipStream_t);
extern template hipError_t launch_m<FP4G_MXFP4, 2, EPI_SILU>(int, const GemvParams&, unsigned, hipStream_t);
extern template hipError_t launch_m<FP4G_FP8_ROW, 1, EPI_STORE>(int, const GemvParams&, unsigned, hipStream_t);

// Shared validation + launch of the single-matrix product (any format).
int32_t run_gemv(const fp4g_weight* W, bool want_fp4, const uint16_t* X, int32_t M, float* Y, void* ws,
                 uint64_t ws_bytes, void* stream) {
  fp4g_status st = check_weight(W, want_fp4);
  if (st != FP4G_OK) return st;
  if (!X || !Y) return FP4G_E_NULL;
  if (M < 1 || M > kMaxM) return FP4G_E_SHAPE;
  if (!aligned(X, 16) || !aligned(Y, 16)) return FP4G_E_ALIGN;
  const int64_t R = row_groups(W->d_out), C = chunks(W->d_in);
  const uint64_t need = gemv_ws_bytes(R, C, 1, M);
  if (need && !ws) return FP4G_E_NULL;
  if (ws_bytes < need) return FP4G_E_WORKSPACE;
  if (need && !aligned(ws, 256)) return FP4G_E_ALIGN;
  const size_t ybytes = (size_t)M * W->d_out * 4, xbytes = (size_t)M * W->d_in * 2;
  if (overlap(Y, ybytes, X, xbytes) || overlap(Y, ybytes, W->packed, W->packed_bytes) ||
      overlap(Y, ybytes, ws, need) || overlap(ws, need, X, xbytes) || overlap(ws, need, W->packed, W->packed_bytes))
    return FP4G_E_ALIAS;
  const Plan pl = plan_for(R, C, 1);
  GemvParams p{};
  p.w[0] = p.w[1] = (const uint8_t*)W->packed;
  p.tscale[0] = p.tscale[1] = W->tensor_scale;
  p.x = X;
  p.y = Y;
  p.counters = (unsigned*)ws;
  p.part = need ? (float*)((uint8_t*)ws + kCounterBytes) : nullptr;
  p.d_out = W->d_out;
  p.d_in = W->d_in;
  p.R = (int)R;
  p.C = (int)C;
  p.S = pl.S;
  p.wg_chunks = pl.wg_chunks;
  const unsigned grid = (unsigned)(R * pl.S);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (W->format == FP4G_NVFP4)
    e = launch_m<FP4G_NVFP4, 1, EPI_STORE>(M, p, grid, s);
  else if (W->format == FP4G_MXFP4)
    e = launch_m<FP4G_MXFP4, 1, EPI_STORE>(M, p, grid, s);
  else
    e = launch_m<FP4G_FP8_ROW, 1, EPI_STORE>(M, p, grid, s);
  return e == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}

}  // namespace fp4g

using namespace fp4g;

extern "C" {

int32_t fp4_gemv(const fp4g_weight* W, const uint16_t* x, float* y, void* ws, uint64_t ws_bytes, void* stream) {
  return run_gemv(W, true, x, 1, y, ws, ws_bytes, stream);
}

int32_t fp4_skinny_gemm(const fp4g_weight* W, const uint16_t* X, int32_t M, float* Y, int32_t path, void* ws,
                        uint64_t ws_bytes, void* stream) {
  if (path != FP4G_PATH_AUTO && path != FP4G_PATH_VALU) {
    if (path == FP4G_PATH_MFMA) return FP4G_E_PATH;
    return FP4G_E_PATH;
  }
  return run_gemv(W, true, X, M, Y, ws, ws_bytes, stream);
}

int32_t fp8_lmhead_gemv(const fp4g_weight* W, const uint16_t* X, int32_t M, float* logits, void* ws,
                        uint64_t ws_bytes, void* stream) {
  return run_gemv(W, false, X, M, logits, ws, ws_bytes, stream);
}

int32_t fp4_gate_up_silu(const fp4g_weight* Wg, const fp4g_weight* Wu, const uint16_t* X, int32_t M, uint16_t* H,
                         int32_t path, void* ws, uint64_t ws_bytes, void* stream) {
  fp4g_status st = check_weight(Wg, true);
  if (st != FP4G_OK) return st;
  st = check_weight(Wu, true);
  if (st != FP4G_OK) return st;
  if (Wg->format != Wu->format) return FP4G_E_FORMAT;
  if (Wg->d_out != Wu->d_out || Wg->d_in != Wu->d_in) return FP4G_E_SHAPE;
  if (!X || !H) return FP4G_E_NULL;
  if (M < 1 || M > kMaxM) return FP4G_E_SHAPE;
  if (path != FP4G_PATH_AUTO && path != FP4G_PATH_VALU) return FP4G_E_PATH;
  if (!aligned(X, 16) || !aligned(H, 16)) return FP4G_E_ALIGN;
  const int64_t R = row_groups(Wg->d_out), C = chunks(Wg->d_in);
  const uint64_t need = gemv_ws_bytes(R, C, 2, M);
  if (need && !ws) return FP4G_E_NULL;
  if (ws_bytes < need) return FP4G_E_WORKSPACE;
  if (need && !aligned(ws, 256)) return FP4G_E_ALIGN;
  const size_t hbytes = (size_t)M * Wg->d_out * 2, xbytes = (size_t)M * Wg->d_in * 2;
  if (overlap(H, hbytes, X, xbytes) || overlap(H, hbytes, Wg->packed, Wg->packed_bytes) ||
      overlap(H, hbytes, Wu->packed, Wu->packed_bytes) || overlap(H, hbytes, ws, need) ||
      overlap(ws, need, X, xbytes) || overlap(ws, need, Wg->packed, Wg->packed_bytes) ||
      overlap(ws, need, Wu->packed, Wu->packed_bytes))
    return FP4G_E_ALIAS;
  const Plan pl = plan_for(R, C, 2);
  GemvParams p{};
  p.w[0] = (const uint8_t*)Wg->packed;
  p.w[1] = (const uint8_t*)Wu->packed;
  p.tscale[0] = Wg->tensor_scale;
  p.tscale[1] = Wu->tensor_scale;
  p.x = X;
  p.h = H;
  p.counters = (unsigned*)ws;
  p.part = need ? (float*)((uint8_t*)ws + kCounterBytes) : nullptr;
  p.d_out = Wg->d_out;
  p.d_in = Wg->d_in;
  p.R = (int)R;
  p.C = (int)C;
  p.S = pl.S;
  p.wg_chunks = pl.wg_chunks;
  const unsigned grid = (unsigned)(R * pl.S);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = Wg->format == FP4G_NVFP4 ? launch_m<FP4G_NVFP4, 2, EPI_SILU>(M, p, grid, s)
                                          : launch_m<FP4G_MXFP4, 2, EPI_SILU>(M, p, grid, s);
  return e == hipSuccess ? FP4G_OK : FP4G_E_HIP;
}

uint64_t fp4g_workspace_bytes(int32_t op, const void* desc, int32_t M) {
  if (!desc || M < 1 || M > kMaxM) return 0;
  if (op == FP4G_OP_MOE) return moe_ws_bytes((const fp4g_moe*)desc, M);
  const fp4g_weight* W = (const fp4g_weight*)desc;
  const bool fp4 = op != FP4G_OP_LMHEAD;
  if (op != FP4G_OP_GEMV && op != FP4G_OP_GATE_UP && op != FP4G_OP_LMHEAD) return 0;
  if (check_weight(W, fp4) != FP4G_OK) return 0;
  return gemv_ws_bytes(row_groups(W->d_out), chunks(W->d_in), op == FP4G_OP_GATE_UP ? 2 : 1, M);
}

}  // extern "C"
