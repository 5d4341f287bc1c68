// gemv_fp8_silu.hip -- the fused gate/up + SiLU instantiations of the decode GEMV kernel for FP8_ROW weights.
#include "gemv_kernel.hpp"

namespace fp4g {
template hipError_t launch_m<FP4G_FP8_ROW, 2, EPI_SILU>(int, int, const GemvParams&, unsigned, hipStream_t);
}  // namespace fp4g
