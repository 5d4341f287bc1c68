// gemv_fp8.hip -- instantiations of the decode GEMV kernel for FP8_ROW weights.
#include "gemv_kernel.hpp"

namespace fp4g {
template hipError_t launch_m<FP4G_FP8_ROW, 1, EPI_STORE>(int, int, const GemvParams&, unsigned, hipStream_t);
template hipError_t launch_m<FP4G_FP8_ROW, 1, EPI_ARGMAX>(int, int, const GemvParams&, unsigned, hipStream_t);
}  // namespace fp4g
