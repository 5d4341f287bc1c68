// gemv_nvfp4.hip -- instantiations of the decode GEMV kernel for NVFP4 weights.
#include "gemv_kernel.hpp"

namespace fp4g {
template hipError_t launch_m<FP4G_NVFP4, 1, EPI_STORE>(int, int, const GemvParams&, unsigned, hipStream_t);
template hipError_t launch_m<FP4G_NVFP4, 2, EPI_SILU>(int, int, const GemvParams&, unsigned, hipStream_t);
}  // namespace fp4g
