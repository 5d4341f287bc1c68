// gemv_mfma_mxfp4_silu.hip -- MXFP4 fused gate/up + SiLU instantiations of the matrix-core kernel (gemv_mfma.hpp).
#include "gemv_mfma.hpp"

namespace fp4g {
template hipError_t launch_mfma<FP4G_MXFP4, 2, EPI_SILU>(int, const GemvParams&, unsigned, size_t, hipStream_t);
}  // namespace fp4g
