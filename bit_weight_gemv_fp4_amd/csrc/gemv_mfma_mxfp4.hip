// gemv_mfma_mxfp4.hip -- MXFP4 plain-product instantiations of the matrix-core kernel (gemv_mfma.hpp).
#include "gemv_mfma.hpp"

namespace fp4g {
template hipError_t launch_mfma<FP4G_MXFP4, 1, EPI_STORE>(int, const GemvParams&, unsigned, size_t, hipStream_t);
}  // namespace fp4g
