// gemv_mfma_moe.hip -- the mixture-of-experts gate/up and down instantiations of the matrix-core kernel (gemv_mfma.hpp).
#include "gemv_mfma.hpp"

namespace fp4g {
template hipError_t launch_mfma_moe<FP4G_NVFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t, hipStream_t);
template hipError_t launch_mfma_moe<FP4G_MXFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t, hipStream_t);
template hipError_t launch_mfma_moe_down<FP4G_NVFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                     hipStream_t);
template hipError_t launch_mfma_moe_down<FP4G_MXFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                     hipStream_t);
}  // namespace fp4g
