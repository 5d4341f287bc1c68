// gemv_mfma_moe_wide.hip -- the mixture-of-experts instantiations of the matrix-core kernel for 9..16 tokens.
#include "gemv_mfma.hpp"

namespace fp4g {
template hipError_t launch_mfma_moe_wide<FP4G_NVFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                     hipStream_t);
template hipError_t launch_mfma_moe_wide<FP4G_MXFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                     hipStream_t);
template hipError_t launch_mfma_moe_down_wide<FP4G_NVFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                          hipStream_t);
template hipError_t launch_mfma_moe_down_wide<FP4G_MXFP4>(int, const GemvParams&, const MfmaMoe&, unsigned, size_t,
                                                          hipStream_t);
}  // namespace fp4g
