// gemv_a8_moe.hip -- the W4A8 kernel's mixture-of-experts instantiations (gemv_a8.hpp).
#include "gemv_a8.hpp"

namespace fp4g {
hipError_t launch_a8_moe_up_ext(int M, const GemvParams& p, const MfmaMoe& q, unsigned grid, size_t lds,
                                hipStream_t s) {
  return launch_a8_moe<1>(M, p, q, grid, lds, s);
}
hipError_t launch_a8_moe_down_ext(int M, const GemvParams& p, const MfmaMoe& q, unsigned grid, size_t lds,
                                  hipStream_t s) {
  return launch_a8_moe<2>(M, p, q, grid, lds, s);
}
}  // namespace fp4g
