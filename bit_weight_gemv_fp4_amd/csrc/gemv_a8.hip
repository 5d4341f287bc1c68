// gemv_a8.hip -- the W4A8 kernel's instantiations (gemv_a8.hpp).
#include "gemv_a8.hpp"

namespace fp4g {
hipError_t launch_a8_ext(int M, const GemvParams& p, unsigned grid, size_t lds, hipStream_t s) {
  return launch_a8<1, EPI_STORE>(M, p, grid, lds, s);
}
hipError_t launch_a8_silu_ext(int M, const GemvParams& p, unsigned grid, size_t lds, hipStream_t s) {
  return launch_a8<2, EPI_SILU>(M, p, grid, lds, s);
}
}  // namespace fp4g
