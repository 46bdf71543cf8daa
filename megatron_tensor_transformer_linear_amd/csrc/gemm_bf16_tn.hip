// bf16 GEMM kernels of layout LAY_TN (A read M-contiguous: dW = X^T . dY, the
// weight-gradient products).  The kernel is in
// gemm_bf16_kernel.hpp; this unit only instantiates it, so the layouts compile in parallel.
#include "gemm_bf16_kernel.hpp"

namespace tpk {

hipError_t launch_shape_tn(int bm, int bn, const GemmDesc& g, hipStream_t stream) {
  return launch_shape_t<LAY_TN>(bm, bn, g, stream);
}

}  // namespace tpk
