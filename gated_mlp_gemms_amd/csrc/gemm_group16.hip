// The 16-bit backward's dx and weight-gradient GEMMs as one grouped launch
// (gemm_dma_group_kernel, 8-wave 256 x 256 tiles, store epilogue): tile body 0 is the NN product
// dx = dpreact [W_gate; W_up] in the I/O type, tile body 1 the TN products dW = dpreact^T x and
// dout^T a, in the I/O type or added into fp32 (accumulate).
#include "gemm_dma.hpp"
#include "launch.hpp"

namespace gmlp {

template <typename T>
static hipError_t group16(DType gio, const GemmGroup& g, hipStream_t s) {
  if (gio == DT_F32) return launch_gemm_dma_group<T, 256, 256, 8, T, true, false, float, false, false>(g, s);
  return launch_gemm_dma_group<T, 256, 256, 8, T, true, false, T, false, false>(g, s);
}

hipError_t run_gemm_group16(DType in, DType gio, const GemmGroup& g, hipStream_t s) {
  if (g.count < 1 || g.count > kGroupMax) return hipErrorInvalidValue;
  if (in == DT_BF16 && (gio == DT_BF16 || gio == DT_F32)) return group16<bf16>(gio, g, s);
  if (in == DT_F16 && (gio == DT_F16 || gio == DT_F32)) return group16<f16>(gio, g, s);
  return hipErrorInvalidValue;
}

}  // namespace gmlp
