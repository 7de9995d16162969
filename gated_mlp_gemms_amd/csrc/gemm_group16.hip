// Grouped launches of the 16-bit backward (gemm_dma_group_kernel, 8-wave 256 x 256 tiles):
// tile body 0 is an NN product with the epilogue epi0 in the I/O type (dx = dpreact
// [W_gate; W_up] with the store epilogue, or dout W_down with the d-activation epilogue), tile
// body 1 a TN weight gradient (dpreact^T x, dout^T a) with the store epilogue, in the I/O type or
// added into fp32 (accumulate).
#include "gemm_dma.hpp"
#include "launch.hpp"

namespace gmlp {

template <typename T, int EPI0>
static hipError_t group16(DType gio, const GemmGroup& g, hipStream_t s) {
  if (gio == DT_F32)
    return launch_gemm_dma_group<T, 256, 256, 8, T, true, false, EPI0, float, false, false, EPI_STORE>(g, s);
  return launch_gemm_dma_group<T, 256, 256, 8, T, true, false, EPI0, T, false, false, EPI_STORE>(g, s);
}

template <typename T>
static hipError_t group16_epi(int epi0, DType gio, const GemmGroup& g, hipStream_t s) {
  switch (epi0) {
    case EPI_STORE: return group16<T, EPI_STORE>(gio, g, s);
    case EPI_DGATED: return group16<T, EPI_DGATED>(gio, g, s);
    case EPI_DACT: return group16<T, EPI_DACT>(gio, g, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t run_gemm_group16(DType in, DType gio, int epi0, const GemmGroup& g, hipStream_t s) {
  if (g.count < 1 || g.count > kGroupMax) return hipErrorInvalidValue;
  if (in == DT_BF16 && (gio == DT_BF16 || gio == DT_F32)) return group16_epi<bf16>(epi0, gio, g, s);
  if (in == DT_F16 && (gio == DT_F16 || gio == DT_F32)) return group16_epi<f16>(epi0, gio, g, s);
  return hipErrorInvalidValue;
}

}  // namespace gmlp
