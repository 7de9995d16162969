// e5m2 x e4m3 GEMMs (both operands K-major) of the backward with fp8 gradients: dout_q W2^T_q with
// the quantizing d-ReLU^2 epilogue, and the dx / dW1 / dW2 products with the scaled store
// (bf16, or fp32 accumulate) or split-K partials.
#include "gemm_dma.hpp"
#include "launch.hpp"

namespace gmlp {

template <int BM, int BN, int W>
static hipError_t dispatch(DType io, int epi, const GemmArgs& a, int grid, hipStream_t s) {
  switch (epi) {
    case EPI_F8DACT:   // io: the type of the pre-activation it reads
      if (io == DT_BF16) return launch_gemm_dma<f8g, bf16, BM, BN, true, true, EPI_F8DACT, W>(a, grid, s);
      if (io == DT_F32) return launch_gemm_dma<f8g, float, BM, BN, true, true, EPI_F8DACT, W>(a, grid, s);
      return hipErrorInvalidValue;
    case EPI_STORE:
      if (io == DT_BF16) return launch_gemm_dma<f8g, bf16, BM, BN, true, true, EPI_STORE, W>(a, grid, s);
      if (io == DT_F32) return launch_gemm_dma<f8g, float, BM, BN, true, true, EPI_STORE, W>(a, grid, s);
      return hipErrorInvalidValue;
    case EPI_PARTIAL: return launch_gemm_dma<f8g, float, BM, BN, true, true, EPI_PARTIAL, W>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t run_gemm_f8g_nt(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s) {
  switch (tile) {
    case TILE_256x256: return dispatch<256, 256, 4>(io, epi, a, grid, s);
    case TILE_256x128: return dispatch<256, 128, 4>(io, epi, a, grid, s);
    case TILE_128x128: return dispatch<128, 128, 4>(io, epi, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gmlp
