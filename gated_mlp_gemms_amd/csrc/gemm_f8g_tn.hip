// e5m2 x e4m3 weight-gradient GEMMs of the backward with fp8 gradients, both operands read along
// the tokens from their row-major codes (MN-major: dW1 = dpre_q^T x_q, dW2 = dout_q^T post_q),
// through the 8-bit transposing LDS read; scaled store (bf16, or fp32 accumulate) or split-K
// partials.
#include "gemm_dma.hpp"
#include "launch.hpp"

namespace gmlp {

template <int BM, int BN, int W>
static hipError_t dispatch(DType io, int epi, const GemmArgs& a, int grid, hipStream_t s) {
  switch (epi) {
    case EPI_STORE:
      if (io == DT_BF16) return launch_gemm_dma<f8g, bf16, BM, BN, false, false, EPI_STORE, W>(a, grid, s);
      if (io == DT_F32) return launch_gemm_dma<f8g, float, BM, BN, false, false, EPI_STORE, W>(a, grid, s);
      return hipErrorInvalidValue;
    case EPI_PARTIAL: return launch_gemm_dma<f8g, float, BM, BN, false, false, EPI_PARTIAL, W>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t run_gemm_f8g_tn(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s) {
  switch (tile) {
    case TILE_256x256: return dispatch<256, 256, 4>(io, epi, a, grid, s);
    case TILE_256x128: return dispatch<256, 128, 4>(io, epi, a, grid, s);
    case TILE_128x128: return dispatch<128, 128, 4>(io, epi, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gmlp
