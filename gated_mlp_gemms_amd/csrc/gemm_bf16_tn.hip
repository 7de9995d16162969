// bf16 GEMMs with both operands MN-major (dout^T a, dpreact^T x): the weight gradients,
// written in bf16 or added into fp32 buffers, and their split-K partial form.
#include "gemm_dma.hpp"
#include "launch.hpp"

namespace gmlp {

template <int BM, int BN, int W>
static hipError_t dispatch(DType io, int epi, const GemmArgs& a, int grid, hipStream_t s) {
  switch (epi) {
    case EPI_STORE:
      if (io == DT_BF16) return launch_gemm_dma<bf16, bf16, BM, BN, false, false, EPI_STORE, W>(a, grid, s);
      return launch_gemm_dma<bf16, float, BM, BN, false, false, EPI_STORE, W>(a, grid, s);
    case EPI_PARTIAL: return launch_gemm_dma<bf16, float, BM, BN, false, false, EPI_PARTIAL, W>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t run_gemm_bf16_tn(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s) {
  switch (tile) {
    case TILE_256x256: return dispatch<256, 256, 4>(io, epi, a, grid, s);
    case TILE_256x128: return dispatch<256, 128, 4>(io, epi, a, grid, s);
    case TILE_128x128: return dispatch<128, 128, 4>(io, epi, a, grid, s);
    case TILE_256x256_W8: return dispatch<256, 256, 8>(io, epi, a, grid, s);
    case TILE_256x128_W8: return dispatch<256, 128, 8>(io, epi, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gmlp
