// e4m3 x e4m3 GEMMs (both operands K-major) of the ReLU^2 forward: x_q W1_q^T with the
// quantizing ReLU^2 epilogue (pre-activation kept in bf16, or fp32 for the fp8-gradient
// backward), and post_q W2_q^T with the scaled bf16 store (fp32: the recomputed pre-activation).
#include "gemm_dma.hpp"
#include "launch.hpp"

namespace gmlp {

template <int BM, int BN, int W>
static hipError_t dispatch(DType io, int epi, const GemmArgs& a, int grid, hipStream_t s) {
  switch (epi) {
    case EPI_F8ACT:   // io: the type the pre-activation is kept in (bf16; fp32 for the fp8-gradient backward)
      if (io == DT_BF16) return launch_gemm_dma<e4m3, bf16, BM, BN, true, true, EPI_F8ACT, W>(a, grid, s);
      if (io == DT_F32) return launch_gemm_dma<e4m3, float, BM, BN, true, true, EPI_F8ACT, W>(a, grid, s);
      return hipErrorInvalidValue;
    case EPI_STORE:
      if (io == DT_BF16) return launch_gemm_dma<e4m3, bf16, BM, BN, true, true, EPI_STORE, W>(a, grid, s);
      if (io == DT_F32) return launch_gemm_dma<e4m3, float, BM, BN, true, true, EPI_STORE, W>(a, grid, s);
      return hipErrorInvalidValue;
    case EPI_PARTIAL: return launch_gemm_dma<e4m3, float, BM, BN, true, true, EPI_PARTIAL, W>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t run_gemm_e4m3_nt(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s) {
  switch (tile) {
    case TILE_256x256: return dispatch<256, 256, 4>(io, epi, a, grid, s);
    case TILE_256x128: return dispatch<256, 128, 4>(io, epi, a, grid, s);
    case TILE_128x128: return dispatch<128, 128, 4>(io, epi, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gmlp
