// fp32 GEMMs (fp32 MFMA; CDNA4 has no reduced-precision fp32 mode) for every layout and
// epilogue, 128 x 128 tiles.
#include "gemm_kernel.hpp"
#include "launch.hpp"

namespace gmlp {

hipError_t run_gemm_f32(Layout layout, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s) {
  if (tile != TILE_128x128) return hipErrorInvalidValue;
  constexpr int B = 128;
  switch (layout) {
    case NT:
      switch (epi) {
        case EPI_GATED: return launch_gemm<float, float, B, B, true, true, EPI_GATED>(a, grid, s);
        case EPI_ACT: return launch_gemm<float, float, B, B, true, true, EPI_ACT>(a, grid, s);
        case EPI_STORE: return launch_gemm<float, float, B, B, true, true, EPI_STORE>(a, grid, s);
        case EPI_PARTIAL: return launch_gemm<float, float, B, B, true, true, EPI_PARTIAL>(a, grid, s);
        default: return hipErrorInvalidValue;
      }
    case NN:
      switch (epi) {
        case EPI_DGATED: return launch_gemm<float, float, B, B, true, false, EPI_DGATED>(a, grid, s);
        case EPI_DACT: return launch_gemm<float, float, B, B, true, false, EPI_DACT>(a, grid, s);
        case EPI_STORE: return launch_gemm<float, float, B, B, true, false, EPI_STORE>(a, grid, s);
        case EPI_PARTIAL: return launch_gemm<float, float, B, B, true, false, EPI_PARTIAL>(a, grid, s);
        default: return hipErrorInvalidValue;
      }
    case TN:
      switch (epi) {
        case EPI_STORE: return launch_gemm<float, float, B, B, false, false, EPI_STORE>(a, grid, s);
        case EPI_PARTIAL: return launch_gemm<float, float, B, B, false, false, EPI_PARTIAL>(a, grid, s);
        default: return hipErrorInvalidValue;
      }
  }
  return hipErrorInvalidValue;
}

}  // namespace gmlp
