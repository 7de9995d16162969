// bf16 GEMMs in the NN layout (launch table: gemm_dispatch16.hpp).
#include "gemm_dispatch16.hpp"

namespace gmlp {

hipError_t run_gemm_bf16_nn(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s) {
  return run_gemm16<bf16, NN>(io, epi, tile, a, grid, s);
}

}  // namespace gmlp
