// Launch tables of the 16-bit (bf16 / fp16) GEMMs: per layout, the fused epilogues it serves,
// per tile shape the workgroup geometry. One translation unit instantiates each (type, layout).
//   NT (x W^T): the fused gate/up and non-gated forward, the down projection;
//   NN (dout W, dpreact W): the fused d-activation backward and dx;
//   TN (dout^T a, dpreact^T x): the weight gradients, in the I/O type or added into fp32.
#pragma once

#include "gemm_dma.hpp"
#include "launch.hpp"

namespace gmlp {

template <typename T> constexpr DType dtype_of();
template <> constexpr DType dtype_of<bf16>() { return DT_BF16; }
template <> constexpr DType dtype_of<f16>() { return DT_F16; }

template <typename T, int LAYOUT, int BM, int BN, int W>
hipError_t dispatch16(DType io, int epi, const GemmArgs& a, int grid, hipStream_t s) {
  constexpr bool AK = LAYOUT != TN, BK = LAYOUT == NT;
  const bool own = io == dtype_of<T>();
  switch (epi) {
    case EPI_PARTIAL: return launch_gemm_dma<T, float, BM, BN, AK, BK, EPI_PARTIAL, W>(a, grid, s);
    case EPI_STORE:
      if (own) return launch_gemm_dma<T, T, BM, BN, AK, BK, EPI_STORE, W>(a, grid, s);
      if constexpr (LAYOUT == TN) {
        if (io == DT_F32) return launch_gemm_dma<T, float, BM, BN, AK, BK, EPI_STORE, W>(a, grid, s);
      }
      return hipErrorInvalidValue;
    default: break;
  }
  if constexpr (LAYOUT == NT) {
    if (epi == EPI_GATED) return launch_gemm_dma<T, T, BM, BN, true, true, EPI_GATED, W>(a, grid, s);
    if (epi == EPI_ACT) return launch_gemm_dma<T, T, BM, BN, true, true, EPI_ACT, W>(a, grid, s);
  } else if constexpr (LAYOUT == NN) {
    if (epi == EPI_DGATED) return launch_gemm_dma<T, T, BM, BN, true, false, EPI_DGATED, W>(a, grid, s);
    if (epi == EPI_DACT) return launch_gemm_dma<T, T, BM, BN, true, false, EPI_DACT, W>(a, grid, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int LAYOUT>
hipError_t run_gemm16(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s) {
  switch (tile) {
    case TILE_256x256: return dispatch16<T, LAYOUT, 256, 256, 4>(io, epi, a, grid, s);
    case TILE_256x128: return dispatch16<T, LAYOUT, 256, 128, 4>(io, epi, a, grid, s);
    case TILE_128x128: return dispatch16<T, LAYOUT, 128, 128, 4>(io, epi, a, grid, s);
    case TILE_256x256_W8: return dispatch16<T, LAYOUT, 256, 256, 8>(io, epi, a, grid, s);
    case TILE_256x128_W8: return dispatch16<T, LAYOUT, 256, 128, 8>(io, epi, a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gmlp
