// Host-side declarations of every kernel launch the C-ABI layer uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_args.hpp"

namespace gmlp {

// DT_F8G: the fp8-gradient GEMM operand pair (A e5m2, B e4m3); an input type only.
enum DType : int { DT_F32 = 0, DT_BF16 = 1, DT_E4M3 = 2, DT_F16 = 3, DT_F8G = 4 };
enum Layout : int { NT = 0, NN = 1, TN = 2 };   // A K-major/B K-major, A K/B MN, A MN/B MN
// Tile shapes of the bf16 / e4m3 kernel; _W8 runs the tile with 8 waves (two per SIMD).
enum TileShape : int {
  TILE_256x256 = 0, TILE_256x128 = 1, TILE_128x128 = 2, TILE_256x256_W8 = 3, TILE_256x128_W8 = 4, TILE_COUNT = 5
};

// One GEMM launch. `io` is the element type of the epilogue's stored/loaded tensors (for
// EPI_STORE the output type; accumulate mode needs DT_F32). Returns hipErrorInvalidValue for a
// combination that has no instantiation.
hipError_t run_gemm(DType in, DType io, Layout layout, int epi, TileShape tile, const GemmArgs& a,
                    int grid, hipStream_t stream);

// Per-(input dtype, layout) launchers, one translation unit each.
hipError_t run_gemm_bf16_nt(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s);
hipError_t run_gemm_bf16_nn(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s);
hipError_t run_gemm_bf16_tn(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s);
hipError_t run_gemm_f16_nt(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s);
hipError_t run_gemm_f16_nn(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s);
hipError_t run_gemm_f16_tn(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s);
hipError_t run_gemm_f32(Layout layout, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s);
hipError_t run_gemm_e4m3_nt(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s);
hipError_t run_gemm_f8g_nt(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s);
hipError_t run_gemm_f8g_tn(DType io, int epi, TileShape tile, const GemmArgs& a, int grid, hipStream_t s);

// Independent GEMMs of the 16-bit backward in one launch of 8-wave 256 x 256 tiles (GemmGroup):
// kind 0 an NN product with epilogue epi0 (EPI_STORE: dx; EPI_DGATED / EPI_DACT: the
// d-activation GEMM), output `in`; kind 1 a TN weight gradient with the store epilogue, output
// gio (`in`, or DT_F32 to accumulate).
hipError_t run_gemm_group16(DType in, DType gio, int epi0, const GemmGroup& g, hipStream_t s);

// Products with at most kSkinnyMaxRows rows (decode-size token counts), K-major A [M, K] and
// B [N, K] (gated: B0 gate rows, B1 up rows), in `in` = DT_BF16 / DT_F16; K a multiple of 8.
// Epilogues EPI_STORE (C0 = alpha * A B^T), EPI_ACT and EPI_GATED with GemmArgs::flags as in the
// GEMM kernels (bit 0: the pre-activation into aux, bit 1: the activation into C0).
constexpr int kSkinnyMaxRows = 16;
hipError_t run_skinny(DType in, int epi, const GemmArgs& a, hipStream_t s);
// EPI_PARTIAL: the store product with K split over kSkinnyParts workgroups per column block,
// unscaled fp32 partial sums into a.partial [kSkinnyParts][M][N] (then the split-K reduce).
// Taken above 8 tokens for narrow outputs with a long K (skinny_parts_for), where the whole-K
// form has few column blocks and each of them re-reads all of the token rows. LLaMA widths, same
// box: 16 tokens 60.8 -> 57.5 us per inference forward; 8 and 1 tokens 54.3 -> 56.4 and 48.6 ->
// 53.1 us (few token rows to save, one more launch), hence the threshold.
constexpr int kSkinnyParts = 4;
inline bool skinny_parts_for(int64_t M, int64_t N, int64_t K) { return M > 8 && N <= 8192 && K >= 2048; }

// out = alpha * sum_s partial[s] (fixed order), stored as `io` or added into fp32 (accumulate).
// Rows >= c_split go to C1 (row - c_split).
hipError_t run_splitk_reduce(DType io, const float* partial, int splits, int M, int N, void* C0,
                             void* C1, int64_t ldc, int c_split, float alpha, const float* dev0,
                             const float* dev1, int accumulate, hipStream_t s);

// Split-K finish of the gated up projection: g|u = alpha * sum of the fp32 partials [s][M][2H] in
// order; g|u -> preact [M, 2H] when non-NULL; a = act(g, u) -> a [M, H].
hipError_t run_gated_reduce(DType io, const float* partial, int splits, int M, int H, float alpha,
                            const float* dev0, const float* dev1, void* preact, void* a, float gate_mult,
                            int gate_inside, int fn, hipStream_t s);

// a[m][n] = act(g = pre[m][n], u = pre[m][H + n]) (gated), or post = f(alpha * pre); fn: ActFn.
hipError_t run_gated_act(DType io, const void* preact, void* a, int M, int H, float gate_mult,
                         int gate_inside, int fn, hipStream_t s);
hipError_t run_plain_act(DType io, const void* pre, void* post, int64_t n, float alpha,
                         const float* dev0, const float* dev1, int fn, hipStream_t s);

// Per-tensor e4m3 quantization: amax (into ws[0], from per-workgroup maxima in ws[64 ..
// 64 + kQuantizeParts)), then scale and codes. The workspace holds kQuantizeWsBytes.
constexpr int kQuantizeParts = 2048;
constexpr size_t kQuantizeWsBytes = 256 + kQuantizeParts * sizeof(float);
hipError_t run_quantize_e4m3(DType src_t, const void* src, int64_t n, void* dst, float* scale,
                             float* ws, hipStream_t s);
// Exact e4m3 -> bf16 widening (every e4m3 value is a bf16 value).
hipError_t run_dequant_e4m3_bf16(const void* src, void* dst, int64_t n, hipStream_t s);

// fp8 codes of a [rows, cols] row-major matrix (leading dimension ld_src elements), in row-major
// form (dst, leading dimension cols; may be NULL) and transposed (dst_t [cols, ld_t], ld_t >= rows
// a multiple of 16, columns rows .. ld_t-1 zero; may be NULL). src_t: DT_BF16 or DT_F32 (value
// v). relu_sq: quantize max(v, 0)^2 instead of v.
// e5m2: OCP E5M2 codes, else E4M3; code = fmt(v / *scale). cols must be a multiple of 16.
hipError_t run_quantize_fp8_2d(DType src_t, const void* src, int64_t rows, int64_t cols, int64_t ld_src,
                               int relu_sq, int e5m2, const float* scale, void* dst, void* dst_t,
                               int64_t ld_t, hipStream_t s);

// The fp8 weight-cache quantizer (row-major codes into dst, transposed into dst_t; either may be
// NULL): exact = 1 forms *scale from w's own amax (an amax pass first), exact = 0 from the per-tile
// amax the previous call recorded in tile_amax (weight_amax_slots(rows, cols) floats); both record
// w's per-tile amax there. src_t: DT_BF16 or DT_F32; cols a multiple of 16.
int64_t weight_amax_slots(int64_t rows, int64_t cols);
hipError_t run_quantize_weight_e4m3(DType src_t, const void* w, int64_t rows, int64_t cols, int exact, float* scale,
                                    float* tile_amax, void* dst, void* dst_t, int64_t ld_t, hipStream_t s);

}  // namespace gmlp
