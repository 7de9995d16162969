// Memory-bound helper kernels of the MLP engine: the split-K reduction, the activation-only
// pass of the "only dW_down" backward branch, and e4m3 quantize / widen.
#include "common.hpp"
#include "launch.hpp"

#include <algorithm>

namespace gmlp {

namespace {

constexpr int kEwThreads = 256;

inline int ew_grid(int64_t items) {
  int64_t g = (items + kEwThreads - 1) / kEwThreads;
  const int64_t cap = 256 * 64;   // 64 workgroups per CU is plenty for a streaming pass
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

template <typename T> __device__ __forceinline__ void load4(const void* p, float v[4]);
template <> __device__ __forceinline__ void load4<float>(const void* p, float v[4]) {
  f32x4 x = *reinterpret_cast<const f32x4*>(p);
  v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
}
template <typename T> __device__ __forceinline__ void load4_16(const void* p, float v[4]) {
  u32x2 x = *reinterpret_cast<const u32x2*>(p);
  v[0] = Bits16<T>::to_f32(x[0] & 0xffffu); v[1] = Bits16<T>::to_f32(x[0] >> 16);
  v[2] = Bits16<T>::to_f32(x[1] & 0xffffu); v[3] = Bits16<T>::to_f32(x[1] >> 16);
}
template <> __device__ __forceinline__ void load4<bf16>(const void* p, float v[4]) { load4_16<bf16>(p, v); }
template <> __device__ __forceinline__ void load4<f16>(const void* p, float v[4]) { load4_16<f16>(p, v); }
template <typename T> __device__ __forceinline__ void store4(void* p, const float v[4]);
template <> __device__ __forceinline__ void store4<float>(void* p, const float v[4]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
}
template <typename T> __device__ __forceinline__ void store4_16(void* p, const float v[4]) {
  *reinterpret_cast<u32x2*>(p) = u32x2{pack16x2<T>(v[0], v[1]), pack16x2<T>(v[2], v[3])};
}
template <> __device__ __forceinline__ void store4<bf16>(void* p, const float v[4]) { store4_16<bf16>(p, v); }
template <> __device__ __forceinline__ void store4<f16>(void* p, const float v[4]) { store4_16<f16>(p, v); }
template <typename T> constexpr int esize() { return sizeof(T) == 4 ? 4 : 2; }

// ---- split-K reduction: fixed summation order over the splits -----------------------------

template <typename OutT>
__global__ __launch_bounds__(kEwThreads) void splitk_reduce_kernel(
    const float* __restrict__ partial, int splits, int M, int N, void* C0, void* C1, int64_t ldc,
    int c_split, float alpha, const float* dev0, const float* dev1, int accumulate) {
  float a = alpha;
  if (dev0) a *= *dev0;
  if (dev1) a *= *dev1;
  const int n4 = N / 4;
  const int64_t total = (int64_t)M * n4;
  const int64_t plane = (int64_t)M * N;
  for (int64_t i = blockIdx.x * (int64_t)kEwThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kEwThreads) {
    const int m = (int)(i / n4), n = (int)(i % n4) * 4;
    const float* src = partial + (int64_t)m * N + n;
    f32x4 s = *reinterpret_cast<const f32x4*>(src);
    for (int k = 1; k < splits; ++k) s += *reinterpret_cast<const f32x4*>(src + k * plane);
    float v[4] = {a * s[0], a * s[1], a * s[2], a * s[3]};
    const bool lo = m < c_split;
    char* row = reinterpret_cast<char*>(lo ? C0 : C1) + (int64_t)(lo ? m : m - c_split) * ldc * esize<OutT>();
    if (accumulate) {
      float* q = reinterpret_cast<float*>(row) + n;
      f32x4 o = *reinterpret_cast<f32x4*>(q);
      o[0] += v[0]; o[1] += v[1]; o[2] += v[2]; o[3] += v[3];
      *reinterpret_cast<f32x4*>(q) = o;
    } else {
      store4<OutT>(row + (int64_t)n * esize<OutT>(), v);
    }
  }
}

// ---- split-K reduce of the gated up projection ------------------------------------------------
// partial[s][m][0 .. 2H) holds unscaled sums over K-slice s of [g | u]; g, u = alpha * (sum over s
// in order); [g | u] -> preact (when given), a = act(g, u) -> a_out.
template <typename T>
__global__ __launch_bounds__(kEwThreads) void gated_reduce_kernel(const float* partial, int splits, int M,
                                                                  int H, float alpha, const float* dev0,
                                                                  const float* dev1, void* preact, void* a_out,
                                                                  float gm, int inside, int fn) {
  float al = alpha;
  if (dev0) al *= *dev0;
  if (dev1) al *= *dev1;
  const int h4 = H / 4;
  const int64_t total = (int64_t)M * h4;
  const int64_t slice = (int64_t)M * 2 * H;
  for (int64_t i = blockIdx.x * (int64_t)kEwThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kEwThreads) {
    const int m = (int)(i / h4), n = (int)(i % h4) * 4;
    const float* row = partial + (int64_t)m * 2 * H;
    f32x4 g = *reinterpret_cast<const f32x4*>(row + n), u = *reinterpret_cast<const f32x4*>(row + H + n);
    for (int sp = 1; sp < splits; ++sp) {
      g += *reinterpret_cast<const f32x4*>(row + sp * slice + n);
      u += *reinterpret_cast<const f32x4*>(row + sp * slice + H + n);
    }
    float gv[4], uv[4], a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) { gv[r] = al * g[r]; uv[r] = al * u[r]; }
    if (preact) {
      char* prow = reinterpret_cast<char*>(preact) + (int64_t)m * 2 * H * esize<T>();
      store4<T>(prow + (int64_t)n * esize<T>(), gv);
      store4<T>(prow + (int64_t)(H + n) * esize<T>(), uv);
    }
    gated_act<4>(fn, gm, inside, gv, uv, a);
    store4<T>(reinterpret_cast<char*>(a_out) + ((int64_t)m * H + n) * esize<T>(), a);
  }
}

// ---- activation only -------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(kEwThreads) void gated_act_kernel(const void* preact, void* a_out, int M,
                                                               int H, float gm, int inside, int fn) {
  const int h4 = H / 4;
  const int64_t total = (int64_t)M * h4;
  for (int64_t i = blockIdx.x * (int64_t)kEwThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kEwThreads) {
    const int m = (int)(i / h4), n = (int)(i % h4) * 4;
    const char* row = reinterpret_cast<const char*>(preact) + (int64_t)m * 2 * H * esize<T>();
    float g[4], u[4], a[4];
    load4<T>(row + (int64_t)n * esize<T>(), g);
    load4<T>(row + (int64_t)(H + n) * esize<T>(), u);
    gated_act<4>(fn, gm, inside, g, u, a);
    store4<T>(reinterpret_cast<char*>(a_out) + ((int64_t)m * H + n) * esize<T>(), a);
  }
}

template <typename T>
__global__ __launch_bounds__(kEwThreads) void plain_act_kernel(const void* pre, void* post, int64_t n,
                                                               float alpha, const float* dev0,
                                                               const float* dev1, int fn) {
  float a = alpha;
  if (dev0) a *= *dev0;
  if (dev1) a *= *dev1;
  const int64_t n4 = n / 4;
  for (int64_t i = blockIdx.x * (int64_t)kEwThreads + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * kEwThreads) {
    float v[4];
    load4<T>(reinterpret_cast<const char*>(pre) + i * 4 * esize<T>(), v);
    float z[4], f[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) z[r] = a * v[r];
    act_fn<4>(fn, z, f);
    store4<T>(reinterpret_cast<char*>(post) + i * 4 * esize<T>(), f);
  }
}

// ---- e4m3 quantize ---------------------------------------------------------------------------

__global__ void zero_f32_kernel(float* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0.0f;
}

template <typename T> __device__ __forceinline__ float load1(const void* p, int64_t i);
template <> __device__ __forceinline__ float load1<float>(const void* p, int64_t i) {
  return reinterpret_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float load1<bf16>(const void* p, int64_t i) {
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float load1<f16>(const void* p, int64_t i) {
  return Bits16<f16>::to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}

template <typename T>
__global__ __launch_bounds__(kEwThreads) void absmax_kernel(const void* src, int64_t n, float* amax) {
  float m = 0.0f;
  for (int64_t i = blockIdx.x * (int64_t)kEwThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kEwThreads)
    m = fmaxf(m, __builtin_fabsf(load1<T>(src, i)));
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float part[kEwThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kEwThreads / 64; ++w) m = fmaxf(m, part[w]);
    amax_update(amax, m);
  }
}

// scale = max(amax, 1e-12) / 448 (fp32, correctly rounded); q = e4m3(v / scale).
template <typename T>
__global__ __launch_bounds__(kEwThreads) void quantize_kernel(const void* src, int64_t n, uint8_t* dst,
                                                              const float* amax, float* scale_out) {
  const float s = __fdiv_rn(fmaxf(*amax, 1e-12f), 448.0f);
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  for (int64_t i = blockIdx.x * (int64_t)kEwThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kEwThreads)
    dst[i] = (uint8_t)f32_to_e4m3(__fdiv_rn(load1<T>(src, i), s));
}

__global__ __launch_bounds__(kEwThreads) void dequant_kernel(const uint8_t* src, uint16_t* dst, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)kEwThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kEwThreads)
    dst[i] = (uint16_t)(__float_as_uint(e4m3_to_f32(src[i])) >> 16);   // exact: <= 4 significant bits
}

// The same three passes 8 elements per lane per step: a 16-byte load of the source (bf16 / f16:
// one; fp32: two), an 8-byte store of the codes, a 16-byte store of the widened values. Each
// element goes through the same arithmetic as above (the hardware e4m3 conversion after
// saturation encodes exactly as f32_to_e4m3), so the results are bit-identical. The elements
// after the last whole group of 8 are taken one by one by the first workgroup. The host picks
// these kernels only when the pointers are aligned for the vector accesses.
template <typename T> __device__ __forceinline__ void load8(const char* p, float v[8]) {
  if constexpr (sizeof(T) == 4) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int r = 0; r < 4; ++r) { v[r] = a[r]; v[4 + r] = b[r]; }
  } else {
    const u32x4 x = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[2 * r] = Bits16<T>::to_f32(x[r] & 0xffffu);
      v[2 * r + 1] = Bits16<T>::to_f32(x[r] >> 16);
    }
  }
}

// Maximum over a workgroup (the result in thread 0).
__device__ __forceinline__ float block_max(float m) {
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float part[kEwThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < kEwThreads / 64; ++w) m = fmaxf(m, part[w]);
  return m;
}

// The absmax in two passes and no atomics: each workgroup writes the maximum of its grid-stride
// share (four 16-byte loads in flight per lane) to part[workgroup]; one workgroup then reduces
// the parts into *amax. (Many workgroups finishing together on one atomic word serialize there.)
template <typename T>
__global__ __launch_bounds__(kEwThreads) void absmax8_part_kernel(const void* src, int64_t n, float* part) {
  const char* base = reinterpret_cast<const char*>(src);
  const int64_t n8 = n / 8, stride = (int64_t)gridDim.x * kEwThreads;
  float m = 0.0f;
  int64_t j = blockIdx.x * (int64_t)kEwThreads + threadIdx.x;
  for (; j + 3 * stride < n8; j += 4 * stride) {
    float v[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) load8<T>(base + (j + u * stride) * 8 * esize<T>(), v[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 8; ++r) m = fmaxf(m, __builtin_fabsf(v[u][r]));
  }
  for (; j < n8; j += stride) {
    float v[8];
    load8<T>(base + j * 8 * esize<T>(), v);
#pragma unroll
    for (int r = 0; r < 8; ++r) m = fmaxf(m, __builtin_fabsf(v[r]));
  }
  if (blockIdx.x == 0)
    for (int64_t i = n8 * 8 + threadIdx.x; i < n; i += kEwThreads) m = fmaxf(m, __builtin_fabsf(load1<T>(src, i)));
  m = block_max(m);
  if (threadIdx.x == 0) part[blockIdx.x] = m;
}

__global__ __launch_bounds__(kEwThreads) void max_parts_kernel(const float* part, int parts, float* amax) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < parts; i += kEwThreads) m = fmaxf(m, part[i]);
  m = block_max(m);
  if (threadIdx.x == 0) *amax = m;
}

template <typename T>
__global__ __launch_bounds__(kEwThreads) void quantize8_kernel(const void* src, int64_t n, uint8_t* dst,
                                                               const float* amax, float* scale_out) {
  const float s = __fdiv_rn(fmaxf(*amax, 1e-12f), 448.0f);
  const float rs = __fdiv_rn(1.0f, s);
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = s;
  const char* base = reinterpret_cast<const char*>(src);
  const int64_t n8 = n / 8;
  for (int64_t j = blockIdx.x * (int64_t)kEwThreads + threadIdx.x; j < n8; j += (int64_t)gridDim.x * kEwThreads) {
    float v[8];
    load8<T>(base + j * 8 * esize<T>(), v);
    float y[8];
    quot_rn_n<8>(v, s, rs, y);
#pragma unroll
    for (int r = 0; r < 8; ++r) v[r] = y[r];
    *reinterpret_cast<u32x2*>(dst + j * 8) =
        u32x2{f32x4_to_fp8<false>(v[0], v[1], v[2], v[3]), f32x4_to_fp8<false>(v[4], v[5], v[6], v[7])};
  }
  if (blockIdx.x == 0)
    for (int64_t i = n8 * 8 + threadIdx.x; i < n; i += kEwThreads)
      dst[i] = (uint8_t)f32_to_e4m3(__fdiv_rn(load1<T>(src, i), s));
}

__global__ __launch_bounds__(kEwThreads) void dequant8_kernel(const uint8_t* src, uint16_t* dst, int64_t n) {
  const int64_t n8 = n / 8;
  for (int64_t j = blockIdx.x * (int64_t)kEwThreads + threadIdx.x; j < n8; j += (int64_t)gridDim.x * kEwThreads) {
    const u32x2 c = *reinterpret_cast<const u32x2*>(src + j * 8);
    u32x4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint32_t w = c[r >> 1] >> (16 * (r & 1));
      o[r] = (__float_as_uint(e4m3_to_f32(w & 0xffu)) >> 16) | (__float_as_uint(e4m3_to_f32((w >> 8) & 0xffu)) & 0xffff0000u);
    }
    *reinterpret_cast<u32x4*>(dst + j * 8) = o;
  }
  if (blockIdx.x == 0)
    for (int64_t i = n8 * 8 + threadIdx.x; i < n; i += kEwThreads)
      dst[i] = (uint16_t)(__float_as_uint(e4m3_to_f32(src[i])) >> 16);
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// fp8 codes of a [rows, cols] matrix, row-major and / or transposed, one 128 x 128 tile of codes
// at a time through LDS (as 32-bit words, rows padded by one word). Every global access of a wave
// covers whole 128-byte lines: a source row of the tile is 16 lanes x 16 (bf16) or 32 (fp32)
// bytes, and each transposed output column's 128 rows are written by 8 lanes of one wave. For the transposed stores a lane reads a 16-row x 4-column block of codes (16 words),
// regroups its bytes into the 4 columns in registers, and writes 16 bytes to each column. Source
// rows past `rows` (up to the transposed leading dimension) give code 0, which pads the
// transposed output.
__device__ __forceinline__ uint32_t byte_col(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3, int j) {
  const int sh = 8 * j;
  return ((r0 >> sh) & 0xffu) | (((r1 >> sh) & 0xffu) << 8) | (((r2 >> sh) & 0xffu) << 16) | (((r3 >> sh) & 0xffu) << 24);
}

// SRC: 1 bf16 values, 2 fp32 values. tile_amax (may be NULL): slot t = row tile * n_ct + column
// tile of each tile with rows inside the matrix gets the tile's max |v| (of the source values,
// before relu_sq). amax_only: record tile_amax and write no
// codes (the scale is not read).
template <int SRC>
__global__ __launch_bounds__(256) void quant2d_kernel(const void* src, int64_t rows, int64_t cols, int64_t ld_src,
                                                      int relu_sq, int e5m2, const float* scale, uint8_t* dst,
                                                      uint8_t* dst_t, int64_t ld_t, int64_t n_ct, int64_t n_tiles,
                                                      float* tile_amax, int amax_only) {
  constexpr int TW = 33;   // words per LDS row: 128 codes + 1 word of padding
  __shared__ uint32_t tile[128 * TW];
  __shared__ float wave_max[4];
  const int tid = threadIdx.x;
  const float sc = amax_only ? 1.0f : *scale;
  const float rsc = __fdiv_rn(1.0f, sc);
  for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    const int64_t r0 = (t / n_ct) * 128, c0 = (t % n_ct) * 128;
    // 16 lanes x 8 values per row, 16 rows per pass
    float m = 0.0f;
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int lr = (tid >> 4) + 16 * pass, lc = (tid & 15) * 8;
      const int64_t r = r0 + lr, c = c0 + lc;
      uint32_t lo = 0, hi = 0;
      if (r < rows && c < cols) {
        float in[8];
        if constexpr (SRC == 2) {
          const u32x4* q = reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(src) + r * ld_src + c);
          const u32x4 x0 = q[0], x1 = q[1];
#pragma unroll
          for (int k = 0; k < 4; ++k) { in[k] = __uint_as_float(x0[k]); in[4 + k] = __uint_as_float(x1[k]); }
        } else {
          const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(src) + r * ld_src + c);
#pragma unroll
          for (int k = 0; k < 8; ++k) in[k] = bf16_bits_to_f32((k & 1) ? (x[k >> 1] >> 16) : (x[k >> 1] & 0xffffu));
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) m = fmaxf(m, __builtin_fabsf(in[k]));
        if (amax_only) continue;
        float y[8];
        if (relu_sq) {
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const float r = fmaxf(in[k], 0.0f);
            in[k] = r * r;
          }
        }
        quot_rn_n<8>(in, sc, rsc, y);
        if (e5m2) {
          lo = f32x4_to_fp8<true>(y[0], y[1], y[2], y[3]);
          hi = f32x4_to_fp8<true>(y[4], y[5], y[6], y[7]);
        } else {
          lo = f32x4_to_fp8<false>(y[0], y[1], y[2], y[3]);
          hi = f32x4_to_fp8<false>(y[4], y[5], y[6], y[7]);
        }
        if (dst) *reinterpret_cast<u32x2*>(dst + r * cols + c) = u32x2{lo, hi};
      }
      tile[lr * TW + lc / 4] = lo;
      tile[lr * TW + lc / 4 + 1] = hi;
    }
    if (tile_amax) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      if ((tid & 63) == 0) wave_max[tid >> 6] = m;
      __syncthreads();
      if (tid == 0 && r0 < rows)
        tile_amax[t] = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    }
    if (amax_only) {
      __syncthreads();
      continue;
    }
    __syncthreads();
    if (dst_t) {   // lane: rows 16 rb .. 16 rb + 15, columns 4 cw .. 4 cw + 3 of the tile
      const int rb = tid & 7, cw = tid >> 3;
      const int64_t r = r0 + 16 * rb;
      uint32_t w[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) w[k] = tile[(16 * rb + k) * TW + cw];
      if (r < ld_t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t c = c0 + 4 * cw + j;
          if (c < cols)
            *reinterpret_cast<u32x4*>(dst_t + c * ld_t + r) =
                u32x4{byte_col(w[0], w[1], w[2], w[3], j), byte_col(w[4], w[5], w[6], w[7], j),
                      byte_col(w[8], w[9], w[10], w[11], j), byte_col(w[12], w[13], w[14], w[15], j)};
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t run_quantize_fp8_2d(DType src_t, const void* src, int64_t rows, int64_t cols, int64_t ld_src,
                               int relu_sq, int e5m2, const float* scale, void* dst, void* dst_t,
                               int64_t ld_t, hipStream_t s) {
  if (rows < 1 || cols < 16 || cols % 16 || ld_src < cols || ld_src % 16 || (dst_t && (ld_t < rows || ld_t % 16)))
    return hipErrorInvalidValue;
  const int64_t cover = dst_t ? ld_t : rows;
  const int64_t n_ct = (cols + 127) / 128, n_rt = (cover + 127) / 128, n_tiles = n_ct * n_rt;
  const int grid = (int)std::min<int64_t>(n_tiles, 8192);
  uint8_t* d = reinterpret_cast<uint8_t*>(dst);
  uint8_t* dt = reinterpret_cast<uint8_t*>(dst_t);
  if (src_t == DT_BF16)
    hipLaunchKernelGGL(quant2d_kernel<1>, dim3(grid), dim3(256), 0, s, src, rows, cols, ld_src, relu_sq, e5m2,
                       scale, d, dt, ld_t, n_ct, n_tiles, nullptr, 0);
  else if (src_t == DT_F32)
    hipLaunchKernelGGL(quant2d_kernel<2>, dim3(grid), dim3(256), 0, s, src, rows, cols, ld_src, relu_sq, e5m2,
                       scale, d, dt, ld_t, n_ct, n_tiles, nullptr, 0);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

namespace {
// *scale = max(max_i tile_amax[i], 1e-12) / 448 in fp32 (the arithmetic of the per-tensor quantizer).
__global__ __launch_bounds__(kEwThreads) void scale_from_tiles_kernel(const float* tile_amax, int64_t n, float* scale) {
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += kEwThreads) m = fmaxf(m, tile_amax[i]);
  m = block_max(m);
  if (threadIdx.x == 0) *scale = __fdiv_rn(fmaxf(m, 1e-12f), 448.0f);
}
}  // namespace

int64_t weight_amax_slots(int64_t rows, int64_t cols) { return ((rows + 127) / 128) * ((cols + 127) / 128); }

hipError_t run_quantize_weight_e4m3(DType src_t, const void* w, int64_t rows, int64_t cols, int exact, float* scale,
                                    float* tile_amax, void* dst, void* dst_t, int64_t ld_t, hipStream_t s) {
  if (rows < 1 || cols < 16 || cols % 16 || (src_t != DT_BF16 && src_t != DT_F32) || (dst_t && (ld_t < rows || ld_t % 16)))
    return hipErrorInvalidValue;
  const int64_t n_ct = (cols + 127) / 128;
  const int64_t n_slots = weight_amax_slots(rows, cols);
  auto q2d = [&](int amax_only, float* rec) {
    const int64_t cover = (!amax_only && dst_t) ? ld_t : rows;
    const int64_t n_tiles = n_ct * ((cover + 127) / 128);
    const int grid = (int)std::min<int64_t>(n_tiles, 8192);
    uint8_t* d = amax_only ? nullptr : reinterpret_cast<uint8_t*>(dst);
    uint8_t* dt = amax_only ? nullptr : reinterpret_cast<uint8_t*>(dst_t);
    if (src_t == DT_BF16)
      hipLaunchKernelGGL(quant2d_kernel<1>, dim3(grid), dim3(256), 0, s, w, rows, cols, cols, 0, 0, scale, d, dt,
                         ld_t, n_ct, n_tiles, rec, amax_only);
    else
      hipLaunchKernelGGL(quant2d_kernel<2>, dim3(grid), dim3(256), 0, s, w, rows, cols, cols, 0, 0, scale, d, dt,
                         ld_t, n_ct, n_tiles, rec, amax_only);
    return hipGetLastError();
  };
  hipError_t e;
  if (exact) {   // this call's amax, then its scale, then the codes
    if ((e = q2d(1, tile_amax)) != hipSuccess) return e;
    hipLaunchKernelGGL(scale_from_tiles_kernel, dim3(1), dim3(kEwThreads), 0, s, tile_amax, n_slots, scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return q2d(0, nullptr);
  }
  // the previous call's recorded amax gives the scale; the codes pass records this call's amax
  hipLaunchKernelGGL(scale_from_tiles_kernel, dim3(1), dim3(kEwThreads), 0, s, tile_amax, n_slots, scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return q2d(0, tile_amax);
}

hipError_t run_splitk_reduce(DType io, const float* partial, int splits, int M, int N, void* C0,
                             void* C1, int64_t ldc, int c_split, float alpha, const float* dev0,
                             const float* dev1, int accumulate, hipStream_t s) {
  const int grid = ew_grid((int64_t)M * (N / 4));
  if (io == DT_BF16 && !accumulate)
    hipLaunchKernelGGL(splitk_reduce_kernel<bf16>, dim3(grid), dim3(kEwThreads), 0, s, partial, splits, M,
                       N, C0, C1, ldc, c_split, alpha, dev0, dev1, 0);
  else if (io == DT_F16 && !accumulate)
    hipLaunchKernelGGL(splitk_reduce_kernel<f16>, dim3(grid), dim3(kEwThreads), 0, s, partial, splits, M,
                       N, C0, C1, ldc, c_split, alpha, dev0, dev1, 0);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<float>, dim3(grid), dim3(kEwThreads), 0, s, partial, splits, M,
                       N, C0, C1, ldc, c_split, alpha, dev0, dev1, accumulate);
  return hipGetLastError();
}

hipError_t run_gated_reduce(DType io, const float* partial, int splits, int M, int H, float alpha,
                            const float* dev0, const float* dev1, void* preact, void* a, float gate_mult,
                            int gate_inside, int fn, hipStream_t s) {
  const int grid = ew_grid((int64_t)M * (H / 4));
  if (io == DT_BF16)
    hipLaunchKernelGGL(gated_reduce_kernel<bf16>, dim3(grid), dim3(kEwThreads), 0, s, partial, splits, M, H,
                       alpha, dev0, dev1, preact, a, gate_mult, gate_inside, fn);
  else if (io == DT_F16)
    hipLaunchKernelGGL(gated_reduce_kernel<f16>, dim3(grid), dim3(kEwThreads), 0, s, partial, splits, M, H,
                       alpha, dev0, dev1, preact, a, gate_mult, gate_inside, fn);
  else
    hipLaunchKernelGGL(gated_reduce_kernel<float>, dim3(grid), dim3(kEwThreads), 0, s, partial, splits, M, H,
                       alpha, dev0, dev1, preact, a, gate_mult, gate_inside, fn);
  return hipGetLastError();
}

hipError_t run_gated_act(DType io, const void* preact, void* a, int M, int H, float gate_mult,
                         int gate_inside, int fn, hipStream_t s) {
  const int grid = ew_grid((int64_t)M * (H / 4));
  if (io == DT_BF16)
    hipLaunchKernelGGL(gated_act_kernel<bf16>, dim3(grid), dim3(kEwThreads), 0, s, preact, a, M, H, gate_mult,
                       gate_inside, fn);
  else if (io == DT_F16)
    hipLaunchKernelGGL(gated_act_kernel<f16>, dim3(grid), dim3(kEwThreads), 0, s, preact, a, M, H, gate_mult,
                       gate_inside, fn);
  else
    hipLaunchKernelGGL(gated_act_kernel<float>, dim3(grid), dim3(kEwThreads), 0, s, preact, a, M, H, gate_mult,
                       gate_inside, fn);
  return hipGetLastError();
}

hipError_t run_plain_act(DType io, const void* pre, void* post, int64_t n, float alpha,
                         const float* dev0, const float* dev1, int fn, hipStream_t s) {
  const int grid = ew_grid(n / 4);
  if (io == DT_BF16)
    hipLaunchKernelGGL(plain_act_kernel<bf16>, dim3(grid), dim3(kEwThreads), 0, s, pre, post, n, alpha, dev0, dev1, fn);
  else if (io == DT_F16)
    hipLaunchKernelGGL(plain_act_kernel<f16>, dim3(grid), dim3(kEwThreads), 0, s, pre, post, n, alpha, dev0, dev1, fn);
  else
    hipLaunchKernelGGL(plain_act_kernel<float>, dim3(grid), dim3(kEwThreads), 0, s, pre, post, n, alpha, dev0, dev1, fn);
  return hipGetLastError();
}

hipError_t run_quantize_e4m3(DType src_t, const void* src, int64_t n, void* dst, float* scale,
                             float* ws, hipStream_t s) {
  uint8_t* q = reinterpret_cast<uint8_t*>(dst);
  if (aligned(src, 16) && aligned(dst, 8)) {
    const int64_t n8 = n / 8;
    const int parts = (int)std::min<int64_t>(kQuantizeParts, std::max<int64_t>((n8 + 4 * kEwThreads - 1) / (4 * kEwThreads), 1));
    float* part = ws + 64;
    const int grid = ew_grid(std::max<int64_t>(n8, 1));
    if (src_t == DT_BF16) hipLaunchKernelGGL(absmax8_part_kernel<bf16>, dim3(parts), dim3(kEwThreads), 0, s, src, n, part);
    else if (src_t == DT_F16) hipLaunchKernelGGL(absmax8_part_kernel<f16>, dim3(parts), dim3(kEwThreads), 0, s, src, n, part);
    else hipLaunchKernelGGL(absmax8_part_kernel<float>, dim3(parts), dim3(kEwThreads), 0, s, src, n, part);
    hipLaunchKernelGGL(max_parts_kernel, dim3(1), dim3(kEwThreads), 0, s, part, parts, ws);
    if (src_t == DT_BF16) hipLaunchKernelGGL(quantize8_kernel<bf16>, dim3(grid), dim3(kEwThreads), 0, s, src, n, q, ws, scale);
    else if (src_t == DT_F16) hipLaunchKernelGGL(quantize8_kernel<f16>, dim3(grid), dim3(kEwThreads), 0, s, src, n, q, ws, scale);
    else hipLaunchKernelGGL(quantize8_kernel<float>, dim3(grid), dim3(kEwThreads), 0, s, src, n, q, ws, scale);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(zero_f32_kernel, dim3(1), dim3(64), 0, s, ws, 1);
  const int grid = ew_grid(n);
  if (src_t == DT_BF16) {
    hipLaunchKernelGGL(absmax_kernel<bf16>, dim3(grid), dim3(kEwThreads), 0, s, src, n, ws);
    hipLaunchKernelGGL(quantize_kernel<bf16>, dim3(grid), dim3(kEwThreads), 0, s, src, n, q, ws, scale);
  } else if (src_t == DT_F16) {
    hipLaunchKernelGGL(absmax_kernel<f16>, dim3(grid), dim3(kEwThreads), 0, s, src, n, ws);
    hipLaunchKernelGGL(quantize_kernel<f16>, dim3(grid), dim3(kEwThreads), 0, s, src, n, q, ws, scale);
  } else {
    hipLaunchKernelGGL(absmax_kernel<float>, dim3(grid), dim3(kEwThreads), 0, s, src, n, ws);
    hipLaunchKernelGGL(quantize_kernel<float>, dim3(grid), dim3(kEwThreads), 0, s, src, n, q, ws, scale);
  }
  return hipGetLastError();
}

hipError_t run_dequant_e4m3_bf16(const void* src, void* dst, int64_t n, hipStream_t s) {
  const uint8_t* c = reinterpret_cast<const uint8_t*>(src);
  uint16_t* o = reinterpret_cast<uint16_t*>(dst);
  if (aligned(src, 8) && aligned(dst, 16))
    hipLaunchKernelGGL(dequant8_kernel, dim3(ew_grid(std::max<int64_t>(n / 8, 1))), dim3(kEwThreads), 0, s, c, o, n);
  else
    hipLaunchKernelGGL(dequant_kernel, dim3(ew_grid(n)), dim3(kEwThreads), 0, s, c, o, n);
  return hipGetLastError();
}

}  // namespace gmlp
