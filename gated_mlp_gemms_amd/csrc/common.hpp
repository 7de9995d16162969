// Device-side helpers shared by every kernel of the MLP engine (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_args.hpp"

namespace gmlp {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct e4m3 { uint8_t bits; };   // OCP FP8 E4M3 storage
// Operand pair of the fp8-gradient GEMMs: A holds OCP E5M2 codes (a gradient), B E4M3 codes
// (a weight or activation); both one byte per element.
struct f8g { uint8_t bits; };

constexpr int kThreads = 256;    // 4 wave64 per workgroup
constexpr int kWave = 64;

template <typename T> struct ElemTraits;
template <> struct ElemTraits<float> { static constexpr int bytes = 4; };
template <> struct ElemTraits<bf16>  { static constexpr int bytes = 2; };
template <> struct ElemTraits<f16>   { static constexpr int bytes = 2; };
template <> struct ElemTraits<e4m3>  { static constexpr int bytes = 1; };
template <> struct ElemTraits<f8g>   { static constexpr int bytes = 1; };

// ---- conversions -------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// The 16-bit storage types as bits: to fp32 exactly, from fp32 rounded to nearest even (fp16:
// the hardware conversion in the default rounding mode; beyond +-65504 it gives +-inf).
template <typename T> struct Bits16;
template <> struct Bits16<bf16> {
  static __device__ __forceinline__ float to_f32(uint32_t h) { return bf16_bits_to_f32(h); }
  static __device__ __forceinline__ uint32_t from_f32(float f) { return f32_to_bf16_bits(f); }
  // two at once with gfx950's packed conversion (v_cvt_pk_bf16_f32: nearest even, the same
  // bits as f32_to_bf16_bits for every non-NaN input; NaN stays NaN)
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
  }
};
template <> struct Bits16<f16> {
  static __device__ __forceinline__ float to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(f16, (uint16_t)(h & 0xffffu));
  }
  static __device__ __forceinline__ uint32_t from_f32(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (f16)f);
  }
  static __device__ __forceinline__ uint32_t pack2(float lo, float hi) { return from_f32(lo) | (from_f32(hi) << 16); }
};
template <typename T>
__device__ __forceinline__ uint32_t pack16x2(float lo, float hi) { return Bits16<T>::pack2(lo, hi); }

// fp32 -> OCP E4M3 code: nearest, ties to even mantissa, |v| >= 448 saturates to +-448,
// NaN -> NaN code. Every step below is exact in fp32 except the final rint (the rounding).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(v);
  if (a != a) return sign | 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) {                                  // below 2^-6: subnormal codes 0..8
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);  // a * 2^9 is exact
  }
  const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;   // -6 .. 8
  const float m = a * __uint_as_float((uint32_t)(127 - e) << 23);  // in [1, 2), exact
  uint32_t mi = (uint32_t)__builtin_rintf((m - 1.0f) * 8.0f);      // 0..8
  int ee = e + 7;
  if (mi == 8u) { mi = 0u; ee += 1; }
  return sign | ((uint32_t)ee << 3) | mi;
}

// fp32 -> OCP E5M2 code: nearest, ties to even mantissa, |v| >= 57344 saturates to +-57344,
// NaN -> 0x7F. Exact in fp32 up to the final rint, as for e4m3.
__device__ __forceinline__ uint32_t f32_to_e5m2(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = __builtin_fabsf(v);
  if (a != a) return sign | 0x7fu;
  if (a >= 57344.0f) return sign | 0x7bu;
  if (a < 6.103515625e-05f) {                            // below 2^-14: subnormal codes 0..4
    return sign | (uint32_t)__builtin_rintf(a * 65536.0f);  // a * 2^16 is exact
  }
  const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;   // -14 .. 15
  const float m = a * __uint_as_float((uint32_t)(127 - e) << 23);  // in [1, 2), exact
  uint32_t mi = (uint32_t)__builtin_rintf((m - 1.0f) * 4.0f);      // 0..4
  int ee = e + 15;
  if (mi == 4u) { mi = 0u; ee += 1; }
  return sign | ((uint32_t)ee << 2) | mi;
}

// Four codes (byte k from v[k]) with gfx950's packed conversions (v_cvt_pk_fp8_f32 /
// v_cvt_pk_bf8_f32: nearest even) after saturating at the format maximum. Bit-identical to
// f32_to_e4m3 / f32_to_e5m2 on every non-NaN fp32 input (checked on the GPU over all of them);
// the conversion itself maps NaN to an unsigned code, so lanes holding a NaN take the integer
// encoder instead.
template <bool E5M2>
__device__ __forceinline__ uint32_t f32x4_to_fp8(float v0, float v1, float v2, float v3) {
  constexpr float kMax = E5M2 ? 57344.0f : 448.0f;
  const float c0 = __builtin_amdgcn_fmed3f(v0, -kMax, kMax), c1 = __builtin_amdgcn_fmed3f(v1, -kMax, kMax);
  const float c2 = __builtin_amdgcn_fmed3f(v2, -kMax, kMax), c3 = __builtin_amdgcn_fmed3f(v3, -kMax, kMax);
  int w;
  if constexpr (E5M2) {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c0, c1, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c2, c3, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
  }
  if ((v0 != v0) | (v1 != v1) | (v2 != v2) | (v3 != v3)) {
    auto enc = [](float x) { return E5M2 ? f32_to_e5m2(x) : f32_to_e4m3(x); };
    return enc(v0) | (enc(v1) << 8) | (enc(v2) << 16) | (enc(v3) << 24);
  }
  return (uint32_t)w;
}

// The correctly rounded quotients v[i] / s (what IEEE division gives) from the correctly rounded
// reciprocal r = RN(1 / s), computed once per scale: y0 = RN(v r) is within an ulp of v / s, the
// residual e = v - y0 s is exact in one fma, and RN(y0 + e r) is then the correctly rounded
// quotient (Markstein's theorem; Muller et al., Handbook of Floating-Point Arithmetic, the
// division-by-fma chapter). Three instructions instead of a full division. The sign is y0's:
// for v = -0 the correction step would turn the quotient's -0 into +0 (+0 + -0 = +0), which the
// fp8 encoders keep as a different code. A quotient in the fp32 subnormal range may differ in its
// last bit, which no fp8 code can see (such values encode to +-0 either way). If any first
// product of the group is not finite (v infinite or NaN, or v r overflowing), the whole group
// takes the IEEE division: one branch per group.
template <int N>
__device__ __forceinline__ void quot_rn_n(const float (&v)[N], float s, float r, float (&y)[N]) {
  bool finite = true;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float y0 = v[i] * r;
    finite &= __builtin_isfinite(y0);
    y[i] = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-y0, s, v[i]), r, y0), y0);
  }
  if (!finite) {
#pragma unroll
    for (int i = 0; i < N; ++i) y[i] = __fdiv_rn(v[i], s);
  }
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t s = c & 0x80u, e = (c >> 3) & 0xfu, m = c & 7u;
  float mag;
  if (e == 0) mag = (float)m * 0.001953125f;                        // m * 2^-9
  else mag = __uint_as_float(((e + 120u) << 23) | (m << 20));       // 2^(e-7) * (1 + m/8)
  if (e == 15u && m == 7u) mag = __builtin_nanf("");
  return s ? -mag : mag;
}

// *amax = max(*amax, v) for v >= 0 (the float bits of non-negative values order as unsigned
// integers). Every wave of a quantizing epilogue reports its maximum to the same word, and
// same-address atomics serialize in L2, so a wave first reads the word and skips the atomic when
// it cannot raise it (the word only grows: a stale read can only cost an unneeded atomic).
__device__ __forceinline__ void amax_update(float* amax, float v) {
  if (!(v > 0.0f)) return;
  const unsigned int cur = __hip_atomic_load(reinterpret_cast<unsigned int*>(amax), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
  if (__float_as_uint(v) > cur) atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(v));
}

// ---- activations (fp32) -------------------------------------------------------------------

__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// tanh(y) = 1 - 2 / (e^(2y) + 1); saturates to +-1 when e^(2y) over- or underflows
__device__ __forceinline__ float tanhf_(float y) {
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + __expf(2.0f * y));
}

// The activation functions of the fused epilogues: ActFn (gemm_args.hpp).
constexpr float kGeluC = 0.7978845608028654f;   // sqrt(2 / pi)
constexpr float kGeluK = 0.044715f;

// f(z[r]) for N values; the switch on the (uniform) function sits outside the element loop.
template <int N>
__device__ __forceinline__ void act_fn(int fn, const float (&z)[N], float (&f)[N]) {
  switch (fn) {
    case FN_SILU:
#pragma unroll
      for (int r = 0; r < N; ++r) f[r] = z[r] * sigmoidf_(z[r]);
      break;
    case FN_GELU_TANH:   // the same expression as in act_fn_grad, so both give identical bits
#pragma unroll
      for (int r = 0; r < N; ++r) {
        const float z2 = z[r] * z[r];
        f[r] = 0.5f * z[r] * (1.0f + tanhf_(kGeluC * (z[r] + kGeluK * z2 * z[r])));
      }
      break;
    case FN_RELU:
#pragma unroll
      for (int r = 0; r < N; ++r) f[r] = fmaxf(z[r], 0.0f);
      break;
    case FN_SIGMOID:
#pragma unroll
      for (int r = 0; r < N; ++r) f[r] = sigmoidf_(z[r]);
      break;
    default:   // FN_RELU_SQ
#pragma unroll
      for (int r = 0; r < N; ++r) { const float t = fmaxf(z[r], 0.0f); f[r] = t * t; }
  }
}

// f(z[r]) and f'(z[r]).
template <int N>
__device__ __forceinline__ void act_fn_grad(int fn, const float (&z)[N], float (&f)[N], float (&df)[N]) {
  switch (fn) {
    case FN_SILU:
#pragma unroll
      for (int r = 0; r < N; ++r) {
        const float s = sigmoidf_(z[r]);
        f[r] = z[r] * s;
        df[r] = s * (1.0f + z[r] * (1.0f - s));
      }
      break;
    case FN_GELU_TANH:
#pragma unroll
      for (int r = 0; r < N; ++r) {
        const float z2 = z[r] * z[r];
        const float t = tanhf_(kGeluC * (z[r] + kGeluK * z2 * z[r]));
        f[r] = 0.5f * z[r] * (1.0f + t);
        df[r] = 0.5f * (1.0f + t) + 0.5f * z[r] * (1.0f - t * t) * kGeluC * (1.0f + 3.0f * kGeluK * z2);
      }
      break;
    case FN_RELU:
#pragma unroll
      for (int r = 0; r < N; ++r) { f[r] = fmaxf(z[r], 0.0f); df[r] = z[r] > 0.0f ? 1.0f : 0.0f; }
      break;
    case FN_SIGMOID:
#pragma unroll
      for (int r = 0; r < N; ++r) { const float s = sigmoidf_(z[r]); f[r] = s; df[r] = s * (1.0f - s); }
      break;
    default:   // FN_RELU_SQ
#pragma unroll
      for (int r = 0; r < N; ++r) { const float t = fmaxf(z[r], 0.0f); f[r] = t * t; df[r] = 2.0f * t; }
  }
}

// Gated activation of N values: a = gm * f(g) * u (gate multiplier outside) or f(gm * g) * u.
template <int N>
__device__ __forceinline__ void gated_act(int fn, float gm, int inside, const float (&g)[N], const float (&u)[N],
                                          float (&a)[N]) {
  float z[N], f[N];
#pragma unroll
  for (int r = 0; r < N; ++r) z[r] = inside ? gm * g[r] : g[r];
  act_fn<N>(fn, z, f);
#pragma unroll
  for (int r = 0; r < N; ++r) a[r] = (inside ? f[r] : gm * f[r]) * u[r];
}

// Its backward against da: dg, du, and the post-activation a re-emitted.
template <int N>
__device__ __forceinline__ void gated_act_grad(int fn, float gm, int inside, const float (&da)[N], const float (&g)[N],
                                               const float (&u)[N], float (&dg)[N], float (&du)[N], float (&a)[N]) {
  float z[N], f[N], df[N];
#pragma unroll
  for (int r = 0; r < N; ++r) z[r] = inside ? gm * g[r] : g[r];
  act_fn_grad<N>(fn, z, f, df);
#pragma unroll
  for (int r = 0; r < N; ++r) {
    dg[r] = da[r] * gm * u[r] * df[r];
    du[r] = inside ? da[r] * f[r] : da[r] * gm * f[r];
    a[r] = (inside ? f[r] : gm * f[r]) * u[r];
  }
}

// ---- LDS tile geometry -------------------------------------------------------------------
// Every operand tile in LDS is [rows][128 bytes]: the K extent of one pipeline stage is
// 128 bytes of the element type (64 bf16, 32 fp32, 128 e4m3), split in 8 chunks of 16 bytes.
// Chunk c of row r is stored at chunk slot c ^ swz(r); the XOR spreads the 16-byte reads of
// 16 consecutive rows over distinct bank groups.
__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * 128 + ((chunk ^ lds_swz(row)) << 4);
}

// ---- tile scheduling ----------------------------------------------------------------------
// Workgroups are handed to the 8 XCDs round robin (block b on XCD b % 8). Remap the launch
// index so that each XCD works through one contiguous range of the logical tile order, which
// keeps the tiles sharing operands in the same L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  constexpr int kXcd = 8;
  const int q = total / kXcd, r = total % kXcd;
  const int x = b % kXcd, i = b / kXcd;
  return (x < r) ? x * (q + 1) + i : r * (q + 1) + (x - r) * q + i;
}

// Grouped raster: tiles go column-major inside bands of `group_m` tile rows, so consecutive
// tiles reuse the same B columns and a band of A rows.
__device__ __forceinline__ void grouped_tile(int t, int tiles_m, int tiles_n, int group_m,
                                             int& tm, int& tn) {
  const int per_group = group_m * tiles_n;
  const int g = t / per_group;
  const int first_m = g * group_m;
  const int gsize = min(tiles_m - first_m, group_m);
  const int in_g = t - g * per_group;
  tm = first_m + in_g % gsize;
  tn = in_g / gsize;
}

}  // namespace gmlp
