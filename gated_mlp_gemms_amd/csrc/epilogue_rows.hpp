// Fused epilogues that write whole row segments: the accumulators of each 32-row block-row of
// a wave are staged through LDS (free once the K loop is done) and read back so that every
// lane owns 8 consecutive columns of one row. Every global load and store is then 16 bytes of
// a contiguous 128-256 byte row segment, instead of 8 bytes scattered over 32 rows.
#pragma once

#include <type_traits>

#include "gemm_kernel.hpp"

namespace gmlp {

// ---- 8-element row pieces ---------------------------------------------------------------------

template <typename T> struct Vec8;
template <> struct Vec8<float> {
  static __device__ __forceinline__ void load(const void* p, float v[8]) {
    const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
    for (int r = 0; r < 4; ++r) { v[r] = a[r]; v[4 + r] = b[r]; }
  }
  static __device__ __forceinline__ void store(void* p, const float v[8]) {
    reinterpret_cast<f32x4*>(p)[0] = f32x4{v[0], v[1], v[2], v[3]};
    reinterpret_cast<f32x4*>(p)[1] = f32x4{v[4], v[5], v[6], v[7]};
  }
};
template <typename T> struct Vec8Bits16 {
  static __device__ __forceinline__ void load(const void* p, float v[8]) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[2 * r] = Bits16<T>::to_f32(x[r] & 0xffffu);
      v[2 * r + 1] = Bits16<T>::to_f32(x[r] >> 16);
    }
  }
  static __device__ __forceinline__ void store(void* p, const float v[8]) {
    *reinterpret_cast<u32x4*>(p) = u32x4{pack16x2<T>(v[0], v[1]), pack16x2<T>(v[2], v[3]),
                                         pack16x2<T>(v[4], v[5]), pack16x2<T>(v[6], v[7])};
  }
};
template <> struct Vec8<bf16> : Vec8Bits16<bf16> {};
template <> struct Vec8<f16> : Vec8Bits16<f16> {};

// Tensors an epilogue reads besides the accumulators (saved g, u or pre; the fp32 buffer of an
// accumulating store), fetched for a whole round before the round's LDS staging so their
// latency overlaps it. Raw 16-byte pieces: bf16 x 8 or fp32 x 4 (two pieces for fp32 x 8).
struct AuxPiece { u32x4 a, b, c; };

template <int EPI, typename IoT>
__device__ __forceinline__ void epi_prefetch(const GemmArgs& p, int m, int n, AuxPiece& x) {
  if constexpr (EPI == EPI_DGATED) {
    x.a = *reinterpret_cast<const u32x4*>(elem_ptr<IoT>(p.aux, m, p.ld_aux, n));
    x.b = *reinterpret_cast<const u32x4*>(elem_ptr<IoT>(p.aux, m, p.ld_aux, p.half + n));
  } else if constexpr (EPI == EPI_DACT) {
    x.a = *reinterpret_cast<const u32x4*>(elem_ptr<IoT>(p.aux, m, p.ld_aux, n));
  } else if constexpr (EPI == EPI_STORE) {
    if (p.accumulate) {
      const bool lo = m < p.c_split;
      const float* q = reinterpret_cast<const float*>(elem_ptr<float>(lo ? p.C0 : p.C1, lo ? m : m - p.c_split, p.ldc0, n));
      x.a = reinterpret_cast<const u32x4*>(q)[0];
      x.c = reinterpret_cast<const u32x4*>(q)[1];
    }
  }
}

template <typename T>
__device__ __forceinline__ void unpack16x8(const u32x4 x, float (&v)[8]) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    v[2 * r] = Bits16<T>::to_f32(x[r] & 0xffffu);
    v[2 * r + 1] = Bits16<T>::to_f32(x[r] >> 16);
  }
}

// The epilogue function on 8 consecutive columns n .. n+7 of row m. v = alpha * acc (or the
// raw accumulator for split-K partials); u = the up-projection values for the gated epilogue;
// x = what epi_prefetch fetched for this piece. (The quantizing epilogues take 16 columns:
// epi_row16.)
template <int EPI, typename IoT>
__device__ __forceinline__ void epi_row8(const GemmArgs& p, int m, int n, int split, const float (&v)[8],
                                         const float (&u)[8], const AuxPiece& x, float& local_amax) {
  static_assert(EPI != EPI_F8ACT && EPI != EPI_F8DACT, "the quantizing epilogues are 16 columns wide");
  if constexpr (EPI == EPI_STORE) {
    const bool lo = m < p.c_split;
    void* base = lo ? p.C0 : p.C1;
    const int row = lo ? m : m - p.c_split;
    if (p.accumulate) {
      float* q = reinterpret_cast<float*>(elem_ptr<float>(base, row, p.ldc0, n));
      float o[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o[r] = __uint_as_float(x.a[r]) + v[r];
        o[4 + r] = __uint_as_float(x.c[r]) + v[4 + r];
      }
      Vec8<float>::store(q, o);
    } else {
      Vec8<IoT>::store(elem_ptr<IoT>(base, row, p.ldc0, n), v);
    }
  } else if constexpr (EPI == EPI_PARTIAL) {
    const int64_t prow = (int64_t)split * p.M + m;
    Vec8<float>::store(elem_ptr<float>(p.partial, prow, p.N, n), v);
  } else if constexpr (EPI == EPI_GATED) {
    if (p.flags & 1) {
      Vec8<IoT>::store(elem_ptr<IoT>(p.aux, m, p.ld_aux, n), v);
      Vec8<IoT>::store(elem_ptr<IoT>(p.aux, m, p.ld_aux, p.half + n), u);
    }
    if (p.flags & 2) {
      float a[8];
      gated_act<8>(p.act, p.gate_mult, p.gate_inside, v, u, a);
      Vec8<IoT>::store(elem_ptr<IoT>(p.C0, m, p.ldc0, n), a);
    }
  } else if constexpr (EPI == EPI_ACT) {
    if (p.flags & 1) Vec8<IoT>::store(elem_ptr<IoT>(p.aux, m, p.ld_aux, n), v);
    if (p.flags & 2) {
      float q[8];
      act_fn<8>(p.act, v, q);
      Vec8<IoT>::store(elem_ptr<IoT>(p.C0, m, p.ldc0, n), q);
    }
  } else if constexpr (EPI == EPI_DGATED) {
    static_assert(ElemTraits<IoT>::bytes == 2, "row-staged d-activation epilogues read 16-bit aux data");
    float gg[8], uu[8], dg[8], du[8], a[8];
    unpack16x8<IoT>(x.a, gg);
    unpack16x8<IoT>(x.b, uu);
    gated_act_grad<8>(p.act, p.gate_mult, p.gate_inside, v, gg, uu, dg, du, a);
    Vec8<IoT>::store(elem_ptr<IoT>(p.C0, m, p.ldc0, n), dg);
    Vec8<IoT>::store(elem_ptr<IoT>(p.C0, m, p.ldc0, p.half + n), du);
    if (p.flags & 2) Vec8<IoT>::store(elem_ptr<IoT>(p.C1, m, p.ldc1, n), a);
  } else if constexpr (EPI == EPI_DACT) {
    static_assert(ElemTraits<IoT>::bytes == 2, "row-staged d-activation epilogues read 16-bit aux data");
    float pre[8], dpre[8], post[8];
    unpack16x8<IoT>(x.a, pre);
    act_fn_grad<8>(p.act, pre, post, dpre);
#pragma unroll
    for (int r = 0; r < 8; ++r) dpre[r] *= v[r];
    Vec8<IoT>::store(elem_ptr<IoT>(p.C0, m, p.ldc0, n), dpre);
    if (p.flags & 2) Vec8<IoT>::store(elem_ptr<IoT>(p.C1, m, p.ldc1, n), post);
  }
}

// The quantizing epilogues on 16 consecutive columns n .. n+15 of row m (widths a multiple of
// 16), so that each tensor of 1-byte codes is written as one 16-byte store per lane (two 8-byte
// stores cost about twice one: a store instruction costs about the same whatever its width).
// x: the pre-activation's 16 values (F8DACT), 4 (fp32) or 2 (16-bit) 16-byte pieces. The e4m3
// forward's fp32 pre-activation is stored by the caller, in a layout of its own.
template <int EPI, typename IoT>
__device__ __forceinline__ void epi_row16(const GemmArgs& p, int m, int n, const float (&v)[16],
                                          const u32x4 (&x)[4], float& local_amax) {
  static_assert(EPI == EPI_F8ACT || EPI == EPI_F8DACT, "the quantizing epilogues");
  if constexpr (EPI == EPI_F8ACT) {
    if (ElemTraits<IoT>::bytes == 2 && (p.flags & 1)) {
      Vec8<IoT>::store(elem_ptr<IoT>(p.aux, m, p.ld_aux, n), reinterpret_cast<const float(&)[8]>(v[0]));
      Vec8<IoT>::store(elem_ptr<IoT>(p.aux, m, p.ld_aux, n + 8), reinterpret_cast<const float(&)[8]>(v[8]));
    }
    const float sp = *p.s_post;
    const float rp = __fdiv_rn(1.0f, sp);
    float post[16], y[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float t = fmaxf(v[r], 0.0f);
      post[r] = t * t;
      local_amax = fmaxf(local_amax, post[r]);
    }
    quot_rn_n<16>(post, sp, rp, y);
    *reinterpret_cast<u32x4*>(elem_ptr<e4m3>(p.C0, m, p.ldc0, n)) =
        u32x4{f32x4_to_fp8<false>(y[0], y[1], y[2], y[3]), f32x4_to_fp8<false>(y[4], y[5], y[6], y[7]),
              f32x4_to_fp8<false>(y[8], y[9], y[10], y[11]), f32x4_to_fp8<false>(y[12], y[13], y[14], y[15])};
  } else {
    float pre[16];
    if constexpr (ElemTraits<IoT>::bytes == 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r) pre[4 * k + r] = __uint_as_float(x[k][r]);
    } else {
      unpack16x8<IoT>(x[0], reinterpret_cast<float(&)[8]>(pre[0]));
      unpack16x8<IoT>(x[1], reinterpret_cast<float(&)[8]>(pre[8]));
    }
    const float sd = *p.s_post;
    const float rd = __fdiv_rn(1.0f, sd);
    float dpre[16], y[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dpre[r] = v[r] * (2.0f * fmaxf(pre[r], 0.0f));
      local_amax = fmaxf(local_amax, __builtin_fabsf(dpre[r]));
    }
    quot_rn_n<16>(dpre, sd, rd, y);
    *reinterpret_cast<u32x4*>(elem_ptr<e4m3>(p.C0, m, p.ldc0, n)) =
        u32x4{f32x4_to_fp8<true>(y[0], y[1], y[2], y[3]), f32x4_to_fp8<true>(y[4], y[5], y[6], y[7]),
              f32x4_to_fp8<true>(y[8], y[9], y[10], y[11]), f32x4_to_fp8<true>(y[12], y[13], y[14], y[15])};
    if (p.C1) {   // relu(pre)^2 codes for dW2, the arithmetic of the 2-D quantizer's relu^2 mode
      const float sp = *p.s_c1;
      const float rp = __fdiv_rn(1.0f, sp);
      float post[16], z[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float t = fmaxf(pre[r], 0.0f);
        post[r] = t * t;
      }
      quot_rn_n<16>(post, sp, rp, z);
      *reinterpret_cast<u32x4*>(elem_ptr<e4m3>(p.C1, m, p.ldc1, n)) =
          u32x4{f32x4_to_fp8<false>(z[0], z[1], z[2], z[3]), f32x4_to_fp8<false>(z[4], z[5], z[6], z[7]),
                f32x4_to_fp8<false>(z[8], z[9], z[10], z[11]), f32x4_to_fp8<false>(z[12], z[13], z[14], z[15])};
    }
  }
}

// Rows of a block-row staged per round: 32 with 4 waves, 16 with 8 (the staging of all waves
// must fit the ring's LDS).
template <int WAVES> constexpr int epilogue_rows_per_round() { return WAVES == 8 ? 16 : 32; }

// Bytes of LDS the row-staged epilogue uses (waves x rows per round x padded WN fp32 columns).
template <int BN, int WAVES>
constexpr int epilogue_lds_bytes() { return WAVES * epilogue_rows_per_round<WAVES>() * ((BN / 2) * 4 + 16); }

// acc[i][j]: the MFMA layout of the wave's WM x WN tile (see epilogue()). lds: this
// workgroup's LDS, at least epilogue_lds_bytes<BN>() bytes, not in use by any wave.
template <int EPI, typename IoT, int BM, int BN, int MI, int NI, int WAVES, typename AccV>
__device__ __forceinline__ void epilogue_rows(const GemmArgs& p, AccV (&acc)[MI][NI], int m0, int n0,
                                              int split, int wm, int wn, int lane, int wave, char* lds) {
  constexpr bool GATED = EPI == EPI_GATED;
  // 32x32 blocks (16 values per lane: rows l%32, columns 8g + 4(l/32) + r) or 16x16 blocks
  // (4 values per lane: row l%16, columns 4(l/16) + r)
  constexpr bool B16 = sizeof(AccV) == 4 * sizeof(float);
  constexpr int BLK = B16 ? 16 : 32;
  constexpr int WM = BM / (WAVES / 2), WN = BN / 2;
  constexpr int RR = epilogue_rows_per_round<WAVES>();   // rows staged per round
  constexpr int STRIDE = WN * 4 + 16;                 // padded: rows 16 bytes apart in bank space
  constexpr int UNITS = GATED ? WN / 2 : WN;          // output columns of the wave
  // columns per lane: 16 for the quantizing epilogues (16-byte code stores), else 8
  constexpr int PW = (EPI == EPI_F8DACT || EPI == EPI_F8ACT) ? 16 : 8;
  constexpr int LPR = UNITS / PW;                     // lanes per row
  constexpr int RPI = 64 / LPR;                       // rows per pass
  static_assert(RR % RPI == 0, "passes must cover a round's rows");
  static_assert(RR <= BLK, "a round stays within one block row");
  const int frow = lane & (BLK - 1), fhalf = lane >> 5, fq = lane >> 4;
  char* wbuf = lds + wave * RR * STRIDE;

  float alpha = p.alpha;
  if (p.alpha_dev0) alpha *= *p.alpha_dev0;
  if (p.alpha_dev1) alpha *= *p.alpha_dev1;
  const float scale = EPI == EPI_PARTIAL ? 1.0f : alpha;   // partials stay unscaled
  float local_amax = 0.0f;

  const int nbase = GATED ? n0 + wn * (WN / 2) : n0 + wn * WN;
  const int rl = lane / LPR, cl = (lane % LPR) * PW;      // this lane's row-in-pass / column
#pragma unroll
  for (int i = 0; i < MI; ++i) {
#pragma unroll
    for (int h = 0; h < BLK / RR; ++h) {
      const int mrow0 = m0 + wm * WM + i * BLK + h * RR;
      AuxPiece x[PW == 8 ? RR / RPI : 1];
      u32x4 x16[PW == 16 ? RR / RPI : 1][4];   // 16-wide: the pre-activation's pieces
#pragma unroll
      for (int pass = 0; pass < RR / RPI; ++pass) {
        const int m = mrow0 + pass * RPI + rl, n = nbase + cl;
        if constexpr (PW == 16) {
          if (EPI == EPI_F8DACT && m < p.M && n < p.N) {
            constexpr int NP = ElemTraits<IoT>::bytes == 4 ? 4 : 2;   // 16-byte pieces of 16 values
#pragma unroll
            for (int k = 0; k < NP; ++k)
              x16[pass][k] = *reinterpret_cast<const u32x4*>(elem_ptr<IoT>(p.aux, m, p.ld_aux, n + k * 16 / ElemTraits<IoT>::bytes));
          }
        } else {
          if (m < p.M && n < p.N) epi_prefetch<EPI, IoT>(p, m, n, x[pass]);
        }
      }
      // MFMA layout -> LDS rows: lanes whose row falls in this round write columns
      // j*32 + 8g + 4*fhalf .. +3 of row (frow - h*RR)
      if (frow / RR == h) {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          if constexpr (B16) {
            const f32x4 v = {scale * acc[i][j][0], scale * acc[i][j][1], scale * acc[i][j][2], scale * acc[i][j][3]};
            *reinterpret_cast<f32x4*>(wbuf + (frow - h * RR) * STRIDE + (j * 16 + 4 * fq) * 4) = v;
          } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 v = {scale * acc[i][j][4 * g], scale * acc[i][j][4 * g + 1],
                               scale * acc[i][j][4 * g + 2], scale * acc[i][j][4 * g + 3]};
              *reinterpret_cast<f32x4*>(wbuf + (frow - h * RR) * STRIDE + (j * 32 + 8 * g + 4 * fhalf) * 4) = v;
            }
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      if constexpr (EPI == EPI_F8ACT && ElemTraits<IoT>::bytes == 4) {
        // an fp32 pre-activation first, read back in a layout of its own: 4 columns per lane, so
        // each store instruction writes whole 128-byte lines of 4 rows (with the 16 columns per
        // lane of the codes, an fp32 store covers a quarter of a line in each of 16 rows;
        // measured 266 vs 282 us on the GPT-shape up projection)
        if (p.flags & 1) {
          constexpr int CA = 4;                             // columns per 16-byte store
          constexpr int LPA = UNITS / CA, RPA = 64 / LPA;   // lanes per row, rows per pass
          static_assert(RR % RPA == 0, "passes must cover a round's rows");
          const int ra = lane / LPA, ca = (lane % LPA) * CA;
#pragma unroll
          for (int pa = 0; pa < RR / RPA; ++pa) {
            const int r = pa * RPA + ra;
            const int m = mrow0 + r, n = nbase + ca;
            const f32x4* src = reinterpret_cast<const f32x4*>(wbuf + r * STRIDE + ca * 4);
            const f32x4 a = src[0];
            if (m < p.M && n < p.N) *reinterpret_cast<f32x4*>(elem_ptr<IoT>(p.aux, m, p.ld_aux, n)) = a;
          }
        }
      }
#pragma unroll
      for (int pass = 0; pass < RR / RPI; ++pass) {
        const int r = pass * RPI + rl;
        const int m = mrow0 + r;
        const int n = nbase + cl;
        if constexpr (PW == 16) {
          float v16[16];
          const f32x4* src = reinterpret_cast<const f32x4*>(wbuf + r * STRIDE + cl * 4);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const f32x4 a = src[k];
#pragma unroll
            for (int q = 0; q < 4; ++q) v16[4 * k + q] = a[q];
          }
          if (m < p.M && n < p.N) epi_row16<EPI, IoT>(p, m, n, v16, x16[pass], local_amax);
        } else {
          float v[8], u[8];
          const f32x4* src = reinterpret_cast<const f32x4*>(wbuf + r * STRIDE + cl * 4);
          f32x4 a0 = src[0], a1 = src[1];
#pragma unroll
          for (int q = 0; q < 4; ++q) { v[q] = a0[q]; v[4 + q] = a1[q]; }
          if constexpr (GATED) {
            const f32x4* su = reinterpret_cast<const f32x4*>(wbuf + r * STRIDE + (UNITS + cl) * 4);
            a0 = su[0];
            a1 = su[1];
#pragma unroll
            for (int q = 0; q < 4; ++q) { u[q] = a0[q]; u[4 + q] = a1[q]; }
          }
          if (m < p.M && n < p.N) epi_row8<EPI, IoT>(p, m, n, split, v, u, x[pass], local_amax);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);       // reads done before the next round's writes
      __builtin_amdgcn_wave_barrier();
    }
  }
  if constexpr (EPI == EPI_F8ACT || EPI == EPI_F8DACT) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) local_amax = fmaxf(local_amax, __shfl_xor(local_amax, off));
    if (lane == 0) amax_update(p.amax, local_amax);
  }
}

}  // namespace gmlp
