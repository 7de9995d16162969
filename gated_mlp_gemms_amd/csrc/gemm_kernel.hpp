// One GEMM kernel template for every contraction of the MLP forward and backward, with the
// activation work fused into its epilogue.
//
//   C[m][n] = sum_k A(m, k) * B(n, k)       (fp32 accumulation in MFMA registers)
//
// Operand storage (per template flags):
//   A_KMAJ:  A(m, k) = A[m * lda + k]          else  A(m, k) = A[k * lda + m]
//   B_KMAJ:  B(n, k) = B0[n * ldb + k]          else  B(n, k) = Bsrc(k)[k' * ldb + n]
//            (the MN-major B may come from two buffers split along K at b_split: rows
//             k < b_split from B0, the rest from B1 — the stacked [W_gate; W_up] of dx)
// The gated epilogue reads its B tile from two buffers split along N instead: the first half
// of the tile's rows are W_gate rows, the second half the same W_up rows, so the gate and up
// accumulators of one hidden unit sit in the same lane (flash-swiglu-mlp README, "design
// points": one kernel computes gate_proj and up_proj from one x tile, G/U stay in registers).
//
// Work split: a workgroup of 4 wave64 computes one BM x BN tile (2 x 2 waves, each WM x WN);
// each wave issues 32x32 MFMAs. Operands are staged through LDS in [rows][128 B] tiles, two
// stages deep: the global loads of K-step k+1 are in flight while the MFMAs of step k run.
#pragma once

#include "common.hpp"
#include "gemm_args.hpp"

namespace gmlp {

// ---- 4-element row segments in the epilogue ----------------------------------------------

template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ void load(const void* p, float v[4]) {
    f32x4 x = *reinterpret_cast<const f32x4*>(p);
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  }
  static __device__ __forceinline__ void store(void* p, const float v[4]) {
    f32x4 x = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p) = x;
  }
};
template <typename T> struct Vec4Bits16 {
  static __device__ __forceinline__ void load(const void* p, float v[4]) {
    u32x2 x = *reinterpret_cast<const u32x2*>(p);
    v[0] = Bits16<T>::to_f32(x[0] & 0xffffu); v[1] = Bits16<T>::to_f32(x[0] >> 16);
    v[2] = Bits16<T>::to_f32(x[1] & 0xffffu); v[3] = Bits16<T>::to_f32(x[1] >> 16);
  }
  static __device__ __forceinline__ void store(void* p, const float v[4]) {
    u32x2 x = {pack16x2<T>(v[0], v[1]), pack16x2<T>(v[2], v[3])};
    *reinterpret_cast<u32x2*>(p) = x;
  }
};
template <> struct Vec4<bf16> : Vec4Bits16<bf16> {};
template <> struct Vec4<f16> : Vec4Bits16<f16> {};

template <typename T>
__device__ __forceinline__ char* elem_ptr(void* base, int64_t row, int64_t ld, int64_t col) {
  return reinterpret_cast<char*>(base) + (row * ld + col) * (int64_t)ElemTraits<T>::bytes;
}
template <typename T>
__device__ __forceinline__ const char* elem_ptr(const void* base, int64_t row, int64_t ld, int64_t col) {
  return reinterpret_cast<const char*>(base) + (row * ld + col) * (int64_t)ElemTraits<T>::bytes;
}

// ---- register transposes for MN-major operands --------------------------------------------
// in[i] = 16 bytes of storage row i (k = i), columns j (m or n); out[j][.] = column j along k.

__device__ __forceinline__ void transpose_block(const u32x4 in[8], u32x4 out[8], bf16) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1;
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      out[j][ii] = __builtin_amdgcn_perm(in[2 * ii + 1][w], in[2 * ii][w], sel);
  }
}
__device__ __forceinline__ void transpose_block(const u32x4 in[4], u32x4 out[4], float) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) out[j][i] = in[i][j];
}

// ---- MFMA step over one LDS substep ---------------------------------------------------------
// Each lane contributes the same K subset to its A and B fragments, so the K assignment inside
// an instruction does not need to match any particular documented layout; only the output
// layout matters: for a 32x32 block, lane l holds column-of-B-operand (l % 32) and, in
// register r, row 8*(r/4) + 4*(l/32) + r%4 of the A operand.

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int kSub = 4;     // 4 x K=16 per 64-element stage
  static constexpr int kChunks = 1;  // 16-byte chunks per lane per fragment per substep
  static __device__ __forceinline__ int chunk(int s, int half, int c) { return 2 * s + half; }
  static __device__ __forceinline__ void mma(const u32x4* a, const u32x4* b, f32x16& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                   __builtin_bit_cast(bf16x8, b[0]), acc, 0, 0, 0);
  }
};
template <> struct Mma<f16> {
  static constexpr int kSub = 4;     // 4 x K=16 per 64-element stage
  static constexpr int kChunks = 1;
  static __device__ __forceinline__ int chunk(int s, int half, int c) { return 2 * s + half; }
  static __device__ __forceinline__ void mma(const u32x4* a, const u32x4* b, f32x16& acc) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a[0]),
                                                  __builtin_bit_cast(f16x8, b[0]), acc, 0, 0, 0);
  }
};
// 16x16x32 MFMA of the two-wave-per-SIMD kernels (v_mfma_f32_16x16x32_bf16 / _f16): one 16 x 16
// fp32 block, 4 values per lane; with two waves per SIMD it issues closer to its nominal rate
// than the 32x32x16 form does.
template <typename T> struct Mma16;
template <> struct Mma16<bf16> {
  static __device__ __forceinline__ void mma(const u32x4& a, const u32x4& b, f32x4& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   acc, 0, 0, 0);
  }
};
template <> struct Mma16<f16> {
  static __device__ __forceinline__ void mma(const u32x4& a, const u32x4& b, f32x4& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b),
                                                  acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int kSub = 4;     // 4 x (4 x K=2) per 32-element stage
  static constexpr int kChunks = 1;
  static __device__ __forceinline__ int chunk(int s, int half, int c) { return 2 * s + half; }
  static __device__ __forceinline__ void mma(const u32x4* a, const u32x4* b, f32x16& acc) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[0][e]), __uint_as_float(b[0][e]),
                                                  acc, 0, 0, 0);
  }
};
template <> struct Mma<e4m3> {
  static constexpr int kSub = 2;     // 2 x K=64 per 128-element stage
  static constexpr int kChunks = 2;
  static __device__ __forceinline__ int chunk(int s, int half, int c) { return 4 * s + 2 * half + c; }
  static __device__ __forceinline__ void mma(const u32x4* a, const u32x4* b, f32x16& acc) {
    i32x8 av, bv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[i] = (int)a[0][i]; av[4 + i] = (int)a[1][i];
      bv[i] = (int)b[0][i]; bv[4 + i] = (int)b[1][i];
    }
    // e4m3 x e4m3 (format code 0), unit block scales (E8M0 127 = 2^0)
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
  }
};

// A in e5m2, B in e4m3. The kernel passes the B fragment as the instruction's first source and
// the A fragment as its second, so the format codes are e4m3 (0) for the first and e5m2 (1) for
// the second.
template <> struct Mma<f8g> {
  static constexpr int kSub = 2;
  static constexpr int kChunks = 2;
  static __device__ __forceinline__ int chunk(int s, int half, int c) { return 4 * s + 2 * half + c; }
  static __device__ __forceinline__ void mma(const u32x4* a, const u32x4* b, f32x16& acc) {
    i32x8 av, bv;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      av[i] = (int)a[0][i]; av[4 + i] = (int)a[1][i];
      bv[i] = (int)b[0][i]; bv[4 + i] = (int)b[1][i];
    }
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 1, 0, 127, 0, 127);
  }
};

// ---- operand tile loaders ---------------------------------------------------------------------

// K-major operand: ROWS rows of 8 chunks; thread t loads chunk (t % 8) of rows t/8 + 32 i.
template <typename T, int ROWS>
struct KMajorTile {
  static constexpr int kIt = ROWS / 32;
  static constexpr int E = 16 / ElemTraits<T>::bytes;
  const char* ptr[kIt];
  bool ok[kIt];
  u32x4 reg[kIt];

  // row_base(i) -> pointer to element (row, k = 0) of tile row i, or nullptr when the row is
  // outside the matrix.
  template <typename RowPtr>
  __device__ __forceinline__ void init(int tid, int kbeg, RowPtr row_base) {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const char* b = row_base((tid >> 3) + 32 * i);
      ok[i] = b != nullptr;
      ptr[i] = ok[i] ? b + (int64_t)(kbeg + c * E) * ElemTraits<T>::bytes : nullptr;
    }
  }
  __device__ __forceinline__ void load(int tid, int k_rel, int k_left) {
    const bool kok = (tid & 7) * E + k_rel < k_left;
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      if (ok[i] && kok) reg[i] = *reinterpret_cast<const u32x4*>(ptr[i] + (int64_t)k_rel * ElemTraits<T>::bytes);
      else reg[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < kIt; ++i)
      *reinterpret_cast<u32x4*>(lds + lds_off((tid >> 3) + 32 * i, c)) = reg[i];
  }
};

// MN-major operand: global rows are K, columns the tile's ROWS. Thread t owns E x E blocks
// (E k-rows x E columns), transposes them in registers and writes E LDS rows of one chunk.
template <typename T, int ROWS>
struct MNMajorTile {
  static constexpr int E = 16 / ElemTraits<T>::bytes;
  static constexpr int kBlkCols = ROWS / E;
  static constexpr int kBlocks = kBlkCols * 8;
  static constexpr int kBpt = (kBlocks + kThreads - 1) / kThreads;
  u32x4 reg[kBpt][E];

  // src(k) -> pointer to element (k, col 0 of the tile) or nullptr; col_ok(col) says whether
  // the 16-byte column chunk starting at tile column col is inside the matrix.
  template <typename SrcRow, typename ColOk>
  __device__ __forceinline__ void load(int tid, int k0, int kend, SrcRow src, ColOk col_ok) {
#pragma unroll
    for (int j = 0; j < kBpt; ++j) {
      const int b = tid + kThreads * j;
      const int cb = b % kBlkCols, kb = b / kBlkCols;
      const bool bok = (kBlocks % kThreads == 0 || b < kBlocks) && col_ok(cb * E);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const int k = k0 + kb * E + i;
        const char* s = (bok && k < kend) ? src(k) : nullptr;
        if (s) reg[j][i] = *reinterpret_cast<const u32x4*>(s + (int64_t)cb * E * ElemTraits<T>::bytes);
        else reg[j][i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < kBpt; ++j) {
      const int b = tid + kThreads * j;
      if (kBlocks % kThreads != 0 && b >= kBlocks) continue;
      const int cb = b % kBlkCols, kb = b / kBlkCols;
      u32x4 t[E];
      transpose_block(reg[j], t, T{});
#pragma unroll
      for (int i = 0; i < E; ++i)
        *reinterpret_cast<u32x4*>(lds + lds_off(cb * E + i, kb)) = t[i];
    }
  }
};

template <bool KMAJ, typename T, int ROWS> struct TileSel;
template <typename T, int ROWS> struct TileSel<true, T, ROWS> { using type = KMajorTile<T, ROWS>; };
template <typename T, int ROWS> struct TileSel<false, T, ROWS> { using type = MNMajorTile<T, ROWS>; };

// ---- fused epilogue ---------------------------------------------------------------------------
// acc[i][j] holds the 32x32 block (i, j) of the wave's WM x WN tile with the MFMA operands
// swapped (B tile rows as the instruction's rows): lane l owns output row m = l % 32 of the
// block and, in register 4g + r, column 8g + 4(l / 32) + r.
template <int EPI, typename IoT, int BM, int BN, int MI, int NI>
__device__ __forceinline__ void epilogue(const GemmArgs& p, f32x16 (&acc)[MI][NI], int m0, int n0,
                                         int split, int wm, int wn, int lane) {
  constexpr bool GATED = EPI == EPI_GATED;
  constexpr int WM = BM / 2, WN = BN / 2;
  const int frow = lane & 31, fhalf = lane >> 5;
  float alpha = p.alpha;
  if (p.alpha_dev0) alpha *= *p.alpha_dev0;
  if (p.alpha_dev1) alpha *= *p.alpha_dev1;
  float local_amax = 0.0f;
  (void)local_amax;

  constexpr int NJ = GATED ? NI / 2 : NI;
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = m0 + wm * WM + i * 32 + frow;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int nb = GATED ? n0 + wn * (BN / 4) + j * 32 : n0 + wn * WN + j * 32;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = nb + 8 * g + 4 * fhalf;
        if (n >= p.N) continue;
        // split-K partials stay unscaled: the reduce kernel applies alpha once
        const float scale = EPI == EPI_PARTIAL ? 1.0f : alpha;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = scale * acc[i][j][4 * g + r];

        if constexpr (EPI == EPI_STORE) {
          const bool lo = m < p.c_split;
          void* base = lo ? p.C0 : p.C1;
          const int row = lo ? m : m - p.c_split;
          if (p.accumulate) {
            float* q = reinterpret_cast<float*>(elem_ptr<float>(base, row, p.ldc0, n));
            float o[4];
            Vec4<float>::load(q, o);
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] += v[r];
            Vec4<float>::store(q, o);
          } else {
            Vec4<IoT>::store(elem_ptr<IoT>(base, row, p.ldc0, n), v);
          }
        } else if constexpr (EPI == EPI_PARTIAL) {
          const int64_t prow = (int64_t)split * p.M + m;
          Vec4<float>::store(elem_ptr<float>(p.partial, prow, p.N, n), v);
        } else if constexpr (EPI == EPI_GATED) {
          float u[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) u[r] = alpha * acc[i][j + NJ][4 * g + r];
          if (p.flags & 1) {
            Vec4<IoT>::store(elem_ptr<IoT>(p.aux, m, p.ld_aux, n), v);
            Vec4<IoT>::store(elem_ptr<IoT>(p.aux, m, p.ld_aux, p.half + n), u);
          }
          if (p.flags & 2) {
            float a[4];
            gated_act<4>(p.act, p.gate_mult, p.gate_inside, v, u, a);
            Vec4<IoT>::store(elem_ptr<IoT>(p.C0, m, p.ldc0, n), a);
          }
        } else if constexpr (EPI == EPI_ACT) {
          if (p.flags & 1) Vec4<IoT>::store(elem_ptr<IoT>(p.aux, m, p.ld_aux, n), v);
          if (p.flags & 2) {
            float q[4];
            act_fn<4>(p.act, v, q);
            Vec4<IoT>::store(elem_ptr<IoT>(p.C0, m, p.ldc0, n), q);
          }
        } else if constexpr (EPI == EPI_DGATED) {
          float gg[4], uu[4], dg[4], du[4], a[4];
          Vec4<IoT>::load(elem_ptr<IoT>(p.aux, m, p.ld_aux, n), gg);
          Vec4<IoT>::load(elem_ptr<IoT>(p.aux, m, p.ld_aux, p.half + n), uu);
          gated_act_grad<4>(p.act, p.gate_mult, p.gate_inside, v, gg, uu, dg, du, a);
          Vec4<IoT>::store(elem_ptr<IoT>(p.C0, m, p.ldc0, n), dg);
          Vec4<IoT>::store(elem_ptr<IoT>(p.C0, m, p.ldc0, p.half + n), du);
          if (p.flags & 2) Vec4<IoT>::store(elem_ptr<IoT>(p.C1, m, p.ldc1, n), a);
        } else if constexpr (EPI == EPI_DACT) {
          float pre[4], dpre[4], post[4];
          Vec4<IoT>::load(elem_ptr<IoT>(p.aux, m, p.ld_aux, n), pre);
          act_fn_grad<4>(p.act, pre, post, dpre);
#pragma unroll
          for (int r = 0; r < 4; ++r) dpre[r] *= v[r];
          Vec4<IoT>::store(elem_ptr<IoT>(p.C0, m, p.ldc0, n), dpre);
          if (p.flags & 2) Vec4<IoT>::store(elem_ptr<IoT>(p.C1, m, p.ldc1, n), post);
        } else if constexpr (EPI == EPI_F8ACT) {
          if (p.flags & 1) Vec4<IoT>::store(elem_ptr<IoT>(p.aux, m, p.ld_aux, n), v);
          const float sp = *p.s_post;
          uint32_t packed = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float t = fmaxf(v[r], 0.0f);
            const float post = t * t;
            local_amax = fmaxf(local_amax, post);
            packed |= f32_to_e4m3(__fdiv_rn(post, sp)) << (8 * r);
          }
          *reinterpret_cast<uint32_t*>(elem_ptr<e4m3>(p.C0, m, p.ldc0, n)) = packed;
        }
      }
    }
  }
  if constexpr (EPI == EPI_F8ACT) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) local_amax = fmaxf(local_amax, __shfl_xor(local_amax, off));
    if (lane == 0) amax_update(p.amax, local_amax);
  }
}

// ---- the kernel --------------------------------------------------------------------------------

template <typename T, typename IoT, int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const GemmArgs p) {
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must split into 2x2 waves of 32x32 blocks");
  static_assert(EPI != EPI_GATED || B_KMAJ, "gated epilogue reads K-major weights");
  constexpr int ES = ElemTraits<T>::bytes;
  constexpr int E = 16 / ES;
  constexpr int BK = 8 * E;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
  constexpr bool GATED = EPI == EPI_GATED;
  static_assert(!GATED || NI % 2 == 0, "gated tile needs gate and up blocks per wave");

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles = p.tiles_m * p.tiles_n;
  const int split = lid / tiles;
  lid -= split * tiles;
  int tm, tn;
  grouped_tile(lid, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
  const int m0 = tm * BM;
  const int n0 = tn * (GATED ? BN / 2 : BN);
  const int kbeg = split * p.k_per_split;
  const int kend = min(p.K, kbeg + p.k_per_split);
  const int nk = (kend - kbeg + BK - 1) / BK;

  // ---- operand loaders
  typename TileSel<A_KMAJ, T, BM>::type ta;
  typename TileSel<B_KMAJ, T, BN>::type tb;

  if constexpr (A_KMAJ) {
    ta.init(tid, kbeg, [&](int r) -> const char* {
      const int m = m0 + r;
      return m < p.M ? elem_ptr<T>(p.A, m, p.lda, 0) : nullptr;
    });
  }
  if constexpr (B_KMAJ) {
    tb.init(tid, kbeg, [&](int r) -> const char* {
      if constexpr (GATED) {
        const int half = BN / 2;
        const int n = n0 + (r < half ? r : r - half);
        if (n >= p.N) return nullptr;
        return elem_ptr<T>(r < half ? p.B0 : p.B1, n, p.ldb, 0);
      } else {
        const int n = n0 + r;
        return n < p.N ? elem_ptr<T>(p.B0, n, p.ldb, 0) : nullptr;
      }
    });
  }

  auto load_tiles = [&](int kt) {
    const int k0 = kbeg + kt * BK;
    if constexpr (A_KMAJ) {
      ta.load(tid, kt * BK, kend - kbeg);
    } else {
      ta.load(tid, k0, kend,
              [&](int k) -> const char* { return elem_ptr<T>(p.A, k, p.lda, m0); },
              [&](int c) { return m0 + c < p.M; });
    }
    if constexpr (B_KMAJ) {
      tb.load(tid, kt * BK, kend - kbeg);
    } else {
      tb.load(tid, k0, kend,
              [&](int k) -> const char* {
                return k < p.b_split ? elem_ptr<T>(p.B0, k, p.ldb, n0)
                                     : elem_ptr<T>(p.B1, k - p.b_split, p.ldb, n0);
              },
              [&](int c) { return n0 + c < p.N; });
    }
  };
  auto store_tiles = [&](int stage) {
    char* base = smem + stage * STAGE;
    ta.store(base, tid);
    tb.store(base + A_BYTES, tid);
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // LDS rows this lane reads its fragments from
  const int frow = lane & 31, fhalf = lane >> 5;
  int a_row[MI], b_row[NI];
#pragma unroll
  for (int i = 0; i < MI; ++i) a_row[i] = wm * WM + i * 32 + frow;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    if constexpr (GATED) {
      constexpr int NH = NI / 2;
      b_row[j] = (j < NH ? wn * (BN / 4) + j * 32 : BN / 2 + wn * (BN / 4) + (j - NH) * 32) + frow;
    } else {
      b_row[j] = wn * WN + j * 32 + frow;
    }
  }

  if (nk > 0) {
    load_tiles(0);
    store_tiles(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) load_tiles(kt + 1);
    const char* sa = smem + cur * STAGE;
    const char* sb = sa + A_BYTES;
#pragma unroll
    for (int s = 0; s < Mma<T>::kSub; ++s) {
      u32x4 af[MI][Mma<T>::kChunks], bfr[NI][Mma<T>::kChunks];
#pragma unroll
      for (int c = 0; c < Mma<T>::kChunks; ++c) {
        const int ch = Mma<T>::chunk(s, fhalf, c);
#pragma unroll
        for (int i = 0; i < MI; ++i) af[i][c] = *reinterpret_cast<const u32x4*>(sa + lds_off(a_row[i], ch));
#pragma unroll
        for (int j = 0; j < NI; ++j) bfr[j][c] = *reinterpret_cast<const u32x4*>(sb + lds_off(b_row[j], ch));
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) Mma<T>::mma(bfr[j], af[i], acc[i][j]);
    }
    if (more) store_tiles(cur ^ 1);
    __syncthreads();
  }

  epilogue<EPI, IoT, BM, BN, MI, NI>(p, acc, m0, n0, split, wm, wn, lane);
}

template <typename T, typename IoT, int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI>
hipError_t launch_gemm(const GemmArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_kernel<T, IoT, BM, BN, A_KMAJ, B_KMAJ, EPI>), dim3(grid), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace gmlp
