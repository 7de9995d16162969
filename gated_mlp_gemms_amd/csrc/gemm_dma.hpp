// The bf16 / e4m3 GEMM kernel: the same contraction and fused epilogues as gemm_kernel.hpp,
// with operands moved HBM -> LDS by the LDS-DMA form of the global load (no VGPR staging, no
// LDS store instructions) and a software-pipelined MFMA loop.
//
// Per workgroup (4 wave64, 2 x 2 waves of WM x WN): two LDS stages of BK = 128 bytes of K.
//  * K-major operand tiles are [rows][128 B], 16-byte chunks XOR-swizzled by row (lds_off).
//  * MN-major operand tiles are [64 k-rows][rows * 2 B] (bf16), 16-byte chunks XOR-swizzled
//    by (k-row % 4); fragments come out of LDS through the transposing 64-bit read, which hands
//    each lane four consecutive k of one column.
//  * K-step kt+1 is in flight (DMA) while step kt is multiplied; inside a step the fragments of
//    substep s+1 are read while the MFMAs of substep s run. One barrier per K-step, placed
//    before the last substep's MFMAs.
#pragma once

#include <type_traits>

#include "gemm_kernel.hpp"

namespace gmlp {

// The DMA source of every tile slot that lies outside a matrix: 16 zero bytes.
static __device__ __attribute__((aligned(16))) uint32_t g_zero_chunk[4];

#define GMLP_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ void dma16(const void* src, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, GMLP_LDS(lds_wave_base), 16, 0, 0);
}

__device__ __forceinline__ void wait_dma() {
  // vmcnt(0); expcnt and lgkmcnt left at their maxima (no wait on them)
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

// ---- K-major operand: ROWS rows x 128 B per stage ------------------------------------------
// One DMA instruction fills 1 KB = 8 rows: lane l -> row 8j + l/8, slot l%8, which holds the
// row's logical chunk (l%8) ^ swz(row).
template <typename T, int ROWS>
struct KTileDma {
  static constexpr int ES = ElemTraits<T>::bytes;
  static constexpr int E = 16 / ES;
  static constexpr int kInst = ROWS / 32;   // per wave per stage
  const char* ptr[kInst];
  int kc[kInst];

  template <typename RowPtr>
  __device__ __forceinline__ void init(int wave, int lane, int kbeg, RowPtr row_base) {
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
      const int j = wave * kInst + i;
      const int row = 8 * j + (lane >> 3);
      const int c = (lane & 7) ^ lds_swz(row);
      const char* b = row_base(row);
      kc[i] = c * E;
      ptr[i] = b ? b + (int64_t)(kbeg + c * E) * ES : nullptr;
    }
  }
  __device__ __forceinline__ void issue(char* tile, int wave, int k_rel, int k_left) const {
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
      const int j = wave * kInst + i;
      const void* src = (ptr[i] && k_rel + kc[i] < k_left) ? (const void*)(ptr[i] + (int64_t)k_rel * ES)
                                                           : (const void*)g_zero_chunk;
      dma16(src, tile + j * 1024);
    }
  }
  // 16-byte chunk `ch` of LDS row `row`
  static __device__ __forceinline__ u32x4 read(const char* tile, int row, int ch) {
    return *reinterpret_cast<const u32x4*>(tile + lds_off(row, ch));
  }
};

// ---- MN-major bf16 operand: 64 k-rows x ROWS columns per stage --------------------------------
template <int ROWS>
struct MNTileDma {
  static constexpr int ROWB = ROWS * 2;               // bytes per k-row
  static constexpr int kInst = ROWS / 32;             // per wave per stage
  int krow[kInst];
  int col[kInst];

  static __device__ __forceinline__ int phys_chunk(int c, int kr) { return c ^ ((kr & 3) << 2); }

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
      const int j = wave * kInst + i;
      const int byte = j * 1024 + lane * 16;
      const int kr = byte / ROWB;
      const int pc = (byte % ROWB) >> 4;
      krow[i] = kr;
      col[i] = phys_chunk(pc, kr) * 8;                  // the XOR is an involution
    }
  }
  // src(k) -> pointer to element (k, tile column 0); ncols: columns of the matrix left from
  // tile column 0.
  template <typename SrcRow>
  __device__ __forceinline__ void issue(char* tile, int wave, int k0, int kend, int ncols, SrcRow src) const {
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
      const int j = wave * kInst + i;
      const int k = k0 + krow[i];
      const void* s = (k < kend && col[i] < ncols) ? (const void*)(src(k) + (int64_t)col[i] * 2)
                                                   : (const void*)g_zero_chunk;
      dma16(s, tile + j * 1024);
    }
  }
  // Fragment of the 32-column block starting at tile column cb, K substep s (16 k): lane l gets
  // the 8 consecutive k 8*(l/32) .. +7 of column cb + l%32, via two transposing reads of four
  // k each. In each 16-lane group, lane i points at k-row (i/4) of its four and columns
  // 4*(i%4) .. +3 of the group's 16.
  static __device__ __forceinline__ u32x4 read(const char* tile, int cb, int s, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int kr = 16 * s + 8 * (g >> 1) + (i >> 2);
    const int c = cb + 16 * (g & 1) + 4 * (i & 3);
    const int off0 = kr * ROWB + (phys_chunk(c >> 3, kr) << 4) + (c & 7) * 2;
    const int off1 = off0 + 4 * ROWB;                  // k-row + 4: same (k-row % 4)
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + off0));
    const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(tile + off1));
    u32x4 r;
    r[0] = (uint32_t)(uint16_t)v0[0] | ((uint32_t)(uint16_t)v0[1] << 16);
    r[1] = (uint32_t)(uint16_t)v0[2] | ((uint32_t)(uint16_t)v0[3] << 16);
    r[2] = (uint32_t)(uint16_t)v1[0] | ((uint32_t)(uint16_t)v1[1] << 16);
    r[3] = (uint32_t)(uint16_t)v1[2] | ((uint32_t)(uint16_t)v1[3] << 16);
    return r;
  }
};

template <typename T, typename IoT, int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_dma_kernel(const GemmArgs p) {
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must split into 2x2 waves of 32x32 blocks");
  static_assert(A_KMAJ && B_KMAJ || std::is_same<T, bf16>::value, "MN-major operands are bf16 only");
  constexpr int ES = ElemTraits<T>::bytes;
  constexpr int E = 16 / ES;
  constexpr int BK = 8 * E;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MI = WM / 32, NI = WN / 32;
  constexpr int A_BYTES = BM * 128, STAGE = (BM + BN) * 128;
  constexpr bool GATED = EPI == EPI_GATED;
  constexpr int NSUB = Mma<T>::kSub;
  constexpr int KC = Mma<T>::kChunks;
  static_assert(NSUB % 2 == 0, "fragment double buffer alternates per substep");

  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

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

  // ---- DMA loaders
  KTileDma<T, BM> ka;
  KTileDma<T, BN> kb;
  MNTileDma<BM> na;
  MNTileDma<BN> nb;
  if constexpr (A_KMAJ) {
    ka.init(wave, lane, kbeg, [&](int r) -> const char* {
      const int m = m0 + r;
      return m < p.M ? elem_ptr<T>(p.A, m, p.lda, 0) : nullptr;
    });
  } else {
    na.init(wave, lane);
  }
  if constexpr (B_KMAJ) {
    kb.init(wave, lane, kbeg, [&](int r) -> const char* {
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
  } else {
    nb.init(wave, lane);
  }

  auto issue = [&](int kt, int stage) {
    char* sa = smem + stage * STAGE;
    char* sb = sa + A_BYTES;
    if constexpr (A_KMAJ) {
      ka.issue(sa, wave, kt * BK, kend - kbeg);
    } else {
      na.issue(sa, wave, kbeg + kt * BK, kend, p.M - m0,
               [&](int k) -> const char* { return elem_ptr<T>(p.A, k, p.lda, m0); });
    }
    if constexpr (B_KMAJ) {
      kb.issue(sb, wave, kt * BK, kend - kbeg);
    } else {
      nb.issue(sb, wave, kbeg + kt * BK, kend, p.N - n0, [&](int k) -> const char* {
        return k < p.b_split ? elem_ptr<T>(p.B0, k, p.ldb, n0) : elem_ptr<T>(p.B1, k - p.b_split, p.ldb, n0);
      });
    }
  };

  // ---- fragment rows / columns of this lane
  const int frow = lane & 31, fhalf = lane >> 5;
  int a_base[MI], b_base[NI];   // first tile row (K-major) / column (MN-major) of each block
#pragma unroll
  for (int i = 0; i < MI; ++i) a_base[i] = wm * WM + i * 32;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    if constexpr (GATED) {
      constexpr int NH = NI / 2;
      b_base[j] = j < NH ? wn * (BN / 4) + j * 32 : BN / 2 + wn * (BN / 4) + (j - NH) * 32;
    } else {
      b_base[j] = wn * WN + j * 32;
    }
  }

  u32x4 fa[2][MI][KC], fb[2][NI][KC];
  auto read_frags = [&](int stage, int s, int slot) {
    const char* sa = smem + stage * STAGE;
    const char* sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if constexpr (A_KMAJ) fa[slot][i][c] = KTileDma<T, BM>::read(sa, a_base[i] + frow, Mma<T>::chunk(s, fhalf, c));
        else fa[slot][i][c] = MNTileDma<BM>::read(sa, a_base[i], s, lane);
      }
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if constexpr (B_KMAJ) fb[slot][j][c] = KTileDma<T, BN>::read(sb, b_base[j] + frow, Mma<T>::chunk(s, fhalf, c));
        else fb[slot][j][c] = MNTileDma<BN>::read(sb, b_base[j], s, lane);
      }
    }
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (nk > 0) {
    issue(0, 0);
    wait_dma();
    __syncthreads();
    read_frags(0, 0, 0);
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) issue(kt + 1, cur ^ 1);
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      if (s + 1 < NSUB) {
        read_frags(cur, s + 1, (s + 1) & 1);
      } else if (more) {
        wait_dma();
        __syncthreads();
        read_frags(cur ^ 1, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) Mma<T>::mma(fb[s & 1][j], fa[s & 1][i], acc[i][j]);
    }
  }

  epilogue<EPI, IoT, BM, BN, MI, NI>(p, acc, m0, n0, split, wm, wn, lane);
}

template <typename T, typename IoT, int BM, int BN, bool A_KMAJ, bool B_KMAJ, int EPI>
hipError_t launch_gemm_dma(const GemmArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_dma_kernel<T, IoT, BM, BN, A_KMAJ, B_KMAJ, EPI>), dim3(grid), dim3(kThreads),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace gmlp
