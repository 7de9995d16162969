// Products with at most 16 rows (decode-size inference: a few tokens against the full weights).
// They are bound by reading the weights once from HBM, so the kernel streams weight rows straight
// into registers, with no LDS staging and no tile of zero-padded token rows:
//  * a workgroup owns 16 or 32 output units (their weight rows; gated: the gate rows and the up
//    rows of the same units) and splits K over its waves;
//  * lane l works on weight row l % 16 and token row l % 16; MFMA c of a 128-wide K block takes
//    the 8 elements k = 32 c + 8 q .. + 7 from lane group q = l / 16 (the instruction's own
//    operand layout), so one 16-byte load per lane reads 64 contiguous bytes of each of 16 weight
//    rows, and a block is four such loads per matrix;
//  * loads run two or three blocks ahead of the MFMAs that use them;
//  * the waves' partial sums meet in LDS and are added in wave order (deterministic), then the
//    first wave runs the epilogue: store, activation, or gated activation (and the pre-activation
//    when training), with the same activation functions as the GEMM epilogues.
// Above 8 tokens the gated product takes a second form (skinny_gated_lds_kernel below) that
// stages the token rows in LDS once per workgroup and shares them between column blocks, and a
// narrow store product with a long K (the down projection) splits K over workgroups into fp32
// partials for the split-K reduce, so that each workgroup reads a quarter of the token rows.
#include "common.hpp"
#include "gemm_kernel.hpp"
#include "launch.hpp"

namespace gmlp {

namespace {

constexpr int kKBlock = 128;       // K per block: four lane groups x 32
constexpr int kTwoBlocksFrom = 1024;   // output column blocks of 16 from which a workgroup takes two

// NCB column blocks of 16 units per workgroup (more units share each load of the token rows);
// NBUF blocks of loads in flight per wave. KQ > 1 (EPI_PARTIAL): workgroup b takes part b % KQ
// of K (in 128-wide blocks) for the column blocks of b / KQ and writes unscaled fp32 partial
// sums, partial[part][token][unit], for the fixed-order split-K reduce; a workgroup then reads
// the token rows of its part only, so per unit of weights streamed it reads KQ x fewer of them.
template <typename T, int EPI, int WAVES, int NCB, int NBUF, int KQ = 1>
__global__ __launch_bounds__(64 * WAVES) void skinny_kernel(const GemmArgs p) {
  static_assert((KQ > 1) == (EPI == EPI_PARTIAL), "K parts across workgroups write partial sums");
  constexpr bool GATED = EPI == EPI_GATED;
  constexpr int NB = GATED ? 2 : 1;   // weight matrices read: gate and up, or one
  constexpr int NACC = NB * NCB;
  __shared__ f32x4 red[WAVES][NACC][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int part = KQ > 1 ? (int)(blockIdx.x % KQ) : 0;
  const int nbase = (KQ > 1 ? (int)(blockIdx.x / KQ) : (int)blockIdx.x) * 16 * NCB + r;   // weight row, block 0
  const bool tok_ok = r < p.M;
  const char* xrow = reinterpret_cast<const char*>(elem_ptr<T>(p.A, tok_ok ? r : 0, p.lda, 0));
  const char* wrow[NB][NCB];
  bool row_ok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int n = nbase + 16 * cb;
    row_ok[cb] = n < p.N;
    wrow[0][cb] = reinterpret_cast<const char*>(elem_ptr<T>(p.B0, row_ok[cb] ? n : 0, p.ldb, 0));
    if constexpr (GATED) wrow[1][cb] = reinterpret_cast<const char*>(elem_ptr<T>(p.B1, row_ok[cb] ? n : 0, p.ldb, 0));
  }
  const int nblk_all = (p.K + kKBlock - 1) / kKBlock;
  const int kb0 = part * nblk_all / KQ, nblk = (part + 1) * nblk_all / KQ - kb0;   // this part's blocks
  const int b0 = kb0 + wave * nblk / WAVES, nb = kb0 + (wave + 1) * nblk / WAVES - b0;
  // each workgroup walks its waves' K ranges from a different block: every workgroup reads the
  // same token rows, and a common order would send all of them to the same lines at once
  const int rot = nb > 0 ? (int)((blockIdx.x / KQ) % (unsigned)nb) : 0;
  auto blk = [&](int i) { const int j = i + rot; return b0 + (j >= nb ? j - nb : j); };

  u32x4 xa[NBUF][4], wa[NBUF][NB][NCB][4];
  // block b into buffer s; a chunk past K (K is a multiple of 8: a chunk is wholly in or out),
  // a token row past M or a weight row past N loads zeros
  auto load = [&](int b, int s) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = b * kKBlock + c * 32 + q * 8;
      const bool k_ok = k < p.K;
      const int64_t off = (int64_t)k * (int64_t)sizeof(T);
      xa[s][c] = (tok_ok && k_ok) ? *reinterpret_cast<const u32x4*>(xrow + off) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          wa[s][m][cb][c] = (row_ok[cb] && k_ok) ? *reinterpret_cast<const u32x4*>(wrow[m][cb] + off)
                                                 : u32x4{0u, 0u, 0u, 0u};
    }
  };
  f32x4 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](int s) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) Mma16<T>::mma(xa[s][c], wa[s][m][cb][c], acc[m * NCB + cb]);
  };
  // NBUF buffers in rotation, indexed by constants only (a register array indexed at run time
  // would go to scratch memory): the i-th block of the walk lives in buffer i % NBUF
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    if (j < nb) load(blk(j), j);
  int i = 0;
  for (; i + NBUF <= nb; i += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      if (i + j + NBUF - 1 < nb) load(blk(i + j + NBUF - 1), (j + NBUF - 1) % NBUF);
      compute(j);
    }
  }
#pragma unroll
  for (int j = 0; j < NBUF; ++j)
    if (i + j < nb) compute(j);

#pragma unroll
  for (int j = 0; j < NACC; ++j) red[wave][j][lane] = acc[j];
  __syncthreads();
  if (wave != 0) return;
  if constexpr (EPI == EPI_PARTIAL) {
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      if (!row_ok[cb]) continue;
      const int n = nbase + 16 * cb;
      f32x4 s0 = red[0][cb][lane];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) s0 += red[w][cb][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // lane l holds tokens 4 q + i of unit n
        const int t = 4 * q + i;
        if (t < p.M) p.partial[((int64_t)part * p.M + t) * p.N + n] = s0[i];
      }
    }
    return;
  }
  float alpha = p.alpha;
  if (p.alpha_dev0) alpha *= *p.alpha_dev0;
  if (p.alpha_dev1) alpha *= *p.alpha_dev1;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    if (!row_ok[cb]) continue;
    const int n = nbase + 16 * cb;
    f32x4 s0 = red[0][cb][lane], s1 = red[0][NACC - NCB + cb][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      s0 += red[w][cb][lane];
      if constexpr (GATED) s1 += red[w][NCB + cb][lane];
    }
    // lane l holds tokens 4 q + i (i = 0..3) of unit n
    float v[4], u[4], o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = alpha * s0[i];
      u[i] = alpha * s1[i];
    }
    auto put = [&](void* base, int64_t ld, int col, const float (&val)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * q + i;
        if (t < p.M) *reinterpret_cast<uint16_t*>(elem_ptr<T>(base, t, ld, col)) = (uint16_t)Bits16<T>::from_f32(val[i]);
      }
    };
    if constexpr (GATED) {
      if (p.flags & 1) {
        put(p.aux, p.ld_aux, n, v);
        put(p.aux, p.ld_aux, p.half + n, u);
      }
      if (p.flags & 2) {
        gated_act<4>(p.act, p.gate_mult, p.gate_inside, v, u, o);
        put(p.C0, p.ldc0, n, o);
      }
    } else if constexpr (EPI == EPI_ACT) {
      if (p.flags & 1) put(p.aux, p.ld_aux, n, v);
      if (p.flags & 2) {
        act_fn<4>(p.act, v, o);
        put(p.C0, p.ldc0, n, o);
      }
    } else {
      put(p.C0, p.ldc0, n, v);
    }
  }
}

// The gated product with the token rows staged in LDS and shared. A workgroup of CB x KQ waves
// owns CB column blocks of 16 units; wave (cb, kq) streams the gate and up rows of block cb over
// the kq-th part of K, NBUF 128-wide blocks ahead, as the kernel above does, but takes its token
// fragments from LDS: the whole of x (16 rows, zeros past M and K) is staged there once, in
// fragment order (one 16-byte slot per K block, MFMA and lane: 4 KB per block), so the rows
// cross from L2 once per CB column blocks instead of once per block. The KQ partial sums of a
// column block meet in LDS (over the staged x, no longer read) and are added in kq order.
constexpr int kLdsBlocks = 32;   // K up to 4096: 128 KB of LDS

template <typename T, int CB, int KQ, int NBUF>
__global__ __launch_bounds__(64 * CB * KQ, 1) void skinny_gated_lds_kernel(const GemmArgs p) {
  constexpr int WAVES = CB * KQ;
  __shared__ u32x4 xs[kLdsBlocks * 4 * 64];
  static_assert(WAVES * 2 * 64 <= kLdsBlocks * 4 * 64, "partial sums fit the staged x's LDS");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int cb = wave % CB, kq = wave / CB;
  const int nblk = (p.K + kKBlock - 1) / kKBlock;

  // x -> LDS: chunk idx of 8 elements runs along each row (coalesced reads); row `row`, chunk kc
  // of its nblk * 16 goes to slot ((kc / 16) * 4 + (kc % 16) / 4) * 64 + (kc % 4) * 16 + row
  {
    const int per_row = nblk * 16, total = 16 * per_row;
    constexpr int BATCH = 2;   // loads in flight per thread before their LDS stores
    for (int base = threadIdx.x; base < total; base += BATCH * 64 * WAVES) {
      u32x4 v[BATCH];
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int idx = base + j * 64 * WAVES;
        const int row = idx / per_row, kc = idx - row * per_row, k = kc * 8;
        const bool ok = idx < total && row < p.M && k < p.K;
        v[j] = ok ? *reinterpret_cast<const u32x4*>(elem_ptr<T>(p.A, row, p.lda, k)) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < BATCH; ++j) {
        const int idx = base + j * 64 * WAVES;
        if (idx < total) {
          const int row = idx / per_row, kc = idx - row * per_row;
          xs[((kc >> 4) * 4 + ((kc & 15) >> 2)) * 64 + (kc & 3) * 16 + row] = v[j];
        }
      }
    }
  }

  const int n = (blockIdx.x * CB + cb) * 16 + r;   // this lane's gate / up row (unit)
  const bool row_ok = n < p.N;
  const char* wrow[2] = {reinterpret_cast<const char*>(elem_ptr<T>(p.B0, row_ok ? n : 0, p.ldb, 0)),
                         reinterpret_cast<const char*>(elem_ptr<T>(p.B1, row_ok ? n : 0, p.ldb, 0))};
  const int b0 = kq * nblk / KQ, nb = (kq + 1) * nblk / KQ - b0;
  u32x4 wa[NBUF][2][4];
  auto load = [&](int b, int s) {   // block b into buffer s; past K or N: zeros
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = b * kKBlock + c * 32 + q * 8;
      const bool ok = row_ok && k < p.K;
      const int64_t off = (int64_t)k * (int64_t)sizeof(T);
#pragma unroll
      for (int m = 0; m < 2; ++m)
        wa[s][m][c] = ok ? *reinterpret_cast<const u32x4*>(wrow[m] + off) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  f32x4 acc[2] = {f32x4{0.0f, 0.0f, 0.0f, 0.0f}, f32x4{0.0f, 0.0f, 0.0f, 0.0f}};
  auto compute = [&](int b, int s) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 xa = xs[(b * 4 + c) * 64 + lane];
      Mma16<T>::mma(xa, wa[s][0][c], acc[0]);
      Mma16<T>::mma(xa, wa[s][1][c], acc[1]);
    }
  };
  // the first weight blocks go out before the wait for the staged x
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    if (j < nb) load(b0 + j, j);
  __syncthreads();
  // NBUF buffers in rotation, indexed by constants only: the i-th block of the part lives in
  // buffer i % NBUF
  int i = 0;
  for (; i + NBUF <= nb; i += NBUF) {
#pragma unroll
    for (int j = 0; j < NBUF; ++j) {
      if (i + j + NBUF - 1 < nb) load(b0 + i + j + NBUF - 1, (j + NBUF - 1) % NBUF);
      compute(b0 + i + j, j);
    }
  }
#pragma unroll
  for (int j = 0; j < NBUF; ++j)
    if (i + j < nb) compute(b0 + i + j, j);

  // partial sums over the staged x (every wave is done reading it)
  __syncthreads();
  f32x4* red = reinterpret_cast<f32x4*>(xs);   // [KQ][CB][2][64]
  red[((kq * CB + cb) * 2 + 0) * 64 + lane] = acc[0];
  red[((kq * CB + cb) * 2 + 1) * 64 + lane] = acc[1];
  __syncthreads();
  if (kq != 0 || !row_ok) return;
  f32x4 s0 = red[(cb * 2 + 0) * 64 + lane], s1 = red[(cb * 2 + 1) * 64 + lane];
#pragma unroll
  for (int w = 1; w < KQ; ++w) {
    s0 += red[((w * CB + cb) * 2 + 0) * 64 + lane];
    s1 += red[((w * CB + cb) * 2 + 1) * 64 + lane];
  }
  float alpha = p.alpha;
  if (p.alpha_dev0) alpha *= *p.alpha_dev0;
  if (p.alpha_dev1) alpha *= *p.alpha_dev1;
  // lane l holds tokens 4 q + t (t = 0..3) of unit n
  float v[4], u[4], o[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    v[t] = alpha * s0[t];
    u[t] = alpha * s1[t];
  }
  auto put = [&](void* base, int64_t ld, int col, const float (&val)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tok = 4 * q + t;
      if (tok < p.M) *reinterpret_cast<uint16_t*>(elem_ptr<T>(base, tok, ld, col)) = (uint16_t)Bits16<T>::from_f32(val[t]);
    }
  };
  if (p.flags & 1) {
    put(p.aux, p.ld_aux, n, v);
    put(p.aux, p.ld_aux, p.half + n, u);
  }
  if (p.flags & 2) {
    gated_act<4>(p.act, p.gate_mult, p.gate_inside, v, u, o);
    put(p.C0, p.ldc0, n, o);
  }
}

template <typename T, int EPI>
hipError_t launch_skinny(const GemmArgs& a, hipStream_t s) {
  if (EPI == EPI_GATED && a.M > 8 && a.K <= kLdsBlocks * kKBlock) {
    // 3 column blocks x 4 parts of K: 48 units per workgroup of 12 waves, one per CU (128 KB of
    // LDS; 230 workgroups at H = 11008). Measured against the kernel above at the LLaMA widths:
    // 16 tokens 63.9 -> 60.5 us per inference forward, 8 tokens even, 1-4 tokens 1.4 us slower
    // (the x rows it saves are few there), hence the 8-token threshold. 4 x 4 blocks (172
    // workgroups) streamed slower than 230 on more CUs.
    hipLaunchKernelGGL((skinny_gated_lds_kernel<T, 3, 4, 3>), dim3((a.N + 47) / 48), dim3(768), 0, s, a);
    return hipGetLastError();
  }
  const int groups = (a.N + 15) / 16;   // column blocks of 16 units
  if (groups >= kTwoBlocksFrom) {
    // wide outputs: two column blocks per workgroup halve the re-reads of the token rows
    hipLaunchKernelGGL((skinny_kernel<T, EPI, 4, 2, 2>), dim3((groups + 1) / 2), dim3(256), 0, s, a);
  } else if (groups >= 512) {
    hipLaunchKernelGGL((skinny_kernel<T, EPI, 4, 1, 3>), dim3(groups), dim3(256), 0, s, a);
  } else {
    // few workgroups: K split over more waves, so enough loads are in flight (the gated body
    // keeps two weight matrices in flight and stops at 8 waves, within its register budget)
    constexpr int W = EPI == EPI_GATED ? 8 : 16;
    hipLaunchKernelGGL((skinny_kernel<T, EPI, W, 1, 3>), dim3(groups), dim3(64 * W), 0, s, a);
  }
  return hipGetLastError();
}

// The store product split along K over workgroups into fp32 partials (a.partial, [parts][M][N]),
// parts = kSkinnyParts; the caller runs the split-K reduce.
template <typename T>
hipError_t launch_skinny_parts(const GemmArgs& a, hipStream_t s) {
  constexpr int NCB = 4, W = 4;
  const int groups = (a.N + 16 * NCB - 1) / (16 * NCB);
  hipLaunchKernelGGL((skinny_kernel<T, EPI_PARTIAL, W, NCB, 3, kSkinnyParts>), dim3(groups * kSkinnyParts),
                     dim3(64 * W), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t skinny_epi(int epi, const GemmArgs& a, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_skinny<T, EPI_STORE>(a, s);
    case EPI_ACT: return launch_skinny<T, EPI_ACT>(a, s);
    case EPI_GATED: return launch_skinny<T, EPI_GATED>(a, s);
    case EPI_PARTIAL: return launch_skinny_parts<T>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t run_skinny(DType in, int epi, const GemmArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > kSkinnyMaxRows || a.N < 1 || a.K < 1 || a.K % 8) return hipErrorInvalidValue;
  if (in == DT_BF16) return skinny_epi<bf16>(epi, a, s);
  if (in == DT_F16) return skinny_epi<f16>(epi, a, s);
  return hipErrorInvalidValue;
}

}  // namespace gmlp
