// Arguments of the MLP engine's GEMM kernel, shared by host dispatch and device code.
#pragma once

#include <stdint.h>

namespace gmlp {

// The activation functions of the fused epilogues (GemmArgs::act): the gate function f of a
// gated activation a = f(g) * u (SwiGLU: silu, GeGLU: gelu_tanh, ReGLU: relu, GLU: sigmoid), or
// the f of a non-gated post = f(pre) (relu^2, relu, gelu_tanh).
enum ActFn : int { FN_SILU = 0, FN_GELU_TANH = 1, FN_RELU = 2, FN_SIGMOID = 3, FN_RELU_SQ = 4 };

enum Epi : int {
  EPI_STORE = 0,    // C = alpha * acc (OutT); accumulate: C(f32) += alpha * acc; rows >= c_split go to C1
  EPI_PARTIAL = 1,  // split-K: partial[split][m][n] = acc (fp32); a reduce kernel finishes
  EPI_GATED = 2,    // g, u = alpha * acc pair; aux[m][n], aux[m][half+n] = g, u (flag 1);
                    // C0[m][n] = a = act(g, u) (flag 2), act per GemmArgs::act
  EPI_ACT = 3,      // pre = alpha * acc -> aux (flag 1); post = f(pre) -> C0 (flag 2)
  EPI_DGATED = 4,   // da = alpha * acc; g, u <- aux; dg, du -> C0[m][n], C0[m][half+n];
                    // a -> C1 (flag 2). C0 may equal aux.
  EPI_DACT = 5,     // dpost = alpha * acc; pre <- aux; dpre = dpost * f'(pre) -> C0; post -> C1 (flag 2)
  EPI_F8ACT = 6,    // pre = alpha * acc -> aux (bf16 or fp32, flag 1); post = relu(pre)^2;
                    // C0 = e4m3(post / *s_post); *amax = max(*amax, max post)
  EPI_F8DACT = 7,   // dpre = alpha * acc * 2 max(pre, 0), pre <- aux (bf16 or fp32);
                    // C0 = e5m2(dpre / *s_post) (s_post holds the dpre scale here);
                    // *amax = max(*amax, max |dpre|); C1 set: C1 = e4m3(relu(pre)^2 / *s_c1)
};

struct GemmArgs {
  int M, N, K;
  const void* A; int64_t lda;
  // B from two matrices when B1 is set: MN-major B stacked along K (rows k >= b_split from B1,
  // the [W_gate; W_up] of dx); K-major non-gated B stacked along N (rows n >= b_split from B1)
  const void* B0; const void* B1; int64_t ldb; int b_split;
  void* C0; int64_t ldc0; void* C1; int64_t ldc1; int c_split;
  void* aux; int64_t ld_aux; int half;
  float alpha; const float* alpha_dev0; const float* alpha_dev1;
  float gate_mult; int gate_inside;
  int act;          // ActFn of the GATED / DGATED / ACT / DACT epilogues (F8ACT is relu^2)
  int accumulate;
  int flags;
  const float* s_post; float* amax;
  int k_per_split; float* partial;
  int tiles_m, tiles_n, group_m;
  const float* s_c1;   // F8DACT: scale of the e4m3 relu(pre)^2 codes written to C1
};

// Up to kGroupMax independent GEMMs run by one launch (gemm_dma_group_kernel): member j covers
// workgroups [begin[j], begin[j+1]) (multiples of 8 apart), has items[j] tiles (one per
// workgroup, no split) and takes tile body kind[j] (0 or 1) of the kernel's two.
constexpr int kGroupMax = 3;
struct GemmGroup {
  GemmArgs g[kGroupMax];
  int begin[kGroupMax + 1];
  int items[kGroupMax];
  int kind[kGroupMax];
  int count;
};

}  // namespace gmlp
