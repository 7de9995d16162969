/*
 * gated_mlp: fused transformer-MLP forward and backward on AMD Instinct MI355X (gfx950).
 *
 *   gated:     g = x W_gate^T, u = x W_up^T, a = act(g, u), out = down_mult * a W_down^T
 *   non-gated: pre = x W1^T, post = f(pre),               out = down_mult * post W2^T
 *
 * The headline gated activation is SwiGLU: a = gate_mult * silu(g) * u (flash-swiglu-mlp
 * README, "Falcon H1 style models"), or a = silu(gate_mult * g) * u with MLP_GATE_INSIDE; the
 * headline non-gated one is modded-nanogpt gpt.py's ReLUSqrdMLP (relu(x @ W1.T)^2 @ W2.T). The
 * other members of quack mlp.py's Activation set are provided with their standard definitions
 * (see mlp_act). The backward follows
 * quack mlp.py's MLPRecomputeFunc.backward: d-activation applied to dout W2 against the
 * pre-activation (saved, or recomputed from x), dW2 = dout^T postact, dx = dpreact W1,
 * dW1 = dpreact^T x, optionally added into existing fp32 gradient buffers
 * (_compute_weight_grad with fuse_grad_accum).
 *
 * Conventions for every entry point:
 *  - All tensors are dense row-major device buffers. x [M, d_in]; W_gate, W_up, W1 [H, d_in];
 *    W_down, W2 [d_out, H] (nn.Linear layout); out, dout [M, d_out]; dx [M, d_in].
 *  - The caller owns every buffer, including the workspace. The library never allocates or
 *    frees device memory and never synchronizes: work is enqueued on `stream` (a hipStream_t;
 *    NULL is the null stream) and the call returns once it is enqueued.
 *  - Every argument check runs on the host before any HIP call; a failed check enqueues nothing
 *    and returns a status (never aborts). mlp_last_error() then describes it (thread-local).
 *    MLP_ERR_HIP reports a failed launch; faults inside kernels surface at the caller's next
 *    synchronization.
 *  - Device pointers must be 16-byte aligned. d_in, hidden and d_out must be multiples of 8
 *    (bf16) or 4 (f32): rows must be 16-byte aligned (flash-swiglu-mlp README, supported
 *    configurations; quack mlp.py's MLP.forward fast-path conditions). The e4m3 path needs
 *    multiples of 16. M >= 1 is arbitrary.
 *  - Size limits (MLP_ERR_UNSUPPORTED, before any HIP call): M, d_in, d_out < 2^30 and
 *    hidden < 2^29; every leading dimension below 2^25 elements (d_in, d_out, 2 * hidden for a
 *    gated activation or hidden otherwise), since a GEMM operand is addressed
 *    as a base plus a 32-bit offset spanning up to 64 rows; and no matrix of the problem (x, the
 *    pre-activation, out, the weights) above 2^37 elements, more than one GPU's memory holds.
 */
#ifndef GATED_MLP_H
#define GATED_MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mlp_status {
  MLP_OK = 0,
  MLP_ERR_INVALID_ARG = 1,   /* null/extra pointer, bad size, bad enum, inconsistent flags */
  MLP_ERR_UNSUPPORTED = 2,   /* a valid combination this library does not implement */
  MLP_ERR_ALIGNMENT = 3,     /* pointer not 16-byte aligned, or a dim not a multiple of 8/4/16 */
  MLP_ERR_WORKSPACE = 4,     /* workspace smaller than mlp_workspace_bytes() */
  MLP_ERR_HIP = 5            /* a HIP launch failed */
} mlp_status;

/* Activations (quack mlp.py's Activation set; it names them, the definitions are the standard
 * ones). Gated (w_gate and w_up; a = f(g) * u with the gate multiplier per mlp_gate_mode):
 *   MLP_ACT_SWIGLU  f = silu(z) = z sigmoid(z)     MLP_ACT_GEGLU  f = gelu_tanh
 *   MLP_ACT_REGLU   f = relu                       MLP_ACT_GLU    f = sigmoid
 * Non-gated (w_gate holds W1, w_up is NULL; post = f(pre); gate_mult and gate_mode ignored):
 *   MLP_ACT_RELU_SQ f = relu(z)^2                  MLP_ACT_RELU   f = relu(z) = max(z, 0)
 *   MLP_ACT_GELU_TANH f = z/2 (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))
 * relu's derivative is taken as 0 at z = 0. */
typedef enum mlp_act {
  MLP_ACT_SWIGLU = 0,
  MLP_ACT_RELU_SQ = 1,
  MLP_ACT_GEGLU = 2,
  MLP_ACT_REGLU = 3,
  MLP_ACT_GLU = 4,
  MLP_ACT_GELU_TANH = 5,
  MLP_ACT_RELU = 6
} mlp_act;
/* I/O type of x, the weights, out, dout, dx, the saved / d pre-activation and fresh gradients.
 * Accumulation and epilogue math are fp32 for all three; bf16 and fp16 use the 16-bit MFMA. */
typedef enum mlp_dtype { MLP_F32 = 0, MLP_BF16 = 1, MLP_F16 = 2 } mlp_dtype;
/* where gate_mult enters a gated activation: outside = gate_mult * f(g) * u (the README's formula
 * for SwiGLU), inside = f(gate_mult * g) * u. Identical at gate_mult = 1. */
typedef enum mlp_gate_mode { MLP_GATE_OUTSIDE = 0, MLP_GATE_INSIDE = 1 } mlp_gate_mode;
typedef enum mlp_phase { MLP_PHASE_FWD = 0, MLP_PHASE_FWD_INFER = 1, MLP_PHASE_BWD = 2 } mlp_phase;

typedef struct mlp_desc {
  int64_t M;          /* tokens: rows of x (the flattened [B, S]) */
  int64_t d_in;       /* width of x */
  int64_t hidden;     /* intermediate size H */
  int64_t d_out;      /* width of out */
  int32_t act;        /* mlp_act */
  int32_t dtype;      /* mlp_dtype of x, weights, out, dout, dx, saved/d preact, fresh grads */
  float gate_mult;    /* gate multiplier of a gated activation (1.0 = none); ignored otherwise */
  float down_mult;    /* scalar on the down projection's output (1.0 = none) */
  int32_t gate_mode;  /* mlp_gate_mode */
  int32_t recompute;  /* 1: nothing is saved; mlp_bwd recomputes the pre-activation from x */
  int32_t fp8_fwd;    /* 1: e4m3 forward GEMMs (ReLU^2, bf16 only); see mlp_fp8 */
  int32_t fp8_bwd;    /* 1: fp8 backward GEMMs with e5m2 gradients (needs fp8_fwd); see mlp_fp8.
                       * The pre-activation saved by mlp_fwd is then fp32. */
  int32_t save_act;   /* 1: mlp_fwd also keeps the activation a = act(g) * u (non-gated: post =
                       * f(pre)) after the pre-activation in saved_preact, and mlp_bwd reads it
                       * there instead of re-forming it in the d-activation GEMM, so dW_down no
                       * longer waits for that GEMM (flash-swiglu-mlp README, "design points":
                       * the forward keeps A, G and U). Needs recompute = 0 and fp8_fwd = 0. */
} mlp_desc;

/*
 * e4m3 operands of the ReLU^2 forward (modded-nanogpt gpt.py: FP8 MLP constants,
 * _mlp_fp8_args, _refresh_delayed_scale). Each quantized tensor carries one fp32 scale, its
 * dequantized value being scale * e4m3_value. relu(pre)^2 is quantized with the delayed scale
 * *s_post before the down projection, and max|relu(pre)^2| of the call is max-reduced into
 * *post_amax (so the host can form the next s_post with mlp_fp8_next_scale). All pointers are
 * device pointers; the scales are single floats.
 */
/*
 * With desc->fp8_bwd the backward runs every product in fp8 too (modded-nanogpt gpt.py: FP8
 * MLP constants FP8_GRAD_SCALE and FP8_DPRE_HEADROOM, init_mlp_fp8's weight caches and
 * _mlp_fp8_args): dout is quantized to e5m2 with the static scale *s_grad; dpre = down_mult *
 * (dout_q W2) * 2 relu(pre) is quantized to e5m2 with the delayed scale *s_dpre, and its
 * max|dpre| is max-reduced into *dpre_amax (the host forms the next s_dpre with
 * mlp_fp8_next_scale, gain 1.25/57344, floor 1e-12); dx = dpre_q W1, dW1 = dpre_q^T x_q and
 * dW2 = down_mult * dout_q^T post_q with post_q = e4m3(relu(pre)^2 / *s_post). The products
 * take the transposed weight caches w1t_q / w2t_q (the same codes as w1_q / w2_q, transposed:
 * the page's column-major caches) so that every fp8 GEMM reads both operands along K.
 */
typedef struct mlp_fp8 {
  const void* x_q;      /* e4m3 [M, d_in] */
  const void* w1_q;     /* e4m3 [H, d_in] */
  const void* w2_q;     /* e4m3 [d_out, H] */
  const float* s_x;     /* scale of x_q */
  const float* s_w1;    /* scale of w1_q (and w1t_q) */
  const float* s_w2;    /* scale of w2_q (and w2t_q) */
  const float* s_post;  /* scale relu(pre)^2 is quantized with (forward; fp8_bwd backward) */
  float* post_amax;     /* in/out: max(*post_amax, max|relu(pre)^2|) (forward only) */
  const void* w1t_q;    /* e4m3 [d_in, H] = W1^T codes (fp8_bwd only, else NULL) */
  const void* w2t_q;    /* e4m3 [H, d_out] = W2^T codes (fp8_bwd only, else NULL) */
  const float* s_grad;  /* static e5m2 scale of dout (fp8_bwd only) */
  const float* s_dpre;  /* delayed e5m2 scale of dpre (fp8_bwd only) */
  float* dpre_amax;     /* in/out: max(*dpre_amax, max|dpre|) (fp8_bwd only) */
} mlp_fp8;

/* fp8 storage formats (OCP 8-bit floating point): E4M3 (max 448, no infinity) and E5M2 (max
 * 57344). Encoders round to nearest even and saturate at the maximum; NaN stays NaN. */
typedef enum mlp_fp8_format { MLP_FP8_E4M3 = 0, MLP_FP8_E5M2 = 1 } mlp_fp8_format;

/* Bytes of workspace the given phase needs for `desc` (upper bound over every skip
 * combination). 0 for an invalid descriptor (see mlp_last_error). Host only. */
size_t mlp_workspace_bytes(const mlp_desc* desc, int phase);

/*
 * Training forward (quack mlp.py: mlp_func with grad enabled; flash-swiglu-mlp README,
 * "design points": fused gate/up forward, then the down projection).
 *   out          [M, d_out]                          written
 *   saved_preact gated: [M, 2H], row = [g | u]; non-gated: [M, H] pre. Written, in
 *                desc->dtype (fp32 with desc->fp8_bwd: the fp8-gradient backward rounds dpre and
 *                relu(pre)^2 to fp8 from it). Must be NULL iff desc->recompute (then nothing is
 *                kept for the backward: quack's MLPRecomputeFunc saves only x and the weights).
 *                With desc->save_act the [M, P] pre-activation (P = 2H gated, H otherwise) is
 *                followed by the [M, H] activation the down projection read (a, or post), in
 *                desc->dtype: M * (P + H) elements in all.
 *   w_up         NULL for a non-gated activation (w_gate then holds W1, w_down holds W2).
 *   fp8          non-NULL iff desc->fp8_fwd; x / w_gate / w_down are then not read.
 */
mlp_status mlp_fwd(const mlp_desc* desc, const void* x, const void* w_gate, const void* w_up,
                   const void* w_down, void* out, void* saved_preact, const mlp_fp8* fp8,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Inference forward: same out as mlp_fwd (bit for bit), keeping no pre-activation
 * (flash-swiglu-mlp README: the inference path saves no G/U). desc->recompute is ignored.
 */
mlp_status mlp_fwd_infer(const mlp_desc* desc, const void* x, const void* w_gate,
                         const void* w_up, const void* w_down, void* out, const mlp_fp8* fp8,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): mlp_fwd_infer with the workspace taken from a
 * static device array the library holds, MLP_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, from the
 * library's load until the process ends. The call allocates and frees nothing (no hipMalloc,
 * hipFree or allocating library routine); the caller still owns x, the weights, out and fp8.
 *   - Everything else is as mlp_fwd_infer, and out is bit for bit what mlp_fwd_infer writes.
 *   - MLP_ERR_WORKSPACE (before any HIP call) when mlp_workspace_bytes(desc,
 *     MLP_PHASE_FWD_INFER) exceeds MLP_NOALLOC_SCRATCH_BYTES. That size follows the planned
 *     split-K partials, so it is not monotone in M: at d_in = 4096, hidden = 11008 in bf16 every
 *     M up to 645 fits, 2048 fits (45 MB) and 3000 does not.
 *   - stream must belong to the calling thread's current device (else MLP_ERR_INVALID_ARG).
 *     The first call on a device looks the array's address up on that device (make it before
 *     a graph capture starts).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in time on the same
 *     GPU (other streams, other threads) race on it and must be serialized by the caller.
 *     Nothing in the array needs to start at zero; a call leaves its intermediates there.
 */
#define MLP_NOALLOC_SCRATCH_BYTES (64u << 20)
mlp_status mlp_fwd_infer_noalloc(const mlp_desc* desc, const void* x, const void* w_gate,
                                 const void* w_up, const void* w_down, void* out, const mlp_fp8* fp8,
                                 void* stream);

/*
 * Backward (quack mlp.py: MLPRecomputeFunc.backward, _compute_weight_grad; flash-swiglu-mlp
 * README, "design points": fused dA/dG/dU with dA never stored, dG/dU written over G/U,
 * merged dW_g/dW_u GEMM, single-accumulator dI).
 *   saved_preact  as written by mlp_fwd; NULL iff desc->recompute. With desc->save_act its
 *                 activation part is read, not written, and dW_down may run in one launch with
 *                 the d-activation GEMM (see mlp_bwd_grouped).
 *   dpreact       gated [M, 2H] = [dg | du], non-gated [M, H]; written. NULL: kept in the
 *                 workspace. May equal saved_preact (its pre-activation part is overwritten in
 *                 place; no other overlap).
 *   dx            [M, d_in], NULL to skip.
 *   dw_gate/dw_up [H, d_in] (non-gated: dw_gate = dW1, dw_up NULL); both or neither (gated).
 *   dw_down       [d_out, H], NULL to skip.
 *   grad_accum    0: weight grads are written in desc->dtype; 1: they are fp32 buffers and the
 *                 new gradient is added in place (buf = fp32(buf + grad)).
 *   fp8           non-NULL iff desc->fp8_fwd: the backward GEMMs then read the dequantized
 *                 x, W1, W2 of the forward (x / w_gate / w_down are not read). With
 *                 desc->fp8_bwd they run in fp8 instead (see mlp_fp8); dpreact must then be
 *                 NULL (dpre exists only as e5m2 codes in the workspace); M may be any
 *                 value >= 1.
 * Skips: with dx and dw_gate/dw_up all NULL only the down-projection gradient is formed
 * (quack's "only dW2 needed" branch); with dw_down NULL it is not.
 */
mlp_status mlp_bwd(const mlp_desc* desc, const void* dout, const void* x, const void* w_gate,
                   const void* w_up, const void* w_down, const void* saved_preact,
                   void* dpreact, void* dx, void* dw_gate, void* dw_up, void* dw_down,
                   int grad_accum, const mlp_fp8* fp8, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Bytes of workspace mlp_quantize_e4m3 needs (8448: the amax and the per-workgroup maxima it
 * reduces). Host only. */
size_t mlp_quantize_workspace_bytes(void);

/*
 * Per-tensor e4m3 quantization with the exact scale (modded-nanogpt gpt.py,
 * _quantize_mlp_weights_and_scales, exact-scale calls): *scale = max(amax|src|, 1e-12) / 448
 * in fp32, dst[i] = e4m3(src[i] / *scale) with IEEE fp32 division, round to nearest even,
 * saturating at +-448 (OCP E4M3). src is f32, bf16 or fp16 (`dtype`), n >= 1 elements; dst and
 * scale are device buffers written here.
 */
mlp_status mlp_quantize_e4m3(const void* src, int dtype, int64_t n, void* dst, float* scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp8 codes with a given scale (modded-nanogpt gpt.py: the dual-layout caches of init_mlp_fp8,
 * row-major and column-major copies of the same codes): code = fmt(v / *scale) with IEEE fp32
 * division, v = src (or max(src, 0)^2 when relu_sq), src a bf16 [rows, cols] row-major matrix.
 * dst [rows, cols] receives the row-major codes and dst_t [cols, ld_t] the transposed ones
 * (ld_t >= rows, a multiple of 16; columns rows .. ld_t-1 of dst_t are set to 0); either may be
 * NULL, not both. cols must be a multiple of 16; buffers 16-byte aligned; scale a device float.
 */
mlp_status mlp_quantize_fp8(const void* src, int dtype, int64_t rows, int64_t cols, int fmt, int relu_sq,
                            const float* scale, void* dst, void* dst_t, int64_t ld_t, void* stream);

/*
 * The fp8 weight-cache quantizer (modded-nanogpt gpt.py: _quantize_mlp_weights_and_scales with
 * FP8_EXACT_SCALE_CALLS, and the per-tile amax buffers of init_mlp_fp8). w is a [rows, cols]
 * row-major weight (bf16 or f32, `dtype`); its e4m3 codes go row-major into dst and/or transposed
 * into dst_t [cols, ld_t] (as mlp_quantize_fp8; either may be NULL, not both), with
 *   exact = 1: *scale = max(amax|w|, 1e-12) / 448 in fp32 from w itself (an amax pass first);
 *   exact = 0: *scale = max(max_i tile_amax[i], 1e-12) / 448 from the amax the previous call
 *              recorded (one call delayed: entries of w beyond 448 * *scale saturate),
 * and codes = e4m3(w / *scale) (IEEE fp32 division, nearest even, saturating). Either way the call
 * records w's amax per 128 x 128 tile into tile_amax, mlp_weight_amax_slots(rows, cols) device
 * floats, for the next call. The page sets the scales exactly for its first 16 calls (pass
 * exact = 1 for them) and takes the delayed ones afterwards. cols must be a multiple of 16.
 */
mlp_status mlp_quantize_weight_e4m3(const void* w, int dtype, int64_t rows, int64_t cols, int exact, float* scale,
                                    float* tile_amax, void* dst, void* dst_t, int64_t ld_t, void* stream);
/* Number of per-tile amax slots mlp_quantize_weight_e4m3 keeps for a [rows, cols] weight
 * (ceil(rows / 128) * ceil(cols / 128)); 0 for sizes it refuses (either below 1 or from 2^31 on).
 * Host only. */
int64_t mlp_weight_amax_slots(int64_t rows, int64_t cols);

/*
 * The next delayed scale of one fp8 tensor from the amax its last call recorded, in fp32
 * (modded-nanogpt gpt.py, the FP8 MLP's delayed scaling): a finite amax above zero gives
 * max(min(amax, 1e12) * gain, floor); any other amax (zero, negative, NaN, infinite) keeps
 * prev_scale. For relu(pre)^2 the page uses gain = 1.03/448, floor = 1e-6; for dpre (fp8_bwd)
 * gain = 1.25/57344, floor = 1e-12. Host only.
 */
float mlp_fp8_next_scale(float amax, float prev_scale, float gain, float floor_);

/*
 * Stages of mlp_fwd / mlp_fwd_infer / mlp_bwd, for mlp_time_stage_once:
 *   UP        x W1^T with the activation epilogue (gated: gate and up together)
 *   DOWN      a W2^T (the down projection, split-K reduce included)
 *   RECOMPUTE the backward's x W1^T when desc->recompute
 *   DACT      dout W2 with the d-activation epilogue (and dW2 with it when mlp_bwd_grouped
 *             says MLP_BWD_DW_DOWN_WITH_DACT)
 *   DW_DOWN   dW2 = dout^T a;   DX  dx = dpreact W1;   DW_UP  dW1 = dpreact^T x
 *   ACT       the activation-only pass of the "only dW2" branch
 *   WIDEN     the e4m3 -> bf16 widening of the e4m3 backward
 *   BWD_GEMMS DX, DW_UP and DW_DOWN (those asked for) as one launch, in place of their own
 *             stages, when mlp_bwd_grouped says so
 */
typedef enum mlp_stage {
  MLP_STAGE_UP = 0, MLP_STAGE_DOWN = 1, MLP_STAGE_RECOMPUTE = 2, MLP_STAGE_DACT = 3,
  MLP_STAGE_DW_DOWN = 4, MLP_STAGE_DX = 5, MLP_STAGE_DW_UP = 6, MLP_STAGE_ACT = 7,
  MLP_STAGE_WIDEN = 8, MLP_STAGE_BWD_GEMMS = 9, MLP_STAGE_COUNT = 10
} mlp_stage;

/*
 * Schedule of mlp_bwd's GEMMs (quack mlp.py, MLPRecomputeFunc backward: dx and the two weight
 * gradients, which its backward runs on a dynamic tile scheduler), for a call that asks for dx,
 * dw_gate (/dw_up) and dw_down. *grouped is a set of flags:
 *   MLP_BWD_DW_DOWN_WITH_DACT  dW_down runs in one launch with the d-activation GEMM (stage
 *                              DACT; only with desc->save_act, which makes them independent);
 *   MLP_BWD_GROUPED            the remaining ones of dx, dW_gate/dW_up and dW_down run as one
 *                              launch (stage BWD_GEMMS) instead of their own (DX, DW_UP, DW_DOWN).
 * A grouped launch lets the long-K tiles of one product and the short ones of another share the
 * CUs, with no split-K. 0: every product alone. A call that asks for fewer products decides the
 * same way for those it asks for (a product alone runs alone). Results do not depend on it
 * beyond the rounding of split-K sums. Host only. Errors: MLP_ERR_INVALID_ARG for a bad desc or
 * a NULL grouped.
 */
#define MLP_BWD_GROUPED 1
#define MLP_BWD_DW_DOWN_WITH_DACT 2
mlp_status mlp_bwd_grouped(const mlp_desc* desc, int* grouped);

/*
 * Timing hook (profiling only): the next time the calling thread's mlp_* call runs `stage`,
 * the library records `begin` on that call's stream before the stage's first launch and `end`
 * after its last one; then the hook is cleared. begin/end are hipEvent_t created by the caller
 * (hipEventCreate). Passing NULL events disarms the stage. Host only; nothing is enqueued here.
 */
mlp_status mlp_time_stage_once(int stage, void* begin, void* end);

/* Human-readable name of a status; text of the last failed check on this thread. */
const char* mlp_status_string(int status);
const char* mlp_last_error(void);

/* Version of this library's ABI (bumped on any change of the declarations above). */
int mlp_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GATED_MLP_H */
