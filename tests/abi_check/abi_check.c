/* Host-side checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer: every
 * entry point is called with arguments that its validation must reject (so no call reaches the
 * GPU), and the host-only calls (workspace sizes, the backward schedule, slot counts, the
 * delayed-scale rule, status strings) over a grid of valid, edge and invalid descriptors. The
 * program is built and run by tests/test_abi_sanitized.py against the library with its host
 * code instrumented; a memory error or undefined behaviour aborts it, a wrong status makes it
 * exit non-zero. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mlp.h"

static int failures = 0;
#define EXPECT(cond)                                                            \
  do {                                                                          \
    if (!(cond)) {                                                              \
      fprintf(stderr, "%s:%d: expected %s (last error: %s)\n", __FILE__, __LINE__, \
              #cond, mlp_last_error());                                         \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

/* 16-byte aligned, never dereferenced: every call below fails validation first */
#define FAKE ((void*)(uintptr_t)0x7F0000000000ull)
#define MISALIGNED ((void*)(uintptr_t)0x7F0000000002ull)

static mlp_desc desc(int64_t M, int64_t d, int64_t H, int64_t o, int act, int dtype) {
  mlp_desc x;
  memset(&x, 0, sizeof x);
  x.M = M;
  x.d_in = d;
  x.hidden = H;
  x.d_out = o;
  x.act = act;
  x.dtype = dtype;
  x.gate_mult = 1.0f;
  x.down_mult = 1.0f;
  return x;
}

static int gated(int act) {
  return act == MLP_ACT_SWIGLU || act == MLP_ACT_GEGLU || act == MLP_ACT_REGLU || act == MLP_ACT_GLU;
}

/* the host-only planning calls over a grid of descriptors, valid or not */
static void sweep_descriptors(void) {
  const int64_t Ms[] = {-1, 0, 1, 15, 16, 300, 2048, 49152, (int64_t)1 << 24, ((int64_t)1 << 30) - 16,
                        (int64_t)1 << 30, INT64_MAX};
  const int64_t Ds[] = {0, 8, 16, 264, 768, 4096, ((int64_t)1 << 25) - 16, (int64_t)1 << 25, INT64_MIN};
  const int acts[] = {-1, MLP_ACT_SWIGLU, MLP_ACT_RELU_SQ, MLP_ACT_GEGLU, MLP_ACT_RELU, 7};
  const int dtypes[] = {MLP_F32, MLP_BF16, MLP_F16, 3};
  size_t n_valid = 0;
  for (size_t a = 0; a < sizeof Ms / sizeof *Ms; ++a)
    for (size_t b = 0; b < sizeof Ds / sizeof *Ds; ++b)
      for (size_t c = 0; c < sizeof Ds / sizeof *Ds; ++c)
        for (size_t e = 0; e < sizeof acts / sizeof *acts; ++e)
          for (size_t t = 0; t < sizeof dtypes / sizeof *dtypes; ++t)
            for (int flags = 0; flags < 16; ++flags) {
              mlp_desc x = desc(Ms[a], Ds[b], Ds[c], Ds[b], acts[e], dtypes[t]);
              x.recompute = flags & 1;
              x.fp8_fwd = (flags >> 1) & 1;
              x.fp8_bwd = (flags >> 2) & 1;
              x.save_act = (flags >> 3) & 1;
              int ok = 1;
              for (int phase = -1; phase <= 3; ++phase) {
                const size_t need = mlp_workspace_bytes(&x, phase);
                if (phase < 0 || phase > 2) EXPECT(need == 0);
                else ok = ok && need > 0;
              }
              int grouped = -1;
              const mlp_status st = mlp_bwd_grouped(&x, &grouped);
              if (ok) {
                ++n_valid;
                EXPECT(st == MLP_OK);
                EXPECT(grouped >= 0 && grouped <= (MLP_BWD_GROUPED | MLP_BWD_DW_DOWN_WITH_DACT));
                EXPECT(mlp_bwd_grouped(&x, NULL) == MLP_ERR_INVALID_ARG);
              } else {
                EXPECT(st != MLP_OK);
                EXPECT(strlen(mlp_last_error()) > 0);
              }
            }
  EXPECT(n_valid > 0);
  EXPECT(mlp_workspace_bytes(NULL, MLP_PHASE_FWD) == 0);
}

static void rejected_calls(void) {
  const mlp_desc ok = desc(300, 264, 712, 200, MLP_ACT_SWIGLU, MLP_BF16);
  const mlp_desc bad = desc(0, 264, 712, 200, MLP_ACT_SWIGLU, MLP_BF16);
  const size_t ws_f = mlp_workspace_bytes(&ok, MLP_PHASE_FWD);
  const size_t ws_b = mlp_workspace_bytes(&ok, MLP_PHASE_BWD);
  EXPECT(ws_f > 0 && ws_b > 0);
  /* forward */
  EXPECT(mlp_fwd(NULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, ws_f, NULL) == MLP_ERR_INVALID_ARG);
  EXPECT(mlp_fwd(&bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, ws_f, NULL) == MLP_ERR_INVALID_ARG);
  EXPECT(mlp_fwd(&ok, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, ws_f, NULL) == MLP_ERR_INVALID_ARG);
  EXPECT(mlp_fwd(&ok, MISALIGNED, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, ws_f, NULL) == MLP_ERR_ALIGNMENT);
  EXPECT(mlp_fwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, ws_f, NULL) == MLP_ERR_INVALID_ARG);
  EXPECT(mlp_fwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, ws_f - 1, NULL) == MLP_ERR_WORKSPACE);
  EXPECT(mlp_fwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, ws_f, NULL) != MLP_OK);
  EXPECT(mlp_fwd_infer(&ok, FAKE, FAKE, NULL, FAKE, FAKE, NULL, FAKE, 1 << 30, NULL) == MLP_ERR_INVALID_ARG);
  EXPECT(mlp_fwd_infer(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 0, NULL) == MLP_ERR_WORKSPACE);
  /* fp8 arguments without fp8_fwd, and fp8_fwd without them */
  mlp_fp8 f;
  memset(&f, 0, sizeof f);
  EXPECT(mlp_fwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, &f, FAKE, ws_f, NULL) == MLP_ERR_INVALID_ARG);
  mlp_desc f8 = desc(256, 256, 704, 256, MLP_ACT_RELU_SQ, MLP_BF16);
  f8.fp8_fwd = 1;
  EXPECT(mlp_fwd(&f8, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, NULL, FAKE, 1 << 30, NULL) == MLP_ERR_INVALID_ARG);
  EXPECT(mlp_fwd(&f8, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, &f, FAKE, 1 << 30, NULL) == MLP_ERR_INVALID_ARG);
  /* the no-allocation forward: checks and the static-scratch limit come before any HIP call */
  const mlp_desc big = desc(3000, 4096, 11008, 4096, MLP_ACT_SWIGLU, MLP_BF16);
  EXPECT(mlp_fwd_infer_noalloc(&big, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL) == MLP_ERR_WORKSPACE);
  EXPECT(mlp_fwd_infer_noalloc(&ok, NULL, FAKE, FAKE, FAKE, FAKE, NULL, NULL) == MLP_ERR_INVALID_ARG);
  EXPECT(mlp_fwd_infer_noalloc(NULL, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL) == MLP_ERR_INVALID_ARG);
  /* backward */
  EXPECT(mlp_bwd(&ok, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, 0, NULL, FAKE, ws_b, NULL) ==
         MLP_ERR_INVALID_ARG);
  EXPECT(mlp_bwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, NULL, FAKE, 0, NULL, FAKE, ws_b, NULL) ==
         MLP_ERR_INVALID_ARG);
  EXPECT(mlp_bwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, 2, NULL, FAKE, ws_b, NULL) ==
         MLP_ERR_INVALID_ARG);
  EXPECT(mlp_bwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, 0, NULL, FAKE, ws_b - 1, NULL) ==
         MLP_ERR_WORKSPACE);
  EXPECT(mlp_bwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, FAKE, FAKE, FAKE, 0, NULL, FAKE, ws_b, NULL) ==
         MLP_ERR_INVALID_ARG);
  EXPECT(mlp_bwd(&ok, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE, FAKE, 0, NULL, FAKE, ws_b,
                 NULL) == MLP_ERR_ALIGNMENT);
  mlp_desc rc = ok;
  rc.recompute = 1;
  rc.save_act = 1;
  EXPECT(mlp_bwd(&rc, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL, FAKE, FAKE, FAKE, FAKE, 0, NULL, FAKE, 1 << 30, NULL) ==
         MLP_ERR_INVALID_ARG);
  /* quantizers */
  char ws_q[16];
  EXPECT(mlp_quantize_e4m3(FAKE, MLP_BF16, 0, FAKE, FAKE, FAKE, mlp_quantize_workspace_bytes(), NULL) ==
         MLP_ERR_INVALID_ARG);
  EXPECT(mlp_quantize_e4m3(FAKE, 7, 16, FAKE, FAKE, FAKE, mlp_quantize_workspace_bytes(), NULL) ==
         MLP_ERR_INVALID_ARG);
  EXPECT(mlp_quantize_e4m3(FAKE, MLP_BF16, 16, FAKE, FAKE, ws_q, sizeof ws_q, NULL) != MLP_OK);
  EXPECT(mlp_quantize_fp8(FAKE, MLP_BF16, 0, 16, MLP_FP8_E4M3, 0, FAKE, FAKE, NULL, 0, NULL) != MLP_OK);
  EXPECT(mlp_quantize_fp8(FAKE, MLP_BF16, 16, 16, 9, 0, FAKE, FAKE, NULL, 0, NULL) != MLP_OK);
  EXPECT(mlp_quantize_fp8(FAKE, MLP_BF16, 16, 16, MLP_FP8_E4M3, 0, FAKE, NULL, NULL, 0, NULL) != MLP_OK);
  EXPECT(mlp_quantize_weight_e4m3(FAKE, MLP_F16, 64, 64, 1, FAKE, FAKE, FAKE, NULL, 0, NULL) ==
         MLP_ERR_UNSUPPORTED);
  EXPECT(mlp_quantize_weight_e4m3(FAKE, MLP_BF16, 64, 40, 1, FAKE, FAKE, FAKE, NULL, 0, NULL) ==
         MLP_ERR_ALIGNMENT);
  EXPECT(mlp_quantize_weight_e4m3(FAKE, MLP_BF16, INT64_MAX, 64, 1, FAKE, FAKE, FAKE, NULL, 0, NULL) != MLP_OK);
  /* stage hooks: host only */
  EXPECT(mlp_time_stage_once(-1, NULL, NULL) == MLP_ERR_INVALID_ARG);
  EXPECT(mlp_time_stage_once(MLP_STAGE_COUNT, NULL, NULL) == MLP_ERR_INVALID_ARG);
  EXPECT(mlp_time_stage_once(MLP_STAGE_UP, FAKE, NULL) == MLP_ERR_INVALID_ARG);
  EXPECT(mlp_time_stage_once(MLP_STAGE_UP, NULL, NULL) == MLP_OK);
}

static void host_rules(void) {
  /* slot counts: empty sizes give 0; very large ones must not overflow */
  EXPECT(mlp_weight_amax_slots(3072, 768) == 24 * 6);
  EXPECT(mlp_weight_amax_slots(0, 16) == 0);
  EXPECT(mlp_weight_amax_slots(-5, 16) == 0);
  EXPECT(mlp_weight_amax_slots(INT64_MAX, INT64_MAX) == 0);
  EXPECT(mlp_weight_amax_slots(((int64_t)1 << 31) - 1, ((int64_t)1 << 31) - 1) == ((int64_t)1 << 24) * ((int64_t)1 << 24));
  EXPECT(mlp_weight_amax_slots(INT64_MIN, 1) == 0);
  /* the delayed-scale rule over special values */
  const float vals[] = {0.0f, -0.0f, 1.0f, -1.0f, 1e-45f, 1e30f, 3.4e38f, INFINITY, -INFINITY, NAN};
  for (size_t i = 0; i < sizeof vals / sizeof *vals; ++i) {
    const float s = mlp_fp8_next_scale(vals[i], 0.5f, 1.03f / 448.0f, 1e-6f);
    EXPECT(isfinite(s) && s > 0.0f);
    if (!(isfinite(vals[i]) && vals[i] > 0.0f)) EXPECT(s == 0.5f);
  }
  EXPECT(mlp_fp8_next_scale(1e30f, 0.5f, 1.0f, 0.0f) == 1e12f);
  /* status strings */
  for (int st = -2; st < 10; ++st) EXPECT(mlp_status_string(st) != NULL);
  EXPECT(mlp_last_error() != NULL);
  EXPECT(mlp_quantize_workspace_bytes() > 0);
  EXPECT(mlp_abi_version() >= 5);
}

int main(void) {
  sweep_descriptors();
  rejected_calls();
  host_rules();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi_check: all checks passed\n");
  return 0;
}
