// C-ABI of the MLP engine: argument checks (all on the host, before any HIP call), workspace
// layout, per-GEMM tile / split-K choice, and the launch sequence of the forward and backward.
//
// Forward (gated):  [gate/up GEMM + SwiGLU epilogue] -> a -> [down GEMM, x down_mult] -> out
// Backward (gated): [recompute g,u]? -> [dout W_down GEMM + d(SwiGLU) epilogue: dg|du, a]
//                   -> dW_down = dm dout^T a -> dx = [dg|du][W_gate; W_up] -> [dW_gate; dW_up]
// (quack mlp.py MLPRecomputeFunc; flash-swiglu-mlp README "design points"). The ReLU^2 MLP
// runs the same sequence with the relu^2 epilogues (modded-nanogpt gpt.py ReLUSqrdMLP).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <vector>
#include <mutex>
#include <string>

#include "launch.hpp"
#include "mlp.h"

using namespace gmlp;

namespace {

thread_local std::string g_last_error;

mlp_status fail(mlp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

// ---- one-shot stage timing (mlp_time_stage_once) ----------------------------------------------

struct StageHook { hipEvent_t begin = nullptr, end = nullptr; };
thread_local StageHook g_hooks[MLP_STAGE_COUNT];

// Records the armed begin event when constructed and the end event when destroyed, on `s`.
struct StageScope {
  StageHook* h = nullptr;
  hipStream_t s;
  StageScope(int stage, hipStream_t stream) : s(stream) {
    if (g_hooks[stage].begin) {
      h = &g_hooks[stage];
      (void)hipEventRecord(h->begin, s);
    }
  }
  ~StageScope() {
    if (h) {
      (void)hipEventRecord(h->end, s);
      h->begin = h->end = nullptr;
    }
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int esize(int dtype) { return dtype == MLP_F32 ? 4 : 2; }

bool is_gated(int act) {
  return act == MLP_ACT_SWIGLU || act == MLP_ACT_GEGLU || act == MLP_ACT_REGLU || act == MLP_ACT_GLU;
}

// The epilogues' function of an mlp_act: the gate function of a gated one, else f itself.
int act_fn_of(int act) {
  switch (act) {
    case MLP_ACT_SWIGLU: return FN_SILU;
    case MLP_ACT_GEGLU: case MLP_ACT_GELU_TANH: return FN_GELU_TANH;
    case MLP_ACT_REGLU: case MLP_ACT_RELU: return FN_RELU;
    case MLP_ACT_GLU: return FN_SIGMOID;
    default: return FN_RELU_SQ;
  }
}
DType dtype_of(int dtype) { return dtype == MLP_BF16 ? DT_BF16 : dtype == MLP_F16 ? DT_F16 : DT_F32; }
DType io_of(const mlp_desc* d) { return dtype_of(d->dtype); }

// ---- GEMM planning -------------------------------------------------------------------------

struct Plan {
  TileShape tile;
  int splits, k_per_split, tiles_m, tiles_n, group_m, grid;
  double est;   // the planner's time model of this plan, seconds
};

struct TileInfo { TileShape t; int bm, bn, slots; double eff; };
// slots: workgroups per CU that fit in LDS (a 2-stage 256x256 ring takes 128 KiB, a 3-stage
// 256x128 one 144 KiB, a 2-stage 128x128 one 64 KiB). eff: the fraction of a CU's peak MFMA rate
// one K-step of the tile sustains with every CU busy, measured per K-step on the bf16 GEMMs of
// the 2048-token 4096 x 11008 SwiGLU step (random data, all three layouts, fused epilogues):
// the 8-wave 256x256 tile takes ~1.95 us per 64-deep K-step, the 4-wave one ~2.1 us, a pair of
// 128x128 workgroups ~1.2 us, and the 256x128 tile ~1.3 us. These were fitted before the 8-wave
// tiles with a K-major A moved their DMAs to one wave per SIMD, which made those K-steps ~3-8 %
// faster; that only widens the 8-wave tiles' lead, which the planner already gives them. The
// 8-wave 256x128 figure was refitted later from forced-plan runs: the LLaMA down projection
// unsplit in 256 such tiles (one round, no reduce) runs 156 us against 164 for split-K 2 over
// 256x256 tiles plus the reduce, i.e. 0.40 of the per-CU peak.
const TileInfo kTiles[] = {
    {TILE_256x256_W8, 256, 256, 1, 0.44},   // 8 waves: two per SIMD hide each other's stalls
    {TILE_256x256, 256, 256, 1, 0.40},
    {TILE_256x128, 256, 128, 1, 0.33},
    {TILE_256x128_W8, 256, 128, 1, 0.40},
    {TILE_128x128, 128, 128, 2, 0.36},
};

bool is_fp8(DType in) { return in == DT_E4M3 || in == DT_F8G; }
int bk_of(DType in) { return is_fp8(in) ? 128 : (in == DT_F32 ? 32 : 64); }

// gated: N counts hidden units and a tile covers bn/2 of them (gate + up rows). only_tile >= 0
// restricts the choice to that tile shape.
Plan plan_gemm(DType in, int64_t M, int64_t N, int64_t K, bool allow_split, bool gated, int only_tile = -1) {
  const int bk = bk_of(in);
  const double per_cu = (is_fp8(in) ? 2.0 : in == DT_F32 ? 1.0 / 16.0 : 1.0) * 9.83e12;
  Plan best{};
  double best_t = 1e300;
  for (const TileInfo& ti : kTiles) {
    if (in == DT_F32 && ti.t != TILE_128x128) continue;
    if (is_fp8(in) && (ti.t == TILE_256x256_W8 || ti.t == TILE_256x128_W8)) continue;
    if (only_tile >= 0 && ti.t != only_tile) continue;
    const int64_t bn_units = gated ? ti.bn / 2 : ti.bn;
    const int64_t tm = (M + ti.bm - 1) / ti.bm, tn = (N + bn_units - 1) / bn_units;
    const int max_split = allow_split ? 16 : 1;
    for (int s = 1; s <= max_split; ++s) {
      const int64_t kps = ((K + s - 1) / s + bk - 1) / bk * bk;
      const int64_t s_eff = (K + kps - 1) / kps;
      if (s_eff != s) continue;
      const int64_t ntile = tm * tn * s;
      const int64_t slots = 256LL * ti.slots;
      const int64_t waves = (ntile + slots - 1) / slots;
      double t = (double)waves * ti.slots * (2.0 * ti.bm * ti.bn * kps) / (ti.eff * per_cu);
      if (s > 1) t += (2.0 * s * M * N * 4.0 + M * N * 4.0) / 6.0e12 + 4e-6;
      if (t < best_t * 0.98) {
        best_t = t;
        best.tile = ti.t;
        best.splits = s;
        best.k_per_split = (int)kps;
        best.tiles_m = (int)tm;
        best.tiles_n = (int)tn;
        // row bands of 8 tiles, column-major inside (32 tiles on an XCD at once share 8 A and
        // 4 B panels); with three tile columns a band of 24 tiles would straddle the XCD's
        // rounds and its A panels be fetched again, so those walk row by row (the GPT-shape
        // down projection and dx: 599 MB fetched for a 302 MB A; same box 247 -> 243 us,
        // 230 -> 228 us)
        best.group_m = tn == 3 ? 1 : (int)std::min<int64_t>(tm, 8);
        best.grid = (int)ntile;
        best.est = t;
      }
    }
  }
  return best;
}

// The fp8 GEMMs whose epilogue quantizes (relu(pre)^2 to e4m3, dpre to e5m2) run 128 x 128
// tiles, two workgroups per CU: their epilogue (an IEEE division and a conversion per value,
// plus the pre-activation store) is long next to a K loop of a few steps at the GPT shape, and a
// second workgroup runs its K loop meanwhile (GPT shape, 4-wave 256x256 -> 128x128: up projection
// 449 -> 272 us, fp8-gradient d-activation 552 -> 349 us). The recompute of the pre-activation
// takes the same plan as the forward.
Plan plan_quantizing(DType in, int64_t M, int64_t N, int64_t K) {
  return plan_gemm(in, M, N, K, false, false, TILE_128x128);
}

size_t partial_bytes(const Plan& p, int64_t M, int64_t N) {
  return p.splits > 1 ? (size_t)p.splits * M * N * sizeof(float) : 0;
}

// A store-epilogue GEMM whose unsplit 8-wave 256 x 256 tiles leave its last round mostly idle
// (the GPT-shape down projection and dx: 576 tiles = 2.25 rounds of 256), cut along M: rows
// [0, m1) in whole rounds of those tiles, rows [m1, M) planned on their own, where split-K fills
// the chip or smaller tiles do (GPT shape: 510 tiles of 48 K-steps, then the other 5632 rows as
// 132 tiles of 8-wave 256 x 128, one round).
// A static form of what a stream-K schedule does for the last round. m1 = 0: `main` covers all.
struct RowsPlan {
  Plan main{};
  int64_t m1 = 0;
  Plan tail{};
};

RowsPlan plan_rows(DType in, int64_t M, int64_t N, int64_t K) {
  RowsPlan r;
  r.main = plan_gemm(in, M, N, K, true, false);
  if (in != DT_BF16 && in != DT_F16) return r;
  // the cut is taken from the 8-wave 256x256 tiling, and kept if it beats the best plain plan
  const Plan w8 = plan_gemm(in, M, N, K, false, false, TILE_256x256_W8);
  const int64_t tn = w8.tiles_n, tiles = (int64_t)w8.tiles_m * tn;
  const int64_t rounds = tiles / 256, rem = tiles % 256;
  if (rounds < 1 || rem == 0 || rem > 128) return r;
  const int64_t m1 = rounds * 256 / tn * 256;   // whole row tiles that fill `rounds` rounds
  if (m1 < 256 || m1 >= M) return r;
  const Plan main = plan_gemm(in, m1, N, K, false, false, TILE_256x256_W8);
  const Plan tail = plan_gemm(in, M - m1, N, K, true, false);
  if (main.est + tail.est + 4e-6 < 0.97 * r.main.est) {
    r.main = main;
    r.m1 = m1;
    r.tail = tail;
  }
  return r;
}

size_t partial_bytes(const RowsPlan& r, int64_t M, int64_t N) {
  return r.m1 ? std::max(partial_bytes(r.main, r.m1, N), partial_bytes(r.tail, M - r.m1, N))
              : partial_bytes(r.main, M, N);
}

// ---- workspace layout ----------------------------------------------------------------------

struct WsLayout {
  size_t act = 0, act_bytes = 0;        // a / post / post_q  [M, H]
  size_t pre = 0, pre_bytes = 0;        // recomputed preact  [M, P]
  size_t dpre = 0, dpre_bytes = 0;      // dpreact when the caller passes none
  size_t xq = 0, xq_bytes = 0;          // widened e4m3 operands of the fp8 backward
  size_t w1q = 0, w1q_bytes = 0;
  size_t w2q = 0, w2q_bytes = 0;
  // fp8-gradient backward, all row-major [M, width]: e5m2 dout, e5m2 dpre, e4m3 relu(pre)^2
  size_t gq = 0, gq_bytes = 0, pq = 0, pq_bytes = 0, post = 0, post_bytes = 0;
  size_t partial = 0, partial_bytes = 0;
  size_t total = 0;
};

// Small-M (decode) gated up projection: when the fused gate/up GEMM has fewer tiles than the
// CUs, run it split along K over the stacked [W_gate; W_up] (N = 2H, 128 x 128 tiles, enough
// slices for two workgroups per CU) into fp32 partials, and apply the activation in the reduce.
// Returns splits = 1 when the fused kernel is the better choice.
Plan plan_gated_split(DType in, int64_t M, int64_t H, int64_t D) {
  Plan none{};
  none.splits = 1;
  if (in != DT_BF16 && in != DT_F16) return none;
  if (M > 128) return none;   // decode sizes: a single 128-row tile
  const Plan fused = plan_gemm(in, M, H, D, false, true);
  const int64_t tm = 1, tn = (2 * H + 127) / 128, tiles = tm * tn;
  if (fused.grid >= 256 || tiles >= 512) return none;
  const int64_t want = std::min<int64_t>(16, (512 + tiles - 1) / tiles);
  const int bk = bk_of(in);
  const int64_t kps = ((D + want - 1) / want + bk - 1) / bk * bk;
  const int64_t s = (D + kps - 1) / kps;
  if (s < 2) return none;
  Plan p{};
  p.tile = TILE_128x128;
  p.splits = (int)s;
  p.k_per_split = (int)kps;
  p.tiles_m = (int)tm;
  p.tiles_n = (int)tn;
  p.group_m = (int)std::min<int64_t>(tm, 8);
  p.grid = (int)(tiles * s);
  return p;
}

struct Gemms {   // the GEMMs a phase may run, in planning form
  Plan up_split;      // forward gated up projection split along K (splits = 1: fused instead)
  RowsPlan down;      // forward down projection
  Plan dw_down;
  RowsPlan dx;
  Plan dw_up;
};

Gemms plan_all(const mlp_desc* d) {
  const DType io = io_of(d);
  const DType fin = d->fp8_fwd ? DT_E4M3 : io;
  const bool gated = is_gated(d->act);
  const int64_t M = d->M, D = d->d_in, H = d->hidden, O = d->d_out, P = gated ? 2 * H : H;
  Gemms g;
  g.up_split = (gated && !d->fp8_fwd) ? plan_gated_split(io, M, H, D) : Plan{TILE_128x128, 1, 0, 0, 0, 0, 0};
  g.down = plan_rows(fin, M, O, H);
  if (d->fp8_bwd) {   // every backward product on fp8 operands
    g.dw_down = plan_gemm(DT_F8G, O, H, M, true, false);
    g.dx.main = plan_gemm(DT_F8G, M, D, H, true, false);
    g.dw_up = plan_gemm(DT_F8G, H, D, M, true, false);
    return g;
  }
  g.dw_down = plan_gemm(io, O, H, M, true, false);
  g.dx = plan_rows(io, M, D, P);
  g.dw_up = plan_gemm(io, P, D, M, true, false);
  return g;
}

// ---- the backward's dx and weight gradients in one launch -----------------------------------
//
// After the d-activation GEMM, dW_down = dout^T a, dx = dpreact [W_gate; W_up] and
// [dW_gate; dW_up] = dpreact^T x are independent. Run one after another, each idles part of the
// chip in its last round (the LLaMA step's dW_gate/dW_up has 1376 tiles = 5.4 rounds of 256) or
// pays split-K for too few tiles (dx: 128 tiles of 344 K-steps, split 2 plus a reduce). One
// launch of all three lets the short weight-gradient tiles fill the CUs around the long dx
// tiles, unsplit: quack's backward runs these GEMMs on a dynamic tile scheduler for the same
// reason (mlp.py, dynamic_scheduler=True), done here with a static order instead of atomics.

enum BwdGemm : int { BG_DW_DOWN = 0, BG_DX = 1, BG_DW_UP = 2, BG_DACT = 3 };

struct BwdGroup {
  int count = 0;              // 0: separate launches
  int member[kGroupMax] = {}; // BwdGemm ids, longest K first
  Plan plan[kGroupMax] = {};  // unsplit 8-wave 256 x 256 plans
};

struct GemmDims { int64_t M, N, K; };

// M, N, K of BwdGemm `which`.
GemmDims bwd_dims(const mlp_desc* d, int which) {
  const int64_t M = d->M, D = d->d_in, H = d->hidden, O = d->d_out, P = is_gated(d->act) ? 2 * H : H;
  switch (which) {
    case BG_DW_DOWN: return {O, H, M};
    case BG_DX: return {M, D, P};
    case BG_DACT: return {M, H, O};
    default: return {P, D, M};
  }
}

// Makespan, in K-steps, of list-scheduling the members' tiles on one XCD (it takes every 8th
// workgroup of each member, in launch order): each tile goes to the first of the 32 CUs to free
// up and holds it for its K-steps plus `overhead` (prologue and epilogue).
double list_makespan(const int64_t* tiles, const int64_t* steps, int count, double overhead) {
  std::vector<double> cu(32, 0.0);
  for (int j = 0; j < count; ++j)
    for (int64_t t = 0, n = (tiles[j] + 7) / 8; t < n; ++t)
      *std::min_element(cu.begin(), cu.end()) += (double)steps[j] + overhead;
  return *std::max_element(cu.begin(), cu.end());
}

// One launch of the products `ids` (at least two), when the time model prefers it to launching
// them one after another (each planned by plan_gemm: split-K allowed for the weight gradients and
// dx, the d-activation GEMM unsplit); count = 0 otherwise.
BwdGroup plan_group(const mlp_desc* d, const int* ids, int n) {
  BwdGroup g;
  const DType io = io_of(d);
  if (n < 2 || d->fp8_bwd || (io != DT_BF16 && io != DT_F16)) return g;
  int64_t tiles[kGroupMax], steps[kGroupMax];
  Plan plans[kGroupMax];
  double t_sep = 0.0;
  for (int j = 0; j < n; ++j) {
    const GemmDims dm = bwd_dims(d, ids[j]);
    plans[j] = plan_gemm(io, dm.M, dm.N, dm.K, false, false, TILE_256x256_W8);
    tiles[j] = plans[j].grid;
    if (tiles[j] > 32 * 256) return g;   // many rounds: a last round's idle CUs cost under 3 %
    steps[j] = (dm.K + 63) / 64;
    t_sep += plan_gemm(io, dm.M, dm.N, dm.K, ids[j] != BG_DACT, false).est;
  }
  // longest K first (stable on ties: the order of ids)
  int order[kGroupMax] = {0, 1, 2};
  std::stable_sort(order, order + n, [&](int a, int b) { return steps[a] > steps[b]; });
  int64_t ot[kGroupMax], os[kGroupMax];
  for (int j = 0; j < n; ++j) {
    ot[j] = tiles[order[j]];
    os[j] = steps[order[j]];
  }
  const TileInfo& w8 = kTiles[0];
  const double t_step = 2.0 * w8.bm * w8.bn * 64 / (w8.eff * 9.83e12);
  const double t_group = list_makespan(ot, os, n, 1.0) * t_step;
  if (!(t_group < 0.97 * t_sep)) return g;
  g.count = n;
  for (int j = 0; j < n; ++j) {
    g.member[j] = ids[order[j]];
    g.plan[j] = plans[order[j]];
  }
  return g;
}

unsigned bwd_mask(const void* dx, const void* dwg, const void* dwd) {
  return (dwd ? 1u << BG_DW_DOWN : 0u) | (dx ? 1u << BG_DX : 0u) | (dwg ? 1u << BG_DW_UP : 0u);
}

// The backward's launches after the (optional) recompute: `dact` groups the d-activation GEMM
// with dW_down (only with save_act: dW_down then reads the forward's activation, not one the
// d-activation GEMM writes); `rest` groups what remains of dx, dW_gate/dW_up and dW_down.
struct BwdSchedule { BwdGroup dact, rest; };

BwdSchedule plan_bwd_schedule(const mlp_desc* d, unsigned mask) {
  BwdSchedule sc;
  const bool need_dpre = mask & ((1u << BG_DX) | (1u << BG_DW_UP));
  if (d->save_act && need_dpre && (mask & (1u << BG_DW_DOWN))) {
    const int ids[2] = {BG_DACT, BG_DW_DOWN};
    sc.dact = plan_group(d, ids, 2);
    if (sc.dact.count > 0) mask &= ~(1u << BG_DW_DOWN);
  }
  int ids[kGroupMax], n = 0;
  for (int m : {BG_DX, BG_DW_UP, BG_DW_DOWN})
    if (mask & (1u << m)) ids[n++] = m;
  sc.rest = plan_group(d, ids, n);
  return sc;
}

// Decode-size problems whose forward products all run on the small-M kernel (no split-K
// partials): at most kSkinnyMaxRows tokens, 16-bit, not e4m3.
bool skinny_ok(const mlp_desc* d) {
  const DType io = io_of(d);
  return (io == DT_BF16 || io == DT_F16) && !d->fp8_fwd && d->M <= kSkinnyMaxRows;
}

WsLayout ws_layout(const mlp_desc* d, int phase) {
  WsLayout L;
  const bool gated = is_gated(d->act);
  const int64_t M = d->M, D = d->d_in, H = d->hidden, O = d->d_out, P = gated ? 2 * H : H;
  const size_t es = esize(d->dtype);
  const Gemms g = plan_all(d);
  size_t off = 0;
  auto take = [&](size_t& at, size_t& sz, size_t bytes) { at = off; sz = bytes; off += round_up(bytes); };
  if (phase == MLP_PHASE_FWD || phase == MLP_PHASE_FWD_INFER) {
    take(L.act, L.act_bytes, (size_t)M * H * (d->fp8_fwd ? 1 : es));
    take(L.partial, L.partial_bytes,
         skinny_ok(d) ? (skinny_parts_for(M, O, H) ? (size_t)kSkinnyParts * M * O * sizeof(float) : 0)
                      : std::max(partial_bytes(g.down, M, O), partial_bytes(g.up_split, M, 2 * H)));
  } else if (d->fp8_bwd) {
    if (d->recompute) take(L.pre, L.pre_bytes, (size_t)M * H * sizeof(float));
    take(L.gq, L.gq_bytes, (size_t)M * O);
    take(L.pq, L.pq_bytes, (size_t)M * H);
    take(L.post, L.post_bytes, (size_t)M * H);
    const size_t pb = std::max({partial_bytes(g.dw_down, O, H), partial_bytes(g.dx, M, D),
                                partial_bytes(g.dw_up, H, D)});
    take(L.partial, L.partial_bytes, pb);
  } else {
    take(L.act, L.act_bytes, (size_t)M * H * es);
    if (d->recompute) take(L.pre, L.pre_bytes, (size_t)M * P * es);
    else take(L.dpre, L.dpre_bytes, (size_t)M * P * es);
    if (d->fp8_fwd) {
      take(L.xq, L.xq_bytes, (size_t)M * D * 2);
      take(L.w1q, L.w1q_bytes, (size_t)H * D * 2);
      take(L.w2q, L.w2q_bytes, (size_t)O * H * 2);
    }
    const size_t pb = std::max({partial_bytes(g.dw_down, O, H), partial_bytes(g.dx, M, D),
                                partial_bytes(g.dw_up, P, D)});
    take(L.partial, L.partial_bytes, pb);
  }
  L.total = off;
  return L;
}

// ---- argument checks -------------------------------------------------------------------------

mlp_status check_desc(const mlp_desc* d) {
  if (!d) return fail(MLP_ERR_INVALID_ARG, "desc is NULL");
  if (d->M < 1 || d->d_in < 1 || d->hidden < 1 || d->d_out < 1)
    return fail(MLP_ERR_INVALID_ARG, "sizes must be >= 1 (M=%lld d_in=%lld hidden=%lld d_out=%lld)",
                (long long)d->M, (long long)d->d_in, (long long)d->hidden, (long long)d->d_out);
  const int64_t lim = (int64_t)1 << 30;
  if (d->M >= lim || d->d_in >= lim || d->hidden >= lim / 2 || d->d_out >= lim)
    return fail(MLP_ERR_UNSUPPORTED, "a size is beyond 2^30 (2^29 for hidden)");
  if (d->act < MLP_ACT_SWIGLU || d->act > MLP_ACT_RELU)
    return fail(MLP_ERR_INVALID_ARG, "act %d is not an mlp_act", d->act);
  // the GEMMs' DMA addresses are a scalar base plus a 32-bit per-lane offset of up to 64 rows of
  // the operand: every leading dimension (d_in, d_out, the gate/up width) must keep 64 row
  // pitches under 4 GiB
  const int64_t ld_lim = (int64_t)1 << 25;
  if (d->d_in >= ld_lim || d->d_out >= ld_lim || (is_gated(d->act) ? 2 : 1) * d->hidden >= ld_lim)
    return fail(MLP_ERR_UNSUPPORTED, "a leading dimension is 2^25 elements or more (d_in, d_out or the gate/up "
                "width): the DMA offsets are 32-bit");
  // no matrix of the problem may exceed 2^37 elements (256 GiB in bf16, beyond one GPU's HBM): tile
  // and workgroup counts then fit an int and size arithmetic has ample headroom
  {
    const int64_t P = (is_gated(d->act) ? 2 : 1) * d->hidden, mat_lim = (int64_t)1 << 37;
    const int64_t rows[] = {d->M, d->M, d->M, P, d->d_out}, cols[] = {d->d_in, P, d->d_out, d->d_in, d->hidden};
    for (int i = 0; i < 5; ++i)
      if (rows[i] > mat_lim / cols[i])
        return fail(MLP_ERR_UNSUPPORTED, "a matrix of the problem has more than 2^37 elements");
  }
  if (d->dtype != MLP_F32 && d->dtype != MLP_BF16 && d->dtype != MLP_F16)
    return fail(MLP_ERR_INVALID_ARG, "dtype %d is not an mlp_dtype", d->dtype);
  if (d->gate_mode != MLP_GATE_OUTSIDE && d->gate_mode != MLP_GATE_INSIDE)
    return fail(MLP_ERR_INVALID_ARG, "gate_mode %d is not an mlp_gate_mode", d->gate_mode);
  if ((d->recompute != 0 && d->recompute != 1) || (d->fp8_fwd != 0 && d->fp8_fwd != 1) ||
      (d->fp8_bwd != 0 && d->fp8_bwd != 1))
    return fail(MLP_ERR_INVALID_ARG, "recompute, fp8_fwd and fp8_bwd must be 0 or 1");
  if (d->fp8_bwd && !d->fp8_fwd) return fail(MLP_ERR_INVALID_ARG, "fp8_bwd needs fp8_fwd");
  if (d->save_act != 0 && d->save_act != 1) return fail(MLP_ERR_INVALID_ARG, "save_act must be 0 or 1");
  if (d->save_act && (d->recompute || d->fp8_fwd))
    return fail(MLP_ERR_INVALID_ARG, "save_act keeps the activation next to the saved pre-activation: it "
                "needs recompute = 0 and fp8_fwd = 0");
  if (!isfinite(d->gate_mult) || !isfinite(d->down_mult))
    return fail(MLP_ERR_INVALID_ARG, "gate_mult and down_mult must be finite");
  if (d->fp8_fwd && (d->act != MLP_ACT_RELU_SQ || d->dtype != MLP_BF16))
    return fail(MLP_ERR_UNSUPPORTED, "the e4m3 forward is implemented for ReLU^2 with bf16 I/O only");
  const int q = d->fp8_fwd ? 16 : (d->dtype == MLP_F32 ? 4 : 8);
  if (d->d_in % q || d->hidden % q || d->d_out % q)
    return fail(MLP_ERR_ALIGNMENT, "d_in, hidden and d_out must be multiples of %d (16-byte rows)", q);
  return MLP_OK;
}

mlp_status need_ptr(const void* p, const char* name, bool align = true) {
  if (!p) return fail(MLP_ERR_INVALID_ARG, "%s is NULL", name);
  if (align && !aligned16(p)) return fail(MLP_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
  if (!align && !aligned4(p)) return fail(MLP_ERR_ALIGNMENT, "%s is not 4-byte aligned", name);
  return MLP_OK;
}

mlp_status need_null(const void* p, const char* name, const char* why) {
  return p ? fail(MLP_ERR_INVALID_ARG, "%s must be NULL %s", name, why) : MLP_OK;
}

#define MLP_TRY(expr)                 \
  do {                                \
    const mlp_status st_ = (expr);    \
    if (st_ != MLP_OK) return st_;    \
  } while (0)

mlp_status check_fp8(const mlp_desc* d, const mlp_fp8* f, bool fwd) {
  if (!d->fp8_fwd) return need_null(f, "fp8", "unless desc->fp8_fwd");
  if (!f) return fail(MLP_ERR_INVALID_ARG, "fp8 is NULL but desc->fp8_fwd is set");
  MLP_TRY(need_ptr(f->x_q, "fp8->x_q"));
  MLP_TRY(need_ptr(f->w1_q, "fp8->w1_q"));
  MLP_TRY(need_ptr(f->w2_q, "fp8->w2_q"));
  MLP_TRY(need_ptr(f->s_x, "fp8->s_x", false));
  MLP_TRY(need_ptr(f->s_w1, "fp8->s_w1", false));
  MLP_TRY(need_ptr(f->s_w2, "fp8->s_w2", false));
  if (fwd) {
    MLP_TRY(need_ptr(f->s_post, "fp8->s_post", false));
    MLP_TRY(need_ptr(f->post_amax, "fp8->post_amax", false));
  } else if (d->fp8_bwd) {
    MLP_TRY(need_ptr(f->w1t_q, "fp8->w1t_q"));
    MLP_TRY(need_ptr(f->w2t_q, "fp8->w2t_q"));
    MLP_TRY(need_ptr(f->s_post, "fp8->s_post", false));
    MLP_TRY(need_ptr(f->s_grad, "fp8->s_grad", false));
    MLP_TRY(need_ptr(f->s_dpre, "fp8->s_dpre", false));
    MLP_TRY(need_ptr(f->dpre_amax, "fp8->dpre_amax", false));
  } else {
    MLP_TRY(need_null(f->w1t_q, "fp8->w1t_q", "unless desc->fp8_bwd"));
    MLP_TRY(need_null(f->w2t_q, "fp8->w2t_q", "unless desc->fp8_bwd"));
  }
  return MLP_OK;
}

mlp_status check_ws(const mlp_desc* d, int phase, const void* ws, size_t ws_bytes) {
  const size_t need = ws_layout(d, phase).total;
  if (ws_bytes < need)
    return fail(MLP_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  if (need && !ws) return fail(MLP_ERR_INVALID_ARG, "workspace is NULL");
  if (ws && !aligned16(ws)) return fail(MLP_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  return MLP_OK;
}

mlp_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MLP_OK;
  return fail(MLP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// a with the problem sizes and the tile grid of plan p
GemmArgs planned(GemmArgs a, const Plan& p, int64_t M, int64_t N, int64_t K) {
  a.M = (int)M;
  a.N = (int)N;
  a.K = (int)K;
  a.tiles_m = p.tiles_m;
  a.tiles_n = p.tiles_n;
  a.group_m = p.group_m;
  a.k_per_split = p.k_per_split;
  return a;
}

// One GEMM, split along K when the plan says so (fp32 partials, then a fixed-order reduce
// that applies the store epilogue).
mlp_status gemm(DType in, DType io, Layout lay, int epi, const Plan& p, GemmArgs a, int64_t M,
                int64_t N, int64_t K, void* partial, hipStream_t s, const char* what) {
  a = planned(a, p, M, N, K);
  if (p.splits > 1) {
    GemmArgs b = a;
    b.partial = reinterpret_cast<float*>(partial);
    MLP_TRY(hip_status(run_gemm(in, DT_F32, lay, EPI_PARTIAL, p.tile, b, p.grid, s), what));
    return hip_status(run_splitk_reduce(io, b.partial, p.splits, (int)M, (int)N, a.C0, a.C1, a.ldc0,
                                        a.c_split, a.alpha, a.alpha_dev0, a.alpha_dev1, a.accumulate, s),
                      what);
  }
  return hip_status(run_gemm(in, io, lay, epi, p.tile, a, p.grid, s), what);
}

// A non-split GEMM over output columns [0, N) as two launches when that fills the CUs better:
// 8-wave 256 x 256 tiles for the columns that make whole rounds of 256 tiles, 8-wave 256 x 128
// tiles for the rest (one launch's last round otherwise idles part of the chip: the
// d-activation GEMM of the LLaMA step has 344 tiles of 256 x 256 = 1.34 rounds, or 688 tiles of
// 256 x 128, whose K loop moves 1.5x the operand bytes per FLOP). Column offsets move B (MN-major:
// by columns; K-major: by rows), C0, C1 and aux; es = bytes per element of the outputs / aux.
// Falls back to `whole` when the split does not apply.
mlp_status gemm_cols_split(DType in, DType io, Layout lay, int epi, const Plan& whole, GemmArgs a, int64_t M,
                           int64_t N, int64_t K, int es, hipStream_t s, const char* what) {
  const int64_t tm = (M + 255) / 256;
  const int64_t n1_tiles = tm > 0 ? 256 / tm : 0;   // N-tiles of one full round
  const int64_t n1 = n1_tiles * 256;
  if (in != DT_BF16 && in != DT_F16) return gemm(in, io, lay, epi, whole, a, M, N, K, nullptr, s, what);
  if (whole.splits != 1 || tm > 256 || n1_tiles < 1 || n1 >= N || (N - n1) % 128 ||
      (N - n1) / 128 * tm > 256)
    return gemm(in, io, lay, epi, whole, a, M, N, K, nullptr, s, what);
  const Plan p1 = plan_gemm(in, M, n1, K, false, false, TILE_256x256_W8);
  const Plan p2 = plan_gemm(in, M, N - n1, K, false, false, TILE_256x128_W8);
  MLP_TRY(gemm(in, io, lay, epi, p1, a, M, n1, K, nullptr, s, what));
  GemmArgs b = a;
  const int ebi = in == DT_F32 ? 4 : 2;
  b.B0 = lay == NT ? static_cast<const char*>(a.B0) + n1 * a.ldb * ebi : static_cast<const char*>(a.B0) + n1 * ebi;
  if (a.C0) b.C0 = static_cast<char*>(a.C0) + n1 * es;
  if (a.C1) b.C1 = static_cast<char*>(a.C1) + n1 * es;
  if (a.aux) b.aux = static_cast<char*>(a.aux) + n1 * es;
  return gemm(in, io, lay, epi, p2, b, M, N - n1, K, nullptr, s, what);
}

// A store-epilogue GEMM planned by plan_rows: rows [0, m1) with `main`, then rows [m1, M) with
// `tail` (A and the output moved down by m1 rows; A is K-major for NT / NN, MN-major for TN).
mlp_status gemm_rows(DType in, DType io, Layout lay, const RowsPlan& r, GemmArgs a, int64_t M, int64_t N,
                     int64_t K, void* partial, hipStream_t s, const char* what) {
  if (r.m1 == 0 || a.C1 != nullptr) return gemm(in, io, lay, EPI_STORE, r.main, a, M, N, K, partial, s, what);
  MLP_TRY(gemm(in, io, lay, EPI_STORE, r.main, a, r.m1, N, K, partial, s, what));
  const int64_t ei = in == DT_F32 ? 4 : (is_fp8(in) ? 1 : 2), eo = io == DT_F32 ? 4 : 2;
  GemmArgs b = a;
  b.A = static_cast<const char*>(a.A) + (lay == TN ? r.m1 : r.m1 * a.lda) * ei;
  b.C0 = static_cast<char*>(a.C0) + r.m1 * a.ldc0 * eo;
  return gemm(in, io, lay, EPI_STORE, r.tail, b, M - r.m1, N, K, partial, s, what);
}

GemmArgs base_args(const mlp_desc* d) {
  GemmArgs a{};
  a.alpha = 1.0f;
  a.gate_mult = d->gate_mult;
  a.gate_inside = d->gate_mode == MLP_GATE_INSIDE;
  a.act = act_fn_of(d->act);
  a.b_split = 1 << 30;
  a.c_split = 1 << 30;
  return a;
}

// Forward GEMM 1: the gated / non-gated / e4m3 ReLU^2 up projection with its activation epilogue.
// preact_out: where g|u or pre goes (NULL: not kept); act_out: where a / post / post_q goes.
// Decode-size problems (at most kSkinnyMaxRows tokens, 16-bit, not e4m3): every product of the
// forward, and the backward's recompute, runs on the small-M kernel (run_skinny), which streams
// the weights once instead of padding the tokens to a 128- or 256-row tile. The training and the
// inference forward and the recompute then share one kernel, so they agree bit for bit.

mlp_status up_projection(const mlp_desc* d, const void* x, const void* wg, const void* wu,
                         const mlp_fp8* f, void* preact_out, void* act_out, void* partial, hipStream_t s) {
  const DType io = io_of(d);
  const int64_t M = d->M, D = d->d_in, H = d->hidden;
  GemmArgs a = base_args(d);
  a.lda = D;
  a.ldb = D;
  a.C0 = act_out;
  a.ldc0 = H;
  a.aux = preact_out;
  a.flags = (preact_out ? 1 : 0) | (act_out ? 2 : 0);
  if (is_gated(d->act)) {
    a.A = x;
    a.B0 = wg;
    a.B1 = wu;
    a.ld_aux = 2 * H;
    a.half = (int)H;
    if (skinny_ok(d))
      return hip_status(run_skinny(io, EPI_GATED, planned(a, Plan{}, M, H, D), s), "gate/up projection (small M)");
    const Plan ps = plan_all(d).up_split;
    if (ps.splits > 1) {   // decode-size: split-K partials of [g | u], activation in the reduce
      GemmArgs b = a;
      b.M = (int)M;
      b.N = (int)(2 * H);
      b.K = (int)D;
      b.b_split = (int)H;
      b.tiles_m = ps.tiles_m;
      b.tiles_n = ps.tiles_n;
      b.group_m = ps.group_m;
      b.k_per_split = ps.k_per_split;
      b.partial = reinterpret_cast<float*>(partial);
      MLP_TRY(hip_status(run_gemm(io, DT_F32, NT, EPI_PARTIAL, ps.tile, b, ps.grid, s), "gate/up projection"));
      return hip_status(run_gated_reduce(io, b.partial, ps.splits, (int)M, (int)H, a.alpha, a.alpha_dev0,
                                         a.alpha_dev1, preact_out, act_out, d->gate_mult,
                                         d->gate_mode == MLP_GATE_INSIDE, a.act, s),
                        "gate/up projection reduce");
    }
    const Plan p = plan_gemm(io, M, H, D, false, true);
    return gemm(io, io, NT, EPI_GATED, p, a, M, H, D, nullptr, s, "gate/up projection");
  }
  a.ld_aux = H;
  if (d->fp8_fwd) {
    a.A = f->x_q;
    a.B0 = f->w1_q;
    a.alpha_dev0 = f->s_x;
    a.alpha_dev1 = f->s_w1;
    a.s_post = f->s_post;
    a.amax = f->post_amax;
    const Plan p = plan_quantizing(DT_E4M3, M, H, D);
    // the fp8-gradient backward takes its rounding decisions on an fp32 pre-activation
    return gemm(DT_E4M3, d->fp8_bwd ? DT_F32 : DT_BF16, NT, EPI_F8ACT, p, a, M, H, D, nullptr, s,
                "e4m3 up projection");
  }
  a.A = x;
  a.B0 = wg;
  if (skinny_ok(d)) return hip_status(run_skinny(io, EPI_ACT, planned(a, Plan{}, M, H, D), s), "up projection (small M)");
  const Plan p = plan_gemm(io, M, H, D, false, false);
  return gemm(io, io, NT, EPI_ACT, p, a, M, H, D, nullptr, s, "up projection");
}

// With save_act: the [M, H] activation after the [M, P] pre-activation in saved_preact.
void* saved_act(const mlp_desc* d, const void* saved) {
  const int64_t P = is_gated(d->act) ? 2 * d->hidden : d->hidden;
  return const_cast<char*>(static_cast<const char*>(saved)) + d->M * P * esize(d->dtype);
}

// Host-side checks of a forward call's arguments (everything but the workspace).
mlp_status fwd_check(const mlp_desc* d, const void* x, const void* wg, const void* wu, const void* wd,
                     const void* out, const void* saved, const mlp_fp8* f, bool infer) {
  MLP_TRY(check_desc(d));
  const bool gated = is_gated(d->act);
  if (!d->fp8_fwd) {
    MLP_TRY(need_ptr(x, "x"));
    MLP_TRY(need_ptr(wg, gated ? "w_gate" : "w_gate (W1)"));
    MLP_TRY(need_ptr(wd, gated ? "w_down" : "w_down (W2)"));
  }
  if (gated) MLP_TRY(need_ptr(wu, "w_up"));
  else MLP_TRY(need_null(wu, "w_up", "for a non-gated activation"));
  MLP_TRY(need_ptr(out, "out"));
  if (!infer) {
    if (d->recompute) MLP_TRY(need_null(saved, "saved_preact", "with recompute"));
    else MLP_TRY(need_ptr(saved, "saved_preact"));
  }
  return check_fp8(d, f, true);
}

// The forward's launches, on arguments that passed fwd_check and a workspace of at least
// ws_layout(d, phase).total bytes.
mlp_status fwd_run(const mlp_desc* d, const void* x, const void* wg, const void* wu, const void* wd,
                   void* out, void* saved, const mlp_fp8* f, void* ws, void* stream, bool infer) {
  const int phase = infer ? MLP_PHASE_FWD_INFER : MLP_PHASE_FWD;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const WsLayout L = ws_layout(d, phase);
  char* w = reinterpret_cast<char*>(ws);
  const int64_t M = d->M, H = d->hidden, O = d->d_out;
  // the activation the down projection reads: kept after the pre-activation with save_act
  void* act = (d->save_act && !infer) ? saved_act(d, saved) : w + L.act;
  {
    StageScope st(MLP_STAGE_UP, s);
    MLP_TRY(up_projection(d, x, wg, wu, f, infer ? nullptr : saved, act, w + L.partial, s));
  }

  const DType io = io_of(d);
  const DType fin = d->fp8_fwd ? DT_E4M3 : io;
  GemmArgs b = base_args(d);
  b.A = act;
  b.lda = H;
  b.B0 = d->fp8_fwd ? f->w2_q : wd;
  b.ldb = H;
  b.C0 = out;
  b.ldc0 = O;
  b.alpha = d->down_mult;
  if (d->fp8_fwd) {
    b.alpha_dev0 = f->s_post;
    b.alpha_dev1 = f->s_w2;
  }
  StageScope st(MLP_STAGE_DOWN, s);
  if (skinny_ok(d)) {
    if (skinny_parts_for(M, O, H)) {   // K split over workgroups, then the fixed-order reduce
      GemmArgs c = planned(b, Plan{}, M, O, H);
      c.partial = reinterpret_cast<float*>(w + L.partial);
      MLP_TRY(hip_status(run_skinny(io, EPI_PARTIAL, c, s), "down projection (small M, K parts)"));
      return hip_status(run_splitk_reduce(io, c.partial, kSkinnyParts, (int)M, (int)O, out, nullptr, O, c.c_split,
                                          c.alpha, c.alpha_dev0, c.alpha_dev1, 0, s),
                        "down projection (small M, reduce)");
    }
    return hip_status(run_skinny(io, EPI_STORE, planned(b, Plan{}, M, O, H), s), "down projection (small M)");
  }
  const RowsPlan p = plan_all(d).down;
  return gemm_rows(fin, io, NT, p, b, M, O, H, w + L.partial, s, "down projection");
}

mlp_status fwd_impl(const mlp_desc* d, const void* x, const void* wg, const void* wu, const void* wd,
                    void* out, void* saved, const mlp_fp8* f, void* ws, size_t ws_bytes, void* stream,
                    bool infer) {
  MLP_TRY(fwd_check(d, x, wg, wu, wd, out, saved, f, infer));
  MLP_TRY(check_ws(d, infer ? MLP_PHASE_FWD_INFER : MLP_PHASE_FWD, ws, ws_bytes));
  return fwd_run(d, x, wg, wu, wd, out, saved, f, ws, stream, infer);
}

// ---- the library-held workspace of mlp_fwd_infer_noalloc ---------------------------------------
// One copy per GPU, held from the library's load until the process ends. In host code `scratch`
// names a host-side stand-in, not the device array: the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address is
// ever handed to a kernel.
static __device__ __attribute__((aligned(256))) unsigned char scratch[MLP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// The scratch array's device address on the device `stream` runs on, which must be the calling
// thread's current device.
mlp_status scratch_address(void* stream, void** out) {
  int dev = -1;
  MLP_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(MLP_ERR_UNSUPPORTED, "device %d is beyond the %d this library tracks", dev, kMaxDevices);
  if (stream) {
    int sdev = -1;
    MLP_TRY(hip_status(hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev), "hipStreamGetDevice"));
    if (sdev != dev)
      return fail(MLP_ERR_INVALID_ARG, "stream belongs to device %d but the current device is %d", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    MLP_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u))
      return fail(MLP_ERR_HIP, "hipGetSymbolAddress(scratch) gave an unusable address %p", p);
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MLP_OK;
}

// Backward with fp8 gradients (ReLU^2, see mlp_fp8; the pre-activation is fp32, so the e5m2 /
// e4m3 rounding decisions on dpre and relu(pre)^2 are taken on an fp32 value): dout -> e5m2
// codes, row-major; dpre_q = e5m2(dm (dout_q W2) 2 relu(pre) / s_dpre) from the e5m2 x e4m3
// product against the transposed W2 cache, which also writes relu(pre)^2's e4m3 codes; dx =
// dpre_q W1 against the transposed W1 cache. The weight gradients dW1 = dpre_q^T x_q and dW2 =
// dm dout_q^T post_q reduce over the tokens: they read the same row-major codes MN-major (the
// 8-bit transposing LDS read), so no code is ever copied transposed.
mlp_status bwd_fp8(const mlp_desc* d, const void* dout, const void* saved, void* dx, void* dw1, void* dw2,
                   int grad_accum, const mlp_fp8* f, char* w, const WsLayout& L, const Gemms& G, hipStream_t s) {
  const int64_t M = d->M, D = d->d_in, H = d->hidden, O = d->d_out;
  const DType gio = grad_accum ? DT_F32 : DT_BF16;
  const bool need_dpre = dx != nullptr || dw1 != nullptr;

  // pre-activation: saved by the forward, or recomputed with the forward's own e4m3 product
  // (same plan, same bits)
  const void* pre = saved;
  if (d->recompute) {
    GemmArgs a = base_args(d);
    a.A = f->x_q;
    a.lda = D;
    a.B0 = f->w1_q;
    a.ldb = D;
    a.C0 = w + L.pre;
    a.ldc0 = H;
    a.alpha_dev0 = f->s_x;
    a.alpha_dev1 = f->s_w1;
    const Plan p = plan_quantizing(DT_E4M3, M, H, D);
    StageScope st(MLP_STAGE_RECOMPUTE, s);
    MLP_TRY(gemm(DT_E4M3, DT_F32, NT, EPI_STORE, p, a, M, H, D, nullptr, s, "recompute pre-activation"));
    pre = w + L.pre;
  }
  void* gq = w + L.gq;
  void* pq = w + L.pq;
  void* post_codes = w + L.post;
  if (need_dpre) {   // dpre_q = e5m2(dm (dout_q W2) 2 relu(pre) / s_dpre), max|dpre| -> dpre_amax
    StageScope st(MLP_STAGE_DACT, s);
    MLP_TRY(hip_status(run_quantize_fp8_2d(DT_BF16, dout, M, O, O, 0, 1, f->s_grad, gq, nullptr, 0, s),
                       "quantize dout"));
    GemmArgs a = base_args(d);
    a.A = gq;
    a.lda = O;
    a.B0 = f->w2t_q;
    a.ldb = O;
    a.C0 = pq;
    a.ldc0 = H;
    a.aux = const_cast<void*>(pre);
    a.ld_aux = H;
    a.alpha = d->down_mult;
    a.alpha_dev0 = f->s_grad;
    a.alpha_dev1 = f->s_w2;
    a.s_post = f->s_dpre;
    a.amax = f->dpre_amax;
    if (dw2) {   // relu(pre)^2's e4m3 codes, row-major, from the pre-activation this GEMM reads
      a.C1 = post_codes;
      a.ldc1 = H;
      a.s_c1 = f->s_post;
    }
    const Plan p = plan_quantizing(DT_F8G, M, H, O);
    MLP_TRY(gemm(DT_F8G, DT_F32, NT, EPI_F8DACT, p, a, M, H, O, nullptr, s, "fp8 d-activation GEMM"));
  } else if (dw2) {
    StageScope st(MLP_STAGE_DW_DOWN, s);
    MLP_TRY(hip_status(run_quantize_fp8_2d(DT_BF16, dout, M, O, O, 0, 1, f->s_grad, gq, nullptr, 0, s),
                       "quantize dout"));
  }
  if (dw2) {   // dW2 (+)= dm dout_q^T post_q, post_q = e4m3(relu(pre)^2 / s_post)
    StageScope st(MLP_STAGE_DW_DOWN, s);
    // relu(pre)^2's codes: the d-activation GEMM wrote them; without that GEMM they are formed
    // here from the fp32 pre-activation
    if (!need_dpre)
      MLP_TRY(hip_status(run_quantize_fp8_2d(DT_F32, pre, M, H, H, 1, 0, f->s_post, post_codes, nullptr, 0, s),
                         "quantize relu(pre)^2"));
    GemmArgs a = base_args(d);
    a.A = gq;
    a.lda = O;
    a.B0 = post_codes;
    a.ldb = H;
    a.C0 = dw2;
    a.ldc0 = H;
    a.alpha = d->down_mult;
    a.alpha_dev0 = f->s_grad;
    a.alpha_dev1 = f->s_post;
    a.accumulate = grad_accum;
    MLP_TRY(gemm(DT_F8G, gio, TN, EPI_STORE, G.dw_down, a, O, H, M, w + L.partial, s, "fp8 dW_down"));
  }
  if (dx) {   // dx = dpre_q W1
    GemmArgs a = base_args(d);
    a.A = pq;
    a.lda = H;
    a.B0 = f->w1t_q;
    a.ldb = H;
    a.C0 = dx;
    a.ldc0 = D;
    a.alpha_dev0 = f->s_dpre;
    a.alpha_dev1 = f->s_w1;
    StageScope st(MLP_STAGE_DX, s);
    MLP_TRY(gemm(DT_F8G, DT_BF16, NT, EPI_STORE, G.dx.main, a, M, D, H, w + L.partial, s, "fp8 dx"));
  }
  if (dw1) {   // dW1 (+)= dpre_q^T x_q
    StageScope st(MLP_STAGE_DW_UP, s);
    GemmArgs a = base_args(d);
    a.A = pq;
    a.lda = H;
    a.B0 = f->x_q;
    a.ldb = D;
    a.C0 = dw1;
    a.ldc0 = D;
    a.alpha_dev0 = f->s_dpre;
    a.alpha_dev1 = f->s_x;
    a.accumulate = grad_accum;
    MLP_TRY(gemm(DT_F8G, gio, TN, EPI_STORE, G.dw_up, a, H, D, M, w + L.partial, s, "fp8 dW1"));
  }
  return MLP_OK;
}

}  // namespace

extern "C" {

int mlp_abi_version(void) { return 5; }

mlp_status mlp_bwd_grouped(const mlp_desc* d, int* grouped) {
  MLP_TRY(check_desc(d));
  if (!grouped) return fail(MLP_ERR_INVALID_ARG, "grouped must not be NULL");
  const BwdSchedule sch = plan_bwd_schedule(d, bwd_mask(d, d, d));
  *grouped = (sch.rest.count > 0 ? MLP_BWD_GROUPED : 0) | (sch.dact.count > 0 ? MLP_BWD_DW_DOWN_WITH_DACT : 0);
  return MLP_OK;
}

const char* mlp_status_string(int st) {
  switch (st) {
    case MLP_OK: return "MLP_OK";
    case MLP_ERR_INVALID_ARG: return "MLP_ERR_INVALID_ARG";
    case MLP_ERR_UNSUPPORTED: return "MLP_ERR_UNSUPPORTED";
    case MLP_ERR_ALIGNMENT: return "MLP_ERR_ALIGNMENT";
    case MLP_ERR_WORKSPACE: return "MLP_ERR_WORKSPACE";
    case MLP_ERR_HIP: return "MLP_ERR_HIP";
    default: return "unknown mlp_status";
  }
}

const char* mlp_last_error(void) { return g_last_error.c_str(); }

size_t mlp_workspace_bytes(const mlp_desc* d, int phase) {
  if (check_desc(d) != MLP_OK) return 0;
  if (phase < MLP_PHASE_FWD || phase > MLP_PHASE_BWD) {
    fail(MLP_ERR_INVALID_ARG, "phase %d is not an mlp_phase", phase);
    return 0;
  }
  return ws_layout(d, phase).total;
}

mlp_status mlp_fwd(const mlp_desc* d, const void* x, const void* wg, const void* wu, const void* wd,
                   void* out, void* saved, const mlp_fp8* f, void* ws, size_t ws_bytes, void* stream) {
  return fwd_impl(d, x, wg, wu, wd, out, saved, f, ws, ws_bytes, stream, false);
}

mlp_status mlp_fwd_infer(const mlp_desc* d, const void* x, const void* wg, const void* wu,
                         const void* wd, void* out, const mlp_fp8* f, void* ws, size_t ws_bytes,
                         void* stream) {
  return fwd_impl(d, x, wg, wu, wd, out, nullptr, f, ws, ws_bytes, stream, true);
}

mlp_status mlp_fwd_infer_noalloc(const mlp_desc* d, const void* x, const void* wg, const void* wu,
                                 const void* wd, void* out, const mlp_fp8* f, void* stream) {
  MLP_TRY(fwd_check(d, x, wg, wu, wd, out, nullptr, f, true));
  const size_t need = ws_layout(d, MLP_PHASE_FWD_INFER).total;
  if (need > (size_t)MLP_NOALLOC_SCRATCH_BYTES)
    return fail(MLP_ERR_WORKSPACE,
                "this inference forward needs %zu bytes of workspace; the library's static scratch holds %zu "
                "(MLP_NOALLOC_SCRATCH_BYTES): call mlp_fwd_infer with a caller-owned workspace instead",
                need, (size_t)MLP_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  MLP_TRY(scratch_address(stream, &ws));
  return fwd_run(d, x, wg, wu, wd, out, nullptr, f, ws, stream, true);
}

mlp_status mlp_bwd(const mlp_desc* d, const void* dout, const void* x, const void* wg, const void* wu,
                   const void* wd, const void* saved, void* dpreact, void* dx, void* dwg, void* dwu,
                   void* dwd, int grad_accum, const mlp_fp8* f, void* ws, size_t ws_bytes,
                   void* stream) {
  MLP_TRY(check_desc(d));
  const bool gated = is_gated(d->act);
  MLP_TRY(need_ptr(dout, "dout"));
  if (!d->fp8_fwd) {
    MLP_TRY(need_ptr(x, "x"));
    MLP_TRY(need_ptr(wg, gated ? "w_gate" : "w_gate (W1)"));
    MLP_TRY(need_ptr(wd, gated ? "w_down" : "w_down (W2)"));
  }
  if (gated) MLP_TRY(need_ptr(wu, "w_up"));
  else MLP_TRY(need_null(wu, "w_up", "for a non-gated activation"));
  if (d->recompute) MLP_TRY(need_null(saved, "saved_preact", "with recompute"));
  else MLP_TRY(need_ptr(saved, "saved_preact"));
  if (dpreact) MLP_TRY(need_ptr(dpreact, "dpreact"));
  if (dx) MLP_TRY(need_ptr(dx, "dx"));
  if (dwd) MLP_TRY(need_ptr(dwd, "dw_down"));
  if (gated) {
    if ((dwg == nullptr) != (dwu == nullptr))
      return fail(MLP_ERR_INVALID_ARG, "dw_gate and dw_up must both be given or both be NULL");
    if (dwg) {
      MLP_TRY(need_ptr(dwg, "dw_gate"));
      MLP_TRY(need_ptr(dwu, "dw_up"));
    }
  } else {
    MLP_TRY(need_null(dwu, "dw_up", "for a non-gated activation"));
    if (dwg) MLP_TRY(need_ptr(dwg, "dw_gate (dW1)"));
  }
  if (grad_accum != 0 && grad_accum != 1) return fail(MLP_ERR_INVALID_ARG, "grad_accum must be 0 or 1");
  MLP_TRY(check_fp8(d, f, false));
  if (d->fp8_bwd) MLP_TRY(need_null(dpreact, "dpreact", "with fp8_bwd (dpre stays e5m2 in the workspace)"));
  MLP_TRY(check_ws(d, MLP_PHASE_BWD, ws, ws_bytes));

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const WsLayout L = ws_layout(d, MLP_PHASE_BWD);
  const Gemms G = plan_all(d);
  char* w = reinterpret_cast<char*>(ws);
  void* partial = w + L.partial;
  const DType io = io_of(d);
  const DType gio = grad_accum ? DT_F32 : io;
  const int64_t M = d->M, D = d->d_in, H = d->hidden, O = d->d_out, P = gated ? 2 * H : H;
  if (d->fp8_bwd) return bwd_fp8(d, dout, saved, dx, dwg, dwd, grad_accum, f, w, L, G, s);

  // e4m3 path: the backward reads the exact bf16 widening of the forward's operands; their
  // scales enter each GEMM's epilogue.
  const float *sx = nullptr, *sw1 = nullptr, *sw2 = nullptr;
  if (d->fp8_fwd) {
    StageScope st(MLP_STAGE_WIDEN, s);
    MLP_TRY(hip_status(run_dequant_e4m3_bf16(f->x_q, w + L.xq, M * D, s), "widen x_q"));
    MLP_TRY(hip_status(run_dequant_e4m3_bf16(f->w1_q, w + L.w1q, H * D, s), "widen w1_q"));
    MLP_TRY(hip_status(run_dequant_e4m3_bf16(f->w2_q, w + L.w2q, O * H, s), "widen w2_q"));
    x = w + L.xq;
    wg = w + L.w1q;
    wd = w + L.w2q;
    sx = f->s_x;
    sw1 = f->s_w1;
    sw2 = f->s_w2;
  }

  // pre-activation: saved by the forward, or recomputed from x (one extra GEMM)
  const void* pre = saved;
  if (d->recompute) {
    GemmArgs a = base_args(d);
    a.A = x;
    a.lda = D;
    a.B0 = wg;
    a.B1 = wu;
    a.ldb = D;
    a.aux = w + L.pre;
    a.ld_aux = P;
    a.half = (int)H;
    a.flags = 1;
    a.alpha_dev0 = sx;
    a.alpha_dev1 = sw1;
    const int epi = gated ? EPI_GATED : EPI_ACT;
    StageScope st(MLP_STAGE_RECOMPUTE, s);
    if (skinny_ok(d)) {
      MLP_TRY(hip_status(run_skinny(io, epi, planned(a, Plan{}, M, H, D), s), "recompute pre-activation (small M)"));
    } else {
      const Plan p = plan_gemm(io, M, H, D, false, gated);
      MLP_TRY(gemm(io, io, NT, epi, p, a, M, H, D, nullptr, s, "recompute pre-activation"));
    }
    pre = w + L.pre;
  }

  const bool need_dpre = dx != nullptr || dwg != nullptr;
  void* dpre = dpreact ? dpreact : (d->recompute ? w + L.pre : w + L.dpre);
  // the activation dW_down reads: the forward's (save_act), else re-emitted by the d-activation
  // GEMM or the activation-only pass into the workspace
  void* act = d->save_act ? saved_act(d, saved) : w + L.act;

  // da = dm * dout W_down, fused with d(act) against the pre-activation; re-emits a / post
  // when dW_down needs it and the forward did not keep it
  GemmArgs a_dact = base_args(d);
  a_dact.A = dout;
  a_dact.lda = O;
  a_dact.B0 = wd;
  a_dact.ldb = H;
  a_dact.aux = const_cast<void*>(pre);
  a_dact.ld_aux = P;
  a_dact.half = (int)H;
  a_dact.C0 = dpre;
  a_dact.ldc0 = P;
  a_dact.C1 = act;
  a_dact.ldc1 = H;
  a_dact.flags = (dwd && !d->save_act) ? 2 : 0;
  a_dact.alpha = d->down_mult;
  a_dact.alpha_dev0 = sw2;
  // dW_down (+)= dm * dout^T a
  GemmArgs a_dwd = base_args(d);
  a_dwd.A = dout;
  a_dwd.lda = O;
  a_dwd.B0 = act;
  a_dwd.ldb = H;
  a_dwd.C0 = dwd;
  a_dwd.ldc0 = H;
  a_dwd.alpha = d->down_mult;
  a_dwd.accumulate = grad_accum;
  // dx = [dg | du] [W_gate; W_up]  (non-gated: dpre W1)
  GemmArgs a_dx = base_args(d);
  a_dx.A = dpre;
  a_dx.lda = P;
  a_dx.B0 = wg;
  a_dx.B1 = gated ? wu : nullptr;
  a_dx.b_split = (int)H;
  a_dx.ldb = D;
  a_dx.C0 = dx;
  a_dx.ldc0 = D;
  a_dx.alpha_dev0 = sw1;
  // [dW_gate; dW_up] (+)= [dg | du]^T x  (non-gated: dW1 = dpre^T x)
  GemmArgs a_dwg = base_args(d);
  a_dwg.A = dpre;
  a_dwg.lda = P;
  a_dwg.B0 = x;
  a_dwg.ldb = D;
  a_dwg.C0 = dwg;
  a_dwg.C1 = gated ? dwu : nullptr;
  a_dwg.c_split = gated ? (int)H : (int)P;
  a_dwg.ldc0 = D;
  a_dwg.accumulate = grad_accum;
  a_dwg.alpha_dev0 = sx;

  const GemmArgs* args[4] = {&a_dwd, &a_dx, &a_dwg, &a_dact};   // by BwdGemm id
  // one launch of a planned group: member j's workgroups start at a multiple of 8
  auto run_group = [&](const BwdGroup& grp, int epi0, const char* what) {
    GemmGroup gg{};
    int at = 0;
    for (int j = 0; j < grp.count; ++j) {
      const int m = grp.member[j];
      const GemmDims dm = bwd_dims(d, m);
      gg.g[j] = planned(*args[m], grp.plan[j], dm.M, dm.N, dm.K);
      gg.kind[j] = (m == BG_DX || m == BG_DACT) ? 0 : 1;
      gg.items[j] = grp.plan[j].grid;
      gg.begin[j] = at;
      at += (grp.plan[j].grid + 7) / 8 * 8;
    }
    gg.begin[grp.count] = at;
    gg.count = grp.count;
    return hip_status(run_gemm_group16(io, gio, epi0, gg, s), what);
  };

  const BwdSchedule sch = plan_bwd_schedule(d, bwd_mask(dx, dwg, dwd));
  const int dact_epi = gated ? EPI_DGATED : EPI_DACT;
  if (need_dpre) {
    StageScope st(MLP_STAGE_DACT, s);
    if (sch.dact.count > 0)
      MLP_TRY(run_group(sch.dact, dact_epi, "d-activation GEMM and dW_down (one launch)"));
    else
      MLP_TRY(gemm_cols_split(io, io, NN, dact_epi, plan_gemm(io, M, H, O, false, false), a_dact, M, H, O,
                              esize(d->dtype), s, "d-activation GEMM"));
  } else if (dwd && !d->save_act) {
    // only the down-projection gradient: the post-activation from the pre-activation alone
    StageScope st(MLP_STAGE_ACT, s);
    if (gated) MLP_TRY(hip_status(run_gated_act(io, pre, act, (int)M, (int)H, d->gate_mult,
                                                d->gate_mode == MLP_GATE_INSIDE, act_fn_of(d->act), s),
                                  "activation"));
    else MLP_TRY(hip_status(run_plain_act(io, pre, act, M * H, 1.0f, nullptr, nullptr, act_fn_of(d->act), s),
                            "activation"));
  }

  if (sch.rest.count > 0) {
    StageScope st(MLP_STAGE_BWD_GEMMS, s);
    return run_group(sch.rest, EPI_STORE, "dx and weight gradients (one launch)");
  }
  if (dwd && sch.dact.count == 0) {
    StageScope st(MLP_STAGE_DW_DOWN, s);
    MLP_TRY(gemm(io, gio, TN, EPI_STORE, G.dw_down, a_dwd, O, H, M, partial, s, "dW_down"));
  }
  if (dx) {
    StageScope st(MLP_STAGE_DX, s);
    MLP_TRY(gemm_rows(io, io, NN, G.dx, a_dx, M, D, P, partial, s, "dx"));
  }
  if (dwg) {
    StageScope st(MLP_STAGE_DW_UP, s);
    MLP_TRY(gemm(io, gio, TN, EPI_STORE, G.dw_up, a_dwg, P, D, M, partial, s, "dW_gate/dW_up"));
  }
  return MLP_OK;
}

size_t mlp_quantize_workspace_bytes(void) { return kQuantizeWsBytes; }

mlp_status mlp_time_stage_once(int stage, void* begin, void* end) {
  if (stage < 0 || stage >= MLP_STAGE_COUNT) return fail(MLP_ERR_INVALID_ARG, "stage %d is not an mlp_stage", stage);
  if ((begin == nullptr) != (end == nullptr)) return fail(MLP_ERR_INVALID_ARG, "begin and end must both be set or both be NULL");
  g_hooks[stage].begin = reinterpret_cast<hipEvent_t>(begin);
  g_hooks[stage].end = reinterpret_cast<hipEvent_t>(end);
  return MLP_OK;
}

mlp_status mlp_quantize_e4m3(const void* src, int dtype, int64_t n, void* dst, float* scale, void* ws,
                             size_t ws_bytes, void* stream) {
  if (dtype != MLP_F32 && dtype != MLP_BF16 && dtype != MLP_F16)
    return fail(MLP_ERR_INVALID_ARG, "dtype %d is not an mlp_dtype", dtype);
  if (n < 1) return fail(MLP_ERR_INVALID_ARG, "n must be >= 1");
  if (!src || !dst || !scale || !ws) return fail(MLP_ERR_INVALID_ARG, "src, dst, scale and workspace are required");
  if (!aligned4(src) || !aligned4(scale) || !aligned16(ws))
    return fail(MLP_ERR_ALIGNMENT, "src and scale must be 4-byte aligned, workspace 16-byte aligned");
  if (ws_bytes < kQuantizeWsBytes)
    return fail(MLP_ERR_WORKSPACE, "workspace of %zu bytes is smaller than %zu", ws_bytes, kQuantizeWsBytes);
  return hip_status(run_quantize_e4m3(dtype_of(dtype), src, n, dst, scale,
                                      reinterpret_cast<float*>(ws), reinterpret_cast<hipStream_t>(stream)),
                    "quantize");
}

mlp_status mlp_quantize_fp8(const void* src, int dtype, int64_t rows, int64_t cols, int fmt, int relu_sq,
                            const float* scale, void* dst, void* dst_t, int64_t ld_t, void* stream) {
  if (dtype != MLP_BF16) return fail(MLP_ERR_UNSUPPORTED, "mlp_quantize_fp8 reads bf16 sources only");
  if (fmt != MLP_FP8_E4M3 && fmt != MLP_FP8_E5M2) return fail(MLP_ERR_INVALID_ARG, "fmt %d is not an mlp_fp8_format", fmt);
  if (relu_sq != 0 && relu_sq != 1) return fail(MLP_ERR_INVALID_ARG, "relu_sq must be 0 or 1");
  if (rows < 1 || cols < 1 || rows >= ((int64_t)1 << 31) || cols >= ((int64_t)1 << 31))
    return fail(MLP_ERR_INVALID_ARG, "rows and cols must be in [1, 2^31)");
  if (cols % 16) return fail(MLP_ERR_ALIGNMENT, "cols must be a multiple of 16");
  if (!dst && !dst_t) return fail(MLP_ERR_INVALID_ARG, "dst and dst_t are both NULL");
  if (dst_t && (ld_t < rows || ld_t % 16))
    return fail(MLP_ERR_INVALID_ARG, "ld_t must be >= rows and a multiple of 16");
  MLP_TRY(need_ptr(src, "src"));
  MLP_TRY(need_ptr(scale, "scale", false));
  if (dst) MLP_TRY(need_ptr(dst, "dst"));
  if (dst_t) MLP_TRY(need_ptr(dst_t, "dst_t"));
  return hip_status(run_quantize_fp8_2d(DT_BF16, src, rows, cols, cols, relu_sq, fmt == MLP_FP8_E5M2, scale, dst,
                                        dst_t, dst_t ? ld_t : 0, reinterpret_cast<hipStream_t>(stream)),
                    "quantize fp8");
}

int64_t mlp_weight_amax_slots(int64_t rows, int64_t cols) {
  // sizes mlp_quantize_weight_e4m3 refuses have no slots (and the count cannot overflow)
  const int64_t lim = (int64_t)1 << 31;
  if (rows < 1 || cols < 1 || rows >= lim || cols >= lim) return 0;
  return weight_amax_slots(rows, cols);
}

mlp_status mlp_quantize_weight_e4m3(const void* w, int dtype, int64_t rows, int64_t cols, int exact, float* scale,
                                    float* tile_amax, void* dst, void* dst_t, int64_t ld_t, void* stream) {
  if (dtype != MLP_BF16 && dtype != MLP_F32) return fail(MLP_ERR_UNSUPPORTED, "weights must be bf16 or f32");
  if (exact != 0 && exact != 1) return fail(MLP_ERR_INVALID_ARG, "exact must be 0 or 1");
  if (rows < 1 || cols < 1 || rows >= ((int64_t)1 << 31) || cols >= ((int64_t)1 << 31))
    return fail(MLP_ERR_INVALID_ARG, "rows and cols must be in [1, 2^31)");
  if (cols % 16) return fail(MLP_ERR_ALIGNMENT, "cols must be a multiple of 16");
  if (!dst && !dst_t) return fail(MLP_ERR_INVALID_ARG, "dst and dst_t are both NULL");
  if (dst_t && (ld_t < rows || ld_t % 16)) return fail(MLP_ERR_INVALID_ARG, "ld_t must be >= rows and a multiple of 16");
  MLP_TRY(need_ptr(w, "w"));
  MLP_TRY(need_ptr(scale, "scale", false));
  MLP_TRY(need_ptr(tile_amax, "tile_amax", false));
  if (dst) MLP_TRY(need_ptr(dst, "dst"));
  if (dst_t) MLP_TRY(need_ptr(dst_t, "dst_t"));
  return hip_status(run_quantize_weight_e4m3(dtype == MLP_BF16 ? DT_BF16 : DT_F32, w, rows, cols, exact, scale,
                                             tile_amax, dst, dst_t, dst_t ? ld_t : 0,
                                             reinterpret_cast<hipStream_t>(stream)),
                    "quantize weight");
}

float mlp_fp8_next_scale(float amax, float prev_scale, float gain, float floor_) {
  // only a finite amax above zero moves the scale, and it counts at most 1e12
  const float fresh = fminf(amax, 1e12f) * gain;
  return (isfinite(amax) && amax > 0.0f) ? (fresh < floor_ ? floor_ : fresh) : prev_scale;
}

}  // extern "C"

namespace gmlp {

hipError_t run_gemm(DType in, DType io, Layout layout, int epi, TileShape tile, const GemmArgs& a,
                    int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  switch (in) {
    case DT_BF16:
      if (layout == NT) return run_gemm_bf16_nt(io, epi, tile, a, grid, s);
      if (layout == NN) return run_gemm_bf16_nn(io, epi, tile, a, grid, s);
      return run_gemm_bf16_tn(io, epi, tile, a, grid, s);
    case DT_F16:
      if (layout == NT) return run_gemm_f16_nt(io, epi, tile, a, grid, s);
      if (layout == NN) return run_gemm_f16_nn(io, epi, tile, a, grid, s);
      return run_gemm_f16_tn(io, epi, tile, a, grid, s);
    case DT_F32: return run_gemm_f32(layout, epi, tile, a, grid, s);
    case DT_E4M3:
      if (layout == NT) return run_gemm_e4m3_nt(io, epi, tile, a, grid, s);
      return hipErrorInvalidValue;
    case DT_F8G:
      if (layout == NT) return run_gemm_f8g_nt(io, epi, tile, a, grid, s);
      if (layout == TN) return run_gemm_f8g_tn(io, epi, tile, a, grid, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace gmlp
