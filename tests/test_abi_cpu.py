"""CPU tests of the C-ABI library: it loads, exports every declared symbol, rejects bad
arguments on the host before any HIP call, sizes its workspace, and its host-side fp8 scale
rule matches the oracle's. No test here launches a kernel: every call below fails validation
(or is host-only), so nothing reaches the GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import gated_mlp_gemms_amd as gm
import oracle
from gated_mlp_gemms_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000      # 16-byte aligned, never dereferenced: each call fails validation first


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "mlp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlp_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = gm.lib()
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib._SIGNATURES), "binding and header disagree"
    assert L.mlp_abi_version() == 5


def _desc(**kw):
    base = dict(M=300, d_in=264, hidden=712, d_out=200, act="swiglu", dtype="bf16")
    base.update(kw)
    return gm.make_desc(**base)


def _fwd(d, x=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, out=FAKE, saved=FAKE, fp8=None, ws=FAKE, nws=None):
    if nws is None:
        nws = gm.lib().mlp_workspace_bytes(C.byref(d), gm.MLP_PHASE_FWD) if d.M > 0 else 0
    return gm.lib().mlp_fwd(C.byref(d), x, wg, wu, wd, out, saved, C.byref(fp8) if fp8 else None, ws, nws, None)


def _err():
    return gm.lib().mlp_last_error().decode()


def test_descriptor_checks():
    L = gm.lib()
    assert _fwd(_desc(M=0), nws=0) == gm._lib.MLP_ERR_INVALID_ARG
    assert _fwd(_desc(d_in=260)) == gm._lib.MLP_ERR_ALIGNMENT and "multiples of 8" in _err()
    assert _fwd(_desc(hidden=4, dtype="f32", d_in=4, d_out=6)) == gm._lib.MLP_ERR_ALIGNMENT
    d = _desc()
    d.act = 7
    assert _fwd(d) == gm._lib.MLP_ERR_INVALID_ARG
    d = _desc()
    d.fp8_bwd = 2
    assert _fwd(d) == gm._lib.MLP_ERR_INVALID_ARG
    d = _desc(act="relu_sq", fp8_bwd=True, d_in=256, hidden=704, d_out=208)   # fp8_bwd needs fp8_fwd
    assert _fwd(d, wu=None) == gm._lib.MLP_ERR_INVALID_ARG and "fp8_fwd" in _err()
    d = _desc(gate_mult=float("nan"))
    assert _fwd(d) == gm._lib.MLP_ERR_INVALID_ARG
    d = _desc(fp8_fwd=True)            # fp8 forward is ReLU^2 only
    assert _fwd(d) == gm._lib.MLP_ERR_UNSUPPORTED
    d = _desc(act="relu_sq", fp8_fwd=True, d_in=264)
    assert _fwd(d, wu=None) == gm._lib.MLP_ERR_ALIGNMENT   # e4m3 rows need multiples of 16
    assert L.mlp_workspace_bytes(None, 0) == 0
    assert L.mlp_workspace_bytes(C.byref(_desc()), 9) == 0


def test_pointer_checks():
    d = _desc()
    assert _fwd(d, x=None) == gm._lib.MLP_ERR_INVALID_ARG and "x is NULL" in _err()
    assert _fwd(d, wu=None) == gm._lib.MLP_ERR_INVALID_ARG
    assert _fwd(d, x=FAKE + 8) == gm._lib.MLP_ERR_ALIGNMENT
    assert _fwd(d, saved=None) == gm._lib.MLP_ERR_INVALID_ARG          # training needs saved_preact
    dr = _desc(recompute=True)
    assert _fwd(dr, saved=FAKE) == gm._lib.MLP_ERR_INVALID_ARG         # ...and recompute forbids it
    dq = _desc(act="relu_sq")
    assert _fwd(dq) == gm._lib.MLP_ERR_INVALID_ARG and "w_up" in _err()  # ReLU^2 takes no W_up
    fp8 = gm.make_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert _fwd(d, fp8=fp8) == gm._lib.MLP_ERR_INVALID_ARG             # fp8 struct without fp8_fwd
    df = _desc(act="relu_sq", fp8_fwd=True, d_in=256, hidden=704, d_out=208)
    assert _fwd(df, wu=None) == gm._lib.MLP_ERR_INVALID_ARG            # fp8_fwd without the struct
    fp8.s_post = None
    assert _fwd(df, wu=None, fp8=fp8) == gm._lib.MLP_ERR_INVALID_ARG and "s_post" in _err()


def test_workspace_checks():
    d = _desc()
    need = gm.lib().mlp_workspace_bytes(C.byref(d), gm.MLP_PHASE_FWD)
    assert need >= 300 * 712 * 2
    assert _fwd(d, nws=need - 1) == gm._lib.MLP_ERR_WORKSPACE
    assert _fwd(d, ws=None) == gm._lib.MLP_ERR_INVALID_ARG
    assert _fwd(d, ws=FAKE + 4) == gm._lib.MLP_ERR_ALIGNMENT


def test_backward_checks():
    L = gm.lib()
    d = _desc()
    nws = L.mlp_workspace_bytes(C.byref(d), gm.MLP_PHASE_BWD)

    def bwd(dd=d, saved=FAKE, dpre=None, dx=FAKE, dwg=FAKE, dwu=FAKE, dwd=FAKE, acc=0, ws=nws):
        return L.mlp_bwd(C.byref(dd), FAKE, FAKE, FAKE, FAKE, FAKE, saved, dpre, dx, dwg, dwu, dwd, acc,
                         None, FAKE, ws, None)

    assert bwd(dwu=None) == gm._lib.MLP_ERR_INVALID_ARG and "both" in _err()
    assert bwd(acc=2) == gm._lib.MLP_ERR_INVALID_ARG
    assert bwd(saved=None) == gm._lib.MLP_ERR_INVALID_ARG
    assert bwd(dpre=FAKE + 2) == gm._lib.MLP_ERR_ALIGNMENT
    assert bwd(ws=nws - 256) == gm._lib.MLP_ERR_WORKSPACE
    dr = _desc(recompute=True)
    assert bwd(dd=dr, saved=FAKE, ws=L.mlp_workspace_bytes(C.byref(dr), gm.MLP_PHASE_BWD)) == gm._lib.MLP_ERR_INVALID_ARG


def test_workspace_sizes():
    """The forward keeps a [M, H] activation in the workspace; the recompute backward holds the
    recomputed [M, 2H] pre-activation instead of a dpreact buffer, so the caller saves the
    M * 2 * H * dtype_size bytes of saved_preact (quack mlp.py, MLPRecomputeFunc docstring)."""
    L = gm.lib()
    for dt, es in (("bf16", 2), ("f32", 4)):
        d = _desc(dtype=dt, d_in=256, hidden=704, d_out=208)
        fwd = L.mlp_workspace_bytes(C.byref(d), gm.MLP_PHASE_FWD)
        assert fwd >= 300 * 704 * es
        assert L.mlp_workspace_bytes(C.byref(d), gm.MLP_PHASE_FWD_INFER) == fwd
        b0 = L.mlp_workspace_bytes(C.byref(d), gm.MLP_PHASE_BWD)
        dr = _desc(dtype=dt, d_in=256, hidden=704, d_out=208, recompute=True)
        b1 = L.mlp_workspace_bytes(C.byref(dr), gm.MLP_PHASE_BWD)
        assert b1 == b0 >= 300 * 704 * es + 300 * 2 * 704 * es


def test_small_m_workspace_holds_the_down_projection_parts():
    """Up to 16 tokens every forward product runs on the small-M kernel, which needs no split-K
    partials, except that above 8 tokens a narrow down projection with a long K (LLaMA: 4096
    outputs, K = 11008) is split over 4 parts of K into fp32 partials [4][M][d_out]."""
    L = gm.lib()
    llama = dict(d_in=4096, hidden=11008, d_out=4096)
    for phase in (gm.MLP_PHASE_FWD, gm.MLP_PHASE_FWD_INFER):
        for M in (1, 8, 9, 16):
            ws = L.mlp_workspace_bytes(C.byref(_desc(M=M, **llama)), phase)
            act = M * 11008 * 2   # the [M, H] bf16 activation
            parts = 4 * M * 4096 * 4 if M > 8 else 0
            assert act + parts <= ws < act + parts + 4096, (phase, M, ws)
    # a short K keeps the whole-K form
    ws = L.mlp_workspace_bytes(C.byref(_desc(M=16, d_in=256, hidden=1000, d_out=256)), gm.MLP_PHASE_FWD_INFER)
    assert ws < 16 * 1000 * 2 + 4096


def test_quantize_checks():
    L = gm.lib()
    assert L.mlp_quantize_e4m3(FAKE, 1, 0, FAKE, FAKE, FAKE, 256, None) == gm._lib.MLP_ERR_INVALID_ARG
    assert L.mlp_quantize_e4m3(FAKE, 5, 10, FAKE, FAKE, FAKE, 256, None) == gm._lib.MLP_ERR_INVALID_ARG
    assert L.mlp_quantize_e4m3(FAKE, 1, 10, FAKE, FAKE, FAKE, 8, None) == gm._lib.MLP_ERR_WORKSPACE
    # the workspace holds the amax and the per-workgroup maxima (2048 floats after 256 bytes)
    need = gm.mlp_quantize_workspace_bytes()
    assert need == 256 + 2048 * 4
    assert L.mlp_quantize_e4m3(FAKE, 1, 10, FAKE, FAKE, FAKE, need - 1, None) == gm._lib.MLP_ERR_WORKSPACE
    assert L.mlp_quantize_e4m3(None, 1, 10, FAKE, FAKE, FAKE, 256, None) == gm._lib.MLP_ERR_INVALID_ARG


def test_next_scale_matches_oracle():
    rng = np.random.default_rng(0)
    amaxes = list(np.abs(rng.standard_normal(200)).astype(np.float32) * 10.0 ** rng.integers(-8, 14, 200))
    amaxes += [0.0, float("nan"), float("inf"), float("-inf"), 1e-30, 5e11, 2e12, 448.0]
    for gain, floor in ((1.03 / 448.0, 1e-6), (1.25 / 57344.0, 1e-12)):
        for a in amaxes:
            ours = np.float32(gm.mlp_fp8_next_scale(float(a), 0.5, gain, floor))
            ref = oracle.next_delayed_scale(a, 0.5, gain, floor)
            assert ours == ref, (a, gain, ours, ref)


def test_product_and_oracle_share_no_code():
    """The HIP path never imports the oracle and the oracle never imports the HIP path."""
    pat_oracle = re.compile(r"^\s*(from|import)\s+oracle\b", re.M)
    pat_prod = re.compile(r"^\s*(from|import)\s+gated_mlp_gemms_amd\b", re.M)
    pkg = os.path.join(ROOT, "gated_mlp_gemms_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not pat_oracle.search(text), f
                assert "oracle" not in text or f.endswith(".py") and "oracle" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            assert not pat_prod.search(open(os.path.join(ROOT, "oracle", f)).read()), f


@pytest.mark.parametrize("act,gated", [("swiglu", True), ("geglu", True), ("reglu", True), ("glu", True),
                                       ("relu_sq", False), ("relu", False), ("gelu_tanh", False)])
def test_activation_family_checks(act, gated):
    """Every mlp_act passes the descriptor check; a gated one needs w_up, a non-gated one refuses
    it; the e4m3 forward is ReLU^2 only."""
    d = _desc(act=act)
    wu = FAKE if gated else None
    assert _fwd(d, wu=wu, ws=None) == gm._lib.MLP_ERR_INVALID_ARG and "workspace" in _err()
    assert _fwd(d, wu=None if gated else FAKE) == gm._lib.MLP_ERR_INVALID_ARG and "w_up" in _err()
    if act != "relu_sq":
        df = _desc(act=act, fp8_fwd=True, d_in=256, hidden=704, d_out=208)
        assert _fwd(df, wu=wu) == gm._lib.MLP_ERR_UNSUPPORTED


def test_activation_enum_bounds():
    for bad in (-1, 7, 100):
        d = _desc()
        d.act = bad
        assert _fwd(d) == gm._lib.MLP_ERR_INVALID_ARG and "mlp_act" in _err()


def test_fp16_descriptor_checks():
    """fp16 I/O passes the descriptor check with 8-element row alignment; the e4m3 forward stays
    bf16-only."""
    d = _desc(dtype="f16")
    assert _fwd(d, ws=None) == gm._lib.MLP_ERR_INVALID_ARG and "workspace" in _err()
    assert _fwd(_desc(dtype="f16", d_in=260)) == gm._lib.MLP_ERR_ALIGNMENT
    assert _fwd(_desc(act="relu_sq", dtype="f16", fp8_fwd=True, d_in=256, hidden=704, d_out=208),
                wu=None) == gm._lib.MLP_ERR_UNSUPPORTED
    d = _desc()
    d.dtype = 3
    assert _fwd(d) == gm._lib.MLP_ERR_INVALID_ARG and "mlp_dtype" in _err()
    # workspace sizes of fp16 equal bf16's (both 2-byte I/O)
    for ph in (gm.MLP_PHASE_FWD, gm.MLP_PHASE_FWD_INFER, gm.MLP_PHASE_BWD):
        assert gm.lib().mlp_workspace_bytes(C.byref(_desc(dtype="f16")), ph) == \
            gm.lib().mlp_workspace_bytes(C.byref(_desc(dtype="bf16")), ph)


def test_size_limits():
    """Sizes that would overflow the kernels' 32-bit tile indexing are refused before any HIP
    call: M, d_in, d_out >= 2^30, hidden >= 2^29."""
    for kw in (dict(M=1 << 30), dict(d_in=1 << 30), dict(d_out=1 << 30), dict(hidden=1 << 29)):
        assert _fwd(_desc(**kw), nws=0) == gm._lib.MLP_ERR_UNSUPPORTED, kw
        assert "2^30" in _err()


def test_leading_dimension_limits():
    """The GEMMs address an operand as a scalar base plus a 32-bit per-lane offset of up to 64
    row pitches, so every leading dimension stays under 2^25 elements: d_in, d_out, the stacked
    gate/up width 2 * hidden (hidden for a non-gated activation). Refused before any HIP call;
    one below each limit passes. The token count is no leading dimension (the fp8 backward's
    weight gradients read its row-major codes along the tokens), so M = 2^25 passes."""
    big = 1 << 25
    for kw in (dict(d_in=big), dict(d_out=big), dict(hidden=big // 2), dict(act="relu_sq", hidden=big)):
        assert _fwd(_desc(**kw), nws=0) == gm._lib.MLP_ERR_UNSUPPORTED, kw
        assert "2^25" in _err()
    fp8 = dict(act="relu_sq", fp8_fwd=True, fp8_bwd=True, d_in=256, hidden=704, d_out=256)
    assert _fwd(_desc(M=big, **fp8), ws=None) == gm._lib.MLP_ERR_INVALID_ARG
    # just below each limit the size checks pass and the next check (a NULL workspace) fails
    for kw in (dict(d_in=big - 8), dict(d_out=big - 8), dict(hidden=big // 2 - 8), dict(act="relu_sq", hidden=big - 8),
               dict(M=(1 << 30) - 1, d_in=16, hidden=16, d_out=16)):
        assert _fwd(_desc(**kw), ws=None) == gm._lib.MLP_ERR_INVALID_ARG, kw


def test_matrix_size_limit():
    """No matrix of the problem (x, the pre-activation, out, the weights) may exceed 2^37
    elements (more than one GPU holds), which keeps every tile and workgroup count within an int;
    exactly 2^37 passes the size checks."""
    for kw in (dict(M=1 << 20, d_in=(1 << 17) + 8), dict(M=1 << 20, hidden=(1 << 16) + 8),
               dict(M=1 << 20, d_out=(1 << 17) + 8), dict(d_in=1 << 24, hidden=(1 << 13) + 8)):
        assert _fwd(_desc(**kw), nws=0) == gm._lib.MLP_ERR_UNSUPPORTED, kw
        assert "2^37" in _err()
    assert _fwd(_desc(M=1 << 20, d_in=1 << 17, hidden=1 << 10, d_out=1 << 10), ws=None) == gm._lib.MLP_ERR_INVALID_ARG


def test_fp8_backward_checks():
    """The fp8-gradient backward needs the transposed weight caches and the gradient / dpre
    scales, keeps dpre in the workspace (dpreact must be NULL), and the plain fp8 backward must
    not be handed the transposed caches."""
    L = gm.lib()
    d = _desc(act="relu_sq", fp8_fwd=True, fp8_bwd=True, M=300, d_in=256, hidden=704, d_out=208)
    nws = L.mlp_workspace_bytes(C.byref(d), gm.MLP_PHASE_BWD)
    assert nws >= 2 * 300 * 704 + 300 * 208   # dpre and relu(pre)^2 codes, dout codes (row-major)
    full = dict(w1t_q=FAKE, w2t_q=FAKE, s_grad=FAKE, s_dpre=FAKE, dpre_amax=FAKE)

    def bwd(dd=d, dpre=None, ws=nws, **over):
        kw = dict(full)
        kw.update(over)
        f = gm.make_fp8(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, **kw)
        return L.mlp_bwd(C.byref(dd), FAKE, None, None, None, None, FAKE, dpre, FAKE, FAKE, None, FAKE, 0,
                         C.byref(f), FAKE, ws, None)

    for name in full:
        assert bwd(**{name: None}) == gm._lib.MLP_ERR_INVALID_ARG and name in _err()
    assert bwd(dpre=FAKE) == gm._lib.MLP_ERR_INVALID_ARG and "dpreact" in _err()
    assert bwd(ws=nws - 16) == gm._lib.MLP_ERR_WORKSPACE
    d8 = _desc(act="relu_sq", fp8_fwd=True, M=300, d_in=256, hidden=704, d_out=208)
    assert bwd(dd=d8, ws=L.mlp_workspace_bytes(C.byref(d8), gm.MLP_PHASE_BWD)) == gm._lib.MLP_ERR_INVALID_ARG
    assert "w1t_q" in _err()


def test_quantize_fp8_checks():
    L = gm.lib()

    def q(dtype=gm.MLP_BF16, rows=100, cols=64, fmt=gm.MLP_FP8_E5M2, relu=0, scale=FAKE, dst=FAKE, dst_t=FAKE, ld_t=112):
        return L.mlp_quantize_fp8(FAKE, dtype, rows, cols, fmt, relu, scale, dst, dst_t, ld_t, None)

    assert q(dtype=gm.MLP_F32) == gm._lib.MLP_ERR_UNSUPPORTED
    assert q(fmt=2) == gm._lib.MLP_ERR_INVALID_ARG
    assert q(relu=3) == gm._lib.MLP_ERR_INVALID_ARG
    assert q(cols=40) == gm._lib.MLP_ERR_ALIGNMENT
    assert q(rows=0) == gm._lib.MLP_ERR_INVALID_ARG
    assert q(dst=None, dst_t=None) == gm._lib.MLP_ERR_INVALID_ARG
    assert q(ld_t=96) == gm._lib.MLP_ERR_INVALID_ARG          # below rows
    assert q(ld_t=104) == gm._lib.MLP_ERR_INVALID_ARG         # not a multiple of 16
    assert q(scale=None) == gm._lib.MLP_ERR_INVALID_ARG
    assert q(dst_t=FAKE + 8) == gm._lib.MLP_ERR_ALIGNMENT


def test_noalloc_entry_checks_run_before_any_hip_call():
    """mlp_fwd_infer_noalloc: the argument checks and the static-scratch size check come before
    any HIP call (so they run here, without a GPU); the size limit is the header's."""
    text = open(os.path.join(ROOT, "include", "mlp.h")).read()
    m = re.search(r"#define MLP_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gm.MLP_NOALLOC_SCRATCH_BYTES
    L = gm.lib()

    def call(d, x=FAKE, wu=FAKE, fp8=None):
        return L.mlp_fwd_infer_noalloc(C.byref(d), x, FAKE, wu, FAKE, FAKE, C.byref(fp8) if fp8 else None, None)

    assert call(_desc(M=0)) == gm._lib.MLP_ERR_INVALID_ARG
    assert call(_desc(), x=None) == gm._lib.MLP_ERR_INVALID_ARG and "x is NULL" in _err()
    assert call(_desc(act="relu_sq")) == gm._lib.MLP_ERR_INVALID_ARG and "w_up" in _err()
    big = _desc(M=3000, d_in=4096, hidden=11008, d_out=4096)
    need = L.mlp_workspace_bytes(C.byref(big), gm.MLP_PHASE_FWD_INFER)
    assert need > gm.MLP_NOALLOC_SCRATCH_BYTES
    assert call(big) == gm._lib.MLP_ERR_WORKSPACE
    assert "MLP_NOALLOC_SCRATCH_BYTES" in _err() and str(need) in _err()
    fits = _desc(M=512, d_in=4096, hidden=11008, d_out=4096)
    assert L.mlp_workspace_bytes(C.byref(fits), gm.MLP_PHASE_FWD_INFER) <= gm.MLP_NOALLOC_SCRATCH_BYTES


def test_weight_quantizer_checks():
    """mlp_quantize_weight_e4m3 rejects bad arguments on the host; the slot count is per 128 x 128 tile."""
    L = gm.lib()
    assert L.mlp_weight_amax_slots(3072, 768) == 24 * 6
    assert L.mlp_weight_amax_slots(300, 208) == 3 * 2
    assert L.mlp_weight_amax_slots(0, 16) == 0

    def q(dtype=gm.MLP_BF16, rows=64, cols=64, exact=1, scale=FAKE, tiles=FAKE, dst=FAKE, dst_t=None, ld_t=0):
        return L.mlp_quantize_weight_e4m3(FAKE, dtype, rows, cols, exact, scale, tiles, dst, dst_t, ld_t, None)

    assert q(dtype=gm.MLP_F16) == gm._lib.MLP_ERR_UNSUPPORTED
    assert q(exact=2) == gm._lib.MLP_ERR_INVALID_ARG
    assert q(cols=40) == gm._lib.MLP_ERR_ALIGNMENT
    assert q(dst=None) == gm._lib.MLP_ERR_INVALID_ARG
    assert q(dst_t=FAKE, ld_t=60) == gm._lib.MLP_ERR_INVALID_ARG
    assert q(tiles=None) == gm._lib.MLP_ERR_INVALID_ARG and "tile_amax" in _err()
    assert q(scale=None) == gm._lib.MLP_ERR_INVALID_ARG


def test_backward_schedule_query():
    """mlp_bwd_grouped is host-only planning: one launch for the LLaMA and Falcon-H1 backward
    products (many short weight-gradient tiles around long dx tiles), separate launches where the
    weight gradients have few tiles with a very long K (the GPT ReLU^2 shape, whose split-K
    launches beat any single-pass tile order) or the problem is small, and never for fp32 or the
    fp8-gradient backward; a NULL out pointer or a bad descriptor is an argument error."""
    L = gm.lib()
    G, W = gm.MLP_BWD_GROUPED, gm.MLP_BWD_DW_DOWN_WITH_DACT
    assert gm.mlp_bwd_grouped(_desc(M=2048, d_in=4096, hidden=11008, d_out=4096)) == G
    assert gm.mlp_bwd_grouped(_desc(M=8192, d_in=2048, hidden=4864, d_out=2048, recompute=True)) == G
    assert gm.mlp_bwd_grouped(_desc(M=2048, d_in=4096, hidden=11008, d_out=4096, dtype="f16")) == G
    # the kept activation frees dW_down from the d-activation GEMM, and the two share a launch
    # where the d-activation GEMM's own tiles leave a last round to fill (3072 tokens: 516 tiles
    # of 256 x 256); at 2048 tokens it runs alone on 256 x 128 tiles
    assert gm.mlp_bwd_grouped(_desc(M=3072, d_in=4096, hidden=11008, d_out=4096, save_act=True)) == G | W
    assert gm.mlp_bwd_grouped(_desc(M=2048, d_in=4096, hidden=11008, d_out=4096, save_act=True)) == G
    assert not gm.mlp_bwd_grouped(_desc(M=49152, d_in=768, hidden=3072, d_out=768, act="relu_sq"))
    assert not gm.mlp_bwd_grouped(_desc(M=16, d_in=4096, hidden=11008, d_out=4096))
    assert not gm.mlp_bwd_grouped(_desc(M=2048, d_in=4096, hidden=11008, d_out=4096, dtype="f32"))
    assert not gm.mlp_bwd_grouped(_desc(M=49152, d_in=768, hidden=3072, d_out=768, act="relu_sq",
                                        fp8_fwd=True, fp8_bwd=True))
    d = _desc()
    assert L.mlp_bwd_grouped(C.byref(d), None) == _lib.MLP_ERR_INVALID_ARG
    bad = _desc(M=0)
    out = C.c_int(7)
    assert L.mlp_bwd_grouped(C.byref(bad), C.byref(out)) == _lib.MLP_ERR_INVALID_ARG


def test_save_act_checks():
    """save_act is 0 or 1 and keeps the activation next to a saved pre-activation: it cannot be
    combined with recompute (nothing is saved) or the e4m3 forward (its activation is e4m3)."""
    L = gm.lib()
    ok = _desc(save_act=True)
    assert L.mlp_workspace_bytes(C.byref(ok), _lib.MLP_PHASE_BWD) > 0
    for bad in (_desc(save_act=True, recompute=True),
                _desc(act="relu_sq", save_act=True, fp8_fwd=True, d_in=256, hidden=704, d_out=256)):
        assert L.mlp_workspace_bytes(C.byref(bad), _lib.MLP_PHASE_BWD) == 0
        assert b"save_act" in L.mlp_last_error()
    d = _desc()
    d.save_act = 2
    assert L.mlp_workspace_bytes(C.byref(d), _lib.MLP_PHASE_FWD) == 0
    assert b"save_act" in L.mlp_last_error()
