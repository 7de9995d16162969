"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Small problems are compared in full; their sizes span several tiles and end in ragged tails
(M, d_in, hidden, d_out not multiples of the 256/128 tiles). The invariants at the end hold
bit for bit on the GPU: inference forward == training forward, recompute == saved
pre-activation, in-place dpreact == separate buffer, run-to-run determinism, power-of-two
down_mult scaling, and the "only dW_down" skip branch.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, announce, assert_close, check_full, f64, run
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def _w(act, dtype, M, d, H, do, **kw):
    name = f"{act}_{dtype}_m{M}_d{d}_h{H}_o{do}"
    return Workload(name, act, dtype, (M,), d, H, do, **kw)


SMALL_GATED = [
    _w("swiglu", "bf16", 300, 264, 712, 200),
    _w("swiglu", "bf16", 300, 264, 712, 200, gate_mult=1.125, down_mult=2.0),
    _w("swiglu", "bf16", 517, 512, 1400, 520, gate_mult=0.75, down_mult=1.5, seed=3),
    _w("swiglu", "f32", 77, 132, 200, 68, gate_mult=1.125, down_mult=2.0),
]


@pytest.mark.parametrize("w", SMALL_GATED, ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["outside", "inside"])
def test_gated_small(w, mode):
    announce(f"gated {w.name} {mode}")
    t = make_inputs(w)
    r = run(w, t, gate_mode=mode)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r, mode)


def test_swiglu_f32_reference_config():
    w = WORKLOADS["swiglu_f32_m64_d128_h384"]
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.forward_infer()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r)
    assert torch.equal(r.out, r.out_infer)


SAVE_ACT = [
    _w("swiglu", "bf16", 300, 264, 712, 200, gate_mult=1.125, down_mult=2.0, save_act=True),
    _w("relu_sq", "bf16", 300, 264, 712, 200, save_act=True),
    _w("geglu", "f16", 129, 136, 400, 72, down_mult=1.5, save_act=True),
    _w("swiglu", "f32", 77, 132, 200, 68, save_act=True),
]


@pytest.mark.parametrize("w", SAVE_ACT, ids=lambda w: w.name)
def test_save_act_small(w):
    """The forward keeps the activation (a, or post) after the pre-activation: it and every
    output and gradient compared in full with the oracle. The "only dW_down" backward then reads
    the kept activation (no activation pass) and gives the full backward's dW_down bit for bit."""
    announce(f"save_act {w.name}")
    t = make_inputs(w)
    r = run(w, t)
    assert r.saved_act is not None
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r)
    full = r.dw_down.clone()
    r.dw_down.zero_()
    r.backward(dx=False, dw_gate=False)
    torch.cuda.synchronize()
    assert torch.equal(r.dw_down, full)


@pytest.mark.parametrize("mode", ["outside", "inside"])
def test_gated_recompute_accumulate_small(mode):
    w = _w("swiglu", "bf16", 390, 256, 704, 264, gate_mult=1.125, down_mult=2.0, recompute=True, grad_accum=True)
    announce(f"{w.name} recompute+accum {mode}")
    t = make_inputs(w)
    r = run(w, t, gate_mode=mode)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r, mode)


@pytest.mark.parametrize("w", [
    _w("relu_sq", "bf16", 333, 200, 520, 264),
    _w("relu_sq", "bf16", 600, 768, 3072, 768, down_mult=2.0, seed=5),
    _w("relu_sq", "f32", 70, 44, 96, 36),
    _w("relu_sq", "bf16", 257, 136, 392, 128, recompute=True, grad_accum=True),
], ids=lambda w: w.name)
def test_relu_sq_small(w):
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r)


# the other activations of quack's Activation set, through the same kernels
OTHER_GATED = [
    _w("geglu", "bf16", 300, 264, 712, 200, gate_mult=1.125, down_mult=2.0),
    _w("reglu", "bf16", 300, 264, 712, 200, gate_mult=1.125, down_mult=2.0, seed=1),
    _w("glu", "bf16", 300, 264, 712, 200, gate_mult=1.125, down_mult=2.0, seed=2),
    _w("geglu", "f32", 77, 132, 200, 68, gate_mult=0.75),
    _w("glu", "bf16", 517, 512, 1400, 520, seed=4, recompute=True, grad_accum=True),
]


@pytest.mark.parametrize("w", OTHER_GATED, ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["outside", "inside"])
def test_other_gated_small(w, mode):
    announce(f"gated {w.name} {mode}")
    t = make_inputs(w)
    r = run(w, t, gate_mode=mode)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r, mode)


@pytest.mark.parametrize("w", [
    _w("relu", "bf16", 333, 200, 520, 264),
    _w("gelu_tanh", "bf16", 333, 200, 520, 264, down_mult=2.0, seed=1),
    _w("gelu_tanh", "f32", 70, 44, 96, 36),
    _w("relu", "bf16", 257, 136, 392, 128, recompute=True, grad_accum=True, seed=2),
    _w("gelu_tanh", "bf16", 600, 768, 3072, 768, seed=5),
], ids=lambda w: w.name)
def test_other_plain_small(w):
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r)


@pytest.mark.parametrize("act", ["geglu", "reglu", "glu", "gelu_tanh", "relu"])
def test_other_acts_infer_recompute_and_dw_down_only(act):
    """Per activation: inference == training forward, recompute == saved pre-activation, and the
    "only dW_down" branch (act-only kernel) == the full backward's dW_down, bit for bit."""
    w = _w(act, "bf16", 300, 264, 712, 200, gate_mult=1.125 if act in ("geglu", "reglu", "glu") else 1.0)
    announce(f"{act}: infer / recompute / only-dW_down")
    t = make_inputs(w)
    r = run(w, t, gate_mode="inside")
    r.forward()
    r.forward_infer()
    r.backward()
    torch.cuda.synchronize()
    assert torch.equal(r.out, r.out_infer)
    grads = {k: v.clone() for k, v in r.grads().items()}
    full_dwd = r.dw_down.clone()
    rr = run(w.replace(recompute=True), t, gate_mode="inside")
    rr.forward()
    rr.backward()
    torch.cuda.synchronize()
    for k, v in grads.items():
        assert torch.equal(rr.grads()[k], v), k
    r.dw_down.zero_()
    r.backward(dx=False, dw_gate=False)
    torch.cuda.synchronize()
    assert torch.equal(full_dwd, r.dw_down)


def test_m_equals_one():
    w = _w("swiglu", "bf16", 1, 64, 128, 64)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r)


@pytest.mark.parametrize("act,dtype", [("swiglu", "bf16"), ("relu_sq", "bf16"), ("geglu", "f32"), ("glu", "f16")])
def test_smallest_problem(act, dtype):
    """The smallest legal problem: one token, every width one 16-byte row (8 elements; 4 fp32)."""
    n = 4 if dtype == "f32" else 8
    w = _w(act, dtype, 1, n, n, n, gate_mult=1.125, down_mult=2.0)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t, gate_mode="inside")
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r, "inside")


@pytest.mark.parametrize("w", [
    _w("swiglu", "bf16", 16, 512, 1400, 520, gate_mult=1.125, down_mult=2.0),
    _w("geglu", "bf16", 100, 1024, 2048, 512, seed=6),
    _w("swiglu", "f16", 37, 768, 1024, 264, seed=7),
], ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["outside", "inside"])
def test_decode_size_split_up_projection(w, mode):
    """At decode sizes the forward takes its small-M paths: up to 16 tokens the small-M kernel for
    every product, up to 128 the gated up projection split along K over the stacked
    [W_gate; W_up] with the activation applied in the reduce. The training forward (saved g|u),
    the inference forward and the backward against the oracle."""
    announce(f"decode split {w.name} {mode}")
    t = make_inputs(w)
    r = run(w, t, gate_mode=mode)
    r.forward()
    r.forward_infer()
    r.backward()
    torch.cuda.synchronize()
    assert torch.equal(r.out, r.out_infer)
    check_full(w, t, r, mode)


SKINNY = [
    # K = 4104 is 32 blocks of 128 and one chunk of 8; 712 hidden units and 520 / 136 outputs end
    # in a partial group of 16
    _w("swiglu", "bf16", 16, 4104, 712, 520, gate_mult=1.125, down_mult=2.0, seed=21),
    _w("relu_sq", "bf16", 5, 776, 3080, 264, down_mult=1.5, seed=22),
    _w("geglu", "f16", 13, 520, 712, 136, seed=23),
    _w("swiglu", "bf16", 1, 264, 1400, 8, seed=24),
    # 9 to 16 tokens with K <= 4096: the gated product stages x in LDS, shared by 3 column blocks
    # x 4 parts of K; K = 1000 ends in a partial block, 1000 units in a partial workgroup of 48
    _w("swiglu", "bf16", 11, 1000, 1000, 72, gate_mult=1.125, down_mult=2.0, seed=25),
    # 10 tokens, K = 2056 for the gated product (LDS-staged, 5000 units), K = 5000 for the down
    # projection (above 8 tokens split in 4 parts of K over workgroups, then the split-K reduce:
    # partial last blocks, 2056 outputs)
    _w("swiglu", "bf16", 10, 2056, 5000, 2056, down_mult=1.5, seed=26),
    # 12 tokens of ReLU^2: the down projection's 4 parts of K = 3080 (25 blocks, the last partial)
    # over 264 outputs (a partial group of 64)
    _w("relu_sq", "bf16", 12, 776, 3080, 264, down_mult=1.5, seed=27),
    # 9 tokens in fp16: the K-part down projection (K = 2056: 17 blocks, 4 uneven parts) and its
    # reduce in fp16
    _w("swiglu", "f16", 9, 264, 2056, 136, gate_mult=0.75, seed=28),
]


@pytest.mark.parametrize("w", SKINNY, ids=lambda w: w.name)
def test_small_m_kernel(w):
    """Up to 16 tokens every product of the forward runs on the small-M kernel (weights streamed
    once, K split over the waves): compared in full with the oracle, with the training forward
    (saved pre-activation), the inference forward and a recompute backward agreeing bit for bit."""
    announce(f"small-M {w.name}")
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.forward_infer()
    r.backward()
    torch.cuda.synchronize()
    assert torch.equal(r.out, r.out_infer)
    check_full(w, t, r)
    rc = run(w.replace(recompute=True), t)
    rc.backward()
    torch.cuda.synchronize()
    for k, v in r.grads().items():
        assert torch.equal(v, rc.grads()[k]), f"recompute {k}"


def test_small_m_llama_decode():
    """The decode step the bench times: 16 tokens through the LLaMA MLP (4096 x 11008), inference
    forward on the small-M kernel, sampled rows and every output column against the oracle."""
    w = _w("swiglu", "bf16", 16, 4096, 11008, 4096, seed=25)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward_infer()
    torch.cuda.synchronize()
    a = {k: f64(v) for k, v in t.items()}
    f = oracle.gated_forward(a["x"], a["w_gate"], a["w_up"], a["w_down"])
    assert_close("out (decode)", f64(r.out_infer), f["out"], TOL["bf16"])


def test_tall_thin_problem():
    """Many tokens through a hidden layer of one 8-wide row: 1 tile column, ragged rows."""
    w = _w("swiglu", "bf16", 1999, 8, 8, 16)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r)


def test_backward_with_nothing_requested_is_a_no_op():
    """mlp_bwd with dpreact, dx and every weight gradient NULL computes and writes nothing."""
    w = _w("swiglu", "bf16", 300, 264, 712, 200)
    announce("backward with no outputs")
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    for v in r.grads().values():
        v.fill_(7.0)
    torch.cuda.synchronize()
    r.backward(dx=False, dw_gate=False, dw_down=False, dpreact=False)
    torch.cuda.synchronize()
    for k, v in r.grads().items():
        assert bool((v == 7.0).all()), k


@pytest.mark.parametrize("act", ["swiglu", "relu_sq"])
def test_zero_inputs_give_exact_zeros(act):
    """x = 0 gives out = 0 and zero weight gradients of W_gate / W_up (W1) exactly; dout = 0
    gives dx = 0 and all weight gradients 0 exactly (no rounding can make a nonzero)."""
    w = _w(act, "bf16", 300, 264, 712, 200)
    announce(f"zero inputs {act}")
    t = make_inputs(w)
    t["x"] = torch.zeros_like(t["x"])
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    assert not bool(r.out.any())
    assert not bool(r.dw_gate.any())
    t = make_inputs(w)
    t["dout"] = torch.zeros_like(t["dout"])
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    for k, v in r.grads().items():
        assert not bool(v.any()), k


# ---- e4m3 ---------------------------------------------------------------------------------

def test_quantize_e4m3_bit_exact():
    import gated_mlp_gemms_amd as gm
    rng = np.random.default_rng(0)
    for dt, n in ((torch.bfloat16, 4099), (torch.float32, 70001), (torch.bfloat16, 1)):
        announce(f"quantize {dt} n={n}")
        v = torch.from_numpy(rng.standard_normal(n).astype(np.float32) * 3.0).to(dt)
        v[0] = -2.5   # a value with a distinct magnitude
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        scale = torch.empty(1, dtype=torch.float32, device="cuda")
        gm.mlp_quantize_e4m3(v.cuda(), dst, scale)
        torch.cuda.synchronize()
        q_ref, s_ref = oracle.quantize_per_tensor(v.to(torch.float32).numpy())
        assert np.float32(scale.item()) == s_ref
        np.testing.assert_array_equal(dst.cpu().numpy(), q_ref)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("offset", [0, 1])
def test_quantize_e4m3_tail_and_unaligned(dt, offset):
    """The largest magnitude in the elements after the last whole group of 8 (the vector pass
    must not miss it), and source / destination views 4 bytes off their allocations' start
    (allowed by the ABI, not aligned for the vector pass, so the per-element pass runs): codes
    and scale bit-exact."""
    import gated_mlp_gemms_amd as gm
    n = 8 * 1000 + 7
    announce(f"quantize tail {dt} offset={offset}")
    rng = np.random.default_rng(5)
    v = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(dt)
    v[-1] = -37.0
    so = 4 * offset // v.element_size()   # elements in 4 bytes
    src = torch.zeros(n + so, dtype=dt, device="cuda")
    src[so:] = v.cuda()
    dst = torch.full((n + 4 * offset,), 0x55, dtype=torch.uint8, device="cuda")
    scale = torch.empty(1, dtype=torch.float32, device="cuda")
    gm.mlp_quantize_e4m3(src[so:], dst[4 * offset:], scale)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_per_tensor(v.to(torch.float32).numpy())
    assert np.float32(scale.item()) == s_ref == np.float32(37.0) / np.float32(448.0)
    got = dst.cpu().numpy()
    np.testing.assert_array_equal(got[4 * offset:], q_ref)
    assert np.all(got[:4 * offset] == 0x55)


def _fp8_run(w, t, announce_name):
    announce(announce_name)
    r = run(w, t)
    r.quantize()
    r.forward()                   # bootstrap post scale 1.0: records amax
    r.refresh_post_scale()
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    return r


def _fp8_oracle_inputs(r):
    s = r.scales.cpu().numpy()
    return (r.x_q.cpu().numpy(), s[0], r.w1_q.cpu().numpy(), s[1], r.w2_q.cpu().numpy(), s[2], s[3])


# 2900 x 3008: 23 x 24 tiles of 128 x 128 (more than two rounds of two per CU) with ragged last
# tiles in both dimensions
@pytest.mark.parametrize("M,d,H,do,dm", [(300, 256, 704, 208, 1.0), (129, 768, 3072, 768, 2.0),
                                         (2900, 256, 3008, 256, 1.0)])
def test_fp8_forward_small(M, d, H, do, dm):
    w = _w("relu_sq", "bf16", M, d, H, do, down_mult=dm, fp8_fwd=True)
    t = make_inputs(w)
    r = _fp8_run(w, t, w.name)
    xq, sx, w1q, s1, w2q, s2, sp = _fp8_oracle_inputs(r)
    # the quantized operands are bit-exact with the oracle's quantizer
    for name, q, src in (("x", xq, t["x"]), ("w1", w1q, t["w1"]), ("w2", w2q, t["w2"])):
        q_ref, s_ref = oracle.quantize_per_tensor(src.to(torch.float32).numpy())
        np.testing.assert_array_equal(q, q_ref, err_msg=name)
    f = oracle.relu_sq_fp8_forward(xq, sx, w1q, s1, w2q, s2, s_post=sp, down_mult=dm)
    f_noq = oracle.relu_sq_fp8_forward(xq, sx, w1q, s1, w2q, s2, s_post=None, down_mult=dm)
    assert_close("out", f64(r.out), f["out"], TOL["fp8"])
    assert_close("out vs no post-q", f64(r.out), f_noq["out"], TOL["fp8"])
    assert_close("pre", f64(r.saved), f["pre"], TOL["bf16"])
    # the delayed scale came from this run's amax
    # the delayed post scale came from this problem's max relu(pre)^2 (headroom 1.03)
    assert abs(sp / (f["post_amax"] * 1.03 / 448) - 1) < 1e-2
    # the backward is bf16 GEMMs on the exact widening of the e4m3 operands: the bf16 bound
    b = oracle.relu_sq_fp8_backward(f64(r.dout), xq, sx, w1q, s1, w2q, s2, down_mult=dm)
    for name, g, ref in (("dx", r.dx, b["dx"]), ("dw1", r.dw_gate, b["dw1"]), ("dw2", r.dw_down, b["dw2"])):
        assert_close(name, f64(g), ref, TOL["bf16"])


def test_fp8_on_grid_equals_bf16_path():
    """Inputs on the e4m3 grid with amax = 448 * 2^k quantize exactly, so the fp8 forward must
    agree with the bf16 forward up to accumulation order (outputs are then bf16-rounded)."""
    rng = np.random.default_rng(1)
    grid = oracle.e4m3_grid()
    M, d, H = 256, 256, 512

    def on_grid(shape, k):
        v = rng.choice(grid[:110], size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v.flat[0] = 448.0
        return torch.from_numpy((v * 2.0 ** k).astype(np.float32)).to(torch.bfloat16)

    t = {"x": on_grid((M, d), -8), "w1": on_grid((H, d), -12), "w2": on_grid((d, H), -12),
         "dout": torch.randn(M, d, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)}
    w8 = _w("relu_sq", "bf16", M, d, H, d, fp8_fwd=True)
    wb = _w("relu_sq", "bf16", M, d, H, d)
    announce("fp8 on-grid vs bf16")
    r8 = run(w8, t)
    r8.quantize()
    r8.forward()
    rb = run(wb, t)
    rb.forward()
    torch.cuda.synchronize()
    s = r8.scales.cpu().numpy()
    assert s[0] == 2.0 ** -8 and s[1] == 2.0 ** -12 and s[2] == 2.0 ** -12
    # pre is computed in fp32 either way; both sides round it to bf16
    assert_close("pre fp8 vs bf16", f64(r8.saved), f64(rb.saved), 1e-2)


# ---- invariants -------------------------------------------------------------------------------

def test_infer_equals_train_forward_and_determinism():
    w = _w("swiglu", "bf16", 300, 264, 712, 200, gate_mult=1.125, down_mult=2.0)
    announce("infer == train, determinism")
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.forward_infer()
    r.backward()
    torch.cuda.synchronize()
    assert torch.equal(r.out, r.out_infer)
    first = {k: v.clone() for k, v in r.grads().items()}
    out1 = r.out.clone()
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    assert torch.equal(out1, r.out)
    for k, v in r.grads().items():
        assert torch.equal(first[k], v), k


@pytest.mark.parametrize("act", ["swiglu", "relu_sq"])
def test_recompute_equals_saved_and_inplace(act):
    kw = dict(gate_mult=1.125, down_mult=2.0) if act == "swiglu" else {}
    base = _w(act, "bf16", 300, 264, 712, 200, **kw)
    t = make_inputs(base)
    announce(f"recompute/in-place invariants {act}")
    r0 = run(base, t)
    r0.forward()
    r0.backward()
    r1 = run(base.replace(recompute=True), t)
    r1.forward()
    r1.backward()
    r2 = run(base, t, dpreact_in_place=True)
    r2.forward()
    r2.backward()
    torch.cuda.synchronize()
    assert torch.equal(r0.out, r1.out) and torch.equal(r0.out, r2.out)
    for k, v in r0.grads().items():
        assert torch.equal(v, r1.grads()[k]), f"recompute {k}"
        assert torch.equal(v, r2.grads()[k]), f"in-place {k}"


def test_power_of_two_down_mult_is_exact():
    w1 = _w("swiglu", "bf16", 300, 264, 712, 200, gate_mult=1.125)
    w2 = w1.replace(down_mult=2.0)
    t = make_inputs(w1)
    announce("down_mult = 2 exact")
    r1, r2 = run(w1, t), run(w2, t)
    for r in (r1, r2):
        r.forward()
        r.backward()
    torch.cuda.synchronize()
    assert torch.equal(r2.out.float(), 2 * r1.out.float())
    for k, v in r1.grads().items():
        assert torch.equal(r2.grads()[k].float(), 2 * v.float()), k


@pytest.mark.parametrize("act", ["swiglu", "relu_sq"])
def test_only_dw_down_branch(act):
    w = _w(act, "bf16", 300, 264, 712, 200)
    t = make_inputs(w)
    announce(f"only-dW_down branch {act}")
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    full = r.dw_down.clone()
    r.dw_down.zero_()
    r.backward(dx=False, dw_gate=False)
    torch.cuda.synchronize()
    assert torch.equal(full, r.dw_down)


# fp16 I/O (the flash-swiglu README's other supported dtype), same kernels with the fp16 MFMA
@pytest.mark.parametrize("w", [
    _w("swiglu", "f16", 300, 264, 712, 200, gate_mult=1.125, down_mult=2.0),
    _w("swiglu", "f16", 517, 512, 1400, 520, seed=3, recompute=True, grad_accum=True),
    _w("geglu", "f16", 300, 264, 712, 200, seed=1),
    _w("relu_sq", "f16", 333, 200, 520, 264),
    _w("gelu_tanh", "f16", 257, 136, 392, 128, recompute=True, grad_accum=True, seed=2),
], ids=lambda w: w.name)
@pytest.mark.parametrize("mode", ["outside", "inside"])
def test_fp16_small(w, mode):
    announce(f"fp16 {w.name} {mode}")
    t = make_inputs(w)
    r = run(w, t, gate_mode=mode)
    r.forward()
    r.forward_infer()
    r.backward()
    torch.cuda.synchronize()
    assert torch.equal(r.out, r.out_infer)
    check_full(w, t, r, mode)


def test_fp16_quantize_e4m3_matches_oracle():
    """The per-tensor e4m3 quantizer reads fp16 sources too: codes and scale bit-exact."""
    import gated_mlp_gemms_amd as gm
    announce("fp16 quantize")
    rng = np.random.default_rng(21)
    src = torch.tensor(rng.standard_normal(70001) * 3.0, dtype=torch.float16)
    ref_q, ref_s = oracle.quantize_per_tensor(src.double().numpy())
    d = src.cuda()
    q = torch.empty(d.numel(), dtype=torch.uint8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(int(gm.mlp_quantize_workspace_bytes()), dtype=torch.uint8, device="cuda")
    gm.mlp_quantize_e4m3(d, q, sc, ws)
    torch.cuda.synchronize()
    assert float(sc.item()) == np.float32(ref_s)
    assert np.array_equal(q.cpu().numpy(), ref_q)


def _capture(fn):
    """Capture fn() into a HIP graph after one warm-up call on a side stream (default priority)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# (12, 2056): the small-M down projection split over parts of K, then the split-K reduce
@pytest.mark.parametrize("M,H", [(1, 712), (16, 712), (300, 712), (12, 2056)])
def test_graph_replay_of_inference_forward(M, H):
    """mlp_fwd_infer captured in a graph (no allocation, no memset node, no host sync inside):
    every replay equals the eager call, with new inputs copied in eagerly between replays."""
    w = _w("swiglu", "bf16", M, 264, H, 200, gate_mult=1.125, down_mult=2.0)
    announce(f"graph replay, inference forward, M={M}, H={H}")
    t = make_inputs(w)
    r = run(w, t)
    xs = [r.x.clone(), (r.x * 0.5).contiguous(), torch.flip(r.x, [0]).contiguous()]
    refs = []
    for xv in xs:
        r.x.copy_(xv)
        r.forward_infer()
        torch.cuda.synchronize()
        refs.append(r.out_infer.clone())
    g = _capture(r.forward_infer)
    for _ in range(2):
        for xv, ref in zip(xs, refs):
            r.x.copy_(xv)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(r.out_infer, ref)


@pytest.mark.parametrize("w", [
    _w("swiglu", "bf16", 300, 264, 712, 200, gate_mult=1.125, down_mult=2.0),
    # the LLaMA shape: the backward's grouped launch, the d-activation's column split, split-K
    _w("swiglu", "bf16", 2048, 4096, 11008, 4096, seed=26),
    # store GEMMs cut along M (rows split), split-K weight gradients
    _w("relu_sq", "bf16", 30000, 1032, 3080, 1032, down_mult=1.5, seed=27),
], ids=lambda w: w.name)
def test_graph_replay_of_training_step(w):
    """A whole training step (forward + backward, with each shape's launch schedule) replayed
    from a graph gives the eager step's outputs and gradients bit for bit, replay after replay."""
    announce(f"graph replay, training step {w.name}")
    t = make_inputs(w)
    r = run(w, t)

    def step():
        r.forward()
        r.backward()

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in r.grads().items()}
    ref["out"] = r.out.clone()
    g = _capture(step)
    for _ in range(3):
        for v in r.grads().values():
            v.zero_()
        r.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(r.out, ref["out"])
        for k, v in r.grads().items():
            assert torch.equal(v, ref[k]), k


def test_dact_column_split_against_oracle():
    """A shape whose d-activation GEMM runs as two launches over the hidden units (8-wave
    256 x 256 tiles for whole rounds, 256 x 128 tiles for the rest), compared in full."""
    w = _w("swiglu", "bf16", 1800, 256, 8448, 200, gate_mult=1.125, down_mult=2.0, seed=9)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    check_full(w, t, r)
