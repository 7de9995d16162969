"""GPU parity at the full workload sizes, in the launch configuration the bench times (the same
entry points, flags and shapes), against the float64 oracle on sampled outputs.

Sampled entries are computed one by one from their definitions (``oracle.gated_sampled`` /
``relu_sq_sampled``): rows of out and dx, and hidden units of every weight gradient. The samples
include the first and last rows/units and tile boundaries.
"""
import numpy as np
import pytest
import torch

import gated_mlp_gemms_amd as gm
import oracle
from gpu_helpers import TOL, announce, assert_close, f64, run
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def _sample(n, k=24, seed=0):
    rng = np.random.default_rng(seed)
    edges = [0, n - 1] + [b for b in (127, 128, 255, 256, 511, 512) if b < n]
    rest = rng.choice(n, size=max(0, k - len(edges)), replace=False)
    return np.unique(np.concatenate([edges, rest]).astype(np.int64))


def _check_gated(w, t, r, mode):
    a = {k: f64(v) for k, v in t.items()}
    rows, units = _sample(w.M, seed=1), _sample(w.hidden, seed=2)
    s = oracle.gated_sampled(a["dout"], a["x"], a["w_gate"], a["w_up"], a["w_down"], rows, units,
                             w.gate_mult, w.down_mult, mode)
    tol = TOL[w.dtype]
    assert_close("out[rows]", f64(r.out[rows]), s["out_rows"], tol)
    assert_close("dx[rows]", f64(r.dx[rows]), s["dx_rows"], tol)
    grads = [("dw_down[:,u]", r.dw_down[:, units], s["dw_down_cols"], "dw_down", (slice(None), units)),
             ("dw_gate[u]", r.dw_gate[units], s["dw_gate_rows"], "dw_gate", (units,)),
             ("dw_up[u]", r.dw_up[units], s["dw_up_rows"], "dw_up", (units,))]
    for name, g, ref, key, idx in grads:
        if w.grad_accum:
            before = a[key][idx]
            assert_close(name + "+buf", f64(g), oracle.accumulate(before, ref), tol)
            assert_close(name + " delta", f64(g) - before, ref, tol)
        else:
            assert_close(name, f64(g), ref, tol)


def test_llama_swiglu_full_size():
    w = WORKLOADS["llama_swiglu_bf16_m2048_d4096_h11008"]
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.forward_infer()
    r.backward(dpreact=False)
    torch.cuda.synchronize()
    assert torch.equal(r.out, r.out_infer)
    # the saved g|u of sampled rows
    a = {k: f64(v) for k, v in t.items()}
    rows = _sample(w.M, seed=3)
    f = oracle.gated_forward(a["x"][rows], a["w_gate"], a["w_up"], a["w_down"])
    assert_close("g[rows]", f64(r.saved[rows, : w.hidden]), f["g"], TOL["bf16"])
    assert_close("u[rows]", f64(r.saved[rows, w.hidden:]), f["u"], TOL["bf16"])
    _check_gated(w, t, r, "outside")


def test_llama_like_ragged_in_every_dimension():
    """A LLaMA-sized problem with no dimension a multiple of the tile: the same 8-wave tiles as
    the LLaMA step, but with partial row and column tiles (M = 2000, H = 11000, d = 4104) and a
    partial last K-step in every product (K = 4104, 11000, 2000, and 22000 for dx, whose stacked
    [W_gate; W_up] changes matrix inside a K-step). Sampled outputs include the last rows and
    hidden units, which the edge tiles produce."""
    w = Workload("llama_ragged_swiglu_bf16_m2000_d4104_h11000", "swiglu", "bf16", (2000,), 4104, 11000, 4104,
                 gate_mult=1.125, down_mult=2.0, seed=11)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward(dpreact=False)
    torch.cuda.synchronize()
    a = {k: f64(v) for k, v in t.items()}
    rows = _sample(w.M, seed=5)
    f = oracle.gated_forward(a["x"][rows], a["w_gate"], a["w_up"], a["w_down"], w.gate_mult, w.down_mult)
    assert_close("g[rows]", f64(r.saved[rows, : w.hidden]), f["g"], TOL["bf16"])
    assert_close("u[rows]", f64(r.saved[rows, w.hidden:]), f["u"], TOL["bf16"])
    _check_gated(w, t, r, "outside")


def test_llama_like_ragged_fp16_inside():
    """The ragged LLaMA-sized problem in fp16 I/O with the multiplier inside the SiLU: the fp16
    instantiations of the same 8-wave kernels and their edge tiles, at the fp16 bound."""
    w = Workload("llama_ragged_swiglu_f16_m2000_d4104_h11000", "swiglu", "f16", (2000,), 4104, 11000, 4104,
                 gate_mult=1.125, down_mult=2.0, seed=12)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t, gate_mode="inside")
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    _check_gated(w, t, r, "inside")


def test_relu_sq_ragged_in_every_dimension():
    """A GPT-like ReLU^2 problem with no dimension a multiple of the tile (M = 12000, d = 776,
    H = 3080): the 8-wave ReLU^2 and d-ReLU^2 epilogue kernels with partial tiles and partial last
    K-steps, sampled against the oracle."""
    w = Workload("gpt_ragged_relu2_bf16_m12000_d776_h3080", "relu_sq", "bf16", (12000,), 776, 3080, 776, seed=13)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    rows, s = _check_relu(w, t, r)
    assert_close("out[rows]", f64(r.out[rows]), s["out_rows"], TOL["bf16"])


@pytest.mark.parametrize("name", ["llama_swiglu_bf16_tp8_m2048_d4096_h1376", "llama_swiglu_bf16_dp8_m256_d4096_h11008"])
def test_llama_shard_shapes(name):
    """One GPU's share of the LLaMA step under 8-way tensor or data parallelism."""
    w = WORKLOADS[name]
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    _check_gated(w, t, r, "outside")


def test_grouped_backward_equals_separate_launches():
    """At the LLaMA size mlp_bwd runs dx, dW_gate/dW_up and dW_down as one launch (asserted: the
    planner's choice for this shape). A tile of that launch runs the same tile body, tile shape
    and K order as the unsplit 8-wave 256x256 launch its product gets when asked for alone, so
    dW_gate/dW_up alone and dW_down alone equal the grouped results bit for bit. dx, split along
    K when alone, is checked against the oracle on sampled rows (test_llama_swiglu_full_size);
    here a second grouped backward repeats the first bit for bit."""
    w = WORKLOADS["llama_swiglu_bf16_m2048_d4096_h11008"]
    announce(f"{w.name} grouped vs separate")
    t = make_inputs(w)
    r = run(w, t)
    assert gm.mlp_bwd_grouped(r.desc)
    r.forward()
    r.backward(dpreact=False)
    torch.cuda.synchronize()
    first = {k: v.clone() for k, v in r.grads().items()}
    r.dw_gate.zero_()
    r.dw_up.zero_()
    r.backward(dx=False, dw_down=False, dpreact=False)
    torch.cuda.synchronize()
    assert torch.equal(r.dw_gate, first["dw_gate"]) and torch.equal(r.dw_up, first["dw_up"])
    r.dw_down.zero_()
    r.backward(dx=False, dw_gate=False, dpreact=False)
    torch.cuda.synchronize()
    assert torch.equal(r.dw_down, first["dw_down"])
    r.dx.zero_()
    r.backward(dpreact=False)
    torch.cuda.synchronize()
    for k, v in r.grads().items():
        assert torch.equal(v, first[k]), k


def test_save_act_llama_full_size():
    """The LLaMA step with the activation kept by the forward (save_act): the backward runs the
    d-activation GEMM alone, then dx with dW_gate/dW_up and dW_down in one launch (asserted).
    Against the same step without save_act, out, dx, dW_gate and dW_up agree bit for
    bit (the same tiles in the same K order; only dW_down's operand a comes from elsewhere: the
    forward's fp32 epilogue instead of the d-activation GEMM's re-emission from the bf16 g and u);
    dW_down and the kept a are checked against the oracle on sampled rows and units."""
    w = WORKLOADS["llama_swiglu_bf16_m2048_d4096_h11008"].replace(save_act=True)
    announce(f"{w.name} save_act")
    t = make_inputs(w)
    r = run(w, t)
    assert gm.mlp_bwd_grouped(r.desc) == gm.MLP_BWD_GROUPED
    r.forward()
    r.backward(dpreact=False)
    torch.cuda.synchronize()
    _check_gated(w, t, r, "outside")
    a = {k: f64(v) for k, v in t.items()}
    rows = _sample(w.M, seed=4)
    f = oracle.gated_forward(a["x"][rows], a["w_gate"], a["w_up"], a["w_down"])
    assert_close("a[rows] (kept)", f64(r.saved_act[rows]), f["a"], TOL["bf16"])
    r0 = run(w.replace(save_act=False), t)
    r0.forward()
    r0.backward(dpreact=False)
    torch.cuda.synchronize()
    assert torch.equal(r.out, r0.out)
    assert torch.equal(r.saved, r0.saved)
    for k in ("dx", "dw_gate", "dw_up"):
        assert torch.equal(getattr(r, k), getattr(r0, k)), k


def test_save_act_ragged_in_every_dimension():
    """A ragged LLaMA-sized problem (M = 2900, d = 4104, H = 11000) with the activation kept by
    the forward: the d-activation GEMM with dW_down in one launch, dx with dW_gate/dW_up in
    another (both asserted), with partial tiles and partial last K-steps, sampled against the
    oracle."""
    w = Workload("llama_ragged_swiglu_bf16_m2900_d4104_h11000_save_act", "swiglu", "bf16", (2900,), 4104, 11000,
                 4104, gate_mult=1.125, down_mult=2.0, seed=11, save_act=True)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    assert gm.mlp_bwd_grouped(r.desc) == gm.MLP_BWD_GROUPED | gm.MLP_BWD_DW_DOWN_WITH_DACT
    r.forward()
    r.backward(dpreact=False)
    torch.cuda.synchronize()
    _check_gated(w, t, r, "outside")


@pytest.mark.parametrize("mode", ["outside", "inside"])
def test_falcon_h1_recompute_accumulate_full_size(mode):
    w = WORKLOADS["falcon_h1_swiglu_bf16_m8192_d2048_h4864"]
    announce(f"{w.name} {mode}")
    t = make_inputs(w)
    r = run(w, t, gate_mode=mode)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    _check_gated(w, t, r, mode)


def test_recompute_accumulate_ragged_in_every_dimension():
    """Falcon-H1-style recompute + fp32 accumulate-into-grad on a problem with no dimension a
    multiple of the tile (M = 6000, d = 2056, H = 4872): the backward's recompute GEMM and the
    accumulating weight-gradient epilogues with partial tiles and partial last K-steps; the
    accumulated buffers and their deltas against the oracle on sampled outputs."""
    w = Workload("falcon_ragged_swiglu_bf16_m6000_d2056_h4872", "swiglu", "bf16", (6000,), 2056, 4872, 2056,
                 gate_mult=1.125, down_mult=2.0, recompute=True, grad_accum=True, seed=14)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    _check_gated(w, t, r, "outside")


def _check_relu(w, t, r, x64=None, w1=None, w2=None, tol=None, extra_rows=()):
    a = {k: f64(v) for k, v in t.items()}
    x64 = a["x"] if x64 is None else x64
    w1 = a["w1"] if w1 is None else w1
    w2 = a["w2"] if w2 is None else w2
    rows = np.unique(np.concatenate([_sample(w.M, seed=4), np.asarray(extra_rows, np.int64)]))
    units = _sample(w.hidden, seed=5)
    s = oracle.relu_sq_sampled(a["dout"], x64, w1, w2, rows, units, w.down_mult)
    tol = tol or TOL[w.dtype]
    assert_close("dx[rows]", f64(r.dx[rows]), s["dx_rows"], tol)
    assert_close("dw2[:,u]", f64(r.dw_down[:, units]), s["dw2_cols"], tol)
    assert_close("dw1[u]", f64(r.dw_gate[units]), s["dw1_rows"], tol)
    return rows, s


def test_gpt_relu_sq_full_size():
    """The GPT-shape ReLU^2 step. Its down projection and dx (576 tiles of 256 x 256) run cut
    along M: rows below 43520 in two whole rounds, the rest split along K; the rows on both sides
    of the cut are among the samples."""
    w = WORKLOADS["gpt_relu2_bf16_m49152_d768_h3072"]
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    rows, s = _check_relu(w, t, r, extra_rows=(43519, 43520, 43521))
    assert_close("out[rows]", f64(r.out[rows]), s["out_rows"], TOL["bf16"])


def test_rows_split_ragged():
    """A ReLU^2 problem with ragged d and H whose down projection and dx run cut along M
    (M = 30000, d = 1032, H = 3080: 118 x 5 = 590 tiles, rows below 26112 in two whole rounds,
    the last 3888 rows split along K, the last row and column tiles partial); sampled rows
    include both sides of the cut and the last row."""
    w = Workload("relu2_rows_split_bf16_m30000_d1032_h3080", "relu_sq", "bf16", (30000,), 1032, 3080, 1032,
                 down_mult=1.5, seed=15)
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    rows, s = _check_relu(w, t, r, extra_rows=(26111, 26112, 26113, 29999))
    assert_close("out[rows]", f64(r.out[rows]), s["out_rows"], TOL["bf16"])


def test_gpt_relu_sq_fp8_full_size():
    w = WORKLOADS["gpt_relu2_fp8fwd_m49152_d768_h3072"]
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.quantize()
    r.forward()
    r.refresh_post_scale()
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    sc = r.scales.cpu().numpy()
    xq, w1q, w2q = r.x_q.cpu().numpy(), r.w1_q.cpu().numpy(), r.w2_q.cpu().numpy()
    # the quantizer is bit-exact with the oracle's
    for name, q, src, s_gpu in (("x", xq, t["x"], sc[0]), ("w1", w1q, t["w1"], sc[1]), ("w2", w2q, t["w2"], sc[2])):
        q_ref, s_ref = oracle.quantize_per_tensor(src.to(torch.float32).numpy())
        assert s_gpu == s_ref, name
        np.testing.assert_array_equal(q, q_ref, err_msg=name)
    # the delayed post scale the GPU formed from its own max relu(pre)^2 is the rule applied to the
    # oracle's maximum (the GPU's pre is an fp32 sum, so the two maxima differ by rounding only)
    xh, w1h = oracle.dequantize(xq, sc[0]), oracle.dequantize(w1q, sc[1])
    post_amax = max(float(np.max(np.maximum(xh[i:i + 4096] @ w1h.T, 0.0))) ** 2 for i in range(0, w.M, 4096))
    s_ref = oracle.next_delayed_scale(post_amax, 1.0, np.float32(1.03) / np.float32(448.0), 1e-6)
    assert abs(sc[3] / s_ref - 1.0) < 1e-3, (sc[3], s_ref)
    rows = _sample(w.M, seed=6)
    f = oracle.relu_sq_fp8_forward(xq[rows], sc[0], w1q, sc[1], w2q, sc[2], s_post=sc[3], down_mult=w.down_mult)
    assert_close("out[rows]", f64(r.out[rows]), f["out"], TOL["fp8"])
    assert_close("pre[rows]", f64(r.saved[rows]), f["pre"], TOL["bf16"])
    # the backward is bf16 GEMMs on the exact widening of the e4m3 operands: the bf16 bound
    _check_relu(w, t, r, xh, w1h, oracle.dequantize(w2q, sc[2]), TOL["bf16"])


def test_gpt_relu_sq_fp8_backward_full_size():
    """The fp8-gradient backward at the GPT MLP's full size, on sampled outputs. The delayed post
    and dpre scales are formed from the oracle's own maxima of relu(pre)^2 and |dpre|."""
    w = WORKLOADS["gpt_relu2_fp8_m49152_d768_h3072"]
    announce(w.name)
    t = make_inputs(w)
    r = run(w, t)
    r.quantize()
    torch.cuda.synchronize()
    q = []
    for name, src, code, slot in (("x", t["x"], r.x_q, 0), ("w1", t["w1"], r.w1_q, 1), ("w2", t["w2"], r.w2_q, 2)):
        q_ref, s_ref = oracle.quantize_per_tensor(src.to(torch.float32).numpy())
        assert np.float32(r.scales[slot].item()) == s_ref, name
        np.testing.assert_array_equal(code.cpu().numpy(), q_ref, err_msg=name)
        q.append((q_ref, s_ref))
    (xq, sx), (w1q, s1), (w2q, s2) = q
    np.testing.assert_array_equal(r.w1t_q.cpu().numpy(), w1q.T)
    np.testing.assert_array_equal(r.w2t_q.cpu().numpy(), w2q.T)
    # delayed scales from the oracle: max relu(pre)^2 of the forward, max |dpre| of the backward
    xh, w1h, w2h = oracle.dequantize(xq, sx), oracle.dequantize(w1q, s1), oracle.dequantize(w2q, s2)
    pre = xh @ w1h.T
    post_amax = float(np.max(np.maximum(pre, 0.0))) ** 2
    s_grad = np.float32(2.0 ** -6)
    g = oracle.e5m2_decode(oracle.quantize_e5m2(f64(t["dout"]), s_grad)) * np.float64(s_grad)
    dpre_amax = float(np.max(np.abs((w.down_mult * (g @ w2h)) * (2.0 * np.maximum(pre, 0.0)))))
    del pre, g
    s_post = oracle.next_delayed_scale(post_amax, 1.0, np.float32(1.03) / np.float32(448.0), 1e-6)
    s_dpre = oracle.next_delayed_scale(dpre_amax, s_grad, np.float32(1.25) / np.float32(57344.0), 1e-12)
    r.scales[3] = float(s_post)
    r.scales[5] = float(s_grad)
    r.scales[6] = float(s_dpre)
    r.scales[7] = 0.0
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    assert abs(float(r.scales[7].item()) / dpre_amax - 1.0) < 2e-2
    rows, units = _sample(w.M, seed=7), _sample(w.hidden, seed=8)
    s = oracle.relu_sq_fp8_backward_e5m2_sampled(f64(t["dout"]), xq, sx, w1q, s1, w2q, s2, s_post, s_grad, s_dpre,
                                                 rows, units, w.down_mult)
    assert_close("dx[rows]", f64(r.dx[rows]), s["dx_rows"], TOL["fp8"])
    assert_close("dw1[u]", f64(r.dw_gate[units]), s["dw1_rows"], TOL["fp8"])
    assert_close("dw2[:,u]", f64(r.dw_down[:, units]), s["dw2_cols"], TOL["fp8"])
