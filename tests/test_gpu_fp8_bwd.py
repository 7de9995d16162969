"""GPU tests of the backward with fp8 gradients (ReLU^2; dout and dpre in e5m2, weights, x and
relu(pre)^2 in e4m3) and of the 2-D fp8 quantizer it uses, through the C ABI, against the
float64 oracle. Every scale the GPU is given comes from the oracle (the exact per-tensor scales
are checked bit for bit against the oracle's first; the delayed post and dpre scales are formed
from the oracle's own max|relu(pre)^2| and max|dpre|)."""
import numpy as np
import pytest
import torch

import gated_mlp_gemms_amd as gm
import oracle
from gpu_helpers import TOL, announce, assert_close, f64, run
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

GRAD_SCALE = np.float32(2.0 ** -6)


def _w(M, d, H, do, **kw):
    tag = "_".join(f"{k}{v}" for k, v in sorted(kw.items()))
    return Workload(f"relu_sq_fp8bwd_m{M}_d{d}_h{H}_o{do}_{tag}", "relu_sq", "bf16", (M,), d, H, do,
                    fp8_fwd=True, fp8_bwd=True, **kw)


@pytest.mark.parametrize("rows,cols", [(100, 64), (1, 16), (300, 704)])
@pytest.mark.parametrize("fmt,relu_sq", [("e5m2", False), ("e4m3", False), ("e4m3", True)])
def test_quantize_fp8_bit_exact(rows, cols, fmt, relu_sq):
    announce(f"quantize_fp8 {fmt} relu_sq={relu_sq} {rows}x{cols}")
    rng = np.random.default_rng(rows * 7 + cols)
    v = torch.from_numpy((rng.standard_normal((rows, cols)) * 3.0).astype(np.float32)).to(torch.bfloat16)
    sc = np.float32(0.37)
    scale = torch.tensor([sc], dtype=torch.float32, device="cuda")
    ld_t = (rows + 15) // 16 * 16
    dst = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    dst_t = torch.full((cols, ld_t), 0xAB, dtype=torch.uint8, device="cuda")
    gm.mlp_quantize_fp8(v.cuda(), fmt, scale, dst=dst, dst_t=dst_t, ld_t=ld_t, relu_sq=relu_sq)
    torch.cuda.synchronize()
    v32 = v.to(torch.float32).numpy()
    if relu_sq:
        m = np.maximum(v32, np.float32(0.0))
        v32 = m * m                                       # fp32 product, as the kernel forms it
    y = v32 / sc                                          # fp32 division
    ref = oracle.e5m2_encode(y) if fmt == "e5m2" else oracle.e4m3_encode(y)
    np.testing.assert_array_equal(dst.cpu().numpy(), ref)
    t = dst_t.cpu().numpy()
    np.testing.assert_array_equal(t[:, :rows], ref.T)
    assert np.all(t[:, rows:] == 0)


def _prepare(w, t):
    """Runner with the oracle-checked e4m3 operands and the oracle's delayed scales loaded."""
    r = run(w, t)
    r.quantize()
    torch.cuda.synchronize()
    q = {}
    for name, src, code, slot in (("x", t["x"], r.x_q, 0), ("w1", t["w1"], r.w1_q, 1), ("w2", t["w2"], r.w2_q, 2)):
        q_ref, s_ref = oracle.quantize_per_tensor(src.to(torch.float32).numpy())
        np.testing.assert_array_equal(code.cpu().numpy(), q_ref, err_msg=name)
        assert np.float32(r.scales[slot].item()) == s_ref, name
        q[name] = (q_ref, s_ref)
    # the transposed caches hold the same codes
    np.testing.assert_array_equal(r.w1t_q.cpu().numpy(), q["w1"][0].T)
    np.testing.assert_array_equal(r.w2t_q.cpu().numpy(), q["w2"][0].T)
    (xq, sx), (w1q, s1), (w2q, s2) = q["x"], q["w1"], q["w2"]
    f = oracle.relu_sq_fp8_forward(xq, sx, w1q, s1, w2q, s2)
    s_post = oracle.next_delayed_scale(f["post_amax"], 1.0, np.float32(1.03) / np.float32(448.0), 1e-6)
    probe = oracle.relu_sq_fp8_backward_e5m2(f64(t["dout"]), xq, sx, w1q, s1, w2q, s2, s_post, GRAD_SCALE,
                                             GRAD_SCALE, w.down_mult)
    s_dpre = oracle.next_delayed_scale(probe["dpre_amax"], GRAD_SCALE, np.float32(1.25) / np.float32(57344.0),
                                       1e-12)
    r.scales[3] = float(s_post)
    r.scales[5] = float(GRAD_SCALE)
    r.scales[6] = float(s_dpre)
    r.scales[7] = 0.0
    b = oracle.relu_sq_fp8_backward_e5m2(f64(t["dout"]), xq, sx, w1q, s1, w2q, s2, s_post, GRAD_SCALE, s_dpre,
                                         w.down_mult)
    return r, b


# 2900 x 3008: more than two rounds of 128 x 128 tiles, with ragged last tiles in both dimensions
@pytest.mark.parametrize("M,d,H,do,dm", [(300, 256, 704, 208, 1.0), (129, 768, 3072, 768, 2.0),
                                         (1, 256, 512, 256, 1.0), (1000, 128, 384, 128, 1.0),
                                         (2900, 256, 3008, 256, 1.0)])
def test_fp8_backward_matches_oracle(M, d, H, do, dm):
    w = _w(M, d, H, do, down_mult=dm)
    announce(w.name)
    t = make_inputs(w)
    r, b = _prepare(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    for name, g, ref in (("dx", r.dx, b["dx"]), ("dw1", r.dw_gate, b["dw1"]), ("dw2", r.dw_down, b["dw2"])):
        assert_close(name, f64(g), ref, TOL["fp8"])
    amax = float(r.scales[7].item())
    assert abs(amax / b["dpre_amax"] - 1.0) < 2e-2, (amax, b["dpre_amax"])


def test_fp8_backward_recompute_skips_and_accumulate():
    """Recompute gives the saved-pre-activation result bit for bit; each skipped output leaves
    the others unchanged; accumulation adds the fresh gradient into the fp32 buffers."""
    M, d, H = 300, 256, 704
    w = _w(M, d, H, d)
    announce("fp8 backward: recompute, skips, accumulate")
    t = make_inputs(w)
    r, _ = _prepare(w, t)
    r.forward()
    r.backward()
    torch.cuda.synchronize()
    full = {k: v.clone() for k, v in (("dx", r.dx), ("dw1", r.dw_gate), ("dw2", r.dw_down))}
    wr = _w(M, d, H, d, recompute=True)
    rr, _ = _prepare(wr, t)
    rr.forward()
    rr.backward()
    torch.cuda.synchronize()
    for k, v in (("dx", rr.dx), ("dw1", rr.dw_gate), ("dw2", rr.dw_down)):
        assert torch.equal(v, full[k]), f"recompute {k}"
    for kw, keep in ((dict(dw_gate=False, dw_down=False), "dx"), (dict(dx=False, dw_down=False), "dw1"),
                     (dict(dx=False, dw_gate=False), "dw2")):
        for v in (r.dx, r.dw_gate, r.dw_down):
            v.fill_(0)
        r.backward(**kw)
        torch.cuda.synchronize()
        got = {"dx": r.dx, "dw1": r.dw_gate, "dw2": r.dw_down}[keep]
        assert torch.equal(got, full[keep]), f"only {keep}"
    wa = _w(M, d, H, d, grad_accum=True)
    ta = make_inputs(wa)
    ra, _ = _prepare(wa, ta)
    ra.forward()
    ra.backward()
    torch.cuda.synchronize()
    for name, buf, k in (("dw1", ra.dw_gate, "dw1"), ("dw2", ra.dw_down, "dw2")):
        delta = f64(buf) - f64(ra.grad_init[k])
        assert_close(f"{name} delta", delta, f64(full[k]), 1e-2)
