"""Shared pieces of the GPU parity tests: running a workload through the C ABI and comparing
with the float64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from gated_mlp_gemms_amd.runner import runner_for

# fp32 1e-5, bf16 2e-2, e4m3 forward 8e-2 as the hot path's specification states; fp16, which it
# does not name: 5e-3, ten fp16 unit roundoffs (2^-11), the bf16 bound scaled by the two
# formats' roundoff ratio (2^-8 / 2^-11 = 8) with headroom (g, u, a and dpre are stored in fp16)
TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 5e-3, "fp8": 8e-2}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(gpu, ref) -> float:
    """max |gpu - ref| / max |ref| (0 when both are exactly zero)."""
    gpu, ref = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    denom = np.max(np.abs(ref)) if ref.size else 0.0
    diff = np.max(np.abs(gpu - ref)) if ref.size else 0.0
    if denom == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return float(diff / denom)


def assert_close(name, gpu, ref, tol):
    e = rel_err(gpu, ref)
    print(f"    {name:>14}: err {e:.3e} (tol {tol:g})", flush=True)
    assert np.all(np.isfinite(np.asarray(gpu, np.float64))), f"{name}: non-finite values"
    assert e <= tol, f"{name}: max|gpu-ref|/max|ref| = {e:.3e} > {tol:g}"


def announce(msg: str):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def oracle_weights(w, t):
    """float64 numpy copies of the inputs, keyed as the oracle takes them."""
    out = {k: f64(v) for k, v in t.items()}
    return out


def run(w, t, **kw):
    r = runner_for(w, t, **kw)
    return r


def check_full(w, t, r, gate_mode="outside", tol=None):
    """Compare every output of a finished forward+backward of a small problem with the full
    float64 oracle."""
    tol = tol or TOL[w.dtype]
    a = oracle_weights(w, t)
    if w.gated:
        f = oracle.gated_forward(a["x"], a["w_gate"], a["w_up"], a["w_down"], w.gate_mult, w.down_mult, gate_mode,
                                 w.act)
        b = oracle.gated_backward(a["dout"], a["x"], a["w_gate"], a["w_up"], a["w_down"], w.gate_mult,
                                  w.down_mult, gate_mode, w.act)
        pairs = [("out", r.out, f["out"]), ("dx", r.dx, b["dx"])]
        grads = [("dw_gate", r.dw_gate, b["dw_gate"]), ("dw_up", r.dw_up, b["dw_up"]),
                 ("dw_down", r.dw_down, b["dw_down"])]
        if r.saved is not None:
            pairs.append(("g", r.saved[:, : w.hidden], f["g"]))
            pairs.append(("u", r.saved[:, w.hidden:], f["u"]))
        if getattr(r, "saved_act", None) is not None:
            pairs.append(("a (kept)", r.saved_act, f["a"]))
    else:
        f = oracle.act_forward(a["x"], a["w1"], a["w2"], w.down_mult, w.act)
        b = oracle.act_backward(a["dout"], a["x"], a["w1"], a["w2"], w.down_mult, w.act)
        pairs = [("out", r.out, f["out"]), ("dx", r.dx, b["dx"])]
        grads = [("dw1", r.dw_gate, b["dw1"]), ("dw2", r.dw_down, b["dw2"])]
        if r.saved is not None:
            pairs.append(("pre", r.saved, f["pre"]))
        if getattr(r, "saved_act", None) is not None:
            pairs.append(("post (kept)", r.saved_act, f["post"]))
    for name, g, ref in pairs:
        assert_close(name, f64(g), ref, tol)
    for name, g, ref in grads:
        if w.grad_accum:
            key = name if w.gated else name
            before = a[key]
            assert_close(name + "+buf", f64(g), oracle.accumulate(before, ref), tol)
            assert_close(name + " delta", f64(g) - before, ref, tol)
        else:
            assert_close(name, f64(g), ref, tol)
    return f, b
