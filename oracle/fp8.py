"""Per-tensor e4m3 quantization and the ReLU^2 MLP with e4m3 forward GEMMs (oracle; test
infrastructure only).

Follows modded-nanogpt ``gpt.py``:

* exact per-tensor scale (``_quantize_mlp_weights_and_scales``, exact-scale calls): the scale
  is the tensor's absolute maximum, clamped below at 1e-12, divided by the e4m3 maximum 448.
  The page forms it in the weights' bf16; here it is formed in float32 (the absolute maximum
  of a bf16 tensor is exact in float32, so the scale is amax/448 rounded once). The quantized
  value of v is e4m3(v / scale) with the division in float32;
* delayed scale (``_refresh_delayed_scale``): a = nan_to_num(amax) clamped above at 1e12;
  new = max(a * gain, floor); a slot whose a is 0 keeps its previous scale. For the ReLU^2
  output the gain is FP8_POST_HEADROOM / 448 = 1.03/448 and the floor 1e-6. The page does this
  in float32 tensors; so does this function;
* the forward of ``ReLUSqrdMLP`` with fp8 arguments: both forward GEMMs take e4m3 operands with
  per-tensor dequant scales, and relu(pre)^2 is quantized with the delayed post scale before the
  down projection. The backward runs on the dequantized operands;
* the backward with fp8 gradients (``relu_sq_fp8_backward_e5m2``): the incoming gradient is
  quantized to e5m2 with the static scale (FP8_GRAD_SCALE), dpre to e5m2 with the delayed dpre
  scale (FP8_DPRE_HEADROOM / 57344 times the previous call's max|dpre|), and every backward
  product takes fp8 operands: the gradients in e5m2, the weights, x and relu(pre)^2 in e4m3
  (``_mlp_fp8_args`` hands the backward the e4m3 weight caches, the transposed e4m3 x, the
  gradient and dpre scales and the dpre amax).
"""
from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode
from .e5m2 import e5m2_decode, e5m2_encode
from .mlp import drelu_sq, relu_sq, relu_sq_backward

_F32 = np.float32


def per_tensor_scale(v) -> np.float32:
    """max(amax(|v|), 1e-12) / 448 in float32."""
    amax = _F32(np.max(np.abs(np.asarray(v, dtype=np.float32)))) if np.size(v) else _F32(0.0)
    return _F32(max(amax, _F32(1e-12)) / _F32(E4M3_MAX))


def quantize_per_tensor(v, scale=None):
    """(codes, scale): codes = e4m3(fp32(v) / scale) with the scale of ``per_tensor_scale``
    unless one is given."""
    v32 = np.asarray(v, dtype=np.float32)
    s = per_tensor_scale(v32) if scale is None else _F32(scale)
    return e4m3_encode(v32 / s), s


def dequantize(codes, scale) -> np.ndarray:
    """scale * value(codes), in float64."""
    return e4m3_decode(codes) * np.float64(scale)


def next_delayed_scale(amax, prev_scale, gain, floor) -> np.float32:
    """One slot of ``_refresh_delayed_scale``, in float32."""
    a = _F32(np.nan_to_num(_F32(amax), nan=0.0, posinf=0.0, neginf=0.0))
    a = min(a, _F32(1e12))
    new = max(_F32(a * _F32(gain)), _F32(floor))
    return _F32(new) if a > 0 else _F32(prev_scale)


def weight_quantize_calls(weights, exact_calls=16):
    """The weight-cache quantizer over a sequence of calls (``_quantize_mlp_weights_and_scales``
    with FP8_EXACT_SCALE_CALLS): call t < exact_calls sets the scale exactly from that call's
    weights, max(amax|W_t|, 1e-12) / 448; every later call uses the amax the previous call
    recorded, max(amax|W_{t-1}|, 1e-12) / 448 (one call delayed), and e4m3's saturation takes
    entries beyond it to +-448. Both are formed in float32. The page records the amax per tile;
    the maximum over the tiles is the tensor's amax, which is what this function takes.

    weights: a sequence of arrays (one per call). Returns a list of (codes, scale) per call."""
    out = []
    prev_amax = None
    for t, w in enumerate(weights):
        w32 = np.asarray(w, dtype=np.float32)
        amax = _F32(np.max(np.abs(w32))) if w32.size else _F32(0.0)
        basis = amax if (t < exact_calls or prev_amax is None) else prev_amax
        scale = _F32(max(basis, _F32(1e-12)) / _F32(E4M3_MAX))
        out.append((e4m3_encode(w32 / scale), scale))
        prev_amax = amax
    return out


def relu_sq_fp8_forward(x_q, s_x, w1_q, s_w1, w2_q, s_w2, s_post=None, down_mult=1.0):
    """ReLU^2 MLP forward on e4m3 operands: pre = (s_x x_q)(s_w1 W1_q)^T, post = relu(pre)^2,
    out = down_mult * post_hat (s_w2 W2_q)^T, where post_hat = s_post * e4m3(fp32(post)/s_post)
    when a post scale is given and post itself otherwise. Returns dict(pre, post, out,
    post_amax)."""
    xh = dequantize(x_q, s_x)
    w1h = dequantize(w1_q, s_w1)
    w2h = dequantize(w2_q, s_w2)
    pre = xh @ w1h.T
    post = relu_sq(pre)
    if s_post is None:
        post_used = post
    else:
        post_used = dequantize(e4m3_encode(post.astype(np.float32) / _F32(s_post)), s_post)
    out = down_mult * (post_used @ w2h.T)
    return {"pre": pre, "post": post, "out": out, "post_amax": float(np.max(post)) if post.size else 0.0}


def relu_sq_fp8_backward(dout, x_q, s_x, w1_q, s_w1, w2_q, s_w2, down_mult=1.0):
    """Backward of the fp8-forward ReLU^2 MLP: the plain backward applied to the dequantized
    operands s_x x_q, s_w1 W1_q, s_w2 W2_q."""
    return relu_sq_backward(dout, dequantize(x_q, s_x), dequantize(w1_q, s_w1),
                            dequantize(w2_q, s_w2), down_mult)


def quantize_e5m2(v, scale) -> np.ndarray:
    """e5m2(fp32(v) / fp32(scale)) with the division in float32 (as for e4m3)."""
    return e5m2_encode(np.asarray(v, dtype=np.float32) / _F32(scale))


def relu_sq_fp8_backward_e5m2(dout, x_q, s_x, w1_q, s_w1, w2_q, s_w2, s_post, s_grad, s_dpre,
                              down_mult=1.0):
    """Backward of the fp8 ReLU^2 MLP with fp8 gradients, in the order the method takes it:

    1. pre = (s_x x_q)(s_w1 W1_q)^T (the forward's pre-activation, re-derived here);
    2. dout_hat = s_grad * e5m2(dout / s_grad)                 (static gradient scale);
    3. dpre = down_mult * (dout_hat (s_w2 W2_q)) * relu^2'(pre);
    4. dpre_hat = s_dpre * e5m2(dpre / s_dpre)                 (delayed dpre scale);
    5. post_hat = s_post * e4m3(relu(pre)^2 / s_post)          (the forward's post operand);
    6. dx = dpre_hat (s_w1 W1_q);  dW1 = dpre_hat^T (s_x x_q);  dW2 = down_mult * dout_hat^T post_hat.

    Steps 1, 3 and 5 are float64: no page states an intermediate precision for them, so none is
    imposed. Each quantizer takes its input as float32 and divides by its scale in float32 (the
    codec's own definition, as for the e4m3 operands).

    Returns dict(dx, dw1, dw2, dpre (step 3, before quantization), dpre_amax = max|dpre|,
    dout_q, dpre_q (the e5m2 codes))."""
    xh = dequantize(x_q, s_x)
    w1h = dequantize(w1_q, s_w1)
    w2h = dequantize(w2_q, s_w2)
    pre = xh @ w1h.T
    dout_q = quantize_e5m2(dout, s_grad)
    gh = e5m2_decode(dout_q) * np.float64(_F32(s_grad))
    dpre = (down_mult * (gh @ w2h)) * drelu_sq(pre)
    dpre_q = quantize_e5m2(dpre, s_dpre)
    ph = e5m2_decode(dpre_q) * np.float64(_F32(s_dpre))
    post_hat = dequantize(e4m3_encode(relu_sq(pre).astype(np.float32) / _F32(s_post)), s_post)
    return {
        "dx": ph @ w1h,
        "dw1": ph.T @ xh,
        "dw2": down_mult * (gh.T @ post_hat),
        "dpre": dpre,
        "dpre_amax": float(np.max(np.abs(dpre))) if dpre.size else 0.0,
        "dout_q": dout_q,
        "dpre_q": dpre_q,
    }


def relu_sq_fp8_backward_e5m2_sampled(dout, x_q, s_x, w1_q, s_w1, w2_q, s_w2, s_post, s_grad, s_dpre,
                                      rows, units, down_mult=1.0):
    """``relu_sq_fp8_backward_e5m2`` on a sample: dx[rows], dw1[units] and dw2[:, units], each
    entry formed by the same steps restricted to the dpre / post entries it needs (dpre[rows, :]
    for dx, dpre[:, units] and post[:, units] for the weight gradients)."""
    xh = dequantize(x_q, s_x)
    w1h = dequantize(w1_q, s_w1)
    w2h = dequantize(w2_q, s_w2)
    gh = e5m2_decode(quantize_e5m2(dout, s_grad)) * np.float64(_F32(s_grad))

    def dpre_hat(r_idx, u_idx):
        pre = xh[r_idx] @ w1h[u_idx].T
        dpre = (down_mult * (gh[r_idx] @ w2h[:, u_idx])) * drelu_sq(pre)
        return e5m2_decode(quantize_e5m2(dpre, s_dpre)) * np.float64(_F32(s_dpre)), pre

    every_row = np.arange(xh.shape[0])
    every_unit = np.arange(w1h.shape[0])
    ph_rows, _ = dpre_hat(rows, every_unit)
    ph_units, pre_units = dpre_hat(every_row, units)
    post_hat = dequantize(e4m3_encode(relu_sq(pre_units).astype(np.float32) / _F32(s_post)), s_post)
    return {
        "dx_rows": ph_rows @ w1h,
        "dw1_rows": ph_units.T @ xh,
        "dw2_cols": down_mult * (gh.T @ post_hat),
    }
