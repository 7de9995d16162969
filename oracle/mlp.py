"""Float64 definitions of the MLP forward and backward (oracle; test infrastructure only).

Notation: x [M, d_in] holds the flattened tokens (quack ``MLPRecomputeFunc.forward`` reshapes
x to 2-D before the first GEMM; the flash-swiglu README requires a contiguous [B, S, dim] input).
Weights use the ``nn.Linear`` layout: W_gate, W_up, W1 are [H, d_in]; W_down, W2 are [d_out, H]
(flash-swiglu README, module usage: gate_proj/up_proj [intermediate, hidden], down_proj
[hidden, intermediate]).

Gated MLP (flash-swiglu README, computed function and "Falcon H1 style models" section):
    g = x W_gate^T,  u = x W_up^T
    a = gate_mult * silu(g) * u          (gate_mode "outside": the README's formula)
    a = silu(gate_mult * g) * u          (gate_mode "inside": the multiplier on the gate input)
    out = down_mult * a W_down^T
The two gate-multiplier placements agree at gate_mult = 1; the README writes the first, and the
second is kept as an explicit mode.

ReLU^2 MLP (modded-nanogpt ``gpt.py``, the comment on ``ReLUSqrdMLP`` and ``GPT._mlp``):
    pre = x W1^T,  post = relu(pre)^2,  out = down_mult * post W2^T
(down_mult = 1 on that page; its fp8 path folds a per-layer scalar into the down projection's
dequant scale, ``_mlp_fp8_args``, which is the same role.)

Backward (quack ``MLPRecomputeFunc.backward`` and ``_compute_weight_grad``): the activation's
derivative is applied to dout W2 against the pre-activation; then dW2 = dout^T postact,
dx = dpreact W1, dW1 = dpreact^T x. For the gated case W1 = [W_gate; W_up] and
dpreact = [dg, du], so dx = dg W_gate + du W_up and [dW_gate; dW_up] = [dg, du]^T x
(flash-swiglu README, "design points": merged dW_g/dW_u GEMM, single-accumulator dI).
The backward recomputes g, u (or pre) from x: it keeps no state from the forward.

Other activations. quack ``mlp.py`` names the set its MLP accepts (``Activation``: gelu_tanh_approx,
relu, relu_sq, swiglu, swiglu_oai, reglu, geglu, glu; the gated ones are those in its gate map)
but prints no formula; the standard definitions are used, with the gate multiplier placed as for
SwiGLU:
    gelu_tanh(z) = z/2 * (1 + tanh(sqrt(2/pi) * (z + 0.044715 z^3)))   (Hendrycks & Gimpel, 2016,
                                                                       the tanh approximation)
    relu(z) = max(z, 0)                       (derivative 1 for z > 0, else 0)
    glu:   a = sigmoid(g) * u                 (Dauphin et al., 2017)
    reglu: a = relu(g) * u,  geglu: a = gelu_tanh(g) * u,  swiglu: a = silu(g) * u
                                              (Shazeer, 2020, "GLU Variants Improve Transformer")
swiglu_oai has no definition on the pages and is not provided.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def sigmoid(z):
    """Logistic function, evaluated without overflow: 1/(1+e^-z) for z >= 0, e^z/(1+e^z) else."""
    z = _f64(z)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu(z):
    """silu(z) = z * sigmoid(z) (the SiLU of the SwiGLU formula in the flash-swiglu README)."""
    z = _f64(z)
    return z * sigmoid(z)


def dsilu(z):
    """d silu / dz = sigmoid(z) * (1 + z * (1 - sigmoid(z)))."""
    z = _f64(z)
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def relu_sq(z):
    """relu(z)^2 (modded-nanogpt ``gpt.py``: relu(x @ W1.T)^2)."""
    r = np.maximum(_f64(z), 0.0)
    return r * r


def drelu_sq(z):
    """d relu(z)^2 / dz = 2 * max(z, 0)."""
    return 2.0 * np.maximum(_f64(z), 0.0)


def relu(z):
    """max(z, 0)."""
    return np.maximum(_f64(z), 0.0)


def drelu(z):
    """d relu / dz: 1 for z > 0, 0 for z <= 0 (the subgradient 0 at the kink, as relu^2' = 0 there)."""
    return (_f64(z) > 0.0).astype(np.float64)


_GELU_C = np.sqrt(2.0 / np.pi)
_GELU_K = 0.044715


def gelu_tanh(z):
    """z/2 * (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))): the tanh approximation of GELU."""
    z = _f64(z)
    return 0.5 * z * (1.0 + np.tanh(_GELU_C * (z + _GELU_K * z ** 3)))


def dgelu_tanh(z):
    """d gelu_tanh / dz = (1 + t)/2 + z/2 (1 - t^2) sqrt(2/pi) (1 + 3 * 0.044715 z^2), with t the
    tanh of the definition."""
    z = _f64(z)
    t = np.tanh(_GELU_C * (z + _GELU_K * z ** 3))
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * _GELU_C * (1.0 + 3.0 * _GELU_K * z * z)


def dsigmoid(z):
    """d sigmoid / dz = sigmoid(z) (1 - sigmoid(z))."""
    s = sigmoid(z)
    return s * (1.0 - s)


# gate function f and its derivative of each gated activation: a = f(g) * u
GATED_FNS = {"swiglu": (silu, dsilu), "geglu": (gelu_tanh, dgelu_tanh), "reglu": (relu, drelu),
             "glu": (sigmoid, dsigmoid)}
# activation f and its derivative of each non-gated activation: post = f(pre)
PLAIN_FNS = {"relu_sq": (relu_sq, drelu_sq), "relu": (relu, drelu), "gelu_tanh": (gelu_tanh, dgelu_tanh)}


def _gated_fn(act):
    if act not in GATED_FNS:
        raise ValueError(f"gated activation must be one of {sorted(GATED_FNS)}, got {act!r}")
    return GATED_FNS[act]


def _gate_act(g, u, gate_mult, gate_mode, act="swiglu"):
    f, _ = _gated_fn(act)
    if gate_mode == "outside":
        return gate_mult * f(g) * u
    if gate_mode == "inside":
        return f(gate_mult * g) * u
    raise ValueError(f"gate_mode must be 'outside' or 'inside', got {gate_mode!r}")


def _gate_act_grad(da, g, u, gate_mult, gate_mode, act="swiglu"):
    """(dg, du) for a = act(g, u) given da = dL/da (chain rule on the two formulas above)."""
    f, df = _gated_fn(act)
    if gate_mode == "outside":
        return da * gate_mult * u * df(g), da * gate_mult * f(g)
    if gate_mode == "inside":
        return da * u * gate_mult * df(gate_mult * g), da * f(gate_mult * g)
    raise ValueError(f"gate_mode must be 'outside' or 'inside', got {gate_mode!r}")


def gated_forward(x, w_gate, w_up, w_down, gate_mult=1.0, down_mult=1.0, gate_mode="outside",
                  act="swiglu"):
    """SwiGLU MLP forward in float64. Returns dict(g, u, a, out).

    Follows the flash-swiglu README's formula down_multiplier * down_proj(gate_multiplier *
    silu(gate_proj(x)) * up_proj(x)) ("Falcon H1 style models"), with the gate/up split of quack
    ``mlp.py``'s fallback (first operand of the gated function is the gate)."""
    x, w_gate, w_up, w_down = map(_f64, (x, w_gate, w_up, w_down))
    g = x @ w_gate.T
    u = x @ w_up.T
    a = _gate_act(g, u, gate_mult, gate_mode, act)
    out = down_mult * (a @ w_down.T)
    return {"g": g, "u": u, "a": a, "out": out}


def gated_backward(dout, x, w_gate, w_up, w_down, gate_mult=1.0, down_mult=1.0,
                   gate_mode="outside", act="swiglu"):
    """SwiGLU MLP backward in float64, recomputing g, u from x.

    Steps as in quack ``MLPRecomputeFunc.backward``: recompute the pre-activation, apply the
    activation's derivative to dout W_down against it (also giving the post-activation a), then
    dW_down = dout^T a, dx = dpreact W1 and dW1 = dpreact^T x. Returns dict(dx, dw_gate, dw_up,
    dw_down, dg, du, a)."""
    dout, x, w_gate, w_up, w_down = map(_f64, (dout, x, w_gate, w_up, w_down))
    g = x @ w_gate.T
    u = x @ w_up.T
    a = _gate_act(g, u, gate_mult, gate_mode, act)
    da = down_mult * (dout @ w_down)
    dg, du = _gate_act_grad(da, g, u, gate_mult, gate_mode, act)
    return {
        "dw_down": down_mult * (dout.T @ a),
        "dx": dg @ w_gate + du @ w_up,
        "dw_gate": dg.T @ x,
        "dw_up": du.T @ x,
        "dg": dg, "du": du, "a": a,
    }


def gated_sampled(dout, x, w_gate, w_up, w_down, rows, units, gate_mult=1.0, down_mult=1.0,
                  gate_mode="outside", act="swiglu"):
    """The same definitions as ``gated_forward``/``gated_backward``, evaluated only where
    needed for a sample of outputs: out[rows], dx[rows], and the hidden units ``units`` of the
    weight gradients (dw_down[:, units], dw_gate[units, :], dw_up[units, :]).

    Each sampled entry is the plain definition with its sums restricted to the entries it
    depends on: a row of out or dx needs g, u of that row only; a hidden unit's weight gradients
    need g, u, da of that unit only (over all rows)."""
    dout, x, w_gate, w_up, w_down = map(_f64, (dout, x, w_gate, w_up, w_down))
    rows = np.asarray(rows)
    units = np.asarray(units)
    # rows: full hidden width, selected tokens
    xr = x[rows]
    g = xr @ w_gate.T
    u = xr @ w_up.T
    a = _gate_act(g, u, gate_mult, gate_mode, act)
    out_rows = down_mult * (a @ w_down.T)
    da = down_mult * (dout[rows] @ w_down)
    dg, du = _gate_act_grad(da, g, u, gate_mult, gate_mode, act)
    dx_rows = dg @ w_gate + du @ w_up
    # units: all tokens, selected hidden units
    gc = x @ w_gate[units].T
    uc = x @ w_up[units].T
    ac = _gate_act(gc, uc, gate_mult, gate_mode, act)
    dac = down_mult * (dout @ w_down[:, units])
    dgc, duc = _gate_act_grad(dac, gc, uc, gate_mult, gate_mode, act)
    return {
        "out_rows": out_rows, "dx_rows": dx_rows,
        "dw_down_cols": down_mult * (dout.T @ ac),
        "dw_gate_rows": dgc.T @ x, "dw_up_rows": duc.T @ x,
    }


def _plain_fn(act):
    if act not in PLAIN_FNS:
        raise ValueError(f"non-gated activation must be one of {sorted(PLAIN_FNS)}, got {act!r}")
    return PLAIN_FNS[act]


def act_forward(x, w1, w2, down_mult=1.0, act="relu_sq"):
    """Non-gated MLP forward: pre = x W1^T, post = f(pre), out = down_mult * post W2^T
    (modded-nanogpt ``gpt.py`` for f = relu^2: ``ReLUSqrdMLP`` comment and ``GPT._mlp``)."""
    x, w1, w2 = map(_f64, (x, w1, w2))
    f, _ = _plain_fn(act)
    pre = x @ w1.T
    post = f(pre)
    return {"pre": pre, "post": post, "out": down_mult * (post @ w2.T)}


def act_backward(dout, x, w1, w2, down_mult=1.0, act="relu_sq"):
    """Non-gated MLP backward (quack ``MLPRecomputeFunc.backward`` with the non-gated ops):
    dpre = (down_mult * dout W2) * f'(pre); dW2 = down_mult * dout^T post; dx = dpre W1;
    dW1 = dpre^T x. Returns dict(dx, dw1, dw2, dpre, post)."""
    dout, x, w1, w2 = map(_f64, (dout, x, w1, w2))
    f, df = _plain_fn(act)
    pre = x @ w1.T
    post = f(pre)
    dpost = down_mult * (dout @ w2)
    dpre = dpost * df(pre)
    return {
        "dw2": down_mult * (dout.T @ post),
        "dx": dpre @ w1,
        "dw1": dpre.T @ x,
        "dpre": dpre, "post": post,
    }


def act_sampled(dout, x, w1, w2, rows, units, down_mult=1.0, act="relu_sq"):
    """``act_forward``/``act_backward`` evaluated on a sample: out[rows], dx[rows],
    dw2[:, units], dw1[units, :] (sums restricted to the entries each sampled output needs)."""
    dout, x, w1, w2 = map(_f64, (dout, x, w1, w2))
    f, df = _plain_fn(act)
    rows = np.asarray(rows)
    units = np.asarray(units)
    pre = x[rows] @ w1.T
    out_rows = down_mult * (f(pre) @ w2.T)
    dpre = down_mult * (dout[rows] @ w2) * df(pre)
    dx_rows = dpre @ w1
    prec = x @ w1[units].T
    dprec = down_mult * (dout @ w2[:, units]) * df(prec)
    return {
        "out_rows": out_rows, "dx_rows": dx_rows,
        "dw2_cols": down_mult * (dout.T @ f(prec)),
        "dw1_rows": dprec.T @ x,
    }


def relu_sq_forward(x, w1, w2, down_mult=1.0):
    """``act_forward`` with f = relu^2."""
    return act_forward(x, w1, w2, down_mult, "relu_sq")


def relu_sq_backward(dout, x, w1, w2, down_mult=1.0):
    """``act_backward`` with f = relu^2."""
    return act_backward(dout, x, w1, w2, down_mult, "relu_sq")


def relu_sq_sampled(dout, x, w1, w2, rows, units, down_mult=1.0):
    """``act_sampled`` with f = relu^2."""
    return act_sampled(dout, x, w1, w2, rows, units, down_mult, "relu_sq")


def accumulate(buf_before, grad):
    """Gradient accumulation into an existing buffer (quack ``_compute_weight_grad`` with
    fuse_grad_accum: ``gemm_add_inplace`` adds the new product into ``weight.grad``)."""
    return _f64(buf_before) + _f64(grad)
