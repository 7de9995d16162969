"""Pins of the float64 oracle against things other than itself (CPU only).

* central finite differences of L = sum(dout * out) on tiny shapes pin every backward formula;
* torch float64 autograd over library routines (F.linear, F.silu, relu) pins forward and
  backward where the multipliers are 1, and with the multipliers applied as plain tensor ops;
* closed forms of silu / sigmoid / relu^2 and special cases whose outputs are known exactly;
* invariants: linearity of the "outside" gate multiplier, exact power-of-two down multiplier,
  permutation equivariance over hidden units, sampled == full.
"""
import zlib

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RNG = np.random.default_rng(1234)


def _rand(*shape, scale=1.0, rng=RNG):
    return scale * rng.standard_normal(shape)


def _gated_loss(dout, x, wg, wu, wd, gm, dm, mode):
    return float(np.sum(dout * oracle.gated_forward(x, wg, wu, wd, gm, dm, mode)["out"]))


def _relu_loss(dout, x, w1, w2, dm):
    return float(np.sum(dout * oracle.relu_sq_forward(x, w1, w2, dm)["out"]))


def _fd_grad(f, arr, h=1e-6):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + h
        fp = f()
        arr[i] = old - h
        fm = f()
        arr[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


SHAPES = [(3, 4, 5, 4), (2, 8, 6, 3)]   # (M, d_in, H, d_out)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("mode", ["outside", "inside"])
@pytest.mark.parametrize("gm,dm", [(1.0, 1.0), (1.125, 2.0), (0.7, 1.0)])
def test_gated_backward_matches_finite_differences(shape, mode, gm, dm):
    M, d, H, do = shape
    rng = np.random.default_rng(zlib.crc32(repr((shape, mode, gm, dm)).encode()))
    x, wg, wu = _rand(M, d, rng=rng), _rand(H, d, rng=rng), _rand(H, d, rng=rng)
    wd, dout = _rand(do, H, rng=rng), _rand(M, do, rng=rng)
    g = oracle.gated_backward(dout, x, wg, wu, wd, gm, dm, mode)
    loss = lambda: _gated_loss(dout, x, wg, wu, wd, gm, dm, mode)  # noqa: E731
    for name, arr in [("dx", x), ("dw_gate", wg), ("dw_up", wu), ("dw_down", wd)]:
        fd = _fd_grad(loss, arr)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-7, err_msg=name)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("dm", [1.0, 2.0])
def test_relu_sq_backward_matches_finite_differences(shape, dm):
    M, d, H, do = shape
    rng = np.random.default_rng(7 + M + d)
    x, w1, w2, dout = _rand(M, d, rng=rng), _rand(H, d, rng=rng), _rand(do, H, rng=rng), _rand(M, do, rng=rng)
    pre = x @ w1.T
    assert np.min(np.abs(pre)) > 1e-3   # keep the kink of relu^2' out of the stencil
    g = oracle.relu_sq_backward(dout, x, w1, w2, dm)
    loss = lambda: _relu_loss(dout, x, w1, w2, dm)  # noqa: E731
    for name, arr in [("dx", x), ("dw1", w1), ("dw2", w2)]:
        fd = _fd_grad(loss, arr)
        np.testing.assert_allclose(g[name], fd, rtol=1e-6, atol=1e-7, err_msg=name)


def _torch_gated(x, wg, wu, wd, dout, gm, dm, mode):
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, wg, wu, wd)]
    g = F.linear(t[0], t[1])
    u = F.linear(t[0], t[2])
    if mode == "outside":
        a = gm * F.silu(g) * u
    else:
        a = F.silu(gm * g) * u
    out = dm * F.linear(a, t[3])
    out.backward(torch.tensor(dout, dtype=torch.float64))
    return out.detach().numpy(), [v.grad.numpy() for v in t]


@pytest.mark.parametrize("mode", ["outside", "inside"])
@pytest.mark.parametrize("gm,dm", [(1.0, 1.0), (1.125, 2.0)])
def test_gated_matches_torch_float64_autograd(mode, gm, dm):
    rng = np.random.default_rng(99)
    M, d, H, do = 17, 24, 40, 16
    x, wg, wu, wd, dout = (_rand(M, d, rng=rng), _rand(H, d, scale=0.3, rng=rng),
                           _rand(H, d, scale=0.3, rng=rng), _rand(do, H, scale=0.2, rng=rng),
                           _rand(M, do, rng=rng))
    out_t, (dx_t, dwg_t, dwu_t, dwd_t) = _torch_gated(x, wg, wu, wd, dout, gm, dm, mode)
    f = oracle.gated_forward(x, wg, wu, wd, gm, dm, mode)
    b = oracle.gated_backward(dout, x, wg, wu, wd, gm, dm, mode)
    for ours, ref in [(f["out"], out_t), (b["dx"], dx_t), (b["dw_gate"], dwg_t),
                      (b["dw_up"], dwu_t), (b["dw_down"], dwd_t)]:
        np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("dm", [1.0, 2.0])
def test_relu_sq_matches_torch_float64_autograd(dm):
    rng = np.random.default_rng(5)
    M, d, H, do = 13, 16, 48, 24
    x, w1, w2, dout = _rand(M, d, rng=rng), _rand(H, d, scale=0.3, rng=rng), _rand(do, H, scale=0.2, rng=rng), _rand(M, do, rng=rng)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, w1, w2)]
    out = dm * F.linear(torch.relu(F.linear(t[0], t[1])) ** 2, t[2])
    out.backward(torch.tensor(dout))
    f = oracle.relu_sq_forward(x, w1, w2, dm)
    b = oracle.relu_sq_backward(dout, x, w1, w2, dm)
    for ours, ref in [(f["out"], out.detach().numpy()), (b["dx"], t[0].grad.numpy()),
                      (b["dw1"], t[1].grad.numpy()), (b["dw2"], t[2].grad.numpy())]:
        np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_closed_forms():
    assert oracle.silu(0.0) == 0.0
    assert oracle.sigmoid(np.array([0.0]))[0] == 0.5
    assert oracle.dsilu(np.array([0.0]))[0] == 0.5
    # silu(1) = 1/(1+e^-1)
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16
    big = oracle.silu(np.array([80.0, -80.0, 1000.0, -1000.0]))
    assert np.all(np.isfinite(big))
    assert big[0] == 80.0 and big[2] == 1000.0
    assert -1e-30 < big[1] < 0.0 and big[3] == -0.0
    assert np.all(np.isfinite(oracle.dsilu(np.array([-1000.0, 1000.0]))))
    # derivative of silu by a finite difference at a few points
    z = np.array([-3.0, -0.5, 0.25, 2.0])
    fd = (oracle.silu(z + 1e-6) - oracle.silu(z - 1e-6)) / 2e-6
    np.testing.assert_allclose(oracle.dsilu(z), fd, rtol=1e-8)
    # relu^2 and its derivative
    z = np.array([-2.0, -0.0, 0.0, 0.5, 3.0])
    np.testing.assert_array_equal(oracle.relu_sq(z), [0.0, 0.0, 0.0, 0.25, 9.0])
    np.testing.assert_array_equal(oracle.drelu_sq(z), [0.0, 0.0, 0.0, 1.0, 6.0])


def test_relu_sq_all_negative_preactivation_gives_exact_zeros():
    rng = np.random.default_rng(3)
    x = np.abs(_rand(5, 8, rng=rng))
    w1 = -np.abs(_rand(12, 8, rng=rng)) - 0.01
    w2, dout = _rand(8, 12, rng=rng), _rand(5, 8, rng=rng)
    assert np.all(oracle.relu_sq_forward(x, w1, w2)["out"] == 0.0)
    b = oracle.relu_sq_backward(dout, x, w1, w2)
    for k in ("dx", "dw1", "dw2"):
        assert np.all(b[k] == 0.0), k


def test_gated_special_cases():
    rng = np.random.default_rng(4)
    M, d, H = 6, 8, 10
    x, wg, wd, dout = _rand(M, d, rng=rng), _rand(H, d, rng=rng), _rand(d, H, rng=rng), _rand(M, d, rng=rng)
    # W_up = 0: a = 0, so out = 0, dW_down = 0, dg = 0 (du need not vanish)
    zero = np.zeros((H, d))
    assert np.all(oracle.gated_forward(x, wg, zero, wd)["out"] == 0.0)
    b = oracle.gated_backward(dout, x, wg, zero, wd)
    assert np.all(b["dw_down"] == 0.0) and np.all(b["dg"] == 0.0) and np.all(b["dw_gate"] == 0.0)
    assert np.any(b["du"] != 0.0)
    # dout = 0: every gradient vanishes
    b = oracle.gated_backward(np.zeros((M, d)), x, wg, _rand(H, d, rng=rng), wd)
    for k in ("dx", "dw_gate", "dw_up", "dw_down"):
        assert np.all(b[k] == 0.0), k
    # M = 1 is a valid problem and equals the first row of a larger one
    wu = _rand(H, d, rng=rng)
    full = oracle.gated_forward(x, wg, wu, wd)["out"]
    one = oracle.gated_forward(x[:1], wg, wu, wd)["out"]
    np.testing.assert_allclose(one, full[:1], rtol=1e-14)


def test_multiplier_invariants():
    rng = np.random.default_rng(8)
    M, d, H = 7, 8, 12
    x, wg, wu, wd, dout = _rand(M, d, rng=rng), _rand(H, d, rng=rng), _rand(H, d, rng=rng), _rand(d, H, rng=rng), _rand(M, d, rng=rng)
    base = oracle.gated_forward(x, wg, wu, wd, 1.0, 1.0, "outside")
    # the outside gate multiplier scales a linearly
    f = oracle.gated_forward(x, wg, wu, wd, 1.125, 1.0, "outside")
    np.testing.assert_allclose(f["out"], 1.125 * base["out"], rtol=1e-12,
                               atol=1e-13 * np.abs(base["out"]).max())
    # the inside one does not (silu is not homogeneous)
    f_in = oracle.gated_forward(x, wg, wu, wd, 1.125, 1.0, "inside")
    assert np.max(np.abs(f_in["out"] - 1.125 * base["out"])) > 1e-3
    # at gate_mult = 1 the two placements coincide
    np.testing.assert_array_equal(oracle.gated_forward(x, wg, wu, wd, 1.0, 1.0, "inside")["out"], base["out"])
    # a power-of-two down multiplier scales out and the affected gradients exactly
    f2 = oracle.gated_forward(x, wg, wu, wd, 1.0, 2.0)
    np.testing.assert_array_equal(f2["out"], 2.0 * base["out"])
    b1 = oracle.gated_backward(dout, x, wg, wu, wd, 1.0, 1.0)
    b2 = oracle.gated_backward(dout, x, wg, wu, wd, 1.0, 2.0)
    for k in ("dx", "dw_gate", "dw_up", "dw_down"):
        np.testing.assert_array_equal(b2[k], 2.0 * b1[k])
    with pytest.raises(ValueError):
        oracle.gated_forward(x, wg, wu, wd, 1.0, 1.0, "sideways")


def test_hidden_permutation_equivariance():
    rng = np.random.default_rng(9)
    M, d, H = 5, 8, 11
    x, wg, wu, wd, dout = _rand(M, d, rng=rng), _rand(H, d, rng=rng), _rand(H, d, rng=rng), _rand(d, H, rng=rng), _rand(M, d, rng=rng)
    p = rng.permutation(H)
    f = oracle.gated_forward(x, wg, wu, wd, 1.125, 2.0)
    fp = oracle.gated_forward(x, wg[p], wu[p], wd[:, p], 1.125, 2.0)
    np.testing.assert_allclose(fp["out"], f["out"], rtol=1e-12, atol=1e-12)
    b = oracle.gated_backward(dout, x, wg, wu, wd, 1.125, 2.0)
    bp = oracle.gated_backward(dout, x, wg[p], wu[p], wd[:, p], 1.125, 2.0)
    np.testing.assert_allclose(bp["dw_gate"], b["dw_gate"][p], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bp["dw_down"], b["dw_down"][:, p], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bp["dx"], b["dx"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["outside", "inside"])
def test_sampled_equals_full(mode):
    rng = np.random.default_rng(11)
    M, d, H, do = 23, 16, 30, 12
    x, wg, wu, wd, dout = _rand(M, d, rng=rng), _rand(H, d, rng=rng), _rand(H, d, rng=rng), _rand(do, H, rng=rng), _rand(M, do, rng=rng)
    rows, units = np.array([0, 5, 22]), np.array([1, 17, 29])
    f = oracle.gated_forward(x, wg, wu, wd, 1.125, 2.0, mode)
    b = oracle.gated_backward(dout, x, wg, wu, wd, 1.125, 2.0, mode)
    s = oracle.gated_sampled(dout, x, wg, wu, wd, rows, units, 1.125, 2.0, mode)
    np.testing.assert_allclose(s["out_rows"], f["out"][rows], rtol=1e-13)
    np.testing.assert_allclose(s["dx_rows"], b["dx"][rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["dw_down_cols"], b["dw_down"][:, units], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["dw_gate_rows"], b["dw_gate"][units], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["dw_up_rows"], b["dw_up"][units], rtol=1e-12, atol=1e-13)
    w1, w2 = _rand(H, d, rng=rng), _rand(do, H, rng=rng)
    f = oracle.relu_sq_forward(x, w1, w2, 2.0)
    b = oracle.relu_sq_backward(dout, x, w1, w2, 2.0)
    s = oracle.relu_sq_sampled(dout, x, w1, w2, rows, units, 2.0)
    np.testing.assert_allclose(s["out_rows"], f["out"][rows], rtol=1e-13)
    np.testing.assert_allclose(s["dx_rows"], b["dx"][rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["dw2_cols"], b["dw2"][:, units], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s["dw1_rows"], b["dw1"][units], rtol=1e-12, atol=1e-13)


def test_accumulate():
    buf = np.array([1.0, -2.0], dtype=np.float32)
    np.testing.assert_array_equal(oracle.accumulate(buf, np.array([0.5, 0.25])), [1.5, -1.75])


# ---- the other activations of quack's ``Activation`` set (standard definitions) -------------

GATED_OTHER = ["geglu", "reglu", "glu"]
PLAIN_OTHER = ["relu", "gelu_tanh"]


def _torch_gate_fn(act):
    return {"swiglu": F.silu, "geglu": lambda z: F.gelu(z, approximate="tanh"), "reglu": torch.relu,
            "glu": torch.sigmoid}[act]


def _torch_plain_fn(act):
    return {"relu_sq": lambda z: torch.relu(z) ** 2, "relu": torch.relu,
            "gelu_tanh": lambda z: F.gelu(z, approximate="tanh")}[act]


def test_gelu_tanh_is_the_library_tanh_gelu_and_close_to_erf_gelu():
    z = np.linspace(-8.0, 8.0, 4001)
    ref = F.gelu(torch.tensor(z), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(z), ref, rtol=1e-14, atol=1e-15)
    exact = F.gelu(torch.tensor(z)).numpy()                       # z * Phi(z), erf form
    dev = np.abs(oracle.gelu_tanh(z) - exact).max()
    assert 1e-5 < dev < 1e-3                                      # an approximation, a close one
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    assert oracle.dgelu_tanh(np.array([0.0]))[0] == 0.5
    # far tails: gelu(z) -> z for z >> 0, -> 0 for z << 0
    assert abs(oracle.gelu_tanh(np.array([12.0]))[0] - 12.0) < 1e-12
    assert abs(oracle.gelu_tanh(np.array([-12.0]))[0]) < 1e-12


@pytest.mark.parametrize("name", ["gelu_tanh", "sigmoid", "relu"])
def test_scalar_derivatives_match_finite_differences(name):
    f, df = {"gelu_tanh": (oracle.gelu_tanh, oracle.dgelu_tanh), "sigmoid": (oracle.sigmoid, oracle.dsigmoid),
             "relu": (oracle.relu, oracle.drelu)}[name]
    z = np.concatenate([np.linspace(-6.0, -0.01, 300), np.linspace(0.01, 6.0, 300)])   # off relu's kink
    h = 1e-6
    fd = (f(z + h) - f(z - h)) / (2 * h)
    np.testing.assert_allclose(df(z), fd, rtol=1e-7, atol=1e-8)


def test_relu_family_closed_forms():
    z = np.array([-2.0, -0.0, 0.0, 1e-300, 3.5])
    np.testing.assert_array_equal(oracle.relu(z), [0.0, 0.0, 0.0, 1e-300, 3.5])
    np.testing.assert_array_equal(oracle.drelu(z), [0.0, 0.0, 0.0, 1.0, 1.0])
    assert oracle.dsigmoid(np.array([0.0]))[0] == 0.25


@pytest.mark.parametrize("act", GATED_OTHER)
@pytest.mark.parametrize("mode", ["outside", "inside"])
@pytest.mark.parametrize("gm,dm", [(1.0, 1.0), (1.125, 2.0)])
def test_other_gated_match_torch_float64_autograd(act, mode, gm, dm):
    rng = np.random.default_rng(zlib.crc32(repr((act, mode, gm, dm)).encode()))
    M, d, H, do = 11, 16, 24, 8
    x, wg, wu, wd, dout = (_rand(M, d, rng=rng), _rand(H, d, scale=0.3, rng=rng), _rand(H, d, scale=0.3, rng=rng),
                           _rand(do, H, scale=0.2, rng=rng), _rand(M, do, rng=rng))
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, wg, wu, wd)]
    fn = _torch_gate_fn(act)
    g, u = F.linear(t[0], t[1]), F.linear(t[0], t[2])
    a = gm * fn(g) * u if mode == "outside" else fn(gm * g) * u
    out = dm * F.linear(a, t[3])
    out.backward(torch.tensor(dout))
    f = oracle.gated_forward(x, wg, wu, wd, gm, dm, mode, act)
    b = oracle.gated_backward(dout, x, wg, wu, wd, gm, dm, mode, act)
    for ours, ref in [(f["out"], out.detach().numpy()), (b["dx"], t[0].grad.numpy()),
                      (b["dw_gate"], t[1].grad.numpy()), (b["dw_up"], t[2].grad.numpy()),
                      (b["dw_down"], t[3].grad.numpy())]:
        np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("act", PLAIN_OTHER)
@pytest.mark.parametrize("dm", [1.0, 2.0])
def test_other_plain_match_torch_float64_autograd(act, dm):
    rng = np.random.default_rng(zlib.crc32(repr((act, dm)).encode()))
    M, d, H, do = 13, 16, 48, 24
    x, w1, w2, dout = _rand(M, d, rng=rng), _rand(H, d, scale=0.3, rng=rng), _rand(do, H, scale=0.2, rng=rng), _rand(M, do, rng=rng)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, w1, w2)]
    out = dm * F.linear(_torch_plain_fn(act)(F.linear(t[0], t[1])), t[2])
    out.backward(torch.tensor(dout))
    f = oracle.act_forward(x, w1, w2, dm, act)
    b = oracle.act_backward(dout, x, w1, w2, dm, act)
    for ours, ref in [(f["out"], out.detach().numpy()), (b["dx"], t[0].grad.numpy()),
                      (b["dw1"], t[1].grad.numpy()), (b["dw2"], t[2].grad.numpy())]:
        np.testing.assert_allclose(ours, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("act", GATED_OTHER)
@pytest.mark.parametrize("mode", ["outside", "inside"])
def test_other_gated_backward_matches_finite_differences(act, mode):
    M, d, H, do = 3, 4, 5, 4
    rng = np.random.default_rng(zlib.crc32(repr(("fd", act, mode)).encode()))
    x, wg, wu = _rand(M, d, rng=rng), _rand(H, d, rng=rng), _rand(H, d, rng=rng)
    wd, dout = _rand(do, H, rng=rng), _rand(M, do, rng=rng)
    gm, dm = 1.125, 2.0
    if act == "reglu":
        z = (x @ wg.T) * (gm if mode == "inside" else 1.0)
        assert np.min(np.abs(z)) > 1e-3   # keep relu's kink out of the stencil
    g = oracle.gated_backward(dout, x, wg, wu, wd, gm, dm, mode, act)
    loss = lambda: float(np.sum(dout * oracle.gated_forward(x, wg, wu, wd, gm, dm, mode, act)["out"]))  # noqa: E731
    for name, arr in [("dx", x), ("dw_gate", wg), ("dw_up", wu), ("dw_down", wd)]:
        np.testing.assert_allclose(g[name], _fd_grad(loss, arr), rtol=1e-6, atol=1e-7, err_msg=name)


@pytest.mark.parametrize("act", PLAIN_OTHER)
def test_other_plain_backward_matches_finite_differences(act):
    M, d, H, do = 3, 4, 6, 3
    rng = np.random.default_rng(zlib.crc32(repr(("fd", act)).encode()))
    x, w1, w2, dout = _rand(M, d, rng=rng), _rand(H, d, rng=rng), _rand(do, H, rng=rng), _rand(M, do, rng=rng)
    assert np.min(np.abs(x @ w1.T)) > 1e-3
    b = oracle.act_backward(dout, x, w1, w2, 2.0, act)
    loss = lambda: float(np.sum(dout * oracle.act_forward(x, w1, w2, 2.0, act)["out"]))  # noqa: E731
    for name, arr in [("dx", x), ("dw1", w1), ("dw2", w2)]:
        np.testing.assert_allclose(b[name], _fd_grad(loss, arr), rtol=1e-6, atol=1e-7, err_msg=name)


def test_glu_and_reglu_special_cases():
    """glu with a zero gate halves the up projection; reglu with a negative gate gives zeros."""
    rng = np.random.default_rng(3)
    x, wu, wd = _rand(4, 6, rng=rng), _rand(5, 6, rng=rng), _rand(3, 5, rng=rng)
    zero = np.zeros((5, 6))
    f = oracle.gated_forward(x, zero, wu, wd, act="glu")
    np.testing.assert_allclose(f["a"], 0.5 * (x @ wu.T), rtol=0, atol=0)
    neg = -np.abs(_rand(5, 6, rng=rng))
    xp = np.abs(x)
    f = oracle.gated_forward(xp, neg, wu, wd, act="reglu")
    assert np.all(f["a"] == 0.0) and np.all(f["out"] == 0.0)


@pytest.mark.parametrize("act", GATED_OTHER)
def test_other_gated_sampled_equals_full(act):
    rng = np.random.default_rng(11)
    M, d, H, do = 9, 8, 12, 6
    x, wg, wu, wd, dout = (_rand(M, d, rng=rng), _rand(H, d, rng=rng), _rand(H, d, rng=rng), _rand(do, H, rng=rng),
                           _rand(M, do, rng=rng))
    rows, units = np.array([0, 4, 8]), np.array([1, 7, 11])
    f = oracle.gated_forward(x, wg, wu, wd, 1.125, 2.0, "inside", act)
    b = oracle.gated_backward(dout, x, wg, wu, wd, 1.125, 2.0, "inside", act)
    s = oracle.gated_sampled(dout, x, wg, wu, wd, rows, units, 1.125, 2.0, "inside", act)
    np.testing.assert_allclose(s["out_rows"], f["out"][rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s["dx_rows"], b["dx"][rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s["dw_down_cols"], b["dw_down"][:, units], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s["dw_gate_rows"], b["dw_gate"][units], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s["dw_up_rows"], b["dw_up"][units], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("act", PLAIN_OTHER)
def test_other_plain_sampled_equals_full(act):
    rng = np.random.default_rng(12)
    M, d, H, do = 9, 8, 12, 6
    x, w1, w2, dout = _rand(M, d, rng=rng), _rand(H, d, rng=rng), _rand(do, H, rng=rng), _rand(M, do, rng=rng)
    rows, units = np.array([1, 5]), np.array([0, 6, 11])
    f = oracle.act_forward(x, w1, w2, 2.0, act)
    b = oracle.act_backward(dout, x, w1, w2, 2.0, act)
    s = oracle.act_sampled(dout, x, w1, w2, rows, units, 2.0, act)
    np.testing.assert_allclose(s["out_rows"], f["out"][rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s["dx_rows"], b["dx"][rows], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s["dw2_cols"], b["dw2"][:, units], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s["dw1_rows"], b["dw1"][units], rtol=1e-13, atol=1e-13)
