"""Pins of the oracle's e5m2 codec and of its backward with fp8 gradients (CPU only).

The codec is checked against torch's ``float8_e5m2`` conversion (an independent implementation
of the same OCP format) on every code and on every rounding midpoint inside the finite range;
outside it the oracle saturates (its stated reading) where torch gives infinity. The fp8
backward is pinned by (1) a one-unit case worked out by hand, (2) inputs on which every
quantization is exact, where it must equal the plain backward, and (3) the rounding bound of the
two e5m2 and one e4m3 quantizations against the exact backward on random data."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_encode(v32):
    return torch.from_numpy(np.asarray(v32, np.float32)).to(torch.float8_e5m2).view(torch.uint8).numpy()


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e5m2).to(torch.float64).numpy()


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.e5m2_decode(codes), _torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(codes[nan]) == {0x7D, 0x7E, 0x7F, 0xFD, 0xFE, 0xFF}
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert np.isinf(ours[0x7C]) and np.isinf(ours[0xFC])


def test_known_codes():
    dec = oracle.e5m2_decode
    assert dec(0x7B) == 57344.0 and dec(0xFB) == -57344.0
    assert dec(0x01) == 2.0 ** -16 and dec(0x04) == 2.0 ** -14 and dec(0x03) == 3 * 2.0 ** -16
    assert dec(0x3C) == 1.0 and dec(0x3D) == 1.25 and dec(0x38) == 0.5 and dec(0x00) == 0.0
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        assert oracle.E5M2_MAX == json.load(f)["e5m2_max"]["value"]


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7C) != 0x7C], dtype=np.uint8)
    assert codes.size == 248
    np.testing.assert_array_equal(oracle.e5m2_encode(oracle.e5m2_decode(codes)), codes)


def test_midpoints_round_to_even_and_match_torch():
    grid = oracle.e5m2_grid()
    mids = (grid[:-1] + grid[1:]) / 2                       # exact in float32
    for sign in (1.0, -1.0):
        v = (sign * mids).astype(np.float32)
        ours = oracle.e5m2_encode(v)
        assert np.all((ours & 0x7F) % 2 == 0)               # even mantissa
        np.testing.assert_array_equal(ours, _torch_encode(v))
        up = np.nextafter(v, np.float32(sign * np.inf))
        dn = np.nextafter(v, np.float32(0.0))
        np.testing.assert_array_equal(oracle.e5m2_encode(up), _torch_encode(up))
        np.testing.assert_array_equal(oracle.e5m2_encode(dn), _torch_encode(dn))


def test_random_values_match_torch_in_range():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(200000) * np.exp2(rng.uniform(-20, 15, 200000))).astype(np.float32)
    v = v[np.abs(v) < 57344.0]
    np.testing.assert_array_equal(oracle.e5m2_encode(v), _torch_encode(v))


def test_saturation_nan_and_signed_zero():
    enc = oracle.e5m2_encode
    np.testing.assert_array_equal(enc([57344.0, 61440.0, 1e9, np.inf]), [0x7B] * 4)
    np.testing.assert_array_equal(enc([-61440.0, -np.inf]), [0xFB] * 2)
    assert enc(np.nan) == 0x7F
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    # below half the smallest subnormal: zero; at exactly half: ties to even (zero)
    assert enc(2.0 ** -18) == 0x00 and enc(2.0 ** -17) == 0x00 and enc(1.5 * 2.0 ** -16) == 0x02


def _e4m3_codes(values):
    return oracle.e4m3_encode(np.asarray(values, dtype=np.float64))


def _one_unit(dout, s_dpre, dm):
    f = np.float32
    return oracle.relu_sq_fp8_backward_e5m2(
        np.array([[dout]]), _e4m3_codes([[1.5]]), f(1.0), _e4m3_codes([[1.0]]), f(1.0),
        _e4m3_codes([[1.0]]), f(1.0), s_post=f(1.0), s_grad=f(1.0), s_dpre=f(s_dpre), down_mult=dm)


def test_hand_worked_one_unit():
    """x = 1.5, W1 = W2 = 1, dout = 2.6 with unit scales. dout rounds to 2.5 (e5m2 steps of 0.5 in
    [2, 4)); pre = 1.5, so dpre = 2.5 * 2 * 1.5 = 7.5, a tie between 7 (odd mantissa) and 8 (even):
    8. post = 2.25 is an e4m3 value. Hence dx = 8, dW1 = 8 * 1.5 = 12, dW2 = 2.5 * 2.25 = 5.625."""
    r = _one_unit(2.6, 1.0, 1.0)
    assert r["dx"][0, 0] == 8.0 and r["dw1"][0, 0] == 12.0 and r["dw2"][0, 0] == 5.625
    assert r["dpre_amax"] == 7.5 and r["dout_q"][0, 0] == 0x41 and r["dpre_q"][0, 0] == 0x48
    # dpre scale 3: 7.5 / 3 = 2.5 is on the grid, so dpre passes unrounded
    r = _one_unit(2.6, 3.0, 1.0)
    assert r["dx"][0, 0] == 7.5 and r["dw1"][0, 0] == 11.25
    # down_mult 2: dpre = 15, a tie between 14 and 16 (steps of 2 in [8, 16)) -> 16
    r = _one_unit(2.6, 1.0, 2.0)
    assert r["dx"][0, 0] == 16.0 and r["dw1"][0, 0] == 24.0 and r["dw2"][0, 0] == 11.25


def test_exact_quantization_equals_plain_backward():
    """Operands chosen so that dout, dpre and relu(pre)^2 all lie on their fp8 grids: then the fp8
    backward is the plain backward of the dequantized operands."""
    f = np.float32
    x = np.array([[1.0, 0.5], [2.0, 1.0]])
    w1 = np.array([[1.0, 1.0], [0.5, -1.0]])
    w2 = np.array([[1.0, 2.0], [0.5, 1.0]])
    dout = np.array([[1.0, 2.0], [0.5, -1.0]])
    # pre = [[1.5, 0], [3, 0]], post = [[2.25, 0], [9, 0]], dpre = [[6, 0], [0, 0]]
    r = oracle.relu_sq_fp8_backward_e5m2(dout, _e4m3_codes(x), f(1.0), _e4m3_codes(w1), f(1.0),
                                         _e4m3_codes(w2), f(1.0), f(1.0), f(1.0), f(1.0))
    ref = oracle.relu_sq_backward(dout, x, w1, w2)
    np.testing.assert_array_equal(r["dpre"], [[6.0, 0.0], [0.0, 0.0]])
    for k in ("dx", "dw1", "dw2"):
        np.testing.assert_array_equal(r[k], ref[k])


@pytest.mark.parametrize("dm", [1.0, 2.0])
def test_within_rounding_bound_of_exact_backward(dm):
    """Each e5m2 value is within 2^-3 of its input (relative; plus half the smallest subnormal
    step absolute), each e4m3 value within 2^-4 (plus 2^-10). Propagating those bounds through
    the products with absolute values bounds the distance to the exact backward."""
    rng = np.random.default_rng(11)
    M, D, H = 24, 32, 48
    f = np.float32
    x = rng.standard_normal((M, D))
    w1 = rng.uniform(-1, 1, (H, D)) / np.sqrt(D)
    w2 = rng.uniform(-1, 1, (D, H)) / np.sqrt(H)
    dout = rng.standard_normal((M, D))
    x_q, s_x = oracle.quantize_per_tensor(x)
    w1_q, s_w1 = oracle.quantize_per_tensor(w1)
    w2_q, s_w2 = oracle.quantize_per_tensor(w2)
    xh, w1h, w2h = (oracle.dequantize(q, s) for q, s in ((x_q, s_x), (w1_q, s_w1), (w2_q, s_w2)))
    exact = oracle.relu_sq_backward(dout, xh, w1h, w2h, dm)
    s_grad = f(2.0 ** -6)
    s_dpre = f(np.max(np.abs(exact["dpre"])) * 1.25 / 57344.0)
    s_post = f(np.max(exact["post"]) * 1.03 / 448.0)
    r = oracle.relu_sq_fp8_backward_e5m2(dout, x_q, s_x, w1_q, s_w1, w2_q, s_w2, s_post, s_grad, s_dpre, dm)
    pre = xh @ w1h.T
    dr = 2.0 * np.maximum(pre, 0.0)
    g_err = 2.0 ** -3 * np.abs(dout) + 2.0 ** -17 * s_grad
    ghat = oracle.e5m2_decode(r["dout_q"]) * np.float64(s_grad)
    dpre_g = (dm * (ghat @ w2h)) * dr                      # dpre from the rounded dout
    dpre_err = (2.0 ** -3 * np.abs(dpre_g) + 2.0 ** -17 * s_dpre) + abs(dm) * (g_err @ np.abs(w2h)) * dr
    post = np.maximum(pre, 0.0) ** 2
    post_err = 2.0 ** -4 * post + 2.0 ** -10 * s_post
    slack = 1e-9
    assert np.all(np.abs(r["dx"] - exact["dx"]) <= dpre_err @ np.abs(w1h) + slack)
    assert np.all(np.abs(r["dw1"] - exact["dw1"]) <= dpre_err.T @ np.abs(xh) + slack)
    dw2_err = abs(dm) * (g_err.T @ (post + post_err) + np.abs(dout).T @ post_err)
    assert np.all(np.abs(r["dw2"] - exact["dw2"]) <= dw2_err + slack)
    # the quantizations do change the result, and the recorded amax is that of the exact dpre
    # of the rounded dout
    assert np.max(np.abs(r["dx"] - exact["dx"])) > 0
    assert r["dpre_amax"] == np.max(np.abs(dpre_g))


def test_dpre_scale_rule_from_page_constants():
    """The delayed dpre scale uses the same refresh rule as the post scale with gain
    FP8_DPRE_HEADROOM / 57344 and floor 1e-12."""
    with open(os.path.join(GOLDEN, "page_constants.json")) as fh:
        c = json.load(fh)
    gain = np.float32(c["fp8_dpre_headroom"]["value"]) / np.float32(c["e5m2_max"]["value"])
    floor = c["dpre_scale_floor"]["value"]
    assert oracle.next_delayed_scale(57344.0, 1.0, gain, floor) == np.float32(np.float32(57344.0) * gain)
    assert oracle.next_delayed_scale(0.0, 0.25, gain, floor) == np.float32(0.25)
    assert c["fp8_grad_scale"]["value"] == 2.0 ** -6


def test_sampled_backward_equals_full():
    rng = np.random.default_rng(5)
    M, D, H = 40, 32, 48
    x = rng.standard_normal((M, D))
    w1 = rng.uniform(-1, 1, (H, D)) / np.sqrt(D)
    w2 = rng.uniform(-1, 1, (D, H)) / np.sqrt(H)
    dout = rng.standard_normal((M, D))
    q = [oracle.quantize_per_tensor(v) for v in (x, w1, w2)]
    args = (dout, q[0][0], q[0][1], q[1][0], q[1][1], q[2][0], q[2][1], np.float32(0.01), np.float32(2.0 ** -6),
            np.float32(0.002))
    full = oracle.relu_sq_fp8_backward_e5m2(*args, down_mult=2.0)
    rows, units = np.array([0, 7, 39]), np.array([1, 20, 47])
    smp = oracle.relu_sq_fp8_backward_e5m2_sampled(*args, rows, units, down_mult=2.0)
    np.testing.assert_allclose(smp["dx_rows"], full["dx"][rows], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(smp["dw1_rows"], full["dw1"][units], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(smp["dw2_cols"], full["dw2"][:, units], rtol=1e-12, atol=1e-14)
