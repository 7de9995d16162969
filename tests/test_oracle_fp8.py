"""Pins of the oracle's e4m3 codec, per-tensor quantizer, delayed-scale rule and fp8 forward
(CPU only). The codec is checked against torch's ``float8_e4m3fn`` conversion (an independent
implementation of the same OCP format) on every code and on every rounding midpoint."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_encode(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(v32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = oracle.e4m3_decode(codes), _torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and set(codes[nan]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(ours[~nan], ref[~nan])


def test_known_codes():
    dec = oracle.e4m3_decode
    assert dec(0x7E) == 448.0 and dec(0xFE) == -448.0
    assert dec(0x01) == 2.0 ** -9 and dec(0x08) == 2.0 ** -6 and dec(0x07) == 7 * 2.0 ** -9
    assert dec(0x38) == 1.0 and dec(0x30) == 0.5 and dec(0x00) == 0.0
    assert oracle.E4M3_MAX == 448.0


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    np.testing.assert_array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_midpoints_round_to_even_and_match_torch():
    grid = oracle.e4m3_grid()
    mids = (grid[:-1] + grid[1:]) / 2                       # exact in float32
    for sign in (1.0, -1.0):
        v = (sign * mids).astype(np.float32)
        ours = oracle.e4m3_encode(v)
        assert np.all((ours & 0x7F) % 2 == 0)               # even mantissa
        np.testing.assert_array_equal(ours, _torch_encode(v))
        # just above / below a midpoint goes to the nearer neighbour
        up = np.nextafter(v, np.float32(sign * np.inf))
        dn = np.nextafter(v, np.float32(0.0))
        np.testing.assert_array_equal(oracle.e4m3_encode(up), _torch_encode(up))
        np.testing.assert_array_equal(oracle.e4m3_encode(dn), _torch_encode(dn))


def test_random_values_match_torch_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.1, 1.0, 30.0, 150.0)]).astype(np.float32)
    v = v[np.abs(v) <= 464.0]        # torch maps values that round beyond 448 to NaN
    np.testing.assert_array_equal(oracle.e4m3_encode(v), _torch_encode(v))


def test_saturation_nan_and_signed_zero():
    v = np.array([448.0, 449.0, 464.0, 480.0, 1e6, np.inf, -np.inf, -500.0, np.nan, -0.0, -1e-9, 1e-9],
                 dtype=np.float32)
    codes = oracle.e4m3_encode(v)
    assert list(codes[:8]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert codes[8] & 0x7F == 0x7F
    assert list(codes[9:]) == [0x80, 0x80, 0x00]


def test_per_tensor_scale_rule():
    # amax = 448 * 2^k gives the scale 2^k exactly, and on-grid values quantize exactly
    rng = np.random.default_rng(2)
    grid = oracle.e4m3_grid()
    for k in (-6, -1, 0, 3):
        vals = rng.choice(grid, size=500) * rng.choice([-1.0, 1.0], size=500)
        vals[0] = 448.0
        v = (vals * 2.0 ** k).astype(np.float32)
        q, s = oracle.quantize_per_tensor(v)
        assert s == np.float32(2.0 ** k)
        np.testing.assert_array_equal(oracle.dequantize(q, s), v.astype(np.float64))
    # scale is max(amax, 1e-12) / 448 in float32 division
    v = np.array([0.3, -1.7, 0.01], dtype=np.float32)
    assert oracle.per_tensor_scale(v) == np.float32(np.float32(1.7) / np.float32(448.0))
    assert oracle.per_tensor_scale(np.zeros(4, np.float32)) == np.float32(np.float32(1e-12) / np.float32(448.0))
    q, _ = oracle.quantize_per_tensor(np.zeros(4, np.float32))
    assert np.all(q == 0)
    # the largest magnitude always lands on +-448
    q, s = oracle.quantize_per_tensor(np.array([0.5, -3.25, 1.0], np.float32))
    assert q[1] == 0xFE


def test_delayed_scale_rule():
    gain = 1.03 / 448.0
    f32 = np.float32
    assert oracle.next_delayed_scale(100.0, 0.5, gain, 1e-6) == f32(f32(100.0) * f32(gain))
    # zero / NaN / inf amax keep the previous scale
    for a in (0.0, float("nan"), float("inf"), float("-inf")):
        assert oracle.next_delayed_scale(a, 0.5, gain, 1e-6) == f32(0.5)
    # tiny amax floors, huge amax clamps at 1e12 before the gain
    assert oracle.next_delayed_scale(1e-20, 0.5, gain, 1e-6) == f32(1e-6)
    assert oracle.next_delayed_scale(1e30, 0.5, gain, 1e-6) == f32(f32(1e12) * f32(gain))


def test_fp8_forward_reduces_to_bf16_on_grid_inputs():
    """With inputs on the e4m3 grid and power-of-two scales, quantizing is the identity, so the
    fp8 forward equals the plain forward on the same values."""
    rng = np.random.default_rng(6)
    grid = oracle.e4m3_grid()
    M, d, H = 9, 16, 24

    def on_grid(shape, k):
        v = rng.choice(grid[:100], size=shape) * rng.choice([-1.0, 1.0], size=shape)
        v.flat[0] = 448.0
        return (v * 2.0 ** k).astype(np.float32)

    x, w1, w2 = on_grid((M, d), -5), on_grid((H, d), -9), on_grid((d, H), -9)
    (xq, sx), (w1q, s1), (w2q, s2) = (oracle.quantize_per_tensor(a) for a in (x, w1, w2))
    f8 = oracle.relu_sq_fp8_forward(xq, sx, w1q, s1, w2q, s2)
    ref = oracle.relu_sq_forward(x, w1, w2)
    np.testing.assert_array_equal(f8["out"], ref["out"])
    np.testing.assert_array_equal(f8["pre"], ref["pre"])
    # quantizing post with a scale that does not saturate moves each post by at most half an
    # e4m3 step: 2^-4 relative in the normal range, 2^-10 * s_post in the subnormal one
    s_post = 2.0 ** np.ceil(np.log2(ref["post"].max() / 448.0))
    f8p = oracle.relu_sq_fp8_forward(xq, sx, w1q, s1, w2q, s2, s_post=s_post)
    bound = (2.0 ** -4 * ref["post"] + 2.0 ** -10 * s_post) @ np.abs(w2.astype(np.float64)).T
    assert np.all(np.abs(f8p["out"] - ref["out"]) <= bound * (1 + 1e-12))
    assert np.any(f8p["out"] != ref["out"])
    dout = rng.standard_normal((M, d))
    b8 = oracle.relu_sq_fp8_backward(dout, xq, sx, w1q, s1, w2q, s2)
    b = oracle.relu_sq_backward(dout, x, w1, w2)
    for k in ("dx", "dw1", "dw2"):
        np.testing.assert_array_equal(b8[k], b[k])


def test_page_constants():
    """Constants the pages print, kept as a cited fixture."""
    with open(os.path.join(GOLDEN, "page_constants.json")) as f:
        c = json.load(f)
    assert oracle.E4M3_MAX == c["e4m3_max"]["value"] == torch.finfo(torch.float8_e4m3fn).max
    assert c["e5m2_max"]["value"] == torch.finfo(torch.float8_e5m2).max
    # the static x scale 2^-4 cannot saturate an RMS-normed 768-wide row: sqrt(768) < 448 * 2^-4
    assert np.sqrt(c["gpt_model_dim"]["value"]) < c["e4m3_max"]["value"] * c["fp8_mlp_x_scale"]["value"]
    assert round(float(np.sqrt(c["gpt_model_dim"]["value"])), 1) == c["sqrt_model_dim_printed"]["value"]
    assert c["fp8_post_headroom"]["value"] == 1.03 and c["multiplier_default"]["value"] == 1.0


def test_weight_scale_bootstrap_then_delayed_by_hand():
    """Exact weight scales for the first 16 calls, then the previous call's amax (gpt.py
    FP8_EXACT_SCALE_CALLS = 16, _quantize_mlp_weights_and_scales). B has amax 1.75 = 448 * 2^-8, so
    c * B has the exact scale c * 2^-8 and the codes below follow from the OCP E4M3 table by hand:
    448 -> 0x7E, 128 -> 0x70, -64 -> 0xE8, 256 -> 0x78, -128 -> 0xF0, 0 -> 0x00."""
    with open(os.path.join(GOLDEN, "page_constants.json")) as fh:
        n_exact = int(json.load(fh)["fp8_exact_scale_calls"]["value"])
    assert n_exact == 16
    B = np.array([[1.75, 0.5], [-0.25, 0.0]])
    c = [1.0] * 16 + [2.0, 2.0, 0.5]             # the weights double at call 16, halve at call 18
    res = oracle.weight_quantize_calls([ci * B for ci in c], exact_calls=n_exact)
    base = np.array([[0x7E, 0x70], [0xE8, 0x00]], dtype=np.uint8)
    for t in range(16):                           # exact: scale 2^-8, B / 2^-8 = [[448, 128], [-64, 0]]
        assert res[t][1] == np.float32(2.0 ** -8)
        np.testing.assert_array_equal(res[t][0], base)
    # call 16: delayed scale from call 15's amax (1.75 -> 2^-8); 2B / 2^-8 = [[896, 256], [-128, 0]]:
    # 896 saturates to 448
    assert res[16][1] == np.float32(2.0 ** -8)
    np.testing.assert_array_equal(res[16][0], np.array([[0x7E, 0x78], [0xF0, 0x00]], dtype=np.uint8))
    # call 17: call 16's amax was 3.5 -> scale 2^-7; 2B / 2^-7 = [[448, 128], [-64, 0]]
    assert res[17][1] == np.float32(2.0 ** -7)
    np.testing.assert_array_equal(res[17][0], base)
    # call 18: B/2 quantized with call 17's scale 2^-7: [[112, 32], [-16, 0]]: 112 = 2^6 * 1.75 -> exponent
    # field 6 + 7 = 13, mantissa 6 -> (13 << 3) | 6 = 0x6E,
    # 32 = 2^5 -> 0x60, -16 = -2^4 -> 0xD8
    assert res[18][1] == np.float32(2.0 ** -7)
    np.testing.assert_array_equal(res[18][0], np.array([[0x6E, 0x60], [0xD8, 0x00]], dtype=np.uint8))
    # the codes decode to what the hand arithmetic says
    np.testing.assert_array_equal(oracle.e4m3_decode(res[18][0]) * 2.0 ** -7, np.array([[0.875, 0.25], [-0.125, 0.0]]))


def test_weight_scale_exact_calls_equal_per_tensor_quantizer():
    """Every exact call is the per-tensor quantizer, and a delayed call with unchanged weights is too."""
    rng = np.random.default_rng(3)
    ws = [rng.uniform(-0.05, 0.05, (24, 40)) * (1 + 0.1 * t) for t in range(4)]
    res = oracle.weight_quantize_calls(ws, exact_calls=2)
    for t in range(2):
        q, sc = oracle.quantize_per_tensor(ws[t])
        assert res[t][1] == sc
        np.testing.assert_array_equal(res[t][0], q)
    # call 2 uses call 1's amax: the scale is per_tensor_scale(ws[1]) and ws[2] (10 % larger) saturates
    assert res[2][1] == oracle.per_tensor_scale(ws[1])
    assert np.any(oracle.e4m3_decode(res[2][0]) == 448.0) or np.any(oracle.e4m3_decode(res[2][0]) == -448.0)
    same = oracle.weight_quantize_calls([ws[0], ws[0], ws[0]], exact_calls=1)
    for codes, sc in same:
        np.testing.assert_array_equal(codes, same[0][0])
        assert sc == same[0][1]
