"""GPU test of the fp8 weight-cache quantizer (mlp_quantize_weight_e4m3) over a sequence of calls,
through the C ABI, against the oracle's (modded-nanogpt gpt.py, FP8_EXACT_SCALE_CALLS and
_quantize_mlp_weights_and_scales): exact scales for the first 16 calls, then the amax the previous
call recorded per tile. Codes (row-major and transposed) and scales are compared bit for bit on
every call, including the call where the weights grow past the delayed scale and saturate."""
import numpy as np
import pytest
import torch

import gated_mlp_gemms_amd as gm
import oracle
from gpu_helpers import announce

pytestmark = pytest.mark.gpu

EXACT = 16
FACTORS = [1.0] * 15 + [1.03, 2.0, 2.0, 0.75]   # call 16 (2.0) exceeds call 15's amax by ~2x


@pytest.mark.parametrize("rows,cols", [(3072, 768), (300, 208)])
def test_weight_quantizer_calls_bit_exact(rows, cols):
    announce(f"weight quantizer over {len(FACTORS)} calls, {rows}x{cols}")
    rng = np.random.default_rng(rows + cols)
    w0 = rng.uniform(-1.0, 1.0, (rows, cols)) / np.sqrt(cols)
    ws = [torch.from_numpy((c * w0).astype(np.float32)).to(torch.bfloat16) for c in FACTORS]
    ref = oracle.weight_quantize_calls([w.to(torch.float32).numpy() for w in ws], exact_calls=EXACT)
    ld_t = (rows + 15) // 16 * 16
    scale = torch.zeros(1, dtype=torch.float32, device="cuda")
    tiles = torch.zeros(gm.mlp_weight_amax_slots(rows, cols), dtype=torch.float32, device="cuda")
    assert tiles.numel() == ((rows + 127) // 128) * ((cols + 127) // 128)
    dst = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    dst_t = torch.full((cols, ld_t), 0xAB, dtype=torch.uint8, device="cuda")
    saturated = 0
    for t, w in enumerate(ws):
        wd = w.cuda()
        gm.mlp_quantize_weight_e4m3(wd, t < EXACT, scale, tiles, dst=dst, dst_t=dst_t, ld_t=ld_t)
        torch.cuda.synchronize()
        codes, sc = ref[t]
        assert np.float32(scale.item()) == sc, (t, scale.item(), sc)
        np.testing.assert_array_equal(dst.cpu().numpy(), codes, err_msg=f"call {t}")
        d_t = dst_t.cpu().numpy()
        np.testing.assert_array_equal(d_t[:, :rows], codes.T, err_msg=f"call {t} transposed")
        assert np.all(d_t[:, rows:] == 0)
        # the record this call leaves is w's amax per tile
        assert float(tiles.max().item()) == float(np.max(np.abs(w.to(torch.float32).numpy())))
        saturated += int(np.sum((codes & 0x7F) == 0x7E))
    # the sequence does exercise the delayed scale's saturation (call 16 and 17 at 2x)
    assert saturated > 0


def _midpoints(grid):
    g = np.unique(np.abs(grid[np.isfinite(grid)]))
    return (g[:-1] + g[1:]) / 2.0


@pytest.mark.parametrize("amax_frac", [0.731, 0.9999, 0.37, 1.0])
def test_per_tensor_quantizer_at_rounding_midpoints(amax_frac):
    """Quotients v / scale placed at and within a few fp32 ulps of every e4m3 rounding midpoint (and
    at the saturation edge): the GPU codes equal the oracle's, whose quotient is one IEEE fp32
    division."""
    announce(f"e4m3 quantizer at rounding midpoints, amax {amax_frac} * 448")
    amax = np.float32(448.0 * amax_frac)
    s = np.float32(max(amax, np.float32(1e-12)) / np.float32(448.0))
    mids = _midpoints(oracle.e4m3_grid())
    base = (mids.astype(np.float64) * np.float64(s)).astype(np.float32)
    vals = [base]
    for k in range(1, 5):
        up, dn = base.copy(), base.copy()
        for _ in range(k):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(0))
        vals += [up, dn]
    v = np.concatenate(vals)
    v = np.concatenate([v, -v, [amax, -amax * np.float32(0.999)]]).astype(np.float32)
    v = v[np.abs(v) <= amax]
    pad = (-len(v)) % 8
    v = np.concatenate([v, np.zeros(pad, np.float32)])
    src = torch.from_numpy(v).cuda()
    dst = torch.empty(len(v), dtype=torch.uint8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(int(gm.mlp_quantize_workspace_bytes()), dtype=torch.uint8, device="cuda")
    gm.mlp_quantize_e4m3(src, dst, sc, ws)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_per_tensor(v)
    assert np.float32(sc.item()) == s_ref
    np.testing.assert_array_equal(dst.cpu().numpy(), q_ref)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("relu_sq", [False, True])
def test_2d_quantizer_every_bf16_value(fmt, relu_sq):
    """Every finite bf16 value, quantized with three scales (one a power of two): the codes equal
    the oracle's encoder of the fp32 quotient."""
    announce(f"2-D quantizer over all finite bf16 values, {fmt}, relu_sq={relu_sq}")
    bits = np.arange(65536, dtype=np.uint32)
    f = (bits << 16).view(np.float32)
    f = f[np.isfinite(f)]
    f = f[: len(f) // 16 * 16].reshape(-1, 16)
    src = torch.from_numpy(f).to(torch.bfloat16)
    assert torch.equal(src.to(torch.float32), torch.from_numpy(f))
    for scale in (np.float32(0.37), np.float32(2.0 ** -5), np.float32(3.3e-3)):
        sc = torch.tensor([scale], dtype=torch.float32, device="cuda")
        dst = torch.empty(f.shape, dtype=torch.uint8, device="cuda")
        gm.mlp_quantize_fp8(src.cuda(), fmt, sc, dst=dst, relu_sq=relu_sq)
        torch.cuda.synchronize()
        x = f
        if relu_sq:
            m = np.maximum(x, np.float32(0.0))
            x = m * m
        y = x / scale
        ref = oracle.e5m2_encode(y) if fmt == "e5m2" else oracle.e4m3_encode(y)
        np.testing.assert_array_equal(dst.cpu().numpy(), ref, err_msg=f"scale {scale}")
