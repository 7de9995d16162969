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
