"""GPU test of mlp_fwd_infer_noalloc (the inference forward on the library's static per-GPU
scratch) through the C ABI: its output equals mlp_fwd_infer's (caller workspace) bit for bit, on
two calls in a row, the second with a smaller problem, for the LLaMA MLP at 64 tokens (whose up
projection runs split along K into fp32 partials held in the scratch) then 16 (the small-M
kernel), a ragged SwiGLU problem, a ReLU^2 problem and the e4m3 forward."""
import pytest
import torch

import gated_mlp_gemms_amd as gm
from gpu_helpers import announce
from workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _pair(w, t, fp8=False):
    """(mlp_fwd_infer out, mlp_fwd_infer_noalloc out) for workload w."""
    from gated_mlp_gemms_amd.runner import runner_for

    r = runner_for(w, t)
    if fp8:
        r.quantize()
    r.forward_infer()
    ref = r.out_infer.clone()
    out = torch.full_like(ref, float("nan"))
    gm.mlp_fwd_infer_noalloc(r.desc, r.x, r.w_gate, r.w_up, r.w_down, out, r.fp8_args)
    torch.cuda.synchronize()
    return ref, out


CASES = [
    # (act, M_first, M_second, d, H, d_out, extra)
    ("swiglu", 64, 16, 4096, 11008, 4096, {}),
    ("swiglu", 300, 100, 264, 712, 200, {"gate_mult": 1.125, "down_mult": 2.0}),
    ("relu_sq", 200, 64, 256, 704, 208, {}),
    ("relu_sq", 129, 16, 768, 3072, 768, {"fp8_fwd": True}),
]


@pytest.mark.parametrize("act,m1,m2,d,H,do,extra", CASES)
def test_noalloc_matches_workspace_entry(act, m1, m2, d, H, do, extra):
    for M in (m1, m2):
        w = Workload(f"noalloc_{act}_m{M}_d{d}_h{H}_o{do}", act, "bf16", (M,), d, H, do, **extra)
        announce(w.name)
        desc = gm.make_desc(M, d, H, do, act, torch.bfloat16, fp8_fwd=extra.get("fp8_fwd", False))
        assert gm.workspace_bytes(desc, "fwd_infer") <= gm.MLP_NOALLOC_SCRATCH_BYTES
        ref, out = _pair(w, make_inputs(w), fp8=extra.get("fp8_fwd", False))
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(out, ref), f"{w.name}: noalloc differs from mlp_fwd_infer"


def test_noalloc_rejects_beyond_scratch():
    """A problem whose inference workspace exceeds the scratch is refused before any launch and
    leaves out untouched."""
    M, d, H = 3000, 4096, 11008
    desc = gm.make_desc(M, d, H, d, "swiglu", torch.bfloat16)
    assert gm.workspace_bytes(desc, "fwd_infer") > gm.MLP_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(M, d, dtype=torch.bfloat16, device="cuda")
    wg = torch.zeros(H, d, dtype=torch.bfloat16, device="cuda")
    wd = torch.zeros(d, H, dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, d), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gm.MlpError, match="MLP_NOALLOC_SCRATCH_BYTES"):
        gm.mlp_fwd_infer_noalloc(desc, x, wg, wg, wd, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
