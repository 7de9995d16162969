"""CPU checks of bench.py's command line (no GPU use): it parses, and asking for more than one
GPU exits with a message instead of timing anything."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_help_lists_contract_flags():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def test_stage_flops_cover_the_step_under_every_schedule():
    """Whatever the backward schedule, the timed stages' FLOP add up to the model's count, each
    product counted once (dW_down inside the d-activation stage or the grouped stage)."""
    sys.path.insert(0, ROOT)
    import bench
    from workloads import WORKLOADS

    for name in ("llama_swiglu_bf16_m2048_d4096_h11008", "gpt_relu2_bf16_m49152_d768_h3072"):
        w = WORKLOADS[name]
        for sched in (0, 1, 2, 3):
            f = bench.stage_flops(w, sched)
            stages = ["up", "down", "dact"] + bench.bwd_stages(sched)
            assert abs(sum(f[s] for s in stages) - w.model_flops()) <= 1e-9 * w.model_flops(), (name, sched)
    assert bench.bwd_stages(0) == ["dw_down", "dx", "dw_up"]
    assert bench.bwd_stages(2) == ["dx", "dw_up"]
    assert bench.bwd_stages(1) == bench.bwd_stages(3) == ["bwd_gemms"]
