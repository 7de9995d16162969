#!/usr/bin/env python3
"""Throughput of one fused SwiGLU MLP training step (forward + backward) on one MI355X.

A step is ``mlp_fwd`` (training: g|u saved) followed by ``mlp_bwd`` (dx, dW_gate, dW_up,
dW_down) of the LLaMA-shaped MLP: x [2, 1024, 4096] (M = 2048 tokens), W_gate/W_up
[11008, 4096], W_down [4096, 11008], bf16 storage, fp32 accumulation. Inputs are synthetic
(``workloads.py``) and resident in HBM before timing starts.

Prints one JSON line: TFLOP/s on the model FLOP count 18*M*d*H (2*M*N*K per GEMM), the
fraction of the bf16 MFMA peak, the roofline of the slowest kernel stage (timed with HIP events
on the library's stream inside the timed region; priced at the dense peak of that stage's operand
type: bf16, fp32, or fp8 for the e4m3 / e5m2 products of the fp8 workloads), and the float64
oracle's throughput on a bounded sample on the host CPU.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (published)
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP32_TFLOPS = 157.3       # MI355X dense fp32 (published)
PEAK_HBM_GBS = 8000.0
METRIC = "fused SwiGLU MLP fwd+bwd TFLOP/s and % bf16 MFMA peak, 4096×11008, 2048 tok"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through the HIP runtime (the library records them on its stream)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")

    def create(self):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, ev):
        self.hip.hipEventDestroy(ev)


def host_info() -> dict:
    """This host's CPU: logical CPUs, the ones this process may run on, and the model name."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)), "cpu_model": model}


def device_info() -> dict:
    """The GPU the step ran on: name, architecture and compute-unit count (torch), the maximum
    shader clock and CU count rocminfo reports for the gfx agent, and the ROCm / HIP versions."""
    import subprocess

    import torch

    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "hip": torch.version.hip, "rocm": None, "max_sclk_mhz": None}
    try:
        with open("/opt/rocm/.info/version") as fh:
            info["rocm"] = fh.read().strip()
    except OSError:
        pass
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        for agent in out.split("Agent ")[1:]:
            if "gfx9" not in agent:
                continue
            for line in agent.splitlines():
                line = line.strip()
                if line.startswith("Max Clock Freq. (MHz):"):
                    info["max_sclk_mhz"] = int(line.split(":")[1].split()[0])
                elif line.startswith("Compute Unit:"):
                    info["rocminfo_cus"] = int(line.split(":")[1].split()[0])
            break
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    return info


def stage_flops(w, sched: int = 0) -> dict:
    """FLOP of each stage's products; `sched` is the library's backward schedule (mlp_bwd_grouped
    flags: 1 = dx and the weight gradients left as one launch, 2 = dW_down with the d-activation
    GEMM)."""
    M, D, H, O = w.M, w.d_in, w.hidden, w.d_out
    P = 2 * H if w.gated else H
    f = {
        "up": 2.0 * M * D * P, "down": 2.0 * M * H * O, "dact": 2.0 * M * O * H,
        "dw_down": 2.0 * O * H * M, "dx": 2.0 * M * P * D, "dw_up": 2.0 * P * D * M,
        "recompute": 2.0 * M * D * P,
    }
    with_dact = bool(sched & 2)
    if with_dact:
        f["dact"] += f["dw_down"]
    f["bwd_gemms"] = f["dx"] + f["dw_up"] + (0.0 if with_dact else f["dw_down"])
    return f


def bwd_stages(sched: int) -> list:
    """The backward's stages after the d-activation GEMM for a schedule (see stage_flops)."""
    if sched & 1:
        return ["bwd_gemms"]
    return ([] if sched & 2 else ["dw_down"]) + ["dx", "dw_up"]


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` from the committed PMC summary of this workload, if the
    kernel sources are the ones the counters were taken on (else None)."""
    from gated_mlp_gemms_amd.profile_summary import kernel_sources_sha256

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None, None
    rec = json.load(open(path))
    if rec.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None, f"{os.path.basename(path)} (stale: kernels changed since)"
    st = rec.get("stages", {}).get(stage)
    return (st["traffic_bytes"] if st else None), os.path.basename(path)


def vendor_gemm_reference(w, tensors, reps: int = 20) -> dict:
    """The same six matrix products timed through torch.matmul (hipBLASLt on ROCm): operands in
    the layouts this engine reads, plain bf16 outputs, no activation, no epilogue and no
    elementwise kernels. Context only: it times a different, unfused computation."""
    import torch

    dev = "cuda"
    x = tensors["x"].to(dev)
    dout = tensors["dout"].to(dev)
    if w.gated:
        w_in = torch.cat([tensors["w_gate"], tensors["w_up"]]).to(dev)    # [2H, d]
        w_out = tensors["w_down"].to(dev)
    else:
        w_in, w_out = tensors["w1"].to(dev), tensors["w2"].to(dev)
    P = w_in.shape[0]
    act = torch.randn(w.M, w.hidden, device=dev, dtype=x.dtype)
    dpre = torch.randn(w.M, P, device=dev, dtype=x.dtype)
    cases = {"up": lambda: x @ w_in.t(), "down": lambda: act @ w_out.t(), "dact": lambda: dout @ w_out,
             "dw_down": lambda: dout.t() @ act, "dx": lambda: dpre @ w_in, "dw_up": lambda: dpre.t() @ x}
    res = {}
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for k, fn in cases.items():
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        res[k] = round(1e3 * a.elapsed_time(b) / reps, 2)
    res["sum"] = round(sum(res.values()), 2)
    return res


def decode_latency(w, tensors, tokens: int, reps: int = 50) -> dict:
    """Inference forward at decode size (`tokens` rows of x, the workload's weights): average time
    per call launched eagerly from Python and replayed from a captured HIP graph, and the weight
    bytes per call over the graph time (a decode step reads every weight once)."""
    import torch
    from gated_mlp_gemms_amd.runner import runner_for

    wd = w.replace(batch=(tokens,), grad_accum=False)
    td = {k: v for k, v in tensors.items() if not k.startswith("dw")}
    td["x"] = tensors["x"][:tokens].clone()
    td["dout"] = tensors["dout"][:tokens].clone()
    r = runner_for(wd, td)
    if w.fp8_fwd:
        r.quantize()
    for _ in range(3):
        r.forward_infer()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        r.forward_infer()
    b.record()
    torch.cuda.synchronize()
    eager_us = 1e3 * a.elapsed_time(b) / reps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        r.forward_infer()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r.forward_infer()
    g.replay()
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    graph_us = 1e3 * a.elapsed_time(b) / reps
    wbytes = (w.hidden * w.d_in * (2 if w.gated else 1) + w.d_out * w.hidden) * (1 if w.fp8_fwd else w.elem_bytes)
    del g, r
    return {"tokens": tokens, "eager_us": round(eager_us, 2), "graph_us": round(graph_us, 2),
            "weight_bytes": wbytes, "weight_GBps": round(wbytes / (graph_us * 1e-6) / 1e9, 1)}


def cpu_baseline(w, tensors, rows: int) -> dict:
    """The float64 oracle (as it stands) on the first `rows` tokens of the workload, all of d
    and H: forward + backward, timed on this host's cores."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle

    f64 = lambda t: t[:rows].to(torch.float64).numpy() if t.shape[0] == w.M else t.to(torch.float64).numpy()  # noqa: E731
    a = {k: f64(v) for k, v in tensors.items()}
    t0 = time.perf_counter()
    if w.gated:
        oracle.gated_forward(a["x"], a["w_gate"], a["w_up"], a["w_down"], w.gate_mult, w.down_mult)
        oracle.gated_backward(a["dout"], a["x"], a["w_gate"], a["w_up"], a["w_down"], w.gate_mult, w.down_mult)
    else:
        oracle.relu_sq_forward(a["x"], a["w1"], a["w2"], w.down_mult)
        oracle.relu_sq_backward(a["dout"], a["x"], a["w1"], a["w2"], w.down_mult)
    secs = time.perf_counter() - t0
    sample = w.replace(batch=(rows,))
    threads = sum(p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas") or 1
    host = host_info()
    return {"value": round(sample.model_flops() / secs / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(secs, 3), "cores_meaning": "BLAS threads the oracle's matmuls ran on",
            "host_nproc": host["nproc"], "host_usable_cpus": host["usable_cpus"], "cpu_model": host["cpu_model"],
            "sample": f"first {rows} of {w.M} tokens, full d={w.d_in} H={w.hidden}: float64 numpy forward + "
                      f"backward ({sample.model_flops() / 1e9:.1f} GFLOP on the model count)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="workload name (default: the headline one)")
    ap.add_argument("--cpu-rows", type=int, default=2048, help="tokens in the oracle's CPU sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-tokens", type=int, default=16,
                    help="also time the inference forward at this many tokens, eager and from a graph (0: skip)")
    ap.add_argument("--vendor-gemm-reference", action="store_true",
                    help="also time the six plain GEMMs through torch.matmul (hipBLASLt), for context")
    ap.add_argument("--save-act", choices=("workload", "on", "off"), default="workload",
                    help="keep the activation from the forward for the backward (mlp_desc.save_act): as the "
                         "workload says, or forced on / off")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before warmup (a known-size "
                         "reference for profiler byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this engine is single-GPU "
              "and has no multi-GPU path to time.", file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_mlp_gemms_amd as gm
    from gated_mlp_gemms_amd.runner import runner_for
    from workloads import HEADLINE, WORKLOADS, make_inputs

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    w = WORKLOADS[args.workload or HEADLINE]
    if args.save_act != "workload":
        w = w.replace(save_act=args.save_act == "on")
    log(f"[bench] workload {w.name}: building inputs")
    tensors = make_inputs(w)
    r = runner_for(w, tensors)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        if w.fp8_fwd:
            r.quantize()
            r.forward()
            r.refresh_post_scale()
            r.backward()
            if w.fp8_bwd:
                r.refresh_dpre_scale()
        else:
            r.step()
        r.reset_grads()
    torch.cuda.synchronize()

    ev = HipEvents()
    # the library groups backward GEMMs into one launch when its planner prefers that
    sched = gm.mlp_bwd_grouped(r.desc)
    stages = ["up", "down", "dact"] + bwd_stages(sched) + (["recompute"] if w.recompute else [])
    stage_id = {n: gm._lib.STAGES.index(n) for n in stages}

    def run_steps(hooked):
        """K steps with HIP event pairs around the `hooked` stages (recorded by the library on
        its stream) and one torch event at every step boundary (the same stream); returns the
        event pairs, the average ms per step, the K per-step times and the wall time."""
        pairs = [[(ev.create(), ev.create()) for _ in hooked] for _ in range(args.steps)]
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        marks[0].record()
        for i in range(args.steps):
            for n, (b, e) in zip(hooked, pairs[i]):
                gm._lib.check(gm.lib().mlp_time_stage_once(stage_id[n], b, e), "mlp_time_stage_once")
            r.step()
            marks[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps)]
        return pairs, marks[0].elapsed_time(marks[-1]) / args.steps, per, wall

    def spread_of(per_step):
        v = sorted(per_step)
        q = lambda f: v[min(len(v) - 1, int(round(f * (len(v) - 1))))]  # noqa: E731
        return {"median": round(q(0.5), 4), "min": round(v[0], 4), "p90": round(q(0.9), 4),
                "mean": round(sum(v) / len(v), 4)}

    def avg_us(pairs, j):
        return 1e3 * sum(ev.elapsed_ms(*pairs[i][j]) for i in range(args.steps)) / args.steps

    # stage pass: every stage's events (each record adds a little queue work, so this pass is not
    # the one the headline is timed on)
    log(f"[bench] stage pass: {args.steps} steps with events around every stage")
    pairs, _, _, _ = run_steps(stages)
    sf = stage_flops(w, sched)
    stage_us, stage_tf = {}, {}
    for j, n in enumerate(stages):
        us = avg_us(pairs, j)
        stage_us[n] = round(us, 2)
        stage_tf[n] = round(sf[n] / (us * 1e-6) / 1e12, 1)
    fwd_us = round(stage_us["up"] + stage_us["down"], 2)
    bwd_us = round(sum(v for k, v in stage_us.items() if k not in ("up", "down")), 2)
    for row in pairs:
        for b, e in row:
            ev.destroy(b)
            ev.destroy(e)
    dom = max(stage_us, key=stage_us.get)

    # timed pass (the headline): events only around the dominant stage, whose average launch
    # duration in these steps gives the roofline's achieved rate
    log(f"[bench] timing {args.steps} steps (events around the {dom} stage)")
    pairs, ms, per_step, wall = run_steps([dom])
    spread = spread_of(per_step)
    dom_us = avg_us(pairs, 0)
    for row in pairs:
        for b, e in row:
            ev.destroy(b)
            ev.destroy(e)
    flops = w.model_flops()
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS
    traffic, traffic_src = measured_traffic(w.name, dom)
    # the dominant stage's product is priced at the peak of its own operand type
    fp8_stages = ({"up", "down", "recompute"} if w.fp8_fwd else set()) | \
        ({"dact", "dw_down", "dx", "dw_up"} if w.fp8_bwd else set())
    stage_peak = PEAK_FP8_TFLOPS if dom in fp8_stages else (PEAK_FP32_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS)
    dom_tf = round(sf[dom] / (dom_us * 1e-6) / 1e12, 1)
    roof = {"bound": "mfma", "achieved": dom_tf, "peak": stage_peak, "unit": "TFLOP/s",
            "frac": round(dom_tf / stage_peak, 4), "traffic": traffic, "kernel_stage": dom,
            "flop_per_launch": sf[dom], "avg_launch_us": round(dom_us, 2), "traffic_source": traffic_src}
    log(f"[bench] {ms:.3f} ms/step, {tflops:.1f} TFLOP/s ({100 * tflops / peak:.1f}% of bf16 peak); "
        f"stages us {stage_us}")

    # inference forward (no saved pre-activation), and the training step with cold caches: a
    # 512 MiB write between steps evicts the operands from L2 and the last-level cache
    n_side = max(1, min(args.steps, 20))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n_side):
        r.forward_infer()
    b.record()
    torch.cuda.synchronize()
    infer_us = round(1e3 * a.elapsed_time(b) / n_side, 2)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for _ in range(n_side):
        flush.fill_(1)
        a.record()
        r.step()
        b.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    cold_ms = round(sorted(cold)[len(cold) // 2], 4)
    log(f"[bench] timed steps: median {spread['median']} ms (min {spread['min']}, p90 {spread['p90']}); fwd {fwd_us} us, "
        f"bwd {bwd_us} us; inference fwd {infer_us} us; cold-cache step {cold_ms} ms")

    decode = None
    if args.decode_tokens > 0:
        decode = decode_latency(w, tensors, args.decode_tokens)
        log(f"[bench] decode {decode}")

    vendor = None
    if args.vendor_gemm_reference:
        vendor = vendor_gemm_reference(w, tensors)
        log(f"[bench] torch.matmul (hipBLASLt) on the six plain GEMMs: {vendor} us")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle on {args.cpu_rows} tokens")
        cpu = cpu_baseline(w, tensors, args.cpu_rows)
        log(f"[bench] oracle {cpu['seconds']} s, {cpu['value']} TFLOP/s on {cpu['cores']} threads")

    dev = device_info()
    log(f"[bench] device {dev}")
    from workloads import digest

    inputs_sha = {k: digest(v) for k, v in tensors.items()}
    dtype = ("fp8-e4m3 fwd / e5m2 x e4m3 bwd" if w.fp8_bwd else "fp8-e4m3 fwd / bf16 bwd") if w.fp8_fwd else w.dtype
    line = {
        "metric": METRIC if w.name == HEADLINE else f"MLP fwd+bwd TFLOP/s (model FLOP count), {w.name}",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "d_in": w.d_in, "hidden": w.hidden, "d_out": w.d_out,
                   "act": w.act, "gate_mult": w.gate_mult, "down_mult": w.down_mult,
                   "recompute": w.recompute, "grad_accum": w.grad_accum, "save_act": w.save_act,
                   "bwd_schedule": {"grouped": bool(sched & 1), "dw_down_with_dact": bool(sched & 2)},
                   "step": "mlp_fwd (training) + mlp_bwd (dx, all weight grads)",
                   "model_flop_per_step": flops, "pct_of_bf16_peak": round(100 * tflops / peak, 2),
                   "wall_s_timed": round(wall, 3)},
        "stages_us": stage_us, "stages_tflops": stage_tf,
        "step_ms": spread, "median_step_tflops": round(flops / (spread["median"] * 1e-3) / 1e12, 2), "fwd_us": fwd_us, "bwd_us": bwd_us,
        "infer_fwd_us": infer_us, "infer_fwd_tflops": round(w.model_flops() / 3 / (infer_us * 1e-6) / 1e12, 1),
        "cold_cache_ms_per_step": cold_ms, "decode": decode,
        "roofline": roof, "cpu_baseline": cpu,
        "device": dev, "host": host_info(), "inputs_sha256": inputs_sha,
    }
    if vendor is not None:
        line["vendor_gemms_us"] = vendor
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
