"""Summaries of rocprofv3 output for the bench step (kernel durations and HBM traffic per stage).

    python -m gated_mlp_gemms_amd.profile_summary trace  <kernel-trace dir> <out.txt>  --command "..."
    python -m gated_mlp_gemms_amd.profile_summary traffic <fetch dir> <write dir> <out.json> --command "..."
    python -m gated_mlp_gemms_amd.profile_summary mfma <pmc dir> <out.json> --command "..."
    python -m gated_mlp_gemms_amd.profile_summary counters <pmc dir> <out.json> --command "..."

The trace summary lists every kernel's dispatch count and average / total duration from the
`*_kernel_stats.csv` rocprofv3 writes with `--kernel-trace --stats --output-format csv`, then the
average duration of each step stage's kernels, from the per-dispatch `*_kernel_trace.csv`, over
the timed steps only (`--first-step`, `--steps`: the bench's warmup and step counts). A kernel
instantiation that serves two stages (the same GEMM shape class for dW_down and dW_gate/dW_up)
thus gets one average per stage, the figure the bench's per-stage HIP events measure.

The traffic summary reads two `--pmc` passes over the same command (FETCH_SIZE, then
WRITE_SIZE, both in KiB per dispatch) that also ran one plain device copy of known size
(`bench.py --copy-probe-mib N`): the copy's counters give the factors that turn each counter into
bytes. Each step's dispatches are assigned to the step's stages in launch order (a split-K reduce
belongs to the GEMM before it), and the per-stage bytes are averaged over the profiled steps. The
output records a SHA-256 of the kernel sources, so a reader can tell whether the kernels changed
since the counters were taken.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

_HERE = os.path.dirname(os.path.abspath(__file__))
STAGE_ORDER_GATED = ["up", "down", "dact", "dw_down", "dx", "dw_up"]
# the backward with activation recompute re-runs the up projection before the d-activation
STAGE_ORDER_RECOMPUTE = ["up", "down", "recompute", "dact", "dw_down", "dx", "dw_up"]
# Grouped launches (gemm_dma_group_kernel) of the backward: the d-activation GEMM with dW_down
# (first tile body with a d-activation epilogue; the "dact" stage then holds dW_down too), and
# dx with the weight gradients (first tile body with the store epilogue): one "bwd_gemms" stage
# in place of the dw_down / dx / dw_up left.
_GROUPED = ("dw_down", "dx", "dw_up")
GROUP_EPI = 100   # gemm_epilogue of a grouped launch: GROUP_EPI + its first body's epilogue
_GROUP_MANGLED = re.compile(r"gemm_dma_group_kernelI.*?Lb[01]ELb[01]ELi(\d)E")
_GROUP_DEMANGLED = re.compile(r"gemm_dma_group_kernel<[^,]+, \d+, \d+, \d+, [^,]+, (?:true|false), (?:true|false), (\d)")


def is_group(name: str) -> bool:
    return "gemm_dma_group_kernel" in name


def group_epilogue(name: str) -> int:
    """The epilogue of a grouped launch's first tile body (0 when the name does not say)."""
    m = _GROUP_MANGLED.search(name) or _GROUP_DEMANGLED.search(name)
    return int(m.group(1)) if m else 0


def grouped_order(stages: list[str], names) -> list[str]:
    """`stages` adjusted to the grouped launches among the dispatch names: dw_down dropped when
    it runs with the d-activation GEMM, and what is left of dw_down, dx and dw_up as one
    bwd_gemms stage when those run as one launch."""
    epis = {group_epilogue(n) for n in names if is_group(n)}
    out = [st for st in stages if not (st == "dw_down" and epis - {0})]
    if 0 not in epis:
        return out
    res = []
    for st in out:
        if st in _GROUPED:
            if "bwd_gemms" not in res:
                res.append("bwd_gemms")
        else:
            res.append(st)
    return res


_BLOCK_COMMENT = re.compile(r"/\*.*?\*/", re.S)
_LINE_COMMENT = re.compile(r"//[^\n]*")


def code_text(src: str) -> str:
    """A C++ source with its comments and blank or trailing space removed: what the hash of the
    kernel sources covers, so that a profile stays current across edits of comments only."""
    src = _LINE_COMMENT.sub("", _BLOCK_COMMENT.sub("", src))
    return "\n".join(line.rstrip() for line in src.splitlines() if line.strip())


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(_HERE, "csrc", "*"))):
        if f.endswith((".hip", ".hpp")):
            h.update(os.path.basename(f).encode())
            h.update(code_text(open(f, encoding="utf-8").read()).encode())
    return h.hexdigest()


def _one(pattern: str) -> str:
    hits = sorted(glob.glob(pattern, recursive=True))
    if not hits:
        raise SystemExit(f"no file matches {pattern}")
    return hits[0]


_GEMM = re.compile(r"gemm_(dma_)?kernelI(.+?)Li(\d+)ELi(\d+)ELb(\d)ELb(\d)ELi(\d)E(?:Li(\d+)E)?")
_EPI = ["STORE", "PARTIAL", "GATED", "ACT", "DGATED", "DACT", "F8ACT", "F8DACT"]


# rocprofv3 prints some instantiations demangled (and their element types garbled)
_GEMM_DEMANGLED = re.compile(r"gmlp::gemm_(dma_)?kernel<(.*), (\d+), (\d+), (true|false), (true|false), (\d)(?:, (\d+))?>")


def _gemm_fields(name: str):
    m = _GEMM.search(name)
    if m:
        return m.groups()
    m = _GEMM_DEMANGLED.search(name)
    if m:
        dma, types, bm, bn, ak, bk, epi, waves = m.groups()
        b = {"true": "1", "false": "0"}
        if int(epi) == 1:
            types += "f"   # split-K partials are fp32
        return dma, types, bm, bn, b[ak], b[bk], epi, waves
    return None


def is_library_kernel(name: str) -> bool:
    return "4gmlp" in name or "gmlp::" in name


def gemm_epilogue(name: str):
    """The epilogue index of one of this library's GEMM kernels (None for other kernels;
    GROUP_EPI for the grouped backward launch)."""
    if is_group(name):
        return GROUP_EPI + group_epilogue(name)
    f = _gemm_fields(name)
    return int(f[6]) if f else None


def short_name(name: str) -> str:
    """A readable name for the engine's kernels (template arguments spelled out)."""
    if is_group(name):
        m = re.search(r"Li(\d+)ELi(\d+)ELi(\d+)E", name) or re.search(r"<[^,]+, (\d+), (\d+), (\d+),", name)
        bm, bn, w = m.groups() if m else ("?", "?", "?")
        t = "f16" if ("DF16_" in name or "_Float16" in name or "half" in name) else "bf16"
        f32 = re.search(r"EfLb0ELb0ELi\dE", name) is not None or ", float, false, false" in name
        return f"gemm_group<{t},NN:{_EPI[group_epilogue(name)]}+TN:STORE,{bm}x{bn},{w}w{',f32 dW out' if f32 else ''}>"
    f = _gemm_fields(name)
    if f:
        dma, types, bm, bn, ak, bk, epi, waves = f
        lay = {("1", "1"): "NT", ("1", "0"): "NN", ("0", "0"): "TN"}.get((ak, bk), "??")
        epin = _EPI[int(epi)]
        t = ("e5m2xe4m3" if "f8g" in types else "e4m3" if "e4m3" in types
             else "f16" if types.startswith("DF16_") else "f32" if types.startswith("ff") else "bf16")
        out = "f32" if "DF16bf" in types or types.endswith("f") else ""
        w = f",{waves}w" if waves else ""
        return f"gemm{'' if dma else '_regstaged'}<{t},{lay},{bm}x{bn}{w},{epin}{',' + out + ' out' if out else ''}>"
    for k in ("splitk_reduce", "gated_reduce", "gated_act", "plain_act", "absmax8_part", "absmax", "max_parts",
              "quantize8", "quantize_kernel", "quant2d", "dequant8", "dequant", "zero_f32", "scale_from_tiles"):
        if k in name:
            return k
    return name.split("(")[0][:60]


def summarize_trace(trace_dir: str, out_txt: str, command: str, first_step: int = 0, steps: int = 0,
                    stages: list[str] = STAGE_ORDER_GATED) -> None:
    stats = _one(os.path.join(trace_dir, "**", "*kernel_stats.csv"))
    rows = list(csv.DictReader(open(stats)))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}", f"# kernel sources sha256: {kernel_sources_sha256()}",
             "", f"{'kernel':64s} {'calls':>6s} {'avg us':>10s} {'total ms':>10s} {'%':>6s}"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
        calls = int(r["Calls"])
        avg_ns = float(r["AverageNs"])
        tot_ns = float(r["TotalDurationNs"])
        pct = float(r.get("Percentage", 0.0))
        lines.append(f"{short_name(name):64s} {calls:6d} {avg_ns / 1e3:10.1f} {tot_ns / 1e6:10.3f} {pct:6.2f}")
    trace = _one(os.path.join(trace_dir, "**", "*kernel_trace.csv"))
    disp = sorted((int(r["Dispatch_Id"]), r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
                  for r in csv.DictReader(open(trace)))
    stages = grouped_order(stages, (n for _, n, _ in disp))
    per_step = _per_step(disp, stages)
    timed = per_step[first_step:first_step + steps] if steps else per_step[first_step:]
    lines += ["", f"# per-stage kernel time, average over {len(timed)} timed steps (dispatch order; a split-K "
                  f"reduce counts with its GEMM)", f"{'stage':10s} {'kernels':64s} {'avg us':>10s}"]
    for st in stages:
        if not timed:
            break
        kern = " + ".join(dict.fromkeys(short_name(n) for n, _ in timed[0][st]))
        avg = sum(sum(d for _, d in s[st]) for s in timed) / len(timed)
        lines.append(f"{st:10s} {kern:64s} {avg:10.1f}")
    open(out_txt, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def is_reduce(name: str) -> bool:
    return "splitk_reduce" in name or "gated_reduce" in name


def _gemm_key(name: str):
    """(layout, epilogue, 16-bit) of a GEMM launch; the grouped launch is its own layout."""
    if is_group(name):
        return ("group", GROUP_EPI + group_epilogue(name), True)
    f = _gemm_fields(name)
    return ((f[4], f[5]), int(f[6]), not ("e4m3" in f[1] or "f8g" in f[1]))


def _continues(prev, cur) -> bool:
    """Whether GEMM launch `cur` belongs to the stage of the launch `prev` before it: the same
    layout with the same epilogue (a stage run as two launches over its output columns), or a
    16-bit split-K launch right after a store launch (a store GEMM cut along M: the rows below
    the cut with the store epilogue, the rest split along K)."""
    if prev is None or prev[0] != cur[0]:
        return False
    return prev[1] == cur[1] or (cur[2] and prev[1] == 0 and cur[1] == 1)


def _per_step(disp, stages):
    """Split this library's dispatches into steps (a step starts at each up-projection) and each
    step into stages. Each GEMM opens the next stage unless it continues the one before it
    (`_continues`). A split-K reduce joins the GEMM before it; other kernels of the library
    (quantize, transpose, widen) prepare an operand and join the GEMM after them. With a
    "recompute" stage, an up-projection GEMM right after the down projection is the backward's
    recompute, not a new step. Only whole steps are returned; launches of other libraries (a fill,
    a copy) are skipped."""
    steps, cur, idx, last_key, pending = [], None, -1, None, []
    rec = stages.index("recompute") if "recompute" in stages else -1
    for _, name, val in disp:
        if not is_library_kernel(name):
            continue
        epi = gemm_epilogue(name)
        if epi is None:
            if is_reduce(name) and cur is not None and 0 <= idx < len(stages):
                cur[stages[idx]].append((name, val))
            elif not is_reduce(name):
                pending.append((name, val))
            continue
        if epi in (2, 3, 6) and not (cur is not None and rec > 0 and idx == rec - 1):   # an up projection
            cur = {st: [] for st in stages}
            steps.append(cur)
            idx = 0
        elif cur is None:
            pending = []
            continue
        elif not _continues(last_key, _gemm_key(name)):
            idx += 1
        last_key = _gemm_key(name)
        if idx < len(stages):
            cur[stages[idx]].extend(pending + [(name, val)])
        else:
            cur["_extra"] = True
        pending = []
    return [s for s in steps if all(s[st] for st in stages) and "_extra" not in s]


def _dispatches(pmc_dir: str, counter: str) -> list[tuple[int, str, float]]:
    path = _one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    out = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    out.sort()
    return out


def _stage_bytes(disp, factor, stages, first_step=0, steps=0):
    """Average bytes per stage over the timed steps."""
    per_step = _per_step(disp, stages)
    full = per_step[first_step:first_step + steps] if steps else per_step[first_step:]
    if not full:
        return {}
    return {st: sum(sum(kib for _, kib in s[st]) for s in full) * 1024.0 * factor / len(full) for st in stages}


def summarize_traffic(fetch_dir: str, write_dir: str, out_json: str, command: str, copy_mib: int,
                      first_step: int = 0, steps: int = 0, stages: list[str] = STAGE_ORDER_GATED) -> None:
    fetch, write = _dispatches(fetch_dir, "FETCH_SIZE"), _dispatches(write_dir, "WRITE_SIZE")
    copy_bytes = copy_mib * 1024 * 1024
    fc = [v for _, n, v in fetch if "copyBuffer" in n]
    wc = [v for _, n, v in write if "copyBuffer" in n]
    if not fc or not wc:
        raise SystemExit("the profiled command ran no device copy (use bench.py --copy-probe-mib)")
    stages = grouped_order(stages, (n for _, n, _ in fetch))
    f_factor = copy_bytes / (fc[0] * 1024.0)
    w_factor = copy_bytes / (wc[0] * 1024.0)
    fb = _stage_bytes(fetch, f_factor, stages, first_step, steps)
    wb = _stage_bytes(write, w_factor, stages, first_step, steps)
    res = {"command": command, "kernel_sources_sha256": kernel_sources_sha256(),
           "copy_probe_bytes": copy_bytes, "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
           "note": "FETCH_SIZE counts L2 misses (last-level-cache hits included), so fetch_bytes is L2-miss traffic",
           "stages": {st: {"fetch_bytes": round(fb.get(st, 0.0)), "write_bytes": round(wb.get(st, 0.0)),
                           "traffic_bytes": round(fb.get(st, 0.0) + wb.get(st, 0.0))} for st in stages}}
    json.dump(res, open(out_json, "w"), indent=1)
    print(json.dumps(res, indent=1))


def _gpu_agent(pmc_dir: str) -> dict:
    path = _one(os.path.join(pmc_dir, "**", "*agent_info.csv"))
    for r in csv.DictReader(open(path)):
        if r.get("Agent_Type", "").upper().endswith("GPU") or r.get("Name", "").startswith("gfx"):
            return r
    raise SystemExit("no GPU agent in the agent info")


def summarize_mfma(pmc_dir: str, out_json: str, command: str, first_step: int = 0, steps: int = 0,
                   stage_order: list[str] = STAGE_ORDER_GATED) -> None:
    """MFMA busy fraction and shader clock per stage from one `--pmc SQ_VALU_MFMA_BUSY_CYCLES
    GRBM_GUI_ACTIVE` pass. SQ_VALU_MFMA_BUSY_CYCLES sums the busy cycles of every SIMD and
    GRBM_GUI_ACTIVE the active cycles of every XCD, so busy / (GUI / XCDs * SIMDs) is the
    fraction of SIMD cycles the matrix units worked, and GUI / XCDs / duration the clock."""
    agent = _gpu_agent(pmc_dir)
    n_xcc, n_simd = int(agent["Num_Xcc"]), int(agent["Simd_Count"])
    path = _one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    per = {}
    for r in csv.DictReader(open(path)):
        d = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"],
                                                   "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    disp = sorted((i, d["name"], (d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0), d.get("GRBM_GUI_ACTIVE", 0.0), d["ns"]))
                  for i, d in per.items())
    stage_order = grouped_order(stage_order, (n for _, n, _ in disp))
    steps_all = _per_step(disp, stage_order)
    timed = steps_all[first_step:first_step + steps] if steps else steps_all[first_step:]
    stages = {}
    for st in stage_order:
        busy = sum(v[0] for s in timed for _, v in s[st])
        gui = sum(v[1] for s in timed for _, v in s[st])
        ns = sum(v[2] for s in timed for _, v in s[st])
        if not timed or gui <= 0 or ns <= 0:
            continue
        cyc = gui / n_xcc
        stages[st] = {"kernel_us": round(ns / len(timed) / 1e3, 1), "sclk_ghz": round(cyc / ns, 3),
                      "mfma_busy": round(busy / (cyc * n_simd), 4)}
    res = {"command": command, "kernel_sources_sha256": kernel_sources_sha256(), "steps": len(timed),
           "xcc": n_xcc, "simds": n_simd, "stages": stages}
    json.dump(res, open(out_json, "w"), indent=1)
    print(json.dumps(res, indent=1))


def summarize_counters(pmc_dir: str, out_json: str, command: str, first_step: int = 0, steps: int = 0,
                       stage_order: list[str] = STAGE_ORDER_GATED) -> None:
    """Per-stage averages (per timed step) of every counter one `--pmc` pass collected, plus the
    ratios a reader usually wants from them (L2 hit rate from TCC_HIT_sum / TCC_MISS_sum, LDS bank
    conflict cycles per LDS-active cycle from SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE)."""
    path = _one(os.path.join(pmc_dir, "**", "*counter_collection.csv"))
    per, names = {}, []
    for r in csv.DictReader(open(path)):
        d = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        if r["Counter_Name"] not in names:
            names.append(r["Counter_Name"])
    disp = sorted((i, d["name"], d) for i, d in per.items())
    stage_order = grouped_order(stage_order, (n for _, n, _ in disp))
    steps_all = _per_step(disp, stage_order)
    timed = steps_all[first_step:first_step + steps] if steps else steps_all[first_step:]
    stages = {}
    for st in stage_order:
        if not timed:
            break
        tot = {c: sum(v.get(c, 0.0) for s in timed for _, v in s[st]) / len(timed) for c in names}
        if "TCC_HIT_sum" in tot and "TCC_MISS_sum" in tot and tot["TCC_HIT_sum"] + tot["TCC_MISS_sum"] > 0:
            tot["l2_hit_rate"] = round(tot["TCC_HIT_sum"] / (tot["TCC_HIT_sum"] + tot["TCC_MISS_sum"]), 4)
        if tot.get("SQ_LDS_IDX_ACTIVE", 0) > 0 and "SQ_LDS_BANK_CONFLICT" in tot:
            tot["lds_bank_conflict_per_active"] = round(tot["SQ_LDS_BANK_CONFLICT"] / tot["SQ_LDS_IDX_ACTIVE"], 5)
        stages[st] = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in tot.items()}
    res = {"command": command, "kernel_sources_sha256": kernel_sources_sha256(), "steps": len(timed),
           "counters": names, "stages": stages}
    json.dump(res, open(out_json, "w"), indent=1)
    print(json.dumps(res, indent=1))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("trace_dir")
    t.add_argument("out_txt")
    t.add_argument("--command", required=True)
    t.add_argument("--first-step", type=int, default=0, help="whole steps to skip (the bench's warmup)")
    t.add_argument("--steps", type=int, default=0, help="whole steps to average (0: all)")
    t.add_argument("--recompute", action="store_true", help="the step's backward recomputes the pre-activation")
    f = sub.add_parser("traffic")
    f.add_argument("fetch_dir")
    f.add_argument("write_dir")
    f.add_argument("out_json")
    f.add_argument("--command", required=True)
    f.add_argument("--copy-mib", type=int, default=256)
    f.add_argument("--first-step", type=int, default=0)
    f.add_argument("--steps", type=int, default=0)
    f.add_argument("--recompute", action="store_true")
    m = sub.add_parser("mfma")
    m.add_argument("pmc_dir")
    m.add_argument("out_json")
    m.add_argument("--command", required=True)
    m.add_argument("--first-step", type=int, default=0)
    m.add_argument("--steps", type=int, default=0)
    m.add_argument("--recompute", action="store_true")
    c = sub.add_parser("counters")
    c.add_argument("pmc_dir")
    c.add_argument("out_json")
    c.add_argument("--command", required=True)
    c.add_argument("--first-step", type=int, default=0)
    c.add_argument("--steps", type=int, default=0)
    c.add_argument("--recompute", action="store_true")
    a = ap.parse_args(argv)
    order = STAGE_ORDER_RECOMPUTE if a.recompute else STAGE_ORDER_GATED
    if a.what == "trace":
        summarize_trace(a.trace_dir, a.out_txt, a.command, a.first_step, a.steps, order)
    elif a.what == "mfma":
        summarize_mfma(a.pmc_dir, a.out_json, a.command, a.first_step, a.steps, order)
    elif a.what == "counters":
        summarize_counters(a.pmc_dir, a.out_json, a.command, a.first_step, a.steps, order)
    else:
        summarize_traffic(a.fetch_dir, a.write_dir, a.out_json, a.command, a.copy_mib, a.first_step, a.steps, order)


if __name__ == "__main__":
    sys.exit(main())
