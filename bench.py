"""Benchmark of the CompileMask hot path on one MI355X.

A step is one pass of the whole path over one batch resident in HBM:
preprocess (metadata -> Execution Descriptor), attention forward, and the
three backward kernels (D, dK/dV, dQ).  The metric is visible-pair TFLOP/s of
forward + backward, 14 * d * V / step time, where V is the exact number of
visible (query, key) pairs of the batch summed over heads (4 d V forward,
10 d V backward); the preprocess time is inside the step and reported alone.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--precision bf16|split]

Prints one JSON line on stdout.  Progress goes to stderr.  Besides the
default workload (reward_model_32k) the line carries `by_workload`: the other
32K workload (retrieval4_32k) and the causal check (causal_8k through the
descriptor and through the maskless causal path, and their ratio), measured
the same way in the same run.

The timed steps call the backward as one `cm_attn_bwd`, as a caller does
(on short grids the library runs dQ beside dK/dV on a second stream);
`ms_per_step` is the wall clock over them, `step_ms` the median and
10th/90th percentiles of HIP events around each step.  A second pass of the
same number of steps calls the three backward kernels one by one, with HIP
events around every kernel: `kernel_ms` and the roofline come from it.

HBM traffic of the dominant kernel comes from rocprofv3 counter runs:

    rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/fetch -o run -- python bench.py --steps 2 --warmup 1 --no-cpu-baseline
    rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/write -o run -- python bench.py --steps 2 --warmup 1 --no-cpu-baseline
    rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/copy_fetch -o run -- python bench.py --copy-calibration
    rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/copy_write -o run -- python bench.py --copy-calibration
    python bench.py --record-traffic OUT

The copy runs time a plain device-to-device copy of known size; the ratio of
its true bytes to what the counters report scales the kernel's counts.

The clock of each kernel comes from a GRBM_GUI_ACTIVE counter run (GPU busy
cycles, summed over the 8 XCDs) over each dispatch's duration:

    rocprofv3 --pmc GRBM_GUI_ACTIVE -f csv -d OUT/clock -o run -- python bench.py --steps 20 --warmup 1 --no-cpu-baseline --no-extra
    python bench.py --record-clock OUT/clock

and the roofline then also reports the fraction of the peak at that clock
(256 CUs x 4096 bf16 flop per CU and cycle x f).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, published
BF16_FLOP_PER_CLK = 256 * 4096  # MI355X: 256 CUs x 4096 dense bf16 flop per CU and cycle
EXTRA_WORKLOADS = (("retrieval4_32k", False), ("causal_8k", False), ("causal_8k", True))
# the step's kernels: their source files (for staleness of recorded counters)
# and the prefix of their names in rocprofv3's output (the dK/dV stage runs
# bwd_dkdv_kernel or bwd_dkdv_wide_kernel, by workload)
KERNEL_SOURCES = {
    "attn_fwd_kernel": ("attn_fwd.hip",),
    "bwd_dkdv_kernel": ("attn_bwd.hip", "attn_dkdv_wide.hip"),
    "bwd_dq_kernel": ("attn_bwd.hip",),
    "preprocess_kernel": ("preprocess.hip", "preprocess_core.h"),
}
KERNEL_MATCH = {"attn_fwd_kernel": "attn_fwd_kernel", "bwd_dkdv_kernel": "bwd_dkdv", "bwd_dq_kernel": "bwd_dq_kernel",
                "preprocess_kernel": "preprocess_kernel"}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_hash(kernel: str) -> str:
    """Hash of the kernel's sources with comments and blank space removed, so
    that a counter record stays valid across edits of comments only."""
    d = os.path.join(ROOT, "runtime_metadata_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(set(KERNEL_SOURCES[kernel]) | {"attn_common.h"}):
        text = open(os.path.join(d, f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic.json),
    or None when no measurement matches the kernel's current source."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(f"{kernel}@{workload}")
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def clock_for(kernel: str, workload: str):
    """Mean clock (GHz) of the kernel over its dispatches in a GRBM_GUI_ACTIVE
    counter run (profiles/clock.json), or None when no measurement matches the
    kernel's current source."""
    p = os.path.join(ROOT, "profiles", "clock.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(f"{kernel}@{workload}")
    if not rec or rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("clock_ghz_mean")


def record_clock(csv_dir: str, workload: str = "reward_model_32k"):
    """Per dispatch: GRBM_GUI_ACTIVE / 8 XCDs = the kernel's cycles; over its
    duration in the counter run = its average clock.  Writes profiles/clock.json
    and prints a markdown summary with every dispatch (duration and clock)."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {csv_dir}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != "GRBM_GUI_ACTIVE":
                continue
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            d = per.setdefault(key, {"cycles": 0.0, "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            d["cycles"] += float(r["Counter_Value"])
    path = os.path.join(ROOT, "profiles", "clock.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    lines = ["| kernel | dispatch | duration us | cycles (GRBM_GUI_ACTIVE / 8) | clock GHz |", "|---|---|---|---|---|"]
    for kernel in KERNEL_SOURCES:
        rows = sorted((k[1], v) for k, v in per.items() if KERNEL_MATCH[kernel] in k[0])
        if not rows:
            continue
        clocks = []
        for disp, v in rows:
            cyc = v["cycles"] / 8.0
            ghz = cyc / v["ns"] if v["ns"] > 0 else float("nan")
            clocks.append(ghz)
            lines.append(f"| `{kernel}` | {disp} | {v['ns'] / 1e3:.1f} | {cyc:.4g} | {ghz:.3f} |")
        rec[f"{kernel}@{workload}"] = {"source_hash": source_hash(kernel), "clock_ghz_mean": round(float(np.mean(clocks)), 4),
                                       "clock_ghz_min": round(float(np.min(clocks)), 4),
                                       "clock_ghz_max": round(float(np.max(clocks)), 4), "dispatches": len(clocks),
                                       "duration_us": [round(v["ns"] / 1e3, 1) for _, v in rows],
                                       "clock_ghz": [round(c, 4) for c in clocks]}
    json.dump(rec, open(path, "w"), indent=1, sort_keys=True)
    print("\n".join(lines))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


COPY_BYTES = 1 << 30


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES (three launches) for the counter runs."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 3}), flush=True)


def _pmc_per_dispatch(csv_dir: str, counter: str):
    """{kernel name: [counter value per dispatch]} from a rocprofv3 csv directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {csv_dir}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def record_traffic(out_dir: str, workload: str = "reward_model_32k"):
    """Scale the FETCH_SIZE / WRITE_SIZE counts (KiB per dispatch) of the attention kernels by the copy
    calibration and write profiles/traffic.json; prints a markdown summary."""
    cf = _pmc_per_dispatch(os.path.join(out_dir, "copy_fetch"), "FETCH_SIZE")
    cw = _pmc_per_dispatch(os.path.join(out_dir, "copy_write"), "WRITE_SIZE")
    copy_name = max(cf, key=lambda n: max(cf[n]))
    kib_f, kib_w = max(cf[copy_name]), max(cw[copy_name])
    f_fetch = COPY_BYTES / (kib_f * 1024.0)
    f_write = COPY_BYTES / (kib_w * 1024.0)
    kf = _pmc_per_dispatch(os.path.join(out_dir, "fetch"), "FETCH_SIZE")
    kw = _pmc_per_dispatch(os.path.join(out_dir, "write"), "WRITE_SIZE")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    lines = [f"copy kernel `{copy_name[:60]}`: {COPY_BYTES} B read and written; FETCH_SIZE {kib_f:.0f} KiB "
             f"(factor {f_fetch:.4f}), WRITE_SIZE {kib_w:.0f} KiB (factor {f_write:.4f})", "",
             "| kernel | dispatches | FETCH_SIZE KiB (mean) | WRITE_SIZE KiB (mean) | HBM bytes per launch (scaled) |",
             "|---|---|---|---|---|"]
    for kernel in KERNEL_SOURCES:
        names = [n for n in kf if KERNEL_MATCH[kernel] in n]
        if not names:
            continue
        fv = [x for n in names for x in kf[n]]
        wv = [x for n in names for x in kw.get(n, [])]
        mf, mw = float(np.mean(fv)), float(np.mean(wv)) if wv else 0.0
        total = mf * 1024.0 * f_fetch + mw * 1024.0 * f_write
        rec[f"{kernel}@{workload}"] = {"source_hash": source_hash(kernel), "bytes_per_launch": round(total),
                                       "fetch_kib": round(mf, 1), "write_kib": round(mw, 1),
                                       "fetch_factor": round(f_fetch, 5), "write_factor": round(f_write, 5)}
        lines.append(f"| `{kernel}` | {len(fv)} | {mf:.0f} | {mw:.0f} | {total:.4g} |")
    json.dump(rec, open(path, "w"), indent=1, sort_keys=True)
    print("\n".join(lines))


def visible_pairs(desc, H: int) -> int:
    """V summed over samples and heads, from the descriptor's row runs."""
    words = desc.words()
    off = desc.offsets()
    n = desc.B * desc.N * desc.K_r * 2
    iv = words[off["row_iv"] // 4: off["row_iv"] // 4 + n].reshape(-1, 2).astype(np.int64)
    return int((iv[:, 1] - iv[:, 0]).sum()) * H


def cpu_baseline(name: str, budget_s: float = 20.0):
    """The float64 oracle on a bounded sample of the same workload: the
    forward and backward work of the last query rows of head 0 of sample 0,
    growing the row block until about `budget_s` of CPU time."""
    import threadpoolctl

    from oracle import attention as oa
    from oracle import masks as om
    from workloads import WORKLOADS, make_metadata, make_tensors

    w = WORKLOADS[name]
    md = make_metadata(w)
    t = make_tensors(1, 1, w.N, w.d, w.seed)
    q, k, v, do = (oa._f64(t[n])[0, 0] for n in ("q", "k", "v", "do"))
    fn = om.row_block_fn(w.mask, md)
    cores = len(os.sched_getaffinity(0))
    rows, spent, vis = 64, 0.0, 0
    with threadpoolctl.threadpool_limits(limits=cores, user_api="blas"):
        while True:
            r1 = w.N
            r0 = max(0, r1 - rows)
            t0 = time.perf_counter()
            oa.backward_rows(q, k, v, do, fn, 0, r0, r1)
            spent = time.perf_counter() - t0
            vis = int(fn(0, r0, r1).sum())
            if spent > budget_s / 4 or r0 == 0:
                break
            rows *= 4
    tflops = 14.0 * w.d * vis / spent / 1e12
    return {"value": tflops, "unit": "visible-pair TFLOP/s (fp64 oracle)", "cores": cores, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{name}: sample 0, head 0, query rows {r0}..{r1 - 1} ({vis} visible pairs), forward + "
                      f"backward, {spent:.2f} s with BLAS on {cores} threads", "seconds": spent}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="reward_model_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="leave out the by_workload measurements")
    ap.add_argument("--precision", default="bf16", choices=["bf16", "split"],
                    help="P / dS operand precision (split: hi + lo bf16 pairs)")
    ap.add_argument("--split-cost", action="store_true",
                    help="also time every workload in both operand precisions (JSON lines to stderr)")
    ap.add_argument("--causal-path", action="store_true", help="time the maskless causal path (causal masks only)")
    ap.add_argument("--all", action="store_true",
                    help="also time every workload (and the causal comparator) and write one JSON line per run "
                         "to stderr; the stdout line stays the default workload's")
    ap.add_argument("--ablation", action="store_true",
                    help="also time the unsigned-compare and the ordinary-compare masked-interval kernels against "
                         "the default (run-bitmask) kernels on every masked workload (one JSON line per workload "
                         "to stderr)")
    ap.add_argument("--predicate", action="store_true",
                    help="also time the predicate baseline (block mask rebuilt per step, predicate in partial tiles) "
                         "against the descriptor path on every padded masked workload (JSON lines to stderr)")
    ap.add_argument("--specialize", action="store_true",
                    help="also time the preprocess of every workload with the interpreting kernel and with the "
                         "spec-specialised one (cm_spec_specialize); JSON lines to stderr")
    ap.add_argument("--graph", action="store_true",
                    help="also time every workload's step eagerly and as a HIP graph replay; JSON lines to stderr")
    ap.add_argument("--copy-calibration", action="store_true", help="only run the plain copy for counter scaling")
    ap.add_argument("--record-traffic", metavar="DIR", help="write profiles/traffic.json from counter runs in DIR")
    ap.add_argument("--record-clock", metavar="DIR", help="write profiles/clock.json from a GRBM_GUI_ACTIVE run in DIR")
    a = ap.parse_args()
    if a.record_traffic:
        record_traffic(a.record_traffic, a.workload)
        return
    if a.record_clock:
        record_clock(a.record_clock, a.workload)
        return
    if a.copy_calibration:
        copy_calibration()
        return
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py measures one GPU only: this path has no multi-GPU mode (asked for {a.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import runtime_metadata_attention_amd as cm
    from runtime_metadata_attention_amd import specs
    from workloads import WORKLOADS, make_metadata, make_tensors

    if a.all:
        for name in WORKLOADS:
            for causal in ([False, True] if WORKLOADS[name].mask == "causal" else [False]):
                line = measure(name, causal, a.steps, a.warmup, cpu=False)
                print("[bench-all] " + json.dumps(line), file=sys.stderr, flush=True)
    if a.ablation:
        for name in WORKLOADS:
            if WORKLOADS[name].N < 1024:
                continue
            base = measure(name, False, a.steps, a.warmup, cpu=False)
            uns = measure(name, False, a.steps, a.warmup, cpu=False, check=cm.CM_CHECK_UNSIGNED)
            abl = measure(name, False, a.steps, a.warmup, cpu=False, check=cm.CM_CHECK_ORDINARY_MASKED)
            rec = {"workload": name, "run_bits_ms": base["ms_per_step"], "unsigned_ms": uns["ms_per_step"],
                   "ordinary_masked_ms": abl["ms_per_step"],
                   "reduction": round(1.0 - uns["ms_per_step"] / abl["ms_per_step"], 4),
                   "run_bits_vs_unsigned": round(1.0 - base["ms_per_step"] / uns["ms_per_step"], 4),
                   "run_bits_kernel_ms": base["kernel_ms"], "unsigned_kernel_ms": uns["kernel_ms"],
                   "ordinary_masked_kernel_ms": abl["kernel_ms"]}
            print("[bench-ablation] " + json.dumps(rec), file=sys.stderr, flush=True)
    if a.graph:
        for name in WORKLOADS:
            print("[bench-graph] " + json.dumps(time_graph(name, a.steps, a.warmup)), file=sys.stderr, flush=True)
    if a.specialize:
        for name in WORKLOADS:
            print("[bench-specialize] " + json.dumps(time_preprocess(name, a.steps)), file=sys.stderr, flush=True)
    if a.predicate:
        for name in WORKLOADS:
            if WORKLOADS[name].N < 1024 or WORKLOADS[name].packed:
                continue
            base = measure(name, False, a.steps, a.warmup, cpu=False)
            pred = measure(name, False, a.steps, a.warmup, cpu=False, predicate=True)
            rec = {"workload": name, "descriptor_ms": base["ms_per_step"], "predicate_ms": pred["ms_per_step"],
                   "speedup": round(pred["ms_per_step"] / base["ms_per_step"], 4),
                   "descriptor_build_us": base["preprocess_us"], "blockmask_build_us": pred["preprocess_us"],
                   "descriptor_kernel_ms": base["kernel_ms"], "predicate_kernel_ms": pred["kernel_ms"]}
            print("[bench-predicate] " + json.dumps(rec), file=sys.stderr, flush=True)
    if a.split_cost:
        for name in WORKLOADS:
            base = measure(name, False, a.steps, a.warmup, cpu=False)
            spl = measure(name, False, a.steps, a.warmup, cpu=False, precision="split")
            rec = {"workload": name, "bf16_ms": base["step_ms"]["median"], "split_ms": spl["step_ms"]["median"],
                   "cost": round(spl["step_ms"]["median"] / base["step_ms"]["median"] - 1.0, 4),
                   "bf16_kernel_ms": base["kernel_ms"], "split_kernel_ms": spl["kernel_ms"]}
            print("[bench-split] " + json.dumps(rec), file=sys.stderr, flush=True)
    prec = a.precision
    line = measure(a.workload, a.causal_path, a.steps, a.warmup, cpu=not a.no_cpu_baseline, precision=prec)
    if not a.no_extra:
        extra = {}
        for name, causal in EXTRA_WORKLOADS:
            if name == a.workload and causal == a.causal_path:
                continue
            m = measure(name, causal, a.steps, a.warmup, cpu=False, precision=prec)
            extra[name + ("_maskless_causal" if causal else "")] = {
                k: m[k] for k in ("value", "frac_peak", "ms_per_step", "step_ms", "preprocess_us", "fwd_tflops",
                                  "bwd_tflops", "kernel_ms")} | {"visible_pairs": m["config"]["visible_pairs"],
                                                                 "roofline": m["roofline"]}
        if "causal_8k" in extra and "causal_8k_maskless_causal" in extra:
            extra["causal_8k_descriptor_vs_maskless"] = round(
                extra["causal_8k_maskless_causal"]["step_ms"]["median"] / extra["causal_8k"]["step_ms"]["median"], 4)
        line["by_workload"] = extra
    print(json.dumps(line), flush=True)


def time_preprocess(name: str, steps: int) -> dict:
    """Preprocess (metadata -> descriptor) alone, interpreting kernel vs the
    spec-specialised kernel, on the same buffers; microseconds per build."""
    import torch

    import runtime_metadata_attention_amd as cm
    from runtime_metadata_attention_amd import specs
    from workloads import WORKLOADS, make_metadata

    w = WORKLOADS[name]
    md = make_metadata(w)
    dev = torch.device("cuda", 0)
    dmd = cm.device_metadata(md, dev)
    out = {"workload": name}
    t0 = time.perf_counter()
    for kind in ("interpreted", "specialised"):
        spec = cm.cm_spec_compile(specs.BY_MASK[w.mask])
        if kind == "specialised":
            t0 = time.perf_counter()
            cm.cm_spec_specialize(spec)
            out["specialise_s"] = round(time.perf_counter() - t0, 3)
        desc = cm.Descriptor(spec, w.B, w.N, w.seg_cap, w.tiles, dev, packed=md.B if w.packed else 0)
        for _ in range(3):
            cm.cm_build_descriptor(spec, dmd, desc)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = max(steps, 10)
        e0.record()
        for _ in range(n):
            cm.cm_build_descriptor(spec, dmd, desc)
        e1.record()
        torch.cuda.synchronize()
        out[kind + "_us"] = round(e0.elapsed_time(e1) * 1e3 / n, 2)
    return out


def time_graph(name: str, steps: int, warmup: int) -> dict:
    """One whole step (descriptor build, forward, backward) timed eagerly and
    as a replay of a HIP graph captured once; milliseconds per step."""
    import torch

    import runtime_metadata_attention_amd as cm
    from runtime_metadata_attention_amd import specs
    from workloads import WORKLOADS, make_metadata, make_tensors

    w = WORKLOADS[name]
    md = make_metadata(w)
    dev = torch.device("cuda", 0)
    t = make_tensors(w.B, w.H, w.N, w.d, w.seed)
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    del t
    spec = cm.cm_spec_compile(specs.BY_MASK[w.mask])
    desc = cm.Descriptor(spec, w.B, w.N, w.seg_cap, w.tiles, dev, packed=md.B if w.packed else 0)
    dmd = cm.device_metadata(md, dev)
    args = cm.attn_args(q)
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    ws = torch.empty(cm.cm_attn_bwd_workspace(args) // 4, dtype=torch.float32, device=dev)

    def step():
        cm.cm_build_descriptor(spec, dmd, desc)
        cm.cm_attn_fwd(args, q, k, v, desc, o, lse)
        cm.cm_attn_bwd(args, q, k, v, o, lse, do, desc, dq, dk, dv, ws)

    def timed(fn):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    eager = timed(step)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    graph = timed(g.replay)
    return {"workload": name, "eager_ms": round(eager, 4), "graph_ms": round(graph, 4),
            "saved": round(1.0 - graph / eager, 4)}


def measure(workload: str, causal_path: bool, steps: int, warmup: int, cpu: bool, check: int = 0,
            predicate: bool = False, precision: str = "bf16") -> dict:
    """One bench line.  predicate=True times the predicate baseline: the block
    mask rebuilt from the metadata every step (cm_build_blockmask) and the
    predicate evaluated in partial tiles (check CM_CHECK_PREDICATE)."""
    import torch

    import runtime_metadata_attention_amd as cm
    from runtime_metadata_attention_amd import specs
    from workloads import WORKLOADS, make_metadata, make_tensors

    w = WORKLOADS[workload]
    md = make_metadata(w)
    log(f"workload {w.name}: B={w.B} H={w.H} N={w.N} d={w.d} tiles={w.tiles}"
        + (f" packed samples={md.B}" if w.packed else ""))
    t = make_tensors(w.B, w.H, w.N, w.d, w.seed)
    dev = torch.device("cuda", 0)
    q, k, v, do = (t[n].to(dev) for n in ("q", "k", "v", "do"))
    del t
    spec = cm.cm_spec_compile(specs.BY_MASK[w.mask])
    desc = cm.Descriptor(spec, w.B, w.N, w.seg_cap, w.tiles, dev, packed=md.B if w.packed else 0)
    dmd = cm.device_metadata(md, dev)
    if predicate:
        check = cm.CM_CHECK_PREDICATE
    prec = {"bf16": cm.CM_PRECISION_BF16, "split": cm.CM_PRECISION_SPLIT}[precision]
    args = cm.attn_args(q, causal=causal_path, check=check, precision=prec)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(cm.cm_attn_bwd_workspace(args) // 4, dtype=torch.float32, device=dev)
    use_desc = None if causal_path else desc

    names = ["preprocess_kernel", "attn_fwd_kernel", "bwd_dot_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"]

    def step(events=None, staged=False):
        def mark(i):
            if events is not None:
                events[i].record()
        mark(0)
        if predicate:
            cm.cm_build_blockmask(w.mask, dmd, desc)
        elif not causal_path:  # the maskless causal comparator needs no descriptor
            cm.cm_build_descriptor(spec, dmd, desc)
        mark(1)
        cm.cm_attn_fwd(args, q, k, v, use_desc, o, lse)
        mark(2)
        if staged:
            for s in range(3):
                cm.cm_attn_bwd_stage(s, args, q, k, v, o, lse, do, use_desc, dq, dk, dv, ws)
                mark(3 + s)
        else:
            cm.cm_attn_bwd(args, q, k, v, o, lse, do, use_desc, dq, dk, dv, ws)
            mark(3)

    cm.cm_build_descriptor(spec, dmd, desc)  # (also counts V for the causal comparator)
    torch.cuda.synchronize()
    V = visible_pairs(desc, w.H)
    for i in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done; visible pairs V = {V}")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / steps
    step_ev = np.array([e[0].elapsed_time(e[3]) for e in evs])  # ms, first to last event of each step
    # per-kernel times: the same number of steps again, the backward's kernels called one by one
    sevs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]
    for i in range(steps):
        step(sevs[i], staged=True)
    torch.cuda.synchronize()
    per = np.zeros((steps, 5))
    for i, e in enumerate(sevs):
        for j in range(5):
            per[i, j] = e[j].elapsed_time(e[j + 1])  # ms
    avg = per.mean(axis=0)
    step_ms = {"median": round(float(np.median(step_ev)), 4), "p10": round(float(np.percentile(step_ev, 10)), 4),
               "p90": round(float(np.percentile(step_ev, 90)), 4)}
    log("per-kernel ms: " + ", ".join(f"{n}={x:.4f}" for n, x in zip(names, avg)))

    d = w.d
    flops_fb = 14.0 * d * V
    value = flops_fb / (ms_step * 1e-3) / 1e12
    # algorithmic flops per launch of each attention kernel (visible pairs only):
    # forward S and PV (4 d V); dK/dV kernel S, dP, dV, dK (8 d V); dQ kernel S, dP, dQ (6 d V)
    alg = {"attn_fwd_kernel": 4.0 * d * V, "bwd_dkdv_kernel": 8.0 * d * V, "bwd_dq_kernel": 6.0 * d * V}
    times = dict(zip(names, avg))
    dom = max(alg, key=lambda n: times[n])
    achieved = alg[dom] / (times[dom] * 1e-3) / 1e12
    traffic = traffic_for(dom, w.name) if precision == "bf16" and check == 0 and not causal_path else None
    clock = clock_for(dom, w.name) if precision == "bf16" and check == 0 and not causal_path else None
    pre_bytes = desc.bytes + sum(x.numel() * 4 for x in (dmd.scalars, dmd.seg_bounds, dmd.n_seg, dmd.refs)
                                 if x is not None)
    line = {
        "metric": "masked attn fwd+bwd visible-pair TFLOP/s (% bf16 MFMA peak) at 32K; preprocess us",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": step_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded metadata and N(0,1) bf16 tensors)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "tiles": list(w.tiles),
                   "seed": w.seed, "visible_pairs": V, "path": "causal" if causal_path else "descriptor",
                   "packed_samples": int(md.B) if w.packed else 0,
                   "check": {0: "run_bits", 1: "ordinary_masked", 2: "predicate", 3: "unsigned"}[check],
                   "precision": precision},
        "frac_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "preprocess_us": round(times["preprocess_kernel"] * 1e3, 2),
        "preprocess_GBps": round(pre_bytes / (times["preprocess_kernel"] * 1e-3) / 1e9, 1),
        "fwd_tflops": round(4.0 * d * V / (times["attn_fwd_kernel"] * 1e-3) / 1e12, 2),
        "bwd_tflops": round(10.0 * d * V / ((times["bwd_dot_kernel"] + times["bwd_dkdv_kernel"] +
                                             times["bwd_dq_kernel"]) * 1e-3) / 1e12, 2),
        "kernel_ms": {n: round(float(x), 4) for n, x in times.items()},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "clock_GHz": clock,
                     "peak_at_clock": None if clock is None else round(BF16_FLOP_PER_CLK * clock * 1e9 / 1e12, 1),
                     "frac_at_clock": None if clock is None else
                     round(achieved / (BF16_FLOP_PER_CLK * clock * 1e9 / 1e12), 4)},
    }
    if cpu:
        log("timing the CPU oracle on a bounded sample")
        cb = cpu_baseline(w.name)
        line["cpu_baseline"] = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in cb.items()
                                if k != "seconds"}
    return line


if __name__ == "__main__":
    main()
