"""Throughput of the SAS gated block-sparse attention hot path on one MI355X.

One step = the training pass of the hot path over one batch of the packed
varlen workload (4 sequences of 32768 / 24576 / 16384 / 8192 tokens in one
buffer, 32 query / 8 KV heads, head dim 128, 64-token blocks, budget 2048
tokens = 31 history blocks + current, bf16, selector logits N(0,3) with 5 %
of the key-block columns boosted by +4): gate + Top-K -> gated forward ->
backward (prepare, dQ and log-gate gradient, dK/dV) -> gate backward.
`value` is the step's algorithmic fwd+bwd TFLOP/s over the attended
(selected-block) pairs: 4 d FLOPs per pair and head forward, 10 d backward.

Reported in the same JSON line:
  roofline      the longest-running kernel of the step, credited with its
                algorithmic FLOPs (metrics.py), over its average duration
                from HIP events on the stream the library launches on,
                against the 2.5 PFLOP/s dense bf16 MFMA peak;
  layer16k      the same step on the 16K-token single-layer workload;
  decode        paged batch-32 decode (budget 4096 tokens): append, pooled
                selection, split-K attention; KV GB/s against 8 TB/s; the
                whole step also timed as one unit, launched eagerly and
                replayed from a HIP graph;
  decode_long   one sequence at 131072 and at 524288 tokens (budget 2048);
  measured_peaks  a bf16 MFMA loop and a streaming read on this device;
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload.
Inputs are seeded synthetic tensors, resident in HBM before timing.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload varlen|layer16k]
                    [--no-cpu-baseline] [--no-decode] [--no-extra]

Profile summaries (no GPU needed; they read rocprofv3 csv output):
    python bench.py --summarize-trace DIR --cmd "..." --out profiles/X.md [--skip W]
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --cmd "..." --out profiles/Y.md
    python bench.py --summarize-counters DIR --cmd "..." --out profiles/Z.md
The second also writes profiles/traffic.json: HBM bytes per dispatch of the
library's kernels, from FETCH_SIZE / WRITE_SIZE scaled by what the same
counters read for the 1 GiB device copy this script runs untimed, tagged
with a hash of the kernel sources and the workload; a bench run reports that
traffic only while both still match.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="varlen", choices=["varlen", "layer16k"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the second training workload, the long decode and the peaks")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--summary-dtype", default="f32", choices=["f32", "bf16", "fp8"],
                    help="decode block-summary storage (bf16 / fp8 shrink the selector's scan)")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-counters", metavar="DIR")
    ap.add_argument("--skip", type=int, default=0,
                    help="summaries: leave out each kernel's first N dispatches (warm-up)")
    ap.add_argument("--cmd", default="", help="command line recorded in a summary")
    ap.add_argument("--out", help="markdown file a summary is written to")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
SUMMARY_BYTES = {"f32": 4, "bf16": 2, "fp8": 1}
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CALIBRATION_BYTES = 1 << 30


def _code_only(text, python=False):
    """Source text without comments and whitespace, so that edits to
    comments alone leave the hash unchanged."""
    if python:
        text = re.sub(r"(?m)^\s*#.*$", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return re.sub(r"\s+", "", text)


def source_hash():
    """Hash of the code the library is built from (kernels, headers, build),
    comments and whitespace left out."""
    pkg = os.path.join(ROOT, "trainable_block_sparse_gate_amd")
    files = sorted(glob.glob(os.path.join(pkg, "csrc", "*")) +
                   [os.path.join(pkg, "build.py"), os.path.join(ROOT, "include", "sas.h")])
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read(), python=f.endswith(".py")).encode())
    return h.hexdigest()[:16]


def short_kernel(name):
    if "rocclr_copyBuffer" in name:
        return "copyBuffer"
    if "sas" not in name:
        return None
    m = re.search(r"_ZN3sas\d+([a-z][a-z0-9_]*?_kernel)", name)  # mangled
    if not m:
        m = re.search(r"([a-z][a-z0-9_]*_kernel)", name)
    return m.group(1) if m else None


def read_csvs(d, suffix):
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


# ------------------------------------------------------------ summaries
def summarize_pmc(fetch_dir, write_dir, cmd, out, workload):
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for r in read_csvs(d, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            k = short_kernel(r["Kernel_Name"])
            if k is None:
                continue
            per.setdefault(k, {}).setdefault(counter, []).append(float(r["Counter_Value"]))
    # the calibration copies are the largest copyBuffer dispatches (1 GiB)
    cp = per.get("copyBuffer", {})
    fetch_cp = sorted(cp.get("FETCH_SIZE", []))[-3:]
    write_cp = sorted(cp.get("WRITE_SIZE", []))[-3:]
    if not fetch_cp or not write_cp:
        sys.exit("no calibration copy dispatches found in the counter output")
    f_fetch = CALIBRATION_BYTES / (sum(fetch_cp) / len(fetch_cp) * 1024)
    f_write = CALIBRATION_BYTES / (sum(write_cp) / len(write_cp) * 1024)
    kernels = {}
    for k, c in sorted(per.items()):
        if k == "copyBuffer" or "FETCH_SIZE" not in c or "WRITE_SIZE" not in c:
            continue
        fk = sum(c["FETCH_SIZE"]) / len(c["FETCH_SIZE"])
        wk = sum(c["WRITE_SIZE"]) / len(c["WRITE_SIZE"])
        kernels[k] = {"dispatches": len(c["FETCH_SIZE"]), "fetch_kib": round(fk, 1),
                      "write_kib": round(wk, 1),
                      "bytes_per_launch": int(fk * 1024 * f_fetch + wk * 1024 * f_write)}
    rec = {"source_hash": source_hash(), "workloads": [workload, "paged"], "command": cmd,
           "calibration": {"copy_bytes": CALIBRATION_BYTES, "fetch_kib": round(fetch_cp[-1], 1),
                           "write_kib": round(write_cp[-1], 1), "fetch_factor": round(f_fetch, 4),
                           "write_factor": round(f_write, 4)},
           "kernels": kernels}
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(rec, fh, indent=1)
    lines = ["# HBM traffic per dispatch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Two counter passes over the same bench run, then this summary:", "", "```",
             cmd, "```", "",
             f"Calibration: the untimed 1 GiB device copy reads {fetch_cp[-1]:.0f} KiB "
             f"(FETCH_SIZE) and writes {write_cp[-1]:.0f} KiB (WRITE_SIZE) per dispatch, so "
             f"the counters are scaled by {f_fetch:.4f} (fetch) and {f_write:.4f} (write).  "
             "FETCH_SIZE counts every L2 miss, including those the Infinity Cache serves.",
             f"Source hash {rec['source_hash']}; training kernels on the {workload} workload, "
             "decode kernels on the paged batch-32 workload (the command runs no other).", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | bytes / launch |",
             "|---|---|---|---|---|"]
    for k, v in kernels.items():
        lines.append(f"| `{k}` | {v['dispatches']} | {v['fetch_kib']:.0f} | {v['write_kib']:.0f} | "
                     f"{v['bytes_per_launch']:,} |")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as fh:
            fh.write(text)
    print(text)


def kernel_label(n):
    m = re.match(r"_ZN3sas\d+(\w+?_kernel)I(\w+?)EEvNS_", n)
    if m:  # template arguments: DF16b = bf16, f = float, Li<n>E = n, Lb0E / Lb1E = bool
        args = re.findall(r"DF16b|f|Li\d+E|Lb[01]E", m.group(2))
        args = [{"DF16b": "bf16", "f": "float", "Lb0E": "false", "Lb1E": "true"}.get(a, a[2:-1])
                for a in args]
        return f"{m.group(1)}<{', '.join(args)}>"
    m = re.match(r"_ZN3sas\d+(\w+?_kernel)E", n)
    if m:  # mangled, no template arguments
        return f"sas::{m.group(1)}"
    if short_kernel(n):
        # the profiler's demangler prints the __bf16 template argument (and
        # the one after it) as "bool _Accum, bool, E"
        n = n.replace("bool _Accum, bool, E", "__bf16, ...")
        return re.sub(r"^void ", "", re.sub(r"\(sas::\w+(, sas::\w+)*\)$", "", n))
    m = re.match(r"(?:void )?\(anonymous namespace\)::(\w+_kernel)(<\d+>)?", n)
    if m:  # the measured-peak kernels (csrc/peaks.hip)
        return f"peaks::{m.group(1)}{m.group(2) or ''}"
    if "__amd_rocclr" in n:
        return re.search(r"__amd_rocclr_\w+", n).group(0) + " (HIP runtime)"
    m = re.search(r"at::native::(?:\(anonymous namespace\)::)?[A-Za-z_:]*", n)
    return (m.group(0) if m else n[:48]) + " (torch)"


def summarize_trace(d, cmd, out, skip):
    """Per-kernel durations from a kernel trace: every dispatch, and the
    steady state without each kernel's first `skip` dispatches (warm-up)."""
    rows = read_csvs(d, "kernel_trace.csv")
    if not rows:
        sys.exit(f"no kernel_trace.csv under {d}")
    per = {}
    for r in rows:  # one entry per kernel and launch shape (workloads differ in grid)
        grid = int(r.get("Grid_Size_X", 0) or 0) * int(r.get("Grid_Size_Y", 1) or 1) * \
            int(r.get("Grid_Size_Z", 1) or 1)
        per.setdefault((r["Kernel_Name"], grid), []).append(r)
    total = sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows)
    lines = ["# Kernel trace summary (rocprofv3 --kernel-trace --stats)", "", "```", cmd, "```",
             "", f"Durations in us, one row per kernel and launch grid (the workloads of the "
             f"command differ in grid).  Steady state = every dispatch after the row's first "
             f"{skip} (the warm-up steps of the command).", "",
             "| kernel | WGs | calls | avg (all) | avg (steady) | min | max | % of GPU time | "
             "WG size | LDS B | VGPR | AGPR |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    summary = {}
    for (n, _), rs in sorted(per.items(), key=lambda kv: -sum(int(r["End_Timestamp"]) -
                                                              int(r["Start_Timestamp"])
                                                              for r in kv[1])):
        rs.sort(key=lambda r: int(r["Start_Timestamp"]))
        dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]
        steady = dur[skip:] if len(dur) > skip else dur
        t = rs[0]
        wg = int(t.get("Workgroup_Size_X", 0) or 0) * int(t.get("Workgroup_Size_Y", 1) or 1)
        grid = int(t.get("Grid_Size_X", 0) or 0) * int(t.get("Grid_Size_Y", 1) or 1) * \
            int(t.get("Grid_Size_Z", 1) or 1)
        nwg = grid // wg if wg else 0
        lab = kernel_label(n)
        summary[f"{lab} [{nwg} WGs]"] = {"calls": len(dur), "avg_us": sum(dur) / len(dur),
                                         "steady_avg_us": sum(steady) / len(steady)}
        lines.append(f"| `{lab}` | {nwg} | {len(dur)} | {sum(dur) / len(dur):.1f} | "
                     f"{sum(steady) / len(steady):.1f} | {min(dur):.1f} | {max(dur):.1f} | "
                     f"{100.0 * sum(dur) * 1e3 / total:.1f} | {wg} | "
                     f"{t.get('LDS_Block_Size', '')} | {t.get('VGPR_Count', '')} | "
                     f"{t.get('Accum_VGPR_Count', '')} |")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as fh:
            fh.write(text)
        with open(os.path.splitext(out)[0] + ".json", "w") as fh:
            json.dump({"command": cmd, "skip": skip, "kernels": summary}, fh, indent=1)
    print(text)


XCDS, SIMDS = 8, 1024  # MI355X: accelerator dies (GRBM_GUI_ACTIVE is summed over them), SIMDs


def summarize_counters(d, cmd, out):
    """Average of every counter per kernel over one --pmc pass, and what
    follows from them: MFMA busy (% of the SIMDs' cycles), the clock the
    kernel ran at, LDS bank-conflict share, L2 hit rate."""
    per, dur = {}, {}
    for r in read_csvs(d, "counter_collection.csv"):
        if short_kernel(r["Kernel_Name"]) in (None, "copyBuffer"):
            continue
        k = kernel_label(r["Kernel_Name"])
        per.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        dur.setdefault(k, {})[r["Dispatch_Id"]] = \
            int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    names = sorted({c for v in per.values() for c in v})

    def derived(v, ns):
        out = {}
        g = v.get("GRBM_GUI_ACTIVE")
        if g and v.get("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
            out["mfma_busy_pct"] = 100.0 * v["SQ_VALU_MFMA_BUSY_CYCLES"] / (g / XCDS * SIMDS)
        if g and ns:
            out["clock_ghz"] = g / XCDS / ns
        if v.get("SQ_LDS_IDX_ACTIVE"):
            out["lds_bank_conflict_pct"] = 100.0 * (v.get("SQ_LDS_BANK_CONFLICT") or 0.0) / \
                v["SQ_LDS_IDX_ACTIVE"]
        if v.get("TCC_HIT_sum") is not None and v.get("TCC_MISS_sum") is not None:
            tot = v["TCC_HIT_sum"] + v["TCC_MISS_sum"]
            out["l2_hit_pct"] = 100.0 * v["TCC_HIT_sum"] / tot if tot else None
        if v.get("SQ_INSTS_VALU_MFMA_MOPS_BF16") is not None and ns:
            out["mfma_bf16_tflops"] = v["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / ns / 1e3
        if v.get("SQ_VALU_MFMA_COEXEC_CYCLES") is not None and v.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            out["valu_coexec_pct_of_mfma_busy"] = \
                100.0 * v["SQ_VALU_MFMA_COEXEC_CYCLES"] / v["SQ_VALU_MFMA_BUSY_CYCLES"]
        wc = v.get("SQ_WAVE_CYCLES")
        if wc:
            for n, key in (("SQ_ACTIVE_INST_VALU", "valu_active_pct_of_wave_cycles"),
                           ("SQ_ACTIVE_INST_LDS", "lds_active_pct_of_wave_cycles"),
                           ("SQ_WAIT_ANY", "wait_any_pct_of_wave_cycles")):
                if v.get(n) is not None:
                    out[key] = 100.0 * v[n] / wc
        return out

    rec = {}
    for k, c in sorted(per.items()):
        vals = {n: (sum(c[n]) / len(c[n]) if n in c else None) for n in names}
        ns = sum(dur[k].values()) / len(dur[k]) if dur.get(k) else None
        rec[k] = {"counters": vals, "avg_ns_under_counters": ns, "derived": derived(vals, ns)}
    dnames = sorted({n for v in rec.values() for n in v["derived"]})
    lines = ["# Hardware counters per dispatch (rocprofv3 --pmc)", "", "```", cmd, "```", "",
             "Averages over the dispatches of each kernel.  GRBM_GUI_ACTIVE is summed over the "
             f"{XCDS} accelerator dies; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / "
             f"{XCDS} x {SIMDS} SIMDs); clock = GRBM_GUI_ACTIVE / {XCDS} / dispatch duration; the "
             "MFMA TFLOP/s counts 512 FLOPs per SQ_INSTS_VALU_MFMA_MOPS_BF16 over the dispatch "
             "duration under the counters (which can run slower than unprofiled).", ""]
    if dnames:
        lines += ["| kernel | " + " | ".join(dnames) + " |", "|---|" + "---|" * len(dnames)]
        for k, v in rec.items():
            lines.append(f"| `{k}` | " + " | ".join(
                "" if v["derived"].get(n) is None else f"{v['derived'][n]:.3g}" for n in dnames) +
                " |")
        lines.append("")
    lines += ["| kernel | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for k, v in rec.items():
        vals = v["counters"]
        lines.append(f"| `{k}` | " + " | ".join("" if vals[n] is None else f"{vals[n]:.4g}"
                                                 for n in names) + " |")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as fh:
            fh.write(text)
        with open(os.path.splitext(out)[0] + ".json", "w") as fh:
            json.dump({"command": cmd, "kernels": rec}, fh, indent=1)
    print(text)


def traffic_for(kernel, workload):
    """HBM bytes per launch of `kernel` from profiles/traffic.json, or None
    when there is none, it was taken on another workload, or the kernels
    have changed since it was taken."""
    try:
        with open(TRAFFIC_JSON) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash() or workload not in rec.get("workloads", []):
        return None
    k = rec.get("kernels", {}).get(kernel)
    return k["bytes_per_launch"] if k else None


# ------------------------------------------------------------ timing
class Marks:
    """HIP events between the phases of a step, summed over steps."""

    def __init__(self, torch):
        self.torch = torch
        self.order = []
        self.events = []
        self.total = {}

    def __call__(self, name):
        ev = self.torch.cuda.Event(enable_timing=True)
        ev.record()
        self.events.append((name, ev))

    def collect(self):
        for (n0, e0), (n1, e1) in zip(self.events, self.events[1:]):
            if n0 == "end":
                continue
            self.total[n0] = self.total.get(n0, 0.0) + e0.elapsed_time(e1)
            if n0 not in self.order:
                self.order.append(n0)
        self.events = []


# phase -> the kernels it launches (the first is the one the phase is named for)
PHASE_KERNELS = {"gate_topk": ["gate_topk_kernel"], "fwd": ["fwd_kernel"],
                 "bwd_prepare": ["bwd_csr_kernel", "bwd_seg_scan_kernel"],
                 "bwd_dq": ["bwd_dq_kernel"],
                 "bwd_dkdv": ["bwd_dkdv_kernel", "bwd_dkdv_reduce_kernel"],
                 "gate_bwd": ["gate_bwd_kernel"]}


def train_bench(args, torch, sas, metrics, case, steps, warmup):
    log(f"[bench] workload {case.name}: T={case.T} hq={case.hq} hkv={case.hkv} d={case.d} "
        f"Kb={case.budget_blocks}")
    prob = sas.Varlen(case.lengths, case.hq, case.hkv, case.d, case.budget_blocks)
    dev = "cuda"

    def to_dev(nm):
        return torch.from_numpy(case.bits[nm].view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, dO = (to_dev(n) for n in ("q", "k", "v", "dO"))
    logits = torch.from_numpy(case.logits).to(dev)
    f32, i32 = torch.float32, torch.int32
    sel = torch.empty((prob.hkv, prob.QB, prob.Kb), dtype=i32, device=dev)
    lg = torch.empty((prob.hkv, prob.QB, prob.Kb), dtype=f32, device=dev)
    glse = torch.empty((prob.hkv, prob.QB), dtype=f32, device=dev)
    o = torch.empty((prob.T, prob.hq, prob.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((prob.hq, prob.T), dtype=f32, device=dev)
    dq = torch.empty((prob.T, prob.hq, prob.d), dtype=f32, device=dev)
    dk = torch.empty((prob.T, prob.hkv, prob.d), dtype=f32, device=dev)
    dv = torch.empty((prob.T, prob.hkv, prob.d), dtype=f32, device=dev)
    dlg = torch.empty_like(lg)
    dlogits = torch.empty_like(logits)
    ws = torch.empty(sas.bwd_workspace_bytes(prob), dtype=torch.uint8, device=dev)

    def step(marks):
        marks("gate_topk")
        sas.gate_topk(prob, logits, out=(sel, lg, glse))
        marks("fwd")
        sas.fwd(prob, q, k, v, sel, lg, out=(o, lse))
        sas.bwd_phases(prob, q, k, v, o, dO, lse, sel, lg, (dq, dk, dv, dlg), ws,
                       marks=lambda n: marks("bwd_" + n if n != "end" else "gate_bwd"))
        sas.gate_bwd(prob, logits, sel, glse, dlg, out=dlogits)
        marks("end")

    nop = lambda n: None  # noqa: E731
    for _ in range(warmup):
        step(nop)
    torch.cuda.synchronize()
    marks = Marks(torch)
    t0 = time.perf_counter()
    for _ in range(steps):
        step(marks)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    marks.collect()
    ms_step = wall * 1e3 / steps
    phases = {n: marks.total[n] / steps for n in marks.order}
    fl = metrics.train_flops(case.lengths, case.hq, case.d, case.budget_blocks)
    tflops = (fl["fwd"] + fl["bwd"]) / (ms_step * 1e-3) / 1e12
    log(f"[bench] step {ms_step:.3f} ms  ->  {tflops:.1f} TFLOP/s  phases(ms): " +
        ", ".join(f"{n}={t:.3f}" for n, t in phases.items()))
    # algorithmic FLOPs credited to each kernel (metrics.py)
    credit = {"fwd": fl["fwd"], "bwd_dq": fl["dq_kernel"], "bwd_dkdv": fl["dkdv_kernel"]}
    executed = {"fwd": fl["fwd"], "bwd_dq": fl["dq_kernel_executed"],
                "bwd_dkdv": fl["dkdv_kernel_executed"]}
    per_kernel = {}
    for n in credit:
        tf = credit[n] / (phases[n] * 1e-3) / 1e12
        per_kernel[n] = {"kernels": PHASE_KERNELS[n], "ms": round(phases[n], 4),
                         "algorithmic_tflops": round(tf, 2),
                         "frac": round(tf / metrics.PEAK_BF16_TFLOPS, 4),
                         "executed_tflops": round(executed[n] / (phases[n] * 1e-3) / 1e12, 2)}
    dom = max(credit, key=lambda n: phases.get(n, 0.0))
    achieved = credit[dom] / (phases[dom] * 1e-3) / 1e12
    kname = PHASE_KERNELS[dom][0]
    roof = {"kernel": " + ".join(PHASE_KERNELS[dom]), "bound": "mfma",
            "achieved": round(achieved, 2), "peak": metrics.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / metrics.PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_for(kname, case.name),
            "ms_per_launch": round(phases[dom], 4),
            "algorithmic_flops_per_launch": credit[dom],
            "flops_credit": {"fwd": "4d", "bwd_dq": "4d", "bwd_dkdv": "6d"}[dom] +
                            " per attended pair and head"}
    bwd_ms = phases["bwd_prepare"] + phases["bwd_dq"] + phases["bwd_dkdv"]
    step_kernels_ms = sum(phases.values())
    out = {"ms_per_step": ms_step, "tflops": tflops, "phases_ms": phases, "flops": fl,
           "roofline": roof, "kernels": per_kernel,
           "backward": {"ms": round(bwd_ms, 4),
                        "tflops": round(fl["bwd"] / (bwd_ms * 1e-3) / 1e12, 2),
                        "frac": round(fl["bwd"] / (bwd_ms * 1e-3) / 1e12 /
                                      metrics.PEAK_BF16_TFLOPS, 4)},
           "step_frac": round(tflops / metrics.PEAK_BF16_TFLOPS, 4),
           "step_kernels_ms": round(step_kernels_ms, 4)}
    del q, k, v, dO, o, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return out


def decode_bench(args, torch, sas, wl, metrics, spec):
    log(f"[bench] decode workload {spec.name}: batch {spec.batch}, lengths "
        f"{min(spec.seqlens)}..{max(spec.seqlens)}, Kb={spec.budget_blocks}")
    t = wl.draw_decode_device(spec)
    if spec.paged:
        prob = sas.Decode(spec.seqlens, spec.hq, spec.hkv, spec.d, spec.budget_blocks, True,
                          spec.max_len, page_table=t["page_table"], num_pages=t["k"].shape[0],
                          summary_dtype=args.summary_dtype)
    else:
        prob = sas.Decode(spec.seqlens, spec.hq, spec.hkv, spec.d, spec.budget_blocks, False,
                          spec.max_len, summary_dtype=args.summary_dtype)
    ksum = sas.pool_keys(prob, t["k"])  # cache maintenance, not timed
    sws = sas.decode_select_workspace(prob)
    sel, lg, glse, scores = sas.decode_select(prob, t["q"], ksum, workspace=sws)
    ws = torch.empty(max(1, sas.decode_workspace_bytes(prob)), dtype=torch.uint8, device="cuda")
    o, lse = sas.decode(prob, t["q"], t["k"], t["v"], sel, lg, workspace=ws)
    # Between iterations the caches are refilled by READING a 1 GiB buffer
    # (more than L2 + Infinity Cache), so no kept K/V block is cached when a
    # decode starts and no dirty line of the flush is written back during it.
    flush = torch.zeros(1 << 28, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    # one step's cache maintenance: a new token per (sequence, kv head)
    # written at position L - 1 (and a finished block summarised when L - 1
    # opens a block); timed apart from the selection and the attention
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    k_new, v_new = (torch.randn((spec.batch, spec.hkv, spec.d), device="cuda",
                                generator=gen).to(torch.bfloat16) for _ in range(2))
    torch.cuda.synchronize()
    t_sel = t_dec = t_app = 0.0
    for it in range(args.decode_steps + 3):
        flush.sum()
        ea, e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(4))
        ea.record()
        sas.decode_append(prob, k_new, v_new, t["k"], t["v"], ksum)
        e0.record()
        sas.decode_select(prob, t["q"], ksum, out=(sel, lg, glse, scores), workspace=sws)
        e1.record()
        sas.decode(prob, t["q"], t["k"], t["v"], sel, lg, workspace=ws, out=(o, lse))
        e2.record()
        torch.cuda.synchronize()
        if it >= 3:
            t_app += ea.elapsed_time(e0)
            t_sel += e0.elapsed_time(e1)
            t_dec += e1.elapsed_time(e2)
    n = args.decode_steps
    # the whole step as one unit: launched eagerly, and replayed from a HIP
    # graph captured once (its 4-5 kernels with no host launch between them;
    # the step is idempotent, so every replay does the same work)
    def step():
        sas.decode_append(prob, k_new, v_new, t["k"], t["v"], ksum)
        sas.decode_select(prob, t["q"], ksum, out=(sel, lg, glse, scores), workspace=sws)
        sas.decode(prob, t["q"], t["k"], t["v"], sel, lg, workspace=ws, out=(o, lse))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    t_whole = [0.0, 0.0]  # eager, graph
    for it in range(n + 3):
        for mode in (0, 1):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            if mode == 0:
                step()
            else:
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            if it >= 3:
                t_whole[mode] += e0.elapsed_time(e1)
    del graph
    # the selection with the other summary storages (same cache, same query)
    by_summary = {}
    for sd in ("f32", "bf16", "fp8"):
        if sd == args.summary_dtype:
            continue
        p2 = sas.Decode(spec.seqlens, spec.hq, spec.hkv, spec.d, spec.budget_blocks, spec.paged,
                        spec.max_len, page_table=t["page_table"],
                        num_pages=t["k"].shape[0] if spec.paged else 0, summary_dtype=sd)
        ks2 = sas.pool_keys(p2, t["k"])
        ws2 = sas.decode_select_workspace(p2)
        out2 = sas.decode_select(p2, t["q"], ks2, workspace=ws2)
        tt = 0.0
        for it in range(n + 3):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            sas.decode_select(p2, t["q"], ks2, out=out2, workspace=ws2)
            e1.record()
            torch.cuda.synchronize()
            if it >= 3:
                tt += e0.elapsed_time(e1)
        b2 = metrics.decode_scan_bytes(spec.seqlens, spec.hkv, spec.d, SUMMARY_BYTES[sd])
        by_summary[sd] = {"us": round(tt / n * 1e3, 2), "summary_bytes": b2,
                          "GB/s": round(b2 / (tt / n * 1e-3) / 1e9, 1)}
        del ks2, ws2, out2
    # the hierarchical selection (opt-in approximation): coarse_keep = Kb - 1
    # super-blocks of 8 blocks, then the fine Top-K over their blocks; its
    # time per summary dtype and its recall of the exact kept blocks
    C = spec.budget_blocks - 1
    hier = {"coarse_keep": C, "coarse_blocks": sas.COARSE_BLOCKS}
    for sd in ("f32", "bf16", "fp8"):
        p2 = sas.Decode(spec.seqlens, spec.hq, spec.hkv, spec.d, spec.budget_blocks, spec.paged,
                        spec.max_len, page_table=t["page_table"],
                        num_pages=t["k"].shape[0] if spec.paged else 0, summary_dtype=sd)
        ks2 = sas.pool_keys(p2, t["k"])
        cs2 = sas.pool_coarse(p2, ks2)
        exact = sas.decode_select(p2, t["q"], ks2)[0]
        ws2 = torch.empty(max(1, sas.decode_select_hier_workspace_bytes(p2, C)),
                          dtype=torch.uint8, device="cuda")
        out2 = sas.decode_select_hier(p2, t["q"], ks2, cs2, C, workspace=ws2)
        tt = 0.0
        for it in range(n + 3):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            sas.decode_select_hier(p2, t["q"], ks2, cs2, C, out=out2, workspace=ws2)
            e1.record()
            torch.cuda.synchronize()
            if it >= 3:
                tt += e0.elapsed_time(e1)
        # recall: kept history blocks of the exact selection also kept here
        cur = torch.tensor([(L - 1) // 64 for L in spec.seqlens], device="cuda").repeat_interleave(
            spec.hkv)[:, None]
        ex = exact.long().masked_fill((exact < 0) | (exact == cur), -1)
        hi = out2[0].long().masked_fill((out2[0] < 0) | (out2[0] == cur), -2)
        hits = (ex[:, :, None] == hi[:, None, :]).any(-1).sum().item()
        total = (ex >= 0).sum().item()
        hier[sd] = {"us": round(tt / n * 1e3, 2), "recall": round(hits / max(total, 1), 4)}
        del ks2, cs2, ws2, out2, exact
    kv = metrics.decode_kv_bytes(spec.seqlens, spec.hkv, spec.d, spec.budget_blocks)
    scan = metrics.decode_scan_bytes(spec.seqlens, spec.hkv, spec.d,
                                     SUMMARY_BYTES[args.summary_dtype])
    gbs = kv / (t_dec / n * 1e-3) / 1e9
    scan_gbs = scan / (t_sel / n * 1e-3) / 1e9
    log(f"[bench] decode {t_dec / n * 1e3:.1f} us for {kv / 2**20:.1f} MiB -> {gbs:.0f} GB/s; "
        f"selection {t_sel / n * 1e3:.1f} us over {scan / 2**20:.1f} MiB summaries; "
        f"append {t_app / n * 1e3:.1f} us; whole step {t_whole[0] / n * 1e3:.1f} us eager, "
        f"{t_whole[1] / n * 1e3:.1f} us from a HIP graph")
    del t, flush
    torch.cuda.empty_cache()
    desc = (f"paged: batch {spec.batch}, lengths U[32768,131072]" if spec.paged else
            f"contiguous: batch {spec.batch}, length {spec.seqlens[0]}")
    return {"workload": f"{desc}, 32/8 heads, d128, budget {spec.budget_blocks} blocks",
            "kv_bytes": kv, "us": round(t_dec / n * 1e3, 2), "value": round(gbs, 1),
            "unit": "GB/s", "frac": round(gbs / metrics.PEAK_HBM_GBS, 4),
            "peak": metrics.PEAK_HBM_GBS,
            "traffic": traffic_for("decode_attend_kernel", spec.name),
            "selection": {"us": round(t_sel / n * 1e3, 2), "summary_bytes": scan,
                          "summary_dtype": args.summary_dtype,
                          "GB/s": round(scan_gbs, 1), "other_summary_dtypes": by_summary,
                          "hierarchical": hier},
            "append_us": round(t_app / n * 1e3, 2),
            "step_us": round((t_app + t_sel + t_dec) / n * 1e3, 2),
            "whole_step_us": {"eager": round(t_whole[0] / n * 1e3, 2),
                              "hip_graph": round(t_whole[1] / n * 1e3, 2)}}


def measured_peaks(torch, metrics):
    """A bf16 MFMA loop and a streaming read on this device (libsas_peaks.so)."""
    import ctypes
    from trainable_block_sparse_gate_amd import build
    if not os.path.exists(build.PEAKS_LIB):
        return None
    L = ctypes.CDLL(build.PEAKS_LIB)
    L.sas_peak_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.sas_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_int]
    chains = L.sas_peak_mfma_chains()
    props = torch.cuda.get_device_properties(0)
    cus = props.multi_processor_count
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    sink = torch.empty(cus * 8 * 256, dtype=torch.float32, device="cuda")
    iters = 4096

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    ms = timed(lambda: L.sas_peak_mfma_bf16(cus * 8, iters, ctypes.c_void_p(sink.data_ptr()), st))
    flops = cus * 8 * 4 * iters * chains * 32 * 32 * 16 * 2
    mfma_tf = flops / (ms * 1e-3) / 1e12
    # on random operands, sustained: ten launches back to back as one interval
    L.sas_peak_mfma_bf16_data.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p]
    g = torch.Generator().manual_seed(7)
    ops = torch.randn(1 << 16, generator=g).to(torch.bfloat16).cuda()
    data_iters = 2048

    def data_run():
        for _ in range(10):
            rc = L.sas_peak_mfma_bf16_data(cus * 8, data_iters, ctypes.c_void_p(ops.data_ptr()),
                                           ops.numel() * 2, ctypes.c_void_p(sink.data_ptr()), st)
            if rc != 0:
                raise RuntimeError(f"sas_peak_mfma_bf16_data failed ({rc})")
    ms_d = timed(data_run, reps=3)
    data_tf = 10 * cus * 8 * 4 * data_iters * chains * 32 * 32 * 16 * 2 / (ms_d * 1e-3) / 1e12
    del ops
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    rsink = torch.empty(cus * 32 * 256, dtype=torch.int32, device="cuda")
    reads = {}
    for mode in (0, 1, 2):
        for wgs in (cus * 4, cus * 16, cus * 32):
            ms_r = timed(lambda: L.sas_peak_read(ctypes.c_void_p(buf.data_ptr()), nbytes, wgs,
                                                 ctypes.c_void_p(rsink.data_ptr()), st, mode))
            reads[f"mode{mode}_wgs{wgs}"] = round(nbytes / (ms_r * 1e-3) / 1e9, 1)
    best = max(reads, key=reads.get)
    read_gbs = reads[best]
    # a 64 MiB buffer read over and over: more than the 32 MB of L2, so the
    # repeats are served by the 256 MB Infinity Cache
    small = 64 << 20
    mall = timed(lambda: L.sas_peak_read(ctypes.c_void_p(buf.data_ptr()), small, cus * 4,
                                         ctypes.c_void_p(rsink.data_ptr()), st, 1), reps=10)
    mall_gbs = small / (mall * 1e-3) / 1e9
    del buf, rsink, sink
    torch.cuda.empty_cache()
    log(f"[bench] measured peaks: bf16 MFMA {mfma_tf:.0f} TFLOP/s ({data_tf:.0f} on random "
        f"operands, sustained), streaming read "
        f"{read_gbs:.0f} GB/s ({best}; {reads}), 64 MiB re-read {mall_gbs:.0f} GB/s "
        f"({cus} compute units)")
    return {"bf16_mfma_tflops": round(mfma_tf, 1),
            "bf16_mfma_frac_of_spec": round(mfma_tf / metrics.PEAK_BF16_TFLOPS, 4),
            "bf16_mfma_random_operands_tflops": round(data_tf, 1),
            "bf16_mfma_random_operands_frac_of_spec": round(data_tf / metrics.PEAK_BF16_TFLOPS, 4),
            "stream_read_gbs": round(read_gbs, 1),
            "stream_read_frac_of_spec": round(read_gbs / metrics.PEAK_HBM_GBS, 4),
            "stream_read_variants_gbs": reads,
            "cache_resident_read_gbs": round(mall_gbs, 1),
            "compute_units": cus,
            "how": (f"MFMA: {cus * 8} workgroups x 4 waves, each {iters} x {chains} "
                    "independent 32x32x16 bf16 MFMAs on registers (near-constant operands), best "
                    f"of 5; random operands: the same grid, {data_iters} x {chains} MFMAs per wave "
                    "on N(0,1) bf16 operands that change every instruction, ten launches timed "
                    "as one interval, best of 3; read: 4 GiB, 16-byte loads, "
                    "grid-stride (mode0) or one contiguous chunk per workgroup with 8 / 16 "
                    "nontemporal loads in flight (mode1 / mode2), best of 5 launches each; "
                    "cache-resident: a 64 MiB buffer re-read (Infinity Cache), best of 10")}


def calibration_copy(torch, nbytes=1 << 30, reps=3):
    """A plain device-to-device copy of known size, run untimed so that
    hardware-counter runs of this script see a kernel whose true HBM traffic
    is known (nbytes read + nbytes written per launch)."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, metrics):
    """The oracle as it stands, on a bounded sample of the same workload: the
    last NS query blocks of every kv head (steady state: every row keeps the
    full budget), forward and backward; dk/dv are produced for the same key
    blocks, which only those rows can keep."""
    import oracle
    nb = case.qblocks[-1]
    QB = case.total_qblocks
    rm = np.zeros((case.hkv, QB), np.uint8)
    NS = min(64, nb - case.budget_blocks)
    rm[:, QB - NS:QB] = 1  # last NS query blocks of the last sequence
    t0 = time.perf_counter()
    idx, sl, _ = oracle.gate_topk(case.cu_seqlens, case.logits, case.hkv, case.budget_blocks)
    t1 = time.perf_counter()
    oracle.fwd(case.cu_seqlens, case.q, case.k, case.v, idx, sl, case.budget_blocks,
               case.scale, row_mask=rm)
    t2 = time.perf_counter()
    oracle.bwd(case.cu_seqlens, case.q, case.k, case.v, case.dO, idx, sl, case.budget_blocks,
               case.scale, row_mask=rm, kblk_mask=rm)
    t3 = time.perf_counter()
    # sample pairs: NS rows x hkv kv heads x G heads, each keeping Kb-1 full blocks + own
    pairs = NS * case.hkv * (case.hq // case.hkv) * ((case.budget_blocks - 1) * 64 * 64 +
                                                     64 * 65 // 2)
    flops = 14 * case.d * pairs
    secs = t3 - t1
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": (f"fwd+bwd of the last {NS} query blocks of all {case.hkv} kv heads "
                       f"({NS * case.hkv} rows, {pairs} attended pairs) of the same workload, "
                       f"fp64, algorithmic 14d FLOPs per pair and head; fwd {t2 - t1:.1f} s, "
                       f"bwd {t3 - t2:.1f} s; gate+Top-K of all rows {t1 - t0:.2f} s not "
                       "counted"),
            "seconds": round(secs, 2), "decode_sample": cpu_decode_sample(metrics)}


def cpu_decode_sample(metrics):
    """The oracle's decode path on a bounded sample: one 131072-token
    sequence, 8 query / 2 kv heads (the workloads' group of 4), head_dim 128,
    budget 64 blocks: summaries, pooled selection and decode attention of
    both (sequence, kv head) rows, timed per phase."""
    import oracle
    from trainable_block_sparse_gate_amd import workloads as wl
    L, hq, hkv, d, Kb = 131072, 8, 2, 128, 64
    host = wl.draw_decode_host_small([L], hq, hkv, d, Kb, False, seed=5000)
    G = hq // hkv
    t_pool = t_sel = t_dec = 0.0
    for g in range(hkv):
        K, V = host["k"][0, g, :L], host["v"][0, g, :L]
        qg = host["q"][0, g * G:(g + 1) * G]
        t0 = time.perf_counter()
        kbar = oracle.pool_keys_row(K)
        t1 = time.perf_counter()
        s = oracle.decode_scores_row(qg, kbar)
        idx, lg, _ = oracle.gate_row(s, (L - 1) // 64, Kb)
        t2 = time.perf_counter()
        oracle.decode_row(qg, K, V, idx, lg, Kb, 1.0 / np.sqrt(d))
        t3 = time.perf_counter()
        t_pool, t_sel, t_dec = t_pool + t1 - t0, t_sel + t2 - t1, t_dec + t3 - t2
    kv = metrics.decode_kv_bytes([L], hkv, d, Kb)
    return {"rows": hkv, "context": L, "budget_blocks": Kb,
            "pool_s": round(t_pool, 4), "select_s": round(t_sel, 4),
            "decode_s": round(t_dec, 4), "decode_kv_GB/s": round(kv / t_dec / 1e9, 3),
            "threads": 1, "note": "fp64 oracle (fp32 pooled scores), rows in turn on one host thread"}


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.cmd, args.out, args.skip)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.cmd, args.out,
                      args.workload)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.cmd, args.out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path shards without exchange over kv heads and sequences; this run "
              "uses one GPU)", file=sys.stderr)
        sys.exit(2)
    import torch
    from trainable_block_sparse_gate_amd import metrics, sas
    from trainable_block_sparse_gate_amd import workloads as wl
    sas.lib()  # fail loudly when the library is missing
    t0 = time.perf_counter()
    case = wl.varlen() if args.workload == "varlen" else wl.layer16k()
    log(f"[bench] inputs drawn in {time.perf_counter() - t0:.1f} s")
    tr = train_bench(args, torch, sas, metrics, case, args.steps, args.warmup)
    extra_train = None
    if not args.no_extra:
        other = wl.layer16k() if args.workload == "varlen" else wl.varlen()
        r = train_bench(args, torch, sas, metrics, other, args.steps, args.warmup)
        extra_train = {"workload": other.name, "tokens": other.T,
                       "budget_blocks": other.budget_blocks,
                       "ms_per_step": round(r["ms_per_step"], 4), "tflops": round(r["tflops"], 2),
                       "step_frac": r["step_frac"], "phases_ms":
                       {k: round(v, 4) for k, v in r["phases_ms"].items()},
                       "kernels": r["kernels"], "backward": r["backward"],
                       "roofline": r["roofline"]}
        del other
    dec = None if args.no_decode else decode_bench(args, torch, sas, wl, metrics,
                                                   wl.paged_spec())
    dec_long = None
    if not args.no_decode and not args.no_extra:
        dec_long = {str(c): decode_bench(args, torch, sas, wl, metrics, wl.decode_spec(c))
                    for c in (131072, 524288)}
    peaks = None if args.no_extra else measured_peaks(torch, metrics)
    calibration_copy(torch)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, metrics)
        log(f"[bench] cpu baseline {cpu['value']} TFLOP/s ({cpu['seconds']} s)")
    line = {
        "metric": "gated sparse attn fwd+bwd TFLOP/s (selected blocks) + decode KV GB/s, %roof",
        "value": round(tr["tflops"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(tr["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": ("synthetic (seeded normal q/k/v/dO; selector logits N(0,3) with 5% of key-block "
                 "columns +4)" if case.name == "varlen" else
                 "synthetic (seeded normal q/k/v/dO, selector logits N(0,2))"),
        "config": {"workload": (f"{case.name}: {len(case.lengths)} packed sequences "
                                f"{'/'.join(map(str, case.lengths))} ({case.T} tokens), "
                                f"{case.hq}/{case.hkv} heads, head_dim {case.d}, block 64, "
                                f"budget {case.budget_blocks} blocks (incl. current), "
                                "gate+topk+fwd+bwd+gate_bwd"),
                   "tokens": case.T, "budget_blocks": case.budget_blocks,
                   "attended_pairs": tr["flops"]["pairs"],
                   "fwd_flops": tr["flops"]["fwd"], "bwd_flops": tr["flops"]["bwd"]},
        "step_frac": tr["step_frac"],
        "phases_ms": {k: round(v, 4) for k, v in tr["phases_ms"].items()},
        "kernels": tr["kernels"],
        "backward": tr["backward"],
        "roofline": tr["roofline"],
        extra_train["workload"] if extra_train else "extra_train": extra_train,
        "decode": dec,
        "decode_long": dec_long,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    line["config"]["seeds"] = ("1000 * workload + stream; workloads tiny 1, layer16k 2, varlen 3, "
                               "decode 4, paged 5; streams q 0, k 1, v 2, logits 3, dO 4, "
                               "lengths 5, page permutation 6, boosted columns 7")
    if peaks:
        # the same fractions against the peaks measured in this run
        mf, hb = peaks["bf16_mfma_random_operands_tflops"], peaks["stream_read_gbs"]
        line["frac_of_measured_peaks"] = {
            "mfma_peak_tflops": mf, "hbm_peak_gbs": hb,
            "step": round(tr["tflops"] / mf, 4),
            "kernels": {k: round(v["algorithmic_tflops"] / mf, 4)
                        for k, v in tr["kernels"].items()},
            "backward": round(tr["backward"]["tflops"] / mf, 4),
            "decode": round(dec["value"] / hb, 4) if dec else None,
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
