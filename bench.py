"""Throughput of the SAS gated block-sparse attention hot path on one MI355X.

One step = the training pass of the hot path over one batch of the
Qwen3-4B-shaped layer workload (1 x 16384 tokens, 32 query / 8 KV heads,
head dim 128, 64-token blocks, budget 1024 tokens = 15 history blocks +
current, bf16): gate + Top-K -> gated forward -> backward (prepare, dQ and
log-gate gradient, dK/dV) -> gate backward.  `value` is the step's
algorithmic fwd+bwd TFLOP/s over the attended (selected-block) pairs.

The decode half of the metric is measured in the same run on the batched
paged workload (batch 32, lengths ~ U[32768, 131072], budget 4096 tokens):
pooled selection, then split-K decode; its KV GB/s is reported under
"decode".  Inputs are seeded synthetic tensors, resident in HBM before
timing.  Per-kernel durations come from HIP events recorded on the stream
the library launches on.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

Profile summaries (no GPU needed; they read rocprofv3 csv output):
    python bench.py --summarize-trace DIR --cmd "..." --out profiles/X.md
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --cmd "..." --out profiles/Y.md
The second also writes profiles/traffic.json: HBM bytes per dispatch of the
library's kernels, from FETCH_SIZE / WRITE_SIZE scaled by what the same
counters read for the 1 GiB device copy this script runs untimed, tagged
with a hash of the kernel sources; a bench run reports that traffic only
while the hash still matches.
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
    ap.add_argument("--workload", default="layer16k", choices=["layer16k", "varlen"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=20)
    ap.add_argument("--summary-dtype", default="f32", choices=["f32", "bf16"],
                    help="decode block-summary storage (bf16 halves the selector's scan)")
    ap.add_argument("--decode-workload", default="paged", choices=["paged", "long"],
                    help="paged: batch 32 paged cache (the metric); long: one sequence of "
                         "524288 tokens in a contiguous cache (selection-dominated)")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--cmd", default="", help="command line recorded in a summary")
    ap.add_argument("--out", help="markdown file a summary is written to")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
CALIBRATION_BYTES = 1 << 30


def source_hash():
    """Hash of everything the library is built from (kernels, headers, build)."""
    pkg = os.path.join(ROOT, "trainable_block_sparse_gate_amd")
    files = sorted(glob.glob(os.path.join(pkg, "csrc", "*")) +
                   [os.path.join(pkg, "build.py"), os.path.join(ROOT, "include", "sas.h")])
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
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


def read_counter_csv(d):
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_pmc(fetch_dir, write_dir, cmd, out):
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for r in read_counter_csv(d):
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
    rec = {"source_hash": source_hash(), "command": cmd,
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
             f"the counters are scaled by {f_fetch:.4f} (fetch) and {f_write:.4f} (write).",
             f"Source hash {rec['source_hash']}.", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes / launch |",
             "|---|---|---|---|---|"]
    for k, v in kernels.items():
        lines.append(f"| `{k}` | {v['dispatches']} | {v['fetch_kib']:.0f} | {v['write_kib']:.0f} | "
                     f"{v['bytes_per_launch']:,} |")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as fh:
            fh.write(text)
    print(text)


def summarize_trace(d, cmd, out):
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not stats:
        sys.exit(f"no kernel_stats.csv under {d}")
    with open(stats[0]) as fh:
        rows = list(csv.DictReader(fh))
    info = {}
    if trace:
        with open(trace[0]) as fh:
            for r in csv.DictReader(fh):
                info.setdefault(r["Kernel_Name"], r)

    def name(n):
        m = re.match(r"_ZN3sas\d+(\w+?_kernel)I(\w+?)EEvNS_", n)
        if m:  # template arguments: DF16b = bf16, f = float, Li<n>E = n
            args = re.findall(r"DF16b|f|Li\d+E", m.group(2))
            args = [{"DF16b": "bf16", "f": "float"}.get(a, a[2:-1]) for a in args]
            return f"{m.group(1)}<{', '.join(args)}>"
        m = re.match(r"_ZN3sas\d+(\w+?_kernel)E", n)
        if m:  # mangled, no template arguments
            return f"sas::{m.group(1)}"
        if short_kernel(n):
            return re.sub(r"^void ", "", re.sub(r"\(sas::\w+\)$", "", n))
        m = re.search(r"at::native::[A-Za-z_:]*", n)
        return (m.group(0) if m else n[:48]) + " (torch)"

    lines = ["# Kernel trace summary (rocprofv3 --kernel-trace --stats)", "", "```", cmd, "```",
             "", "| kernel | calls | avg us | total us | % | WGs | WG size | LDS B | VGPR | AGPR |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        n = r["Name"]
        t = info.get(n, {})
        wg = int(t.get("Workgroup_Size_X", 0) or 0)
        grid = int(t.get("Grid_Size_X", 0) or 0) * int(t.get("Grid_Size_Y", 1) or 1) * \
            int(t.get("Grid_Size_Z", 1) or 1)
        nwg = grid // wg if wg else 0
        lines.append(f"| `{name(n)}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['TotalDurationNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} | "
                     f"{nwg} | {wg} | {t.get('LDS_Block_Size', '')} | {t.get('VGPR_Count', '')} | "
                     f"{t.get('Accum_VGPR_Count', '')} |")
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as fh:
            fh.write(text)
    print(text)


def traffic_for(kernel):
    """HBM bytes per launch of `kernel` from profiles/traffic.json, or None
    when there is none or the kernels have changed since it was taken."""
    try:
        with open(TRAFFIC_JSON) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return k["bytes_per_launch"] if k else None


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


def train_bench(args, torch, sas, wl, metrics, case):
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
    for _ in range(args.warmup):
        step(nop)
    torch.cuda.synchronize()
    marks = Marks(torch)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(marks)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    marks.collect()
    ms_step = wall * 1e3 / args.steps
    phases = {n: marks.total[n] / args.steps for n in marks.order}
    fl = metrics.train_flops(case.lengths, case.hq, case.d, case.budget_blocks)
    tflops = (fl["fwd"] + fl["bwd"]) / (ms_step * 1e-3) / 1e12
    log(f"[bench] step {ms_step:.3f} ms  ->  {tflops:.1f} TFLOP/s  phases(ms): " +
        ", ".join(f"{n}={t:.3f}" for n, t in phases.items()))
    # dominant kernel: the largest single-kernel phase
    kern = {"fwd": ("fwd_kernel", fl["fwd"]), "bwd_dq": ("bwd_dq_kernel", fl["dq_kernel"]),
            "bwd_dkdv": ("bwd_dkdv_kernel", fl["dkdv_kernel"])}
    dom = max(kern, key=lambda n: phases.get(n, 0.0))
    achieved = kern[dom][1] / (phases[dom] * 1e-3) / 1e12
    roof = {"kernel": kern[dom][0], "bound": "mfma", "achieved": round(achieved, 2),
            "peak": metrics.PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / metrics.PEAK_BF16_TFLOPS, 4),
            "traffic": traffic_for(kern[dom][0]),
            "ms_per_launch": round(phases[dom], 4)}
    per_kernel = {n: {"ms": round(phases[n], 4),
                      "tflops": round(kern[n][1] / (phases[n] * 1e-3) / 1e12, 2)}
                  for n in kern}
    out = {"ms_per_step": ms_step, "tflops": tflops, "phases_ms": phases, "flops": fl,
           "roofline": roof, "kernels": per_kernel}
    del q, k, v, dO, o, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return out


def decode_bench(args, torch, sas, wl, metrics):
    spec = wl.paged_spec() if args.decode_workload == "paged" else wl.decode_spec(524288)
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
    sel, lg, glse, scores = sas.decode_select(prob, t["q"], ksum)
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
        sas.decode_select(prob, t["q"], ksum, out=(sel, lg, glse, scores))
        e1.record()
        sas.decode(prob, t["q"], t["k"], t["v"], sel, lg, workspace=ws, out=(o, lse))
        e2.record()
        torch.cuda.synchronize()
        if it >= 3:
            t_app += ea.elapsed_time(e0)
            t_sel += e0.elapsed_time(e1)
            t_dec += e1.elapsed_time(e2)
    n = args.decode_steps
    kv = metrics.decode_kv_bytes(spec.seqlens, spec.hkv, spec.d, spec.budget_blocks)
    scan = metrics.decode_scan_bytes(spec.seqlens, spec.hkv, spec.d,
                                     2 if args.summary_dtype == "bf16" else 4)
    gbs = kv / (t_dec / n * 1e-3) / 1e9
    scan_gbs = scan / (t_sel / n * 1e-3) / 1e9
    log(f"[bench] decode {t_dec / n * 1e3:.1f} us for {kv / 2**20:.1f} MiB -> {gbs:.0f} GB/s; "
        f"selection {t_sel / n * 1e3:.1f} us over {scan / 2**20:.1f} MiB summaries; "
        f"append {t_app / n * 1e3:.1f} us")
    del t, flush
    torch.cuda.empty_cache()
    desc = (f"paged: batch {spec.batch}, lengths U[32768,131072]" if spec.paged else
            f"contiguous: batch {spec.batch}, length {spec.seqlens[0]}")
    return {"workload": f"{desc}, 32/8 heads, d128, budget {spec.budget_blocks} blocks",
            "kv_bytes": kv, "us": round(t_dec / n * 1e3, 2), "value": round(gbs, 1),
            "unit": "GB/s", "frac": round(gbs / metrics.PEAK_HBM_GBS, 4),
            "peak": metrics.PEAK_HBM_GBS, "traffic": traffic_for("decode_attend_kernel"),
            "selection": {"us": round(t_sel / n * 1e3, 2), "summary_bytes": scan,
                          "summary_dtype": args.summary_dtype,
                          "GB/s": round(scan_gbs, 1)},
            "append_us": round(t_app / n * 1e3, 2),
            "step_us": round((t_app + t_sel + t_dec) / n * 1e3, 2)}


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


def cpu_baseline(case, metrics):
    """The oracle as it stands, on a bounded sample of the same workload: the
    last NS query blocks of every kv head (steady state: every row keeps the
    full budget), forward and backward; dk/dv are produced for the same key
    blocks, which only those rows can keep."""
    import oracle
    nb = case.qblocks[-1]
    QB = case.total_qblocks
    rm = np.zeros((case.hkv, QB), np.uint8)
    NS = min(128, nb - case.budget_blocks)
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
            "kind": "oracle",
            "sample": (f"fwd+bwd of the last {NS} query blocks of all {case.hkv} kv heads "
                       f"({NS * case.hkv} rows, {pairs} attended pairs) of the same workload, "
                       f"fp64; fwd {t2 - t1:.1f} s, bwd {t3 - t2:.1f} s (bwd parallel over "
                       f"kv heads); gate+Top-K of all rows {t1 - t0:.2f} s not counted"),
            "seconds": round(secs, 2)}


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.cmd, args.out)
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.cmd, args.out)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path shards without exchange over kv heads and sequences)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from trainable_block_sparse_gate_amd import metrics, sas
    from trainable_block_sparse_gate_amd import workloads as wl
    sas.lib()  # fail loudly when the library is missing
    t0 = time.perf_counter()
    case = wl.layer16k() if args.workload == "layer16k" else wl.varlen()
    log(f"[bench] inputs drawn in {time.perf_counter() - t0:.1f} s")
    tr = train_bench(args, torch, sas, wl, metrics, case)
    dec = None if args.no_decode else decode_bench(args, torch, sas, wl, metrics)
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
        "data": "synthetic (seeded normal q/k/v/dO, selector logits N(0,2))",
        "config": {"workload": (f"{case.name}: {len(case.lengths)} x {case.T} tokens, "
                                f"{case.hq}/{case.hkv} heads, head_dim {case.d}, block 64, "
                                f"budget {case.budget_blocks} blocks (incl. current), "
                                "gate+topk+fwd+bwd+gate_bwd"),
                   "tokens": case.T, "budget_blocks": case.budget_blocks,
                   "attended_pairs": tr["flops"]["pairs"],
                   "fwd_flops": tr["flops"]["fwd"], "bwd_flops": tr["flops"]["bwd"]},
        "phases_ms": {k: round(v, 4) for k, v in tr["phases_ms"].items()},
        "kernels": tr["kernels"],
        "roofline": tr["roofline"],
        "decode": dec,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
