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
"""
import argparse
import json
import os
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
    return ap.parse_args()


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
            "frac": round(achieved / metrics.PEAK_BF16_TFLOPS, 4), "traffic": None,
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
    spec = wl.paged_spec()
    log(f"[bench] decode workload {spec.name}: batch {spec.batch}, lengths "
        f"{min(spec.seqlens)}..{max(spec.seqlens)}, Kb={spec.budget_blocks}")
    t = wl.draw_decode_device(spec)
    npages = t["k"].shape[0]
    prob = sas.Decode(spec.seqlens, spec.hq, spec.hkv, spec.d, spec.budget_blocks, True,
                      spec.max_len, page_table=t["page_table"], num_pages=npages)
    ksum = sas.pool_keys(prob, t["k"])  # cache maintenance, not timed
    sel, lg, glse, scores = sas.decode_select(prob, t["q"], ksum)
    ws = torch.empty(max(1, sas.decode_workspace_bytes(prob)), dtype=torch.uint8, device="cuda")
    o, lse = sas.decode(prob, t["q"], t["k"], t["v"], sel, lg, workspace=ws)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")  # > Infinity Cache
    torch.cuda.synchronize()
    t_sel = t_dec = 0.0
    for it in range(args.decode_steps + 3):
        flush.zero_()
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record()
        sas.decode_select(prob, t["q"], ksum, out=(sel, lg, glse, scores))
        e1.record()
        sas.decode(prob, t["q"], t["k"], t["v"], sel, lg, workspace=ws, out=(o, lse))
        e2.record()
        torch.cuda.synchronize()
        if it >= 3:
            t_sel += e0.elapsed_time(e1)
            t_dec += e1.elapsed_time(e2)
    n = args.decode_steps
    kv = metrics.decode_kv_bytes(spec.seqlens, spec.hkv, spec.d, spec.budget_blocks)
    scan = metrics.decode_scan_bytes(spec.seqlens, spec.hkv, spec.d)
    gbs = kv / (t_dec / n * 1e-3) / 1e9
    scan_gbs = scan / (t_sel / n * 1e-3) / 1e9
    log(f"[bench] decode {t_dec / n * 1e3:.1f} us for {kv / 2**20:.1f} MiB -> {gbs:.0f} GB/s; "
        f"selection {t_sel / n * 1e3:.1f} us over {scan / 2**20:.1f} MiB summaries")
    del t, flush
    torch.cuda.empty_cache()
    return {"workload": f"paged: batch {spec.batch}, lengths U[32768,131072], 32/8 heads, d128, "
                        f"budget {spec.budget_blocks} blocks",
            "kv_bytes": kv, "us": round(t_dec / n * 1e3, 2), "value": round(gbs, 1),
            "unit": "GB/s", "frac": round(gbs / metrics.PEAK_HBM_GBS, 4),
            "peak": metrics.PEAK_HBM_GBS,
            "selection": {"us": round(t_sel / n * 1e3, 2), "summary_bytes": scan,
                          "GB/s": round(scan_gbs, 1)}}


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
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the path shards without exchange over kv heads and sequences; see DESIGN.md)",
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
