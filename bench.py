"""Throughput of the MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--no-cpu-baseline]
                    [--backward | --forward-only] [--dtype f32] [--router-grad]
    python bench.py --vendor-gemm      (the vendor library's GEMMs on the same shapes)

A step is one moe_forward call over the whole hot path (router GEMM, routing, dispatch,
grouped expert GEMMs with the shared expert, combine, aux loss) on one batch of seeded
synthetic input already resident in HBM; with the backward (the default for the
forward+backward workload 5, or --backward for any fp32 workload) the step is
moe_forward followed by moe_backward. The default workload is T=16384 tokens, d_model
2048, 256 SwiGLU experts (intermediate 512) at top-8 plus one shared SwiGLU expert,
bf16 data with fp32 routing, capacity factor 1.0, forward.

Passes, after a settle phase (untimed steps for at least --settle-s seconds, while the
GPU's clocks ramp up) and W warm-up steps: (1) exactly K steps between two HIP events on the
launch stream, which give ms_per_step and value (inputs resident in HBM, the same batch
every step); (2) K steps with an event pair each (the per-step median); (3) K steps with
HIP events around every kernel on the stream it is launched on (warm per-kernel times);
(4) K steps, each after a 512 MiB device write that flushes L2 and the MALL, with the
per-kernel events again (cold per-kernel times). The roofline entry for the dominant
kernel (the GEMM with the largest time per step), the per-GEMM MFMA fractions and the
per-kernel HBM fractions come from pass 4; the warm figures of pass 3 sit beside them.
The CPU oracle is timed last, median of three runs on a bounded token sample.

--cold-only flushes before every step (warm-up included) and runs only pass 4 (and the
flushed per-step times), so that a profiler's per-kernel averages over the whole
process are flushed launches; value is then the mean flushed step time.

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="oracle sample size in tokens (0 = sized from a short probe run so "
                         "that the timed oracle run takes about --cpu-seconds)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--backward", action="store_true",
                    help="time forward + backward (fp32 experts)")
    ap.add_argument("--forward-only", action="store_true",
                    help="time the forward only, also for the forward+backward workload")
    ap.add_argument("--dtype", choices=["f32", "bf16"], default=None,
                    help="override the workload's data type")
    ap.add_argument("--router-grad", action="store_true",
                    help="with the backward: also the router weight gradient and dx's "
                         "router term (logits = x W_r)")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="instead of the layer: time the vendor library's bf16 GEMMs (torch "
                         "bmm / mm) on the expert GEMM shapes of the SwiGLU workload, as a "
                         "reference point for the MFMA fraction")
    ap.add_argument("--w-in-layout", choices=["auto", "in_out", "out_in"], default="auto",
                    help="storage of w_in / w_up handed to the library: [E, D, F] (in_out) or "
                         "[E, F, D] (out_in, a torch Linear weight per expert; bf16 forward), "
                         "transposed once before timing. auto: out_in for the bf16 SwiGLU "
                         "forward, whose persistent gated GEMM runs faster on it; else in_out")
    ap.add_argument("--w-out-layout", choices=["auto", "in_out", "out_in"], default="auto",
                    help="storage of w_out: [E, F, D] (in_out) or [E, D, F] (out_in, a torch "
                         "Linear weight per expert; bf16 forward), transposed once before "
                         "timing. auto: out_in for the bf16 SwiGLU forward (GEMM-2 reads "
                         "k-contiguous weight tiles); else in_out")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the cold-cache pass (per-kernel timing with a 512 MiB device "
                         "write before every step); the warm per-kernel pass then gives the "
                         "roofline")
    ap.add_argument("--cold-only", action="store_true",
                    help="flush before every step, warm-up included, and run only the cold "
                         "passes (for profiler runs, whose per-kernel averages then cover "
                         "flushed steps only); value is then the mean flushed step time")
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="before the warm-up steps, run the step untimed for at least this many "
                         "seconds: the first ~20 launches of a process run 10-40%% slower while "
                         "the GPU's clocks ramp up")
    ap.add_argument("--summarize-trace", default=None, metavar="CSV",
                    help="instead of running: print per-kernel durations from a rocprofv3 "
                         "--kernel-trace CSV (kernel_trace.csv), over the last --last dispatches "
                         "of each kernel name")
    ap.add_argument("--last", type=int, default=40)
    ap.add_argument("--summarize-traffic", nargs=2, default=None, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="instead of running: HBM bytes per launch of every moe kernel from two "
                         "rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE; "
                         "counter_collection.csv), calibrated on the largest device copy of the "
                         "run (--calib-copy-mib), as a markdown table")
    ap.add_argument("--record", default=None, metavar="KEY=KERNEL",
                    help="with --summarize-traffic: store the bytes per launch of the kernel "
                         "whose name contains KERNEL in profiles/traffic.json under KEY (with "
                         "the current GEMM source hash)")
    ap.add_argument("--summarize-mfma", default=None, metavar="CSV",
                    help="instead of running: MFMA work, MFMA busy fraction and engine clock per "
                         "GEMM dispatch from a rocprofv3 --pmc pass over "
                         "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES "
                         "GRBM_GUI_ACTIVE, as a markdown table")
    ap.add_argument("--algo", action="append", default=[], metavar="KERNEL=GFLOP",
                    help="with --summarize-mfma: algorithmic GFLOP per launch of the kernel "
                         "whose name contains KERNEL")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before warmup, run one plain device copy of this many MiB (a "
                         "known-size reference for hardware byte counters)")
    return ap.parse_args()


def gemm_table(w, kept, backward, router_grad):
    """Algorithmic FLOPs of one launch of each GEMM kernel a step launches, by kernel
    name: 2 * rows * inner * outer per product, over the kept rows only (the shared expert
    and the router over all T rows). Forward: the first expert GEMM has two weight
    matrices (gate, up) for SwiGLU. Backward, per expert set: dH = dO W_out^T, the
    pre-activation recompute, dW_out = H^T dO, dW_in (and dW_up) = X^T dZ, and the input
    gradient dZ W_in^T (SwiGLU: two launches, one per weight)."""
    T, D, E, Fs = w.T, w.D, w.E, w.shared_F
    F = w.F if w.kind != "linear" else w.D
    mats = 2 if w.kind == "swiglu" else 1
    g1 = 2.0 * kept * D * F * mats
    g2 = 2.0 * kept * F * D
    f = {}
    if w.dtype == "bf16":
        f["expert_gemm1_swiglu" if w.kind == "swiglu" else "expert_gemm1"] = (
            g1 + (4.0 * T * D * Fs if Fs else 0.0))
        f["expert_gemm2"] = (g2 if w.kind != "linear" else 0.0) + (2.0 * T * Fs * D if Fs else 0.0)
        f["router_gemm"] = 2.0 * T * D * E
    else:
        f["expert_gemm1_swiglu_f32" if w.kind == "swiglu" else "expert_gemm1_f32"] = g1
        if w.kind != "linear":
            f["expert_gemm2_f32"] = g2
        if Fs:
            f["shared_gemm1_swiglu_f32"] = 4.0 * T * D * Fs
            f["shared_gemm2_f32"] = 2.0 * T * Fs * D
        f["router_gemm_f32"] = 2.0 * T * D * E
    if backward:
        if w.kind == "linear":
            f["bwd_dx_gemm"] = 2.0 * kept * D * D
            f["bwd_dw_gemm"] = 2.0 * kept * D * D
        else:
            for pre, rows, FF, m in (("bwd_", kept, F, mats), ("bwd_shared_", T, Fs, 2)):
                if pre == "bwd_shared_" and not Fs:
                    continue
                one = 2.0 * rows * D * FF
                f[pre + "dh_gemm"] = one
                f[pre + ("swiglu_recompute" if m == 2 else "gelu_recompute")] = one * m
                f[pre + "dw_out_gemm"] = one
                f[pre + "dw_in_gemm"] = one
                if m == 2:
                    f[pre + "dw_up_gemm"] = one
                f[pre + "dx_gemm"] = one
        if Fs and w.kind == "linear":
            for nm in ("dh_gemm", "swiglu_recompute", "dw_out_gemm", "dw_in_gemm",
                       "dw_up_gemm", "dx_gemm"):
                f["bwd_shared_" + nm] = 2.0 * T * D * Fs * (2 if nm == "swiglu_recompute" else 1)
        if router_grad:
            f["bwd_dw_router_gemm"] = 2.0 * T * D * E
            f["bwd_dx_router_gemm"] = 2.0 * T * D * E
    return f


def hbm_table(w, kept, backward, C=0):
    """Algorithmic HBM bytes of one launch of the memory- and latency-bound kernels: each
    operand read once and each result written once (kept rows only)."""
    T, D, E, k = w.T, w.D, w.E, w.k
    es = 2 if w.dtype == "bf16" else 4
    nb = -(-T // 32)            # routing blocks (32 tokens each): per-block partials
    nc = -(-nb // 16)           # scan chunks (16 routing blocks each)
    b = {}
    # y = r x + Sh + sum_kept g o: kept expert rows, x, Sh, idx/slot/gate; y written
    b["combine"] = es * D * (kept + (T if w.residual else 0) + (T if w.shared_F else 0) + T) \
        + T * k * 12
    # logits read; idx and gate written; per-block expert counts and probability sums
    b["route"] = T * E * 4 + T * k * 8 + nb * E * 8
    if w.logits_mode == "router":
        # x and W_r read, fp32 logits written
        b["router_gemm" if w.dtype == "bf16" else "router_gemm_f32"] = \
            T * D * es + D * E * es + T * E * 4
    # per-block partials read, chunk sums written
    b["chunk_sum"] = nb * E * 8 + nc * E * 8
    # idx, the block partials before each block and the chunk sums read; slot, kept,
    # slot_assign, drops and the per-expert totals (count, used, overflow, prob_sum,
    # aux) written
    b["assign"] = T * k * 4 + nb * E * 4 + nc * E * 8 + T * k * 5 + E * C * 4 + T * 4 + E * 16
    if backward:
        # dy, kept expert rows, logits, idx/gate/slot read; dgate, dlogits written
        b["dgate_router_bwd"] = 4 * D * (T + kept) + T * E * 4 * 2 + T * k * 16
    return b


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_mixture_experts_stable_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_record(kernel, workload_name, src_hash):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        recs = json.load(open(p))
    except Exception:
        return None
    r = recs.get(f"{kernel}:{workload_name}")
    if not r or r.get("source_hash") != src_hash:
        return None
    return r.get("bytes_per_launch")


def cpu_baseline(w, inp, n_tokens, backward=False, router_grad=False):
    """A callable running the oracle (float64 NumPy) once on the first n_tokens tokens of
    the workload, as a batch of their own (capacity recomputed for that batch size): the
    forward, and with ``backward`` the backward after it; it returns the seconds taken
    (input conversion excluded)."""
    import numpy as np
    import oracle.moe_oracle as om
    from workloads import to_numpy_f32

    x = to_numpy_f32(inp["x"][:n_tokens])
    wts = {k: to_numpy_f32(inp[k]) for k in ("w_in", "w_up", "w_out", "b_in", "b_out") if k in inp}
    shared = None
    if "shared_w_in" in inp:
        shared = {"w_in": to_numpy_f32(inp["shared_w_in"]), "w_up": to_numpy_f32(inp["shared_w_up"]),
                  "w_out": to_numpy_f32(inp["shared_w_out"])}
    kw = {}
    if "logits" in inp:
        kw["logits"] = to_numpy_f32(inp["logits"][:n_tokens])
    else:
        kw["w_router"] = to_numpy_f32(inp["w_router"])
    dy = to_numpy_f32(inp["dy"][:n_tokens]) if backward else None

    def once():
        t0 = time.perf_counter()
        f = om.forward(x, w.k, w.kind, wts, cf=w.cf, residual=w.residual, shared=shared,
                       bf16=(w.dtype == "bf16"), **kw)
        if backward:
            om.backward(dy, x, w.kind, wts, f["logits"], f["idx"], f["gate"], f["kept"],
                        f["count"], residual=w.residual, shared=shared,
                        w_router=kw.get("w_router") if router_grad else None)
        return time.perf_counter() - t0

    return once


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
    except Exception:
        return None


def vendor_gemm(steps):
    """The vendor library's bf16 GEMMs on the expert GEMM shapes of the SwiGLU workload
    (E=256 experts x C=512 rows, d_model 2048, intermediate 512): batched (one GEMM per
    expert, gate and up stacked as 1024 columns) and as one dense GEMM over all E*C rows;
    plus a square 8192 GEMM. Same FLOP accounting as the layer's GEMMs."""
    import torch
    bf = torch.bfloat16
    E, C, D, F = 256, 512, 2048, 512
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn(E, C, D, device="cuda", dtype=bf, generator=g)
    w1 = torch.randn(E, D, 2 * F, device="cuda", dtype=bf, generator=g)
    h = torch.randn(E, C, F, device="cuda", dtype=bf, generator=g)
    w2 = torch.randn(E, F, D, device="cuda", dtype=bf, generator=g)
    o1 = torch.empty(E, C, 2 * F, device="cuda", dtype=bf)
    o2 = torch.empty(E, C, D, device="cuda", dtype=bf)
    X, W1, O1 = x.reshape(E * C, D), w1[0].contiguous(), o1.reshape(E * C, 2 * F)
    H, W2, O2 = h.reshape(E * C, F), w2[0].contiguous(), o2.reshape(E * C, D)
    A = torch.randn(8192, 8192, device="cuda", dtype=bf, generator=g)
    B = torch.randn(8192, 8192, device="cuda", dtype=bf, generator=g)
    Cc = torch.empty_like(A)
    cases = [
        ("bmm [256,512,2048] x [256,2048,1024] (GEMM-1 shape)", lambda: torch.bmm(x, w1, out=o1), 2.0 * E * C * D * 2 * F),
        ("bmm [256,512,512] x [256,512,2048] (GEMM-2 shape)", lambda: torch.bmm(h, w2, out=o2), 2.0 * E * C * F * D),
        ("mm [131072,2048] x [2048,1024]", lambda: torch.mm(X, W1, out=O1), 2.0 * E * C * D * 2 * F),
        ("mm [131072,512] x [512,2048]", lambda: torch.mm(H, W2, out=O2), 2.0 * E * C * F * D),
        ("mm [8192,8192] x [8192,8192]", lambda: torch.mm(A, B, out=Cc), 2.0 * 8192 ** 3),
    ]
    res = {}
    for name, fn, fl in cases:
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = fl / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    print(json.dumps({"vendor_gemm": "torch (hipBLASLt) bf16", "peak_tflops": PEAK_BF16_TFLOPS,
                      "results": res}), flush=True)


def summarize_trace(path, last):
    """Per-kernel dispatch durations (microseconds) from a rocprofv3 kernel trace: count,
    average, minimum and maximum over the last `last` dispatches of each kernel name, as a
    markdown table, with the whole-trace average beside it."""
    import csv
    import statistics
    runs = {}
    for r in csv.DictReader(open(path)):
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        runs.setdefault(r["Kernel_Name"], []).append(d)
    print(f"| kernel | dispatches | last {last}: avg us | min us | max us | all: avg us |")
    print("|---|---|---|---|---|---|")
    for name, ds in sorted(runs.items(), key=lambda kv: -sum(kv[1][-last:])):
        tail = ds[-last:]
        short = name.replace("void ", "").split("(")[0]
        print(f"| `{short}` | {len(ds)} | {statistics.mean(tail):.1f} | {min(tail):.1f} | "
              f"{max(tail):.1f} | {statistics.mean(ds):.1f} |")


def _short_name(n):
    return n.replace("void ", "").split("(")[0]


def _pmc_rows(path):
    import csv
    return list(csv.DictReader(open(path)))


def summarize_traffic(fetch_csv, write_csv, record=None):
    """HBM bytes per launch from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled
    by what the counter reads for the run's largest device copy (a copy of G bytes reads
    G and writes G): average over every profiled launch of each moe kernel."""
    import statistics

    def per_kernel(path):
        out = {}
        for r in _pmc_rows(path):
            out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return out

    fe, wr = per_kernel(fetch_csv), per_kernel(write_csv)

    def copy_counter(vals):
        c = [x for n, v in vals.items() if n.startswith("__amd_rocclr_copyBuffer") for x in v]
        if not c:
            sys.exit("no device copy in the counter pass (run it with --calib-copy-mib)")
        return max(c)

    cf, cw = copy_counter(fe), copy_counter(wr)
    gib_kib = (1 << 30) / 1024.0
    ffac, wfac = gib_kib / cf, gib_kib / cw   # calibrated KiB per counter unit (1 GiB copy)
    rows = []
    for n in fe:
        if "moe::" not in n:
            continue
        rd = statistics.mean(fe[n]) * ffac * 1024
        wt = statistics.mean(wr.get(n, [0.0])) * wfac * 1024
        rows.append((n, len(fe[n]), rd, wt))
    rows.sort(key=lambda r: -(r[2] + r[3]))
    print(f"Calibration: the 1 GiB device copy (`__amd_rocclr_copyBuffer`, 1 GiB read and 1 GiB "
          f"written) reads FETCH_SIZE = {cf:.0f} KiB and WRITE_SIZE = {cw:.0f} KiB, so measured "
          f"bytes = FETCH_SIZE x {ffac:.3f} KiB and WRITE_SIZE x {wfac:.3f} KiB.\n")
    print("| kernel | launches | read MB (calibrated) | written MB (calibrated) |")
    print("|---|---|---|---|")
    for n, c, rd, wt in rows:
        print(f"| `{_short_name(n)}` | {c} | {rd / 1e6:.1f} | {wt / 1e6:.1f} |")
    if record:
        key, sub = record.split("=", 1)
        hit = [r for r in rows if sub in r[0]]
        if len(hit) != 1:
            sys.exit(f"--record: {len(hit)} kernels match {sub!r}")
        name, _, rd, wt = hit[0]
        srcs = ("gemm_f32.hip",) if "gemm_f32" in name else ("gemm_bf16.hip", "gemm_bf16_tile.h")
        p = os.path.join(ROOT, "profiles", "traffic.json")
        recs = json.load(open(p)) if os.path.exists(p) else {}
        recs[key] = {"bytes_per_launch": int(rd + wt), "read_bytes": int(rd), "written_bytes": int(wt),
                     "source_hash": source_hash(*srcs),
                     "calibration": {"fetch_kib_factor": round(ffac, 4), "write_kib_factor": round(wfac, 4)}}
        with open(p, "w") as f:
            json.dump(recs, f, indent=1)
            f.write("\n")


def summarize_mfma(path, algo):
    """Per GEMM kernel, over its last 6 profiled dispatches: MFMA FLOPs (MOPS x 512),
    MFMA busy against 2.4 GHz and against the engine clock of the dispatch
    (GRBM_GUI_ACTIVE / 8 XCDs / duration)."""
    import statistics
    d = {}
    for r in _pmc_rows(path):
        e = d.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"], "start": int(r["Start_Timestamp"]),
                                             "end": int(r["End_Timestamp"])})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    per = {}
    for e in d.values():
        if "moe::" in e["name"] and "gemm" in e["name"]:
            per.setdefault(_short_name(e["name"]), []).append(e)
    algo = dict(a.split("=", 1) for a in algo)
    print("| kernel | launches | MFMA FLOPs (G) | algorithmic (G) | duration (us) | MFMA busy | "
          "clock (GHz) | busy at that clock |")
    print("|---|---|---|---|---|---|---|---|")
    for n, es in sorted(per.items(), key=lambda kv: -statistics.mean(x["end"] - x["start"] for x in kv[1])):
        es = es[-6:]
        dur = statistics.mean((x["end"] - x["start"]) * 1e-9 for x in es)
        fl = statistics.mean(x.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for x in es) * 512
        busy = statistics.mean(x.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for x in es)
        clk = statistics.mean(x.get("GRBM_GUI_ACTIVE", 0.0) for x in es) / 8 / dur
        a = next((v for k, v in algo.items() if k in n), "-")
        print(f"| `{n}` | {len(es)} | {fl / 1e9:.1f} | {a} | {dur * 1e6:.1f} | "
              f"{busy / (1024 * 2.4e9 * dur):.1%} | {clk / 1e9:.2f} | {busy / (1024 * clk * dur):.1%} |")


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.last)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, record=args.record)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma, args.algo)
        return
    if args.vendor_gemm:
        vendor_gemm(args.steps)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU "
              "expert parallelism is not implemented.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from sparse_mixture_experts_stable_amd import ops
    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    backward = (w.backward or args.backward) and not args.forward_only
    if args.dtype and args.dtype != w.dtype:
        w = w.scaled(dtype=args.dtype, name=w.name.replace("_bf16", "").replace("_f32", "")
                     + "_" + args.dtype)
    if backward and not w.backward:
        w = w.scaled(backward=True, name=w.name + "_fwd_bwd")
    if backward and w.dtype != "f32":
        print("the backward runs on fp32 experts: add --dtype f32", file=sys.stderr)
        sys.exit(2)
    router_grad = backward and args.router_grad and w.logits_mode == "router"
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    inp = make_inputs(w)
    g = {k: v.to("cuda") for k, v in inp.items()}
    gen_s = time.perf_counter() - t_gen
    layout = args.w_in_layout
    if layout == "auto":
        layout = "out_in" if w.dtype == "bf16" and w.kind == "swiglu" and not backward else "in_out"
    out_layout = args.w_out_layout
    if out_layout == "auto":
        out_layout = "out_in" if w.dtype == "bf16" and w.kind == "swiglu" and not backward else "in_out"
    out_in, wout_t = layout == "out_in", out_layout == "out_in"
    tr = lambda t: t.transpose(-1, -2).contiguous()
    ex = {"kind": w.kind}
    for key in ("w_in", "w_up", "w_out", "b_in", "b_out"):
        if key in g:
            t = (out_in and key in ("w_in", "w_up")) or (wout_t and key == "w_out")
            ex[key] = tr(g[key]) if t else g[key]
    shared = None
    if w.shared_F:
        shared = {"kind": "swiglu", "w_in": g["shared_w_in"][None], "w_up": g["shared_w_up"][None],
                  "w_out": g["shared_w_out"][None]}
        if out_in:
            shared["w_in"], shared["w_up"] = tr(shared["w_in"]), tr(shared["w_up"])
            shared["w_in_layout"] = "out_in"
        if wout_t:
            shared["w_out"] = tr(shared["w_out"])
            shared["w_out_layout"] = "out_in"
    if out_in:
        ex["w_in_layout"] = "out_in"
        for key in ("w_in", "w_up", "shared_w_in", "shared_w_up"):
            g.pop(key, None)  # the transposed copies replace them in device memory
    if wout_t:
        ex["w_out_layout"] = "out_in"
        for key in ("w_out", "shared_w_out"):
            g.pop(key, None)
    C = ops.capacity(w.T, w.k, w.E, w.cf)
    kw = {"logits": g["logits"]} if "logits" in g else {"w_router": g["w_router"]}
    out = ops.forward(g["x"], ex, k=w.k, capacity=C, shared=shared, use_residual=w.residual, **kw)
    calls = [out["_call"]]
    if backward:
        grads = ops.backward(g["dy"], g["x"], ex, out, k=w.k, use_residual=w.residual,
                             shared=shared, w_router=g["w_router"] if router_grad else None)
        calls.append(grads["_call"])

    def step():
        for c in calls:
            c()

    torch.cuda.synchronize()
    kept = int(out["kept"].sum().item())
    stream = torch.cuda.current_stream()
    # L2 (4 MiB per XCD) and the 256 MiB MALL are flushed by a 512 MiB device write
    # before every step of the cold passes; the write is outside the library's launches
    flush_buf = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device="cuda")

    def flush():
        flush_buf.fill_(1)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # settle: untimed steps until the clocks have ramped up (then the W warm-up steps)
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        if args.cold_only:
            flush()
        step()
        torch.cuda.synchronize()
        settle_steps += 1
    for _ in range(args.warmup):
        if args.cold_only:
            flush()
        step()
    torch.cuda.synchronize()

    def timed_steps(cold):
        """Per-step times from HIP events on the launch stream (a flush, if any, runs
        before the step's first event)."""
        evs = []
        for _ in range(args.steps):
            if cold:
                flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    kern_warm = kern_cold = None
    step_ms_warm = step_ms_cold = None
    prof_ms = None
    if not args.cold_only:
        # the timed pass: exactly K steps between two events, synchronised on both sides
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(args.steps):
            step()
        t1.record(stream)
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / args.steps
        step_ms_warm = timed_steps(False)
        # per-kernel pass: HIP events around every kernel, recorded by the library on
        # the stream each kernel is launched on
        ops.profile_enable(True)
        torch.cuda.synchronize()
        p0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        prof_ms = (time.perf_counter() - p0) * 1e3 / args.steps
        ops.profile_enable(False)
        kern_warm = ops.profile_read()
    if flush_buf is not None:
        step_ms_cold = timed_steps(True)
        for _ in range(args.steps):
            flush()
            ops.profile_enable(True)
            step()
            ops.profile_enable(False)
        torch.cuda.synchronize()
        kern_cold = ops.profile_read()
        del flush_buf
    if args.cold_only:
        ms = sum(step_ms_cold) / len(step_ms_cold)

    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    flops = gemm_table(w, kept, backward, router_grad)
    C_ = ops.capacity(w.T, w.k, w.E, w.cf)

    def gemm_rows(kd):
        out = {}
        for name, fl in flops.items():
            if name not in kd or fl <= 0:
                continue
            cnt, tot = kd[name]
            avg = tot / cnt
            ach = fl / (avg * 1e-3) / 1e12
            out[name] = {"ms_per_step": round(tot / args.steps, 4), "avg_launch_ms": round(avg, 4),
                         "tflops": round(ach, 2), "frac": round(ach / peak, 4)}
        return out

    def hbm_rows(kd):
        out = {}
        for name, by in hbm_table(w, kept, backward, C_).items():
            if name not in kd:
                continue
            cnt, tot = kd[name]
            gbs = by / (tot / cnt * 1e-3) / 1e9
            out[name] = {"avg_launch_ms": round(tot / cnt, 4), "bytes_per_launch": by,
                         "GBs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
        return out

    src_hash = source_hash(*(("gemm_bf16.hip", "gemm_bf16_tile.h") if w.dtype == "bf16"
                             else ("gemm_f32.hip",)))

    def roofline_of(kd, caches, with_traffic):
        gemms = gemm_rows(kd)
        dom = max(gemms, key=lambda n: gemms[n]["ms_per_step"])
        dom_ms = kd[dom][1] / kd[dom][0]
        ach = flops[dom] / (dom_ms * 1e-3) / 1e12
        r = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 2), "peak": peak,
             "unit": "TFLOP/s", "frac": round(ach / peak, 4),
             "traffic": (traffic_record(dom, w.name + ("_w_in_out_in" if out_in else ""), src_hash)
                         if with_traffic else None),
             "algorithmic_flops_per_launch": flops[dom], "avg_launch_ms": round(dom_ms, 4),
             "launches": kd[dom][0], "caches": caches}
        return r, gemms

    cold_note = "L2 and MALL flushed before every step (512 MiB device write)"
    roofline = roofline_warm = None
    gemms = gemms_warm = hbm = hbm_warm = None
    if kern_cold is not None:
        roofline, gemms = roofline_of(kern_cold, cold_note, True)
        hbm = hbm_rows(kern_cold)
    if kern_warm is not None:
        roofline_warm, gemms_warm = roofline_of(kern_warm, "warm: the same input on every step",
                                                kern_cold is None)
        hbm_warm = hbm_rows(kern_warm)
    if roofline is None:
        roofline, gemms, hbm = roofline_warm, gemms_warm, hbm_warm
        roofline_warm = gemms_warm = hbm_warm = None
    kern = kern_cold if kern_cold is not None else kern_warm
    kernels = {k: {"launches_per_step": round(c / args.steps, 2), "avg_ms": round(t / c, 4)}
               for k, (c, t) in kern.items()}

    def med(v):
        return None if not v else round(float(np.median(v)), 4)

    cpu = None
    if not args.no_cpu_baseline:
        if args.cpu_tokens:
            n = min(args.cpu_tokens, w.T)
            run = cpu_baseline(w, inp, n, backward, router_grad)
            dt = run()
        else:
            # grow the sample until one run takes at least half of --cpu-seconds (the
            # oracle's per-token rate rises with batch size, so a single probe misjudges)
            n = min(w.T, 512)
            while True:
                run = cpu_baseline(w, inp, n, backward, router_grad)
                dt = run()
                if n >= w.T or dt >= 0.5 * args.cpu_seconds:
                    break
                grow = max(2.0, min(8.0, args.cpu_seconds / max(dt, 1e-3)))
                n = min(w.T, int(n * grow) // 256 * 256)
        # median of three runs at the final sample size (one if a run exceeds 30 s)
        runs = [dt]
        if dt <= 30.0:
            runs += [run(), run()]
        dt = float(np.median(runs))
        what = "forward + backward" if backward else "forward"
        nblas = blas_threads()
        affinity = len(os.sched_getaffinity(0))
        cpu = {"value": round(n / dt, 2), "unit": "tokens/s", "cores": nblas or affinity,
               "kind": "oracle", "seconds": round(dt, 2), "runs_s": [round(r, 2) for r in runs],
               "affinity_cores": affinity, "blas_threads": nblas,
               "sample": f"oracle {what} (float64 NumPy, its matrix products on "
                         f"{nblas or affinity} BLAS threads) on the first {n} tokens of the "
                         f"workload as a batch of their own; median of {len(runs)} runs"}

    rec = {
        "metric": ("MoE layer fwd tokens/s (E=256,k=8,D=2048) + MFMA % / HBM GB/s of peak"
                   if not backward else
                   f"MoE layer fwd+bwd tokens/s (E={w.E},k={w.k},D={w.D}) + MFMA % / HBM GB/s of peak"),
        "value": round(w.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded normal inputs and random-init weights)",
        "config": {"workload": w.name, "T": w.T, "d_model": w.D, "experts": w.E, "top_k": w.k,
                   "expert": w.kind, "d_hidden": w.F, "shared_hidden": w.shared_F,
                   "capacity": C, "capacity_factor": w.cf, "kept_assignments": kept,
                   "step": "forward + backward" if backward else "forward",
                   "router_grad": router_grad, "w_in_layout": layout, "w_out_layout": out_layout,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "gemms": gemms,
        "hbm": hbm,
        "roofline_warm": roofline_warm,
        "gemms_warm": gemms_warm,
        "hbm_warm": hbm_warm,
        "step_ms_median": {"warm": med(step_ms_warm), "cold": med(step_ms_cold)},
        "cpu_baseline": cpu,
        "kernels": kernels,
        "profiled_ms_per_step": None if prof_ms is None else round(prof_ms, 4),
        "settle_steps": settle_steps,
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
