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

Prints one JSON line: throughput (tokens/s), a roofline entry for the dominant kernel
(the GEMM launch with the largest time per step), whose duration comes from HIP events
recorded around that kernel on its own stream over a second timed pass, per-GEMM MFMA
and per-kernel HBM fractions, and the CPU oracle timed on a bounded token sample of the
same workload.
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
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the cold-cache pass (per-kernel timing with a 512 MiB device "
                         "write before every step)")
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


def hbm_table(w, kept, backward):
    """Algorithmic HBM bytes of one launch of the memory-bound kernels: each operand
    read once and each result written once (kept rows only)."""
    T, D, E, k = w.T, w.D, w.E, w.k
    es = 2 if w.dtype == "bf16" else 4
    b = {}
    # y = r x + Sh + sum_kept g o: kept expert rows, x, Sh, idx/slot/gate; y written
    b["combine"] = es * D * (kept + (T if w.residual else 0) + (T if w.shared_F else 0) + T) \
        + T * k * 12
    # logits read; idx, gate and the per-block expert partials written
    b["route"] = T * E * 4 + T * k * 8
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
    """The oracle (float64 NumPy) on the first n_tokens tokens of the workload, as a batch
    of its own (its capacity recomputed for that batch size): the forward, and with
    ``backward`` the backward after it."""
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
    t0 = time.perf_counter()
    f = om.forward(x, w.k, w.kind, wts, cf=w.cf, residual=w.residual, shared=shared,
                   bf16=(w.dtype == "bf16"), **kw)
    if backward:
        om.backward(dy, x, w.kind, wts, f["logits"], f["idx"], f["gate"], f["kept"], f["count"],
                    residual=w.residual, shared=shared,
                    w_router=kw.get("w_router") if router_grad else None)
    dt = time.perf_counter() - t0
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
    except Exception:
        pass
    return n_tokens / dt, dt, threads


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


def main():
    args = parse()
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
    out_in = layout == "out_in"
    ex = {"kind": w.kind}
    for key in ("w_in", "w_up", "w_out", "b_in", "b_out"):
        if key in g:
            ex[key] = g[key].transpose(1, 2).contiguous() if out_in and key in ("w_in", "w_up") else g[key]
    shared = None
    if w.shared_F:
        shared = {"kind": "swiglu", "w_in": g["shared_w_in"][None], "w_up": g["shared_w_up"][None],
                  "w_out": g["shared_w_out"][None]}
        if out_in:
            shared["w_in"] = shared["w_in"].transpose(1, 2).contiguous()
            shared["w_up"] = shared["w_up"].transpose(1, 2).contiguous()
            shared["w_in_layout"] = "out_in"
    if out_in:
        ex["w_in_layout"] = "out_in"
        for key in ("w_in", "w_up", "shared_w_in", "shared_w_up"):
            g.pop(key, None)  # the transposed copies replace them in device memory
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

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps

    # second timed pass: HIP events around every kernel, recorded by the library on the
    # stream each kernel is launched on
    ops.profile_enable(True)
    torch.cuda.synchronize()
    p0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof_ms = (time.perf_counter() - p0) * 1e3 / args.steps
    ops.profile_enable(False)
    kern = ops.profile_read()

    # third pass (unless --no-flush): the same per-kernel timing with L2 and the MALL
    # flushed before every step by a 512 MiB device write outside the library's launches
    kern_cold = None
    if not args.no_flush:
        flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for _ in range(args.steps):
            flush_buf.fill_(1)
            ops.profile_enable(True)
            step()
            ops.profile_enable(False)
        torch.cuda.synchronize()
        kern_cold = ops.profile_read()
        del flush_buf

    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    flops = gemm_table(w, kept, backward, router_grad)

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
        for name, by in hbm_table(w, kept, backward).items():
            if name not in kd:
                continue
            cnt, tot = kd[name]
            gbs = by / (tot / cnt * 1e-3) / 1e9
            out[name] = {"avg_launch_ms": round(tot / cnt, 4), "bytes_per_launch": by,
                         "GBs": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
        return out

    gemms = gemm_rows(kern)
    dom = max(gemms, key=lambda n: gemms[n]["ms_per_step"])
    dom_ms = kern[dom][1] / kern[dom][0]
    achieved = flops[dom] / (dom_ms * 1e-3) / 1e12
    src_hash = source_hash(*(("gemm_bf16.hip", "gemm_bf16_tile.h") if w.dtype == "bf16"
                             else ("gemm_f32.hip",)))
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic_record(dom, w.name + ("_w_in_out_in" if out_in else ""), src_hash),
                "algorithmic_flops_per_launch": flops[dom], "avg_launch_ms": round(dom_ms, 4)}
    hbm = hbm_rows(kern)
    roofline_cold = hbm_cold = None
    if kern_cold is not None and dom in kern_cold:
        cold_ms = kern_cold[dom][1] / kern_cold[dom][0]
        cold = flops[dom] / (cold_ms * 1e-3) / 1e12
        roofline_cold = {"bound": "mfma", "kernel": dom, "achieved": round(cold, 2),
                         "peak": peak, "unit": "TFLOP/s", "frac": round(cold / peak, 4),
                         "avg_launch_ms": round(cold_ms, 4),
                         "caches": "L2 and MALL flushed before every step (512 MiB write)"}
        hbm_cold = hbm_rows(kern_cold)

    kernels = {k: {"launches_per_step": round(c / args.steps, 2), "avg_ms": round(t / c, 4)}
               for k, (c, t) in kern.items()}

    cpu = None
    if not args.no_cpu_baseline:
        if args.cpu_tokens:
            n = min(args.cpu_tokens, w.T)
            v, dt, threads = cpu_baseline(w, inp, n, backward, router_grad)
        else:
            # grow the sample until one run takes at least half of --cpu-seconds (the
            # oracle's per-token rate rises with batch size, so a single probe misjudges)
            n = min(w.T, 512)
            while True:
                v, dt, threads = cpu_baseline(w, inp, n, backward, router_grad)
                if n >= w.T or dt >= 0.5 * args.cpu_seconds:
                    break
                grow = max(2.0, min(8.0, args.cpu_seconds / max(dt, 1e-3)))
                n = min(w.T, int(n * grow) // 256 * 256)
        what = "forward + backward" if backward else "forward"
        cpu = {"value": round(v, 2), "unit": "tokens/s", "cores": threads or os.cpu_count(),
               "kind": "oracle", "seconds": round(dt, 2),
               "sample": f"oracle {what} (float64 NumPy) on the first {n} tokens of the "
                         f"workload as a batch of their own"}

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
                   "router_grad": router_grad, "w_in_layout": layout,
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "gemms": gemms,
        "hbm": hbm,
        "roofline_cold": roofline_cold,
        "hbm_cold": hbm_cold,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "profiled_ms_per_step": round(prof_ms, 4),
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
