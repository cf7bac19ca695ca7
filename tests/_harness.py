"""Shared helpers for the parity tests: moving seeded inputs to the GPU, running the HIP
path through the C ABI, and comparing with the CPU oracle.

Tolerance metric (elementwise): |a - b| <= rtol * (|b| + rms(b)), i.e. relative error on
normal entries with an absolute floor near zeros. fp32 results use rtol 1e-4, bf16
results 2e-2.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle.moe_oracle as om
from workloads import make_inputs, to_numpy_f32

RTOL = {"f32": 1e-4, "bf16": 2e-2}


def assert_close(got, want, rtol, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if want.size == 0:
        return
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = np.abs(got - want)
    bound = rtol * (np.abs(want) + rms)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), want.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{want.size} outside tolerance; worst at {i}: "
            f"got {got[i]!r} want {want[i]!r} (rtol {rtol}, rms {rms:.3e}, "
            f"max normwise {np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300):.3e})")


def gpu_inputs(inp, device="cuda"):
    return {k: v.to(device) for k, v in inp.items()}


def _out_in(t):
    """[.., in, out] -> [.., out, in], contiguous (the OUT_IN storage of w_in / w_up)."""
    return t.transpose(-1, -2).contiguous()


def experts_dict(w, g, layout="in_out"):
    ex = {"kind": w.kind}
    for key in ("w_in", "w_up", "w_out", "b_in", "b_out"):
        if key in g:
            ex[key] = _out_in(g[key]) if layout == "out_in" and key in ("w_in", "w_up") else g[key]
    if layout == "out_in":
        ex["w_in_layout"] = "out_in"
    return ex


def shared_dict(w, g, layout="in_out"):
    if not w.shared_F:
        return None
    sh = {"kind": "swiglu", "w_in": g["shared_w_in"][None], "w_up": g["shared_w_up"][None],
          "w_out": g["shared_w_out"][None]}
    if layout == "out_in":
        sh["w_in"], sh["w_up"] = _out_in(sh["w_in"]), _out_in(sh["w_up"])
        sh["w_in_layout"] = "out_in"
    return sh


def oracle_weights(inp):
    return {k: to_numpy_f32(inp[k]) for k in ("w_in", "w_up", "w_out", "b_in", "b_out") if k in inp}


def oracle_shared(inp):
    if "shared_w_in" not in inp:
        return None
    return {"w_in": to_numpy_f32(inp["shared_w_in"]), "w_up": to_numpy_f32(inp["shared_w_up"]),
            "w_out": to_numpy_f32(inp["shared_w_out"])}


def run_forward(w, inp, g=None, layout="in_out"):
    """moe_forward on the workload's inputs; layout "out_in" hands w_in / w_up over
    transposed ([E, F, D]) with the OUT_IN layout flag (same products)."""
    from sparse_mixture_experts_stable_amd import ops
    g = g if g is not None else gpu_inputs(inp)
    C = ops.capacity(w.T, w.k, w.E, w.cf)
    kw = {}
    if "logits" in g:
        kw["logits"] = g["logits"]
    else:
        kw["w_router"] = g["w_router"]
    out = ops.forward(g["x"], experts_dict(w, g, layout), k=w.k, capacity=C,
                      shared=shared_dict(w, g, layout), use_residual=w.residual,
                      keep_hidden=True, keep_shared_out=True, **kw)
    torch.cuda.synchronize()
    return out, g


def host(out):
    """Copy a dict of device tensors to NumPy (bf16 -> float32)."""
    res = {}
    for k, v in out.items():
        if isinstance(v, torch.Tensor):
            t = v.detach()
            if t.dtype == torch.bfloat16:
                t = t.float()
            res[k] = t.cpu().numpy()
        else:
            res[k] = v
    return res


def check_routing_dispatch(w, inp, h):
    """Bit-exact routing and dispatch given the GPU's fp32 logits; float statistics to
    tolerance. Returns the oracle's routing and dispatch dicts."""
    logits = h["logits"].astype(np.float64)
    T, E = logits.shape
    if "logits" not in inp:
        # logits recomputed in float64 from the same (bf16 or fp32) operands
        want = to_numpy_f32(inp["x"]).astype(np.float64) @ to_numpy_f32(inp["w_router"]).astype(np.float64)
        assert_close(h["logits"], want, 1e-4, "logits")
    else:
        assert np.array_equal(h["logits"], to_numpy_f32(inp["logits"]))
    r = om.route(logits, w.k)
    C = om.capacity(w.T, w.k, w.E, w.cf)
    assert C == h["capacity"]
    d = om.dispatch(r["idx"], E, C)
    assert np.array_equal(h["topk_idx"], r["idx"]), "topk_idx"
    assert np.array_equal(h["expert_count"], r["count"]), "expert_count"
    assert np.array_equal(h["slot"], d["slot"]), "slot"
    assert np.array_equal(h["kept"].astype(bool), d["kept"]), "kept"
    assert np.array_equal(h["slot_assign"], d["slot_assign"]), "slot_assign"
    assert np.array_equal(h["expert_used"], d["used"]), "expert_used"
    assert np.array_equal(h["expert_overflow"], d["overflow"]), "expert_overflow"
    assert np.array_equal(h["token_drops"], d["drops"]), "token_drops"
    assert_close(h["topk_gate"], r["gate"], 1e-4, "topk_gate")
    assert_close(h["prob_sum"], r["prob_sum"], 1e-4, "prob_sum")
    assert abs(float(h["aux_loss"][0]) - r["aux"]) <= 1e-4 * abs(r["aux"]), ("aux", h["aux_loss"], r["aux"])
    return r, d


def check_outputs(w, inp, h, r, d, tokens=None):
    """Expert outputs (kept slots) and y for the given tokens against the oracle."""
    T = w.T
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    bf16 = w.dtype == "bf16"
    rtol = RTOL[w.dtype]
    x = to_numpy_f32(inp["x"])
    wts = oracle_weights(inp)
    o = om.expert_outputs(w.kind, wts, x, r["idx"], d["kept"], tokens=tokens, bf16=bf16)
    # GPU expert_out rows of the kept choices of these tokens
    k = w.k
    got_o = np.zeros_like(o)
    for i, t in enumerate(tokens):
        for j in range(k):
            if d["kept"][t, j]:
                got_o[i, j] = h["expert_out"][r["idx"][t, j], d["slot"][t, j]]
    assert_close(got_o, o, rtol, "expert_out")
    sh = None
    shared = oracle_shared(inp)
    if shared is not None:
        sh = om.shared_apply(shared, x[tokens], bf16=bf16)
        assert_close(h["shared_out"][tokens], sh, rtol, "shared_out")
    y = om.combine(x[tokens], sh, o, r["gate"][tokens], d["kept"][tokens], w.residual)
    if bf16:
        y = om.bf16_round(y)
    assert_close(h["y"][tokens], y, rtol, "y")
