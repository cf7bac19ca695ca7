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


def _layouts(layout):
    """(w_in / w_up transposed, w_out transposed) for a layout name: "in_out" (the pages'
    einsum form), "out_in" (w_in / w_up as torch Linear weights), "out_in_wout" (w_out
    only), "out_in_all" (every weight as a torch Linear weight)."""
    assert layout in ("in_out", "out_in", "out_in_wout", "out_in_all"), layout
    return layout in ("out_in", "out_in_all"), layout in ("out_in_wout", "out_in_all")


def experts_dict(w, g, layout="in_out"):
    tin, tout = _layouts(layout)
    ex = {"kind": w.kind}
    for key in ("w_in", "w_up", "w_out", "b_in", "b_out"):
        if key in g:
            t = (tin and key in ("w_in", "w_up")) or (tout and key == "w_out")
            ex[key] = _out_in(g[key]) if t else g[key]
    if tin:
        ex["w_in_layout"] = "out_in"
    if tout:
        ex["w_out_layout"] = "out_in"
    return ex


def shared_dict(w, g, layout="in_out"):
    if not w.shared_F:
        return None
    tin, tout = _layouts(layout)
    sh = {"kind": "swiglu", "w_in": g["shared_w_in"][None], "w_up": g["shared_w_up"][None],
          "w_out": g["shared_w_out"][None]}
    if tin:
        sh["w_in"], sh["w_up"] = _out_in(sh["w_in"]), _out_in(sh["w_up"])
        sh["w_in_layout"] = "out_in"
    if tout:
        sh["w_out"] = _out_in(sh["w_out"])
        sh["w_out_layout"] = "out_in"
    return sh


def oracle_weights(inp):
    return {k: to_numpy_f32(inp[k]) for k in ("w_in", "w_up", "w_out", "b_in", "b_out") if k in inp}


def oracle_shared(inp):
    if "shared_w_in" not in inp:
        return None
    return {"w_in": to_numpy_f32(inp["shared_w_in"]), "w_up": to_numpy_f32(inp["shared_w_up"]),
            "w_out": to_numpy_f32(inp["shared_w_out"])}


def run_forward(w, inp, g=None, layout="in_out", keep_hidden=False):
    """moe_forward on the workload's inputs; the layouts other than "in_out" hand the
    weights named by _layouts over transposed, with their OUT_IN flags (same products).
    keep_hidden: pass a hidden_cache (returned as "hidden"); without one the hidden
    activation stays in the workspace, as in the benchmark."""
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
                      keep_hidden=keep_hidden, keep_shared_out=True, **kw)
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


def ulp(v, dtype):
    """Spacing of the floating-point grid of ``dtype`` ("bf16" or "f32") at the values v:
    2^(floor(log2|v|) - mantissa bits), and the smallest normal spacing at zero."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    mant = 7 if dtype == "bf16" else 23
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(v > 0, np.exp2(e - mant), np.exp2(-126.0 - mant))


def assert_routed_close(y_got, x, sh_got, o, gate, kept, rms_o, residual, dtype,
                        renormalize=False, what="routed"):
    """The routed part of y, y - r x - Sh, against the oracle's sum over kept choices of
    gate * o. y is rounded once to ``dtype`` after an fp32 sum (x, then Sh, then the
    gated rows), so y - r x - Sh recovers the GPU's routed sum up to half a unit in the
    last place of y plus the fp32 rounding of that sum. The expert rows o themselves are
    held to rtol * (|o| + rms(o)) elementwise, and the gated sum can cancel (two large
    rows of opposite sign), so the bound here is that tolerance carried through the sum:
    rtol * sum_j g_j (|o_j| + rms(o)), plus the two roundings above. This keeps the
    residual's magnitude out of the bound on the experts' contribution."""
    y_got = np.asarray(y_got, dtype=np.float64)
    base = np.zeros_like(y_got)
    if residual:
        base = base + np.asarray(x, dtype=np.float64)
    if sh_got is not None:
        base = base + np.asarray(sh_got, dtype=np.float64)
    routed_got = y_got - base
    o = np.asarray(o, dtype=np.float64)
    g = om.renormalise_kept(gate, kept) if renormalize else np.where(kept, np.asarray(gate, dtype=np.float64), 0.0)
    want = np.einsum("tj,tjd->td", g, o)
    mag = np.einsum("tj,tjd->td", g, np.abs(o)) + rms_o * g.sum(axis=1)[:, None]
    rtol = RTOL[dtype]
    slack = 0.5 * ulp(y_got, dtype) + 8.0 * 2.0 ** -24 * (np.abs(base) + mag)
    err = np.abs(routed_got - want)
    bound = rtol * mag + slack
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), want.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{want.size} outside tolerance; worst at {i}: got "
            f"{routed_got[i]!r} want {want[i]!r} (rtol {rtol}, bound {bound[i]:.3e})")


def gather_kept_rows(h, idx, slot, kept):
    """The GPU's expert_out rows of the kept choices, as [n_tokens, k, D] (zeros where
    dropped), read through the same (expert, slot) pairs the oracle's dispatch gives."""
    eo = h["expert_out"]
    n, k = idx.shape
    got = np.zeros((n, k, eo.shape[-1]), dtype=np.float64)
    tt, jj = np.nonzero(kept)
    got[tt, jj] = eo[idx[tt, jj], slot[tt, jj]]
    return got


def check_outputs(w, inp, h, r, d, tokens=None, idx=None, gate=None, renormalize=False):
    """Every kept expert output row, the shared expert's output, y and the routed part
    of y for the given tokens (all tokens by default), against the oracle. ``idx`` and
    ``gate`` default to the oracle's routing (equal to the GPU's where these are
    called)."""
    T = w.T
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    bf16 = w.dtype == "bf16"
    rtol = RTOL[w.dtype]
    idx = r["idx"] if idx is None else idx
    gate = r["gate"] if gate is None else gate
    x = to_numpy_f32(inp["x"])
    wts = oracle_weights(inp)
    kept = d["kept"][tokens]
    o = om.expert_outputs(w.kind, wts, x, idx, d["kept"], tokens=tokens, bf16=bf16)
    got_o = gather_kept_rows(h, idx[tokens], d["slot"][tokens], kept)
    assert_close(got_o[kept], o[kept], rtol, "expert_out")
    rms_o = float(np.sqrt(np.mean(o[kept] ** 2))) if kept.any() else 0.0
    sh = None
    sh_got = None
    shared = oracle_shared(inp)
    if shared is not None:
        sh = om.shared_apply(shared, x[tokens], bf16=bf16)
        sh_got = h["shared_out"][tokens]
        assert_close(sh_got, sh, rtol, "shared_out")
    y = om.combine(x[tokens], sh, o, gate[tokens], kept, w.residual, renormalize=renormalize)
    if bf16:
        y = om.bf16_round(y)
    assert_close(h["y"][tokens], y, rtol, "y")
    assert_routed_close(h["y"][tokens], x[tokens], sh_got, o, gate[tokens], kept, rms_o,
                        w.residual, w.dtype, renormalize=renormalize)
