"""GPU parity for the router variants of "Module 7. Mixture of Experts": sigmoid scoring
with log-space gates, a selection-only bias, survivor renormalisation and the router
z-loss, through routing, the whole forward and the backward, against the CPU oracle.

Selection is bit-exact wherever it is decided by the logits alone. With a selection bias
the key is the fp32 clean score plus the bias on the GPU and the float64 one in the
oracle; where the oracle's k-th and (k+1)-th keys lie within 1e-6 of each other either
choice is correct, so there the GPU's choice is checked for validity (its keys are a
top-k of the oracle's keys up to that margin) instead of equality.
"""

import numpy as np
import pytest
import torch

import oracle.moe_oracle as om
from tests import _harness as H
from workloads import WORKLOADS, make_inputs, to_numpy_f32

pytestmark = pytest.mark.gpu

TIE = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ops():
    from sparse_mixture_experts_stable_amd import ops
    return ops


def _keys(r, bias):
    """The oracle's selection keys."""
    return r["clean"] + bias[None, :]


def _check_selection(got_idx, r, bias, k, max_frac=0.01):
    """Equal to the oracle's idx, except on tokens whose boundary keys are near-tied;
    there the GPU's choice must be a valid top-k of the oracle's keys. Returns the mask
    of tokens whose choice equals the oracle's."""
    want = r["idx"]
    same = np.all(got_idx == want, axis=1)
    if same.all():
        return same
    assert bias is not None, "selection by logit must be bit-exact"
    keys = _keys(r, bias)
    bad = np.flatnonzero(~same)
    assert bad.size <= max(1, int(max_frac * got_idx.shape[0])), f"{bad.size} tokens differ"
    for t in bad:
        kg = np.sort(keys[t, got_idx[t]])[::-1]
        kw = np.sort(keys[t, want[t]])[::-1]
        assert np.all(np.abs(kg - kw) <= TIE), (t, kg, kw)
        assert len(set(got_idx[t].tolist())) == k
    return same


# ---------------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------------

def test_page_sigmoid_router_example():
    """The printed Module 7 router example (sigmoid, top-4 of 8, with and without the
    selection bias) and its extreme-logit cases, through moe_route."""
    import json
    import os
    ops = _ops()
    ref = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                      "p3_reference.json")))["router"]
    lg = torch.tensor([ref["logits"]], dtype=torch.float32, device="cuda")
    out = ops.route(logits=lg, k=4, scoring="sigmoid")
    assert out["topk_idx"].cpu().tolist() == [ref["selected"]]
    np.testing.assert_allclose(out["topk_gate"].cpu().numpy()[0], ref["gates"], rtol=1e-6)
    b = torch.tensor(ref["bias"], dtype=torch.float32, device="cuda")
    out = ops.route(logits=lg, k=4, scoring="sigmoid", selection_bias=b)
    assert out["topk_idx"].cpu().tolist() == [ref["selected_with_bias"]]
    np.testing.assert_allclose(out["topk_gate"].cpu().numpy()[0], ref["gates_with_bias"], rtol=1e-6)
    for row, want in (([-1002.0, -1000.0, -1001.0], [1, 2]),
                      ([-1002.0, -1000.0, -1001.0, -1003.0], [1, 2])):
        out = ops.route(logits=torch.tensor([row], device="cuda"), k=2, scoring="sigmoid")
        g = out["topk_gate"].cpu().numpy()[0]
        assert out["topk_idx"].cpu().tolist() == [want]
        assert np.all(np.isfinite(g))
        np.testing.assert_allclose(g, [1 / (1 + np.exp(-1)), 1 / (1 + np.exp(1))], rtol=1e-6)


def test_page_z_loss_example():
    """router_z_loss on the printed Module 7 aux logits (13.363987745409077) and the
    two-token square-before-mean example."""
    import json
    import math
    import os
    ops = _ops()
    ref = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                      "p3_reference.json")))["losses"]
    lg = torch.tensor(ref["aux_logits"], dtype=torch.float32, device="cuda")
    out = ops.route(logits=lg, k=1, z_loss=True)
    assert math.isclose(out["z_loss"].item(), ref["z_loss"], rel_tol=1e-6)
    assert math.isclose(out["aux_loss"].item(), ref["switch_aux"], rel_tol=1e-6)
    two = torch.tensor([[0.0, 0.0], [2.0, 2.0]], device="cuda")
    z = ops.route(logits=two, k=1, z_loss=True)["z_loss"].item()
    assert math.isclose(z, (math.log(2) ** 2 + (2 + math.log(2)) ** 2) / 2, rel_tol=1e-6)


@pytest.mark.parametrize("T,E,k", [(1000, 64, 4), (333, 256, 8), (50, 8, 2), (4097, 16, 1)])
@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_route_variants(T, E, k, scoring, with_bias):
    ops = _ops()
    rng = np.random.default_rng(T + E + k)
    logits = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    logits[::7, 1] = logits[::7, 0]            # exact logit ties
    bias = (rng.standard_normal(E) * 0.05).astype(np.float32) if with_bias else None
    out = ops.route(logits=torch.tensor(logits, device="cuda"), k=k, scoring=scoring,
                    selection_bias=torch.tensor(bias, device="cuda") if with_bias else None,
                    z_loss=True)
    torch.cuda.synchronize()
    h = H.host(out)
    b64 = None if bias is None else bias.astype(np.float64)
    r = om.route(logits.astype(np.float64), k, scoring=scoring, selection_bias=b64)
    same = _check_selection(h["topk_idx"], r, b64, k)
    H.assert_close(h["topk_gate"][same], r["gate"][same], 1e-4, "gate")
    np.testing.assert_allclose(h["topk_gate"].sum(1), 1.0, atol=1e-5)
    got_count = np.bincount(h["topk_idx"].ravel(), minlength=E)
    assert np.array_equal(h["expert_count"], got_count)
    if same.all():
        assert np.array_equal(h["expert_count"], r["count"])
        H.assert_close(h["aux_loss"], np.array([r["aux"]]), 1e-4, "aux")
    H.assert_close(h["prob_sum"], r["prob_sum"], 1e-4, "prob_sum")
    H.assert_close(h["z_loss"], np.array([r["z_loss"]]), 1e-4, "z_loss")


# ---------------------------------------------------------------------------------
# whole forward and backward
# ---------------------------------------------------------------------------------

CASES = {
    "gelu_f32": WORKLOADS[1].scaled(backward=True),
    "swiglu_bf16_shared": WORKLOADS[3].scaled(T=1024, D=256, E=32, F=128, shared_F=128),
    "swiglu_f32_shared": WORKLOADS[3].scaled(T=1024, D=256, E=32, F=128, shared_F=128,
                                             dtype="f32", backward=True),
    "linear_f32": WORKLOADS[5].scaled(T=512, D=128, E=8),
}


def _variant_forward(w, scoring, bias_on, renorm):
    ops = _ops()
    inp = make_inputs(w)
    g = H.gpu_inputs(inp)
    rng = np.random.default_rng(3)
    bias = (rng.standard_normal(w.E) * 0.02).astype(np.float32) if bias_on else None
    C = ops.capacity(w.T, w.k, w.E, w.cf)
    out = ops.forward(g["x"], H.experts_dict(w, g), k=w.k, capacity=C, w_router=g["w_router"],
                      shared=H.shared_dict(w, g), use_residual=w.residual, keep_shared_out=True,
                      scoring=scoring, selection_bias=None if bias is None else torch.tensor(bias, device="cuda"),
                      renormalize_kept=renorm, z_loss=True)
    torch.cuda.synchronize()
    return inp, g, out, bias, C


@pytest.mark.parametrize("case,scoring,bias_on,renorm", [
    ("gelu_f32", "sigmoid", False, True), ("gelu_f32", "softmax", True, True),
    ("swiglu_bf16_shared", "sigmoid", True, False), ("swiglu_bf16_shared", "sigmoid", True, True),
    ("linear_f32", "softmax", False, True)])
def test_forward_variants(case, scoring, bias_on, renorm):
    w = CASES[case]
    inp, g, out, bias, C = _variant_forward(w, scoring, bias_on, renorm)
    h = H.host(out)
    b64 = None if bias is None else bias.astype(np.float64)
    x = to_numpy_f32(inp["x"])
    lg = h["logits"].astype(np.float64)
    want = om.forward(x, w.k, w.kind, H.oracle_weights(inp), logits=lg, C=C, residual=w.residual,
                      shared=H.oracle_shared(inp), bf16=(w.dtype == "bf16"), scoring=scoring,
                      selection_bias=b64, renormalize=renorm)
    assert np.array_equal(h["topk_idx"], want["idx"]), "selection (no near-tie at these seeds)"
    for key, wk in (("slot", "slot"), ("slot_assign", "slot_assign"), ("expert_used", "used"),
                    ("expert_overflow", "overflow"), ("token_drops", "drops")):
        assert np.array_equal(h[key], want[wk]), key
    H.assert_close(h["topk_gate"], want["gate"], 1e-4, "gate")
    H.assert_close(h["z_loss"], np.array([want["z_loss"]]), 1e-4, "z_loss")
    H.assert_close(h["aux_loss"], np.array([want["aux"]]), 1e-4, "aux")
    y = want["y"]
    if w.dtype == "bf16":
        y = om.bf16_round(y)
    H.assert_close(h["y"], y, H.RTOL[w.dtype], "y")


@pytest.mark.parametrize("case,scoring,renorm,zscale", [
    ("gelu_f32", "sigmoid", True, 0.5), ("swiglu_f32_shared", "softmax", True, 0.0),
    ("swiglu_f32_shared", "sigmoid", False, 1.0), ("linear_f32", "sigmoid", True, 0.3)])
def test_backward_variants(case, scoring, renorm, zscale):
    ops = _ops()
    w = CASES[case].scaled(backward=True)
    inp, g, out, bias, C = _variant_forward(w, scoring, True, renorm)
    grads = ops.backward(g["dy"], g["x"], H.experts_dict(w, g), out, k=w.k,
                         use_residual=w.residual, aux_grad_scale=0.5,
                         shared=H.shared_dict(w, g), z_grad_scale=zscale)
    torch.cuda.synchronize()
    h = H.host(out)
    lg = h["logits"].astype(np.float64)
    # the oracle takes the GPU's selection (validated above) and dispatch
    r = om.route(lg, w.k, scoring=scoring, selection_bias=bias.astype(np.float64))
    assert np.array_equal(h["topk_idx"], r["idx"]), "selection (no near-tie at these seeds)"
    d = om.dispatch(h["topk_idx"], w.E, C)
    want = om.backward(to_numpy_f32(inp["dy"]), to_numpy_f32(inp["x"]), w.kind,
                       H.oracle_weights(inp), lg, h["topk_idx"], r["gate"], d["kept"],
                       np.bincount(h["topk_idx"].ravel(), minlength=w.E),
                       residual=w.residual, aux_grad_scale=0.5, shared=H.oracle_shared(inp),
                       scoring=scoring, renormalize=renorm, z_grad_scale=zscale)
    for key in ("dgate", "dlogits", "dx"):
        H.assert_close(grads[key].cpu().numpy(), want[key], 1e-4, key)
    for key, v in grads["dexperts"].items():
        H.assert_close(v.cpu().numpy(), want["dexperts"][key], 1e-4, "d" + key)
    if w.shared_F:
        for key, v in grads["dshared"].items():
            H.assert_close(v.cpu().numpy(), want["dshared"][key], 1e-4, "dshared_" + key)


def test_combine_renormalize_standalone():
    """moe_combine with renormalize_kept against the oracle combine, including tokens
    with every choice dropped (y == residual bit for bit)."""
    ops = _ops()
    rng = np.random.default_rng(17)
    T, k, E, C, D = 300, 3, 6, 40, 64
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    d = om.dispatch(idx, E, C)
    gate = rng.random((T, k)).astype(np.float32)
    gate /= gate.sum(1, keepdims=True)
    eo = rng.standard_normal((E, C, D)).astype(np.float32)
    x = rng.standard_normal((T, D)).astype(np.float32)
    y = ops.combine(torch.tensor(eo, device="cuda"), torch.tensor(idx, device="cuda"),
                    torch.tensor(d["slot"].astype(np.int32), device="cuda"),
                    torch.tensor(gate, device="cuda"), residual=torch.tensor(x, device="cuda"),
                    renormalize_kept=True).cpu().numpy()
    o = np.zeros((T, k, D))
    for t in range(T):
        for j in range(k):
            if d["kept"][t, j]:
                o[t, j] = eo[idx[t, j], d["slot"][t, j]]
    want = om.combine(x, None, o, gate.astype(np.float64), d["kept"], True, renormalize=True)
    H.assert_close(y, want, 1e-4, "y")
    full = np.flatnonzero(d["drops"] == k)
    assert full.size > 0
    assert np.array_equal(y[full], x[full])


# ---------------------------------------------------------------------------------
# full sizes, in the launch configuration the bench uses
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,scoring,renorm", [(3, "sigmoid", True), (4, "sigmoid", True),
                                                (3, "softmax", True)])
def test_forward_variants_full_size(cfg, scoring, renorm):
    """The SwiGLU workload and the drop/tie stress workload at full size with a selection
    bias: routing, dispatch and the z-loss everywhere; every kept expert output row, the
    shared expert's output, y and its routed part on every token whose selection equals
    the oracle's."""
    ops = _ops()
    w = WORKLOADS[cfg]
    inp = make_inputs(w)
    g = H.gpu_inputs(inp)
    rng = np.random.default_rng(11)
    bias = (rng.standard_normal(w.E) * 0.02).astype(np.float32)
    C = ops.capacity(w.T, w.k, w.E, w.cf)
    kw = {"logits": g["logits"]} if "logits" in g else {"w_router": g["w_router"]}
    out = ops.forward(g["x"], H.experts_dict(w, g), k=w.k, capacity=C, shared=H.shared_dict(w, g),
                      use_residual=w.residual, keep_shared_out=True, scoring=scoring,
                      selection_bias=torch.tensor(bias, device="cuda"), renormalize_kept=renorm,
                      z_loss=True, **kw)
    torch.cuda.synchronize()
    h = H.host(out)
    lg = h["logits"].astype(np.float64)
    r = om.route(lg, w.k, scoring=scoring, selection_bias=bias.astype(np.float64))
    _check_selection(h["topk_idx"], r, bias.astype(np.float64), w.k, max_frac=1e-3)
    # dispatch follows the GPU's selection exactly
    d = om.dispatch(h["topk_idx"], w.E, C)
    for key, wk in (("slot", "slot"), ("slot_assign", "slot_assign"), ("expert_used", "used"),
                    ("expert_overflow", "overflow"), ("token_drops", "drops")):
        assert np.array_equal(h[key], d[wk]), key
    H.assert_close(h["z_loss"], np.array([r["z_loss"]]), 1e-4, "z_loss")
    # every token whose selection is the oracle's (all but near-tied boundary keys)
    toks = np.flatnonzero(np.all(h["topk_idx"] == r["idx"], axis=1))
    H.check_outputs(w, inp, h, r, d, tokens=toks, idx=h["topk_idx"], gate=r["gate"],
                    renormalize=renorm)


def test_backward_variants_full_size():
    """The single-linear forward + backward workload at full size under the sigmoid router
    with a selection bias, survivor renormalisation and the z-loss term: every gradient."""
    ops = _ops()
    w = WORKLOADS[5]
    inp, g, out, bias, C = _variant_forward(w, "sigmoid", True, True)
    grads = ops.backward(g["dy"], g["x"], H.experts_dict(w, g), out, k=w.k,
                         use_residual=w.residual, aux_grad_scale=1.0, z_grad_scale=0.5)
    torch.cuda.synchronize()
    h = H.host(out)
    lg = h["logits"].astype(np.float64)
    r = om.route(lg, w.k, scoring="sigmoid", selection_bias=bias.astype(np.float64))
    assert np.array_equal(h["topk_idx"], r["idx"]), "selection (no near-tie at this seed)"
    d = om.dispatch(h["topk_idx"], w.E, C)
    want = om.backward(to_numpy_f32(inp["dy"]), to_numpy_f32(inp["x"]), w.kind,
                       H.oracle_weights(inp), lg, h["topk_idx"], r["gate"], d["kept"], r["count"],
                       residual=w.residual, aux_grad_scale=1.0, scoring="sigmoid",
                       renormalize=True, z_grad_scale=0.5)
    for key in ("dgate", "dlogits", "dx"):
        H.assert_close(grads[key].cpu().numpy(), want[key], 1e-4, key)
    H.assert_close(grads["dW"].cpu().numpy(), want["dexperts"]["w_in"], 1e-4, "dW")
