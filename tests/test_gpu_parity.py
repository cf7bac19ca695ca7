"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Routing and dispatch (indices, slots, kept mask, slot table, used, overflow, drops,
counts) must be bit-exact given the GPU's fp32 logits; gates, probability sums and the
aux loss within 1e-4 relative; fp32 outputs and gradients within 1e-4 and bf16 outputs
within 2e-2 (metric in tests/_harness.py).

Sizes: each workload at a reduced size the oracle finishes in seconds (several GEMM
tiles and a ragged tail per expert); mid-size cases whose GEMMs take the 256 x 256 tiles
the full-size workloads run on (the persistent gated kernel, the staged-epilogue kernel,
in both weight layouts, routed loads even and skewed); and every workload at its full
size. Every element is compared in each case: all kept expert output rows, the shared
expert's output, y, and the routed part of y (y minus the residual and the shared term,
so that the residual's magnitude does not set the bound on the experts' contribution).
"""

import numpy as np
import pytest
import torch

import oracle.moe_oracle as om
from tests import _harness as H
from workloads import WORKLOADS, make_inputs, to_numpy_f32

pytestmark = pytest.mark.gpu

SMALL = {
    1: WORKLOADS[1],
    2: WORKLOADS[2].scaled(T=512, D=256, F=512),
    3: WORKLOADS[3].scaled(T=1024, D=256, E=32, F=128, shared_F=128),
    4: WORKLOADS[4].scaled(T=2048, D=256, E=16, F=256),
    5: WORKLOADS[5].scaled(T=512, D=128, E=8),
}


def _ops():
    from sparse_mixture_experts_stable_amd import ops
    return ops


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_forward_small(cfg):
    w = SMALL[cfg]
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


@pytest.mark.parametrize("case", ["many_experts", "many_chunks"])
def test_forward_split_scan_path(case):
    """Shapes past the limits of the scan that runs inside the assignment launch (more than
    256 experts, or more than 16,384 chunk sums): there the scan is a launch of its own."""
    w = {"many_experts": SMALL[3].scaled(T=512, E=384, k=4, F=64, shared_F=0),
         "many_chunks": SMALL[1].scaled(T=70000, D=64, E=256, F=64)}[case]
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


DEGENERATE = {
    # one token, one choice, a shared expert
    "one_token": SMALL[3].scaled(T=1, E=4, k=1, F=128, shared_F=128),
    # every token picks every expert (k = E), no drops, T off every tile size
    "all_experts": SMALL[2].scaled(T=300, E=4, k=4, cf=2.0),
    # a single expert: one group of 700 rows, ragged in the last row tile
    "single_expert": SMALL[3].scaled(T=700, E=1, k=1, cf=1.0, shared_F=0),
    # bf16 single-linear experts (the output GEMM alone)
    "bf16_linear": SMALL[5].scaled(dtype="bf16", D=256, backward=False),
}


@pytest.mark.parametrize("case", sorted(DEGENERATE))
def test_forward_degenerate_shapes(case):
    w = DEGENERATE[case]
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


def test_forward_small_zipf_pmf_variant():
    w = SMALL[4].scaled(logits_mode="zipf_pmf_q")
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


@pytest.mark.parametrize("kind", ["swiglu", "gelu"])
def test_forward_small_f32_mlp(kind):
    """fp32 SwiGLU (gated fp32 kernel) and GELU experts with a shared fp32 expert."""
    base = SMALL[3] if kind == "swiglu" else SMALL[2].scaled(shared_F=128)
    w = base.scaled(dtype="f32")
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


def _gemm_large_tiles(w):
    """Whether each grouped bf16 GEMM launch of the forward (GEMM-1 with the shared expert
    in the same launch, then GEMM-2) runs on the 256 x 256 tiles. Restates the selection
    rule of the bf16 GEMM launcher: every problem of the launch has at least 192 rows
    per group (C for the routed experts, T for the shared one) and the launch has at
    least 128 tiles of 256 rows by 128 (gated) or 256 output columns."""
    if w.dtype != "bf16":
        return None
    from sparse_mixture_experts_stable_amd import ops
    C = ops.capacity(w.T, w.k, w.E, w.cf)
    cdiv = lambda a, b: -(-a // b)
    gated = w.kind == "swiglu"
    n1 = w.F if w.kind != "linear" else w.D
    probs1 = [(C, w.E, n1)] + ([(w.T, 1, w.shared_F)] if w.shared_F else [])
    bnq1 = 128 if gated else 256
    t1 = sum(g * cdiv(r, 256) * cdiv(n, bnq1) for r, g, n in probs1)
    large1 = all(r >= 192 for r, _, _ in probs1) and t1 >= 128
    if w.kind == "linear":
        return large1, None
    probs2 = [(C, w.E, w.D)] + ([(w.T, 1, w.D)] if w.shared_F else [])
    t2 = sum(g * cdiv(r, 256) * cdiv(n, 256) for r, g, n in probs2)
    large2 = all(r >= 192 for r, _, _ in probs2) and t2 >= 128
    return large1, large2


# Mid-size bf16 cases whose expert GEMMs take the 256 x 256 tiles (the kernels the
# full-size workloads and the benchmark run), small enough for the oracle to check every
# element in seconds.
MID = {
    # SwiGLU + shared expert, k = 8: C = 1024, 576 gated GEMM-1 tiles, 288 GEMM-2 tiles
    "swiglu_shared_k8": WORKLOADS[3].scaled(T=4096, D=512, E=32, F=512, shared_F=512),
    # few experts, long row groups: C = 2048, 640 gated tiles, 192 GEMM-2 tiles
    "swiglu_shared_k2": WORKLOADS[3].scaled(T=8192, D=512, E=8, k=2, F=1024, shared_F=512),
    # GELU with biases (bias + GELU epilogues of the large tiles): C = 2560
    "gelu_bias": WORKLOADS[2].scaled(T=8192, D=512, E=8, F=1024),
    # skewed routing (Zipf bias, quarter-grid ties): most experts far below one row tile,
    # a few full; C = 2048
    "swiglu_zipf": WORKLOADS[4].scaled(T=16384, D=512, E=16, F=512),
    # widths that are not multiples of the tile: d_model and d_hidden 320 (five K steps,
    # a last column tile a quarter or half full, partial 32-column hidden pieces per tile)
    "swiglu_ragged_n": WORKLOADS[3].scaled(T=8192, D=320, E=8, k=2, F=320, shared_F=320),
    "gelu_ragged_n": WORKLOADS[2].scaled(T=8192, D=320, E=8, F=320),
}


@pytest.mark.parametrize("layout", ["in_out", "out_in", "out_in_all"])
@pytest.mark.parametrize("case", sorted(MID))
def test_forward_mid_size_large_tiles(case, layout):
    w = MID[case]
    assert _gemm_large_tiles(w) == (True, True), "case must select the 256 x 256 tiles"
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp, layout=layout)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


@pytest.mark.parametrize("case", ["swiglu_shared_k8", "gelu_bias"])
def test_forward_hidden_cache_layout(case):
    """With a caller's hidden_cache the hidden activation is written row-major ([E, C, F]);
    without one the library keeps it in 32-column pieces. Both runs give the same outputs
    bit for bit (the same products in the same order), and the returned hidden rows
    reproduce the expert outputs: expert_out[e] = hidden[e] W_out[e] (+ b_out) in
    float64, to the bf16 tolerance ("Sparse MoE Layer in NumPy", section 2 forward)."""
    w = MID[case]
    inp = make_inputs(w)
    a, g = H.run_forward(w, inp)
    b, _ = H.run_forward(w, inp, g=g, keep_hidden=True)
    used = a["expert_used"].cpu().numpy()
    assert torch.equal(b["expert_used"], a["expert_used"])
    for key in ("y", "shared_out"):
        if a.get(key) is not None:
            assert torch.equal(a[key], b[key]), key
    for e in range(w.E):
        assert torch.equal(a["expert_out"][e, : used[e]], b["expert_out"][e, : used[e]]), e
    wts = H.oracle_weights(inp)
    hid = b["hidden"].float().cpu().numpy().astype(np.float64)
    out = b["expert_out"].float().cpu().numpy()
    for e in sorted({0, w.E // 2, w.E - 1, int(np.argmax(used))}):
        u = int(used[e])
        want = hid[e, :u] @ wts["w_out"][e].astype(np.float64)
        if w.kind == "gelu":
            want = want + wts["b_out"][e].astype(np.float64)
        H.assert_close(out[e, :u], want, H.RTOL["bf16"], f"expert_out[{e}] from hidden")


# Large-tile cases whose K is a single 64-wide step in one GEMM: the persistent kernel
# needs two K steps per tile, so that GEMM runs one block per tile (with the operand
# slots) instead. d_model 64: GEMM-1 (gated, large tiles); d_hidden 64: GEMM-2.
ONE_STEP = {
    "gemm1_k64": (WORKLOADS[3].scaled(T=8192, D=64, E=8, k=2, F=512, shared_F=512), 0),
    "gemm2_k64": (WORKLOADS[3].scaled(T=8192, D=512, E=8, k=2, F=64, shared_F=64), 1),
}


@pytest.mark.parametrize("layout", ["in_out", "out_in_all"])
@pytest.mark.parametrize("case", sorted(ONE_STEP))
def test_forward_large_tiles_single_k_step(case, layout):
    w, which = ONE_STEP[case]
    assert _gemm_large_tiles(w)[which], "case must select the 256 x 256 tiles"
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp, layout=layout)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_forward_full_size(cfg):
    w = WORKLOADS[cfg]
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


def test_forward_full_size_zipf_pmf_variant():
    """The drop/tie stress workload with the pmf-as-bias reading of its Zipf bias."""
    w = WORKLOADS[4].scaled(logits_mode="zipf_pmf_q")
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


# ---------------------------------------------------------------------------------
# w_in / w_up stored [E, F, D] and w_out [E, D, F] (the OUT_IN layouts): same products,
# k-contiguous B tiles
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["out_in", "out_in_wout", "out_in_all"])
@pytest.mark.parametrize("case", ["swiglu_shared", "gelu_bias", "bf16_linear", "one_token"])
def test_forward_out_in_layout_small(case, layout):
    w = {"swiglu_shared": SMALL[3], "gelu_bias": SMALL[2],
         "bf16_linear": DEGENERATE["bf16_linear"], "one_token": DEGENERATE["one_token"]}[case]
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp, layout=layout)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


@pytest.mark.parametrize("cfg,layout", [(2, "out_in"), (3, "out_in"), (4, "out_in"),
                                        (2, "out_in_all"), (3, "out_in_all")])
def test_forward_out_in_layout_full_size(cfg, layout):
    w = WORKLOADS[cfg]
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp, layout=layout)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


def test_out_in_layout_rejections():
    """OUT_IN (w_in / w_up, or w_out) is bf16-forward only, and the routed and shared
    experts must agree."""
    ops = _ops()
    from sparse_mixture_experts_stable_amd import _lib as L
    w = SMALL[3]
    inp = make_inputs(w)
    g = H.gpu_inputs(inp)
    C = ops.capacity(w.T, w.k, w.E, w.cf)
    with pytest.raises(L.MoeError) as e:
        ops.forward(g["x"], H.experts_dict(w, g, "out_in"), k=w.k, capacity=C,
                    shared=H.shared_dict(w, g, "in_out"), w_router=g["w_router"])
    assert e.value.status == L.MOE_ERR_UNSUPPORTED
    w32 = SMALL[5]
    inp32 = make_inputs(w32)
    g32 = H.gpu_inputs(inp32)
    with pytest.raises(L.MoeError) as e:
        ops.forward(g32["x"], H.experts_dict(w32, g32, "out_in"), k=w32.k,
                    capacity=ops.capacity(w32.T, w32.k, w32.E, w32.cf), w_router=g32["w_router"])
    assert e.value.status == L.MOE_ERR_UNSUPPORTED
    # w_out: the same two rules
    with pytest.raises(L.MoeError) as e:
        ops.forward(g["x"], H.experts_dict(w, g, "out_in_all"), k=w.k, capacity=C,
                    shared=H.shared_dict(w, g, "out_in"), w_router=g["w_router"])
    assert e.value.status == L.MOE_ERR_UNSUPPORTED
    w32g = WORKLOADS[1].scaled(T=64)
    inp32g = make_inputs(w32g)
    g32g = H.gpu_inputs(inp32g)
    with pytest.raises(L.MoeError) as e:
        ops.forward(g32g["x"], H.experts_dict(w32g, g32g, "out_in_wout"), k=w32g.k,
                    capacity=ops.capacity(w32g.T, w32g.k, w32g.E, w32g.cf), w_router=g32g["w_router"])
    assert e.value.status == L.MOE_ERR_UNSUPPORTED


def _backward_case(w, aux_scale, tokens=None):
    ops = _ops()
    inp = make_inputs(w)
    out, g = H.run_forward(w, inp)
    grads = ops.backward(g["dy"], g["x"], H.experts_dict(w, g), out, k=w.k,
                         use_residual=w.residual, aux_grad_scale=aux_scale)
    torch.cuda.synchronize()
    h = H.host(out)
    gh = H.host(grads)
    r, d = H.check_routing_dispatch(w, inp, h)
    x = to_numpy_f32(inp["x"])
    W = to_numpy_f32(inp["w_in"])
    dy = to_numpy_f32(inp["dy"])
    want = om.backward_linear(dy, x, W, h["logits"].astype(np.float64), r["idx"], r["gate"],
                              d["kept"], d["slot"], r["count"], residual=w.residual,
                              aux_grad_scale=aux_scale)
    H.assert_close(gh["dgate"], want["dgate"], 1e-4, "dgate")
    H.assert_close(gh["dlogits"], want["dlogits"], 1e-4, "dlogits")
    H.assert_close(gh["dx"], want["dx"], 1e-4, "dx")
    H.assert_close(gh["dW"], want["dW"], 1e-4, "dW")
    # closed form of the router chain: rows sum to zero (task part)
    if aux_scale == 0.0:
        assert np.max(np.abs(gh["dlogits"].sum(1))) < 1e-5


@pytest.mark.parametrize("aux_scale", [0.0, 1.0])
def test_backward_small(aux_scale):
    _backward_case(SMALL[5], aux_scale)


def test_backward_full_size():
    _backward_case(WORKLOADS[5], 0.0)


def test_backward_no_residual_tiny_capacity():
    _backward_case(SMALL[5].scaled(residual=False, cf=0.25), 0.5)


# ---------------------------------------------------------------------------------
# general backward: GELU / SwiGLU experts, shared expert, router weights (fp32)
# ---------------------------------------------------------------------------------

def _backward_general(w, aux_scale, router):
    ops = _ops()
    inp = make_inputs(w)
    out, g = H.run_forward(w, inp)
    grads = ops.backward(g["dy"], g["x"], H.experts_dict(w, g), out, k=w.k,
                         use_residual=w.residual, aux_grad_scale=aux_scale,
                         shared=H.shared_dict(w, g),
                         w_router=g["w_router"] if router else None)
    torch.cuda.synchronize()
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    want = om.backward(to_numpy_f32(inp["dy"]), to_numpy_f32(inp["x"]), w.kind,
                       H.oracle_weights(inp), h["logits"].astype(np.float64), r["idx"], r["gate"],
                       d["kept"], r["count"], residual=w.residual, aux_grad_scale=aux_scale,
                       shared=H.oracle_shared(inp),
                       w_router=to_numpy_f32(inp["w_router"]) if router else None)
    for key in ("dgate", "dlogits", "dx"):
        H.assert_close(grads[key].cpu().numpy(), want[key], 1e-4, key)
    assert set(grads["dexperts"]) == set(want["dexperts"])
    for key, v in grads["dexperts"].items():
        H.assert_close(v.cpu().numpy(), want["dexperts"][key], 1e-4, "d" + key)
    if w.shared_F:
        for key, v in grads["dshared"].items():
            H.assert_close(v.cpu().numpy(), want["dshared"][key], 1e-4, "dshared_" + key)
    if router:
        H.assert_close(grads["dw_router"].cpu().numpy(), want["dw_router"], 1e-4, "dw_router")
    # experts with no kept row get exactly zero gradients
    unused = np.flatnonzero(d["used"] == 0)
    for v in grads["dexperts"].values():
        assert not v[torch.as_tensor(unused, device=v.device)].any()


BWD = {
    "gelu_bias": WORKLOADS[1].scaled(backward=True),
    "gelu_wide": WORKLOADS[2].scaled(T=1024, D=256, F=512, dtype="f32", backward=True),
    "swiglu_shared": WORKLOADS[3].scaled(T=1024, D=256, E=32, F=128, shared_F=128, dtype="f32",
                                         backward=True),
    "linear": SMALL[5],
    # fp32 tiles of 64 x 64 x 32: partial N tiles (F = 80, E = 8) and K tails (F = 80,
    # D = 16, F = 48, shared 32), every GEMM mode and epilogue of the backward
    "gelu_odd": WORKLOADS[1].scaled(T=300, D=64, E=8, F=80, backward=True),
    "swiglu_tiny": WORKLOADS[3].scaled(T=129, D=16, E=4, k=1, F=48, shared_F=32, dtype="f32",
                                       backward=True, cf=1.5),
    # the shared expert's and the router's weight gradients (K = T = 5000 rows, few output
    # tiles) run split over K: 9 ranges of 576 rows, the last one ragged (392 rows)
    "split_k": WORKLOADS[3].scaled(T=5000, D=256, E=16, F=64, shared_F=128, dtype="f32",
                                   backward=True),
    # d_model above 2048: the router backward streams dy for every choice instead of
    # holding it in registers
    "wide_d": WORKLOADS[5].scaled(T=96, D=3072, E=4),
    # k > 64: the router backward reads each choice's metadata from memory, and the
    # per-choice values span two register slots per lane
    "many_choices": WORKLOADS[5].scaled(T=64, D=64, E=128, k=72),
}


@pytest.mark.parametrize("case,aux_scale,router", [
    ("gelu_bias", 0.0, False), ("gelu_bias", 1.0, True), ("gelu_wide", 0.0, True),
    ("swiglu_shared", 0.0, False), ("swiglu_shared", 0.5, True), ("linear", 0.0, True),
    ("gelu_odd", 0.0, True), ("swiglu_tiny", 1.0, True), ("split_k", 0.0, True),
    ("wide_d", 0.5, True), ("many_choices", 1.0, True),
])
def test_backward_general(case, aux_scale, router):
    _backward_general(BWD[case], aux_scale, router)


@pytest.mark.parametrize("case", ["gelu_odd", "swiglu_tiny"])
def test_forward_odd_fp32_shapes(case):
    w = BWD[case]
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.check_outputs(w, inp, h, r, d)


def test_backward_general_no_residual_tiny_capacity():
    w = BWD["swiglu_shared"].scaled(residual=False, cf=0.1, E=16)
    _backward_general(w, 0.25, True)


def test_backward_general_zero_capacity():
    """C = 0: every routed gradient is zero; dx = r dy + shared + router terms."""
    w = BWD["gelu_bias"].scaled(cf=0.0)
    _backward_general(w, 0.0, True)


# ---------------------------------------------------------------------------------
# routing edge cases
# ---------------------------------------------------------------------------------

def _route_case(logits, k):
    ops = _ops()
    g = torch.tensor(logits, dtype=torch.float32, device="cuda")
    out = ops.route(logits=g, k=k)
    torch.cuda.synchronize()
    h = H.host(out)
    r = om.route(np.asarray(logits, dtype=np.float32).astype(np.float64), k)
    assert np.array_equal(h["topk_idx"], r["idx"])
    assert np.array_equal(h["expert_count"], r["count"])
    H.assert_close(h["topk_gate"], r["gate"], 1e-4, "gate")
    H.assert_close(h["prob_sum"], r["prob_sum"], 1e-4, "prob_sum")
    assert abs(float(h["aux_loss"][0]) - r["aux"]) <= 1e-4 * abs(r["aux"])


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (1, 7, 7), (33, 5, 3), (100, 64, 64), (70, 130, 9),
                                   (40, 300, 100), (17, 1000, 256), (50, 513, 2)])
def test_route_shapes_with_ties(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    logits = np.round(rng.standard_normal((T, E)) * 2) / 2      # many exact ties
    _route_case(logits, k)


def test_route_signed_zero_and_page_examples():
    _route_case(np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0], [0.0, 0.0, 0.0]]), 1)
    _route_case(np.zeros((4, 4)), 2)
    ref = [[4.0, 1.0, 0.0, -1.0], [3.0, 1.0, 0.0, -1.0], [4.0, 0.0, 1.0, -1.0], [3.0, 0.0, 1.0, -1.0]]
    _route_case(np.array(ref), 1)


# ---------------------------------------------------------------------------------
# dispatch on caller-supplied choices, including duplicates and invalid indices
# ---------------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E,C", [(1, 1, 1, 1), (300, 3, 7, 50), (1000, 2, 4, 0), (777, 8, 64, 40),
                                     (5000, 1, 3, 2000), (257, 5, 1000, 1), (40000, 2, 128, 700),
                                     (70000, 2, 256, 600)])
def test_dispatch_random_with_duplicates(T, k, E, C):
    ops = _ops()
    rng = np.random.default_rng(T + k + E + C)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    out = ops.dispatch(torch.tensor(idx, device="cuda"), E, C)
    torch.cuda.synchronize()
    h = H.host(out)
    d = om.dispatch(idx.astype(np.int64), E, C)
    assert np.array_equal(h["slot"], d["slot"])
    assert np.array_equal(h["kept"].astype(bool), d["kept"])
    assert np.array_equal(h["slot_assign"], d["slot_assign"])
    assert np.array_equal(h["expert_used"], d["used"])
    assert np.array_equal(h["expert_overflow"], d["overflow"])
    assert np.array_equal(h["token_drops"], d["drops"])


def test_dispatch_flags_invalid_indices():
    ops = _ops()
    E, C = 3, 4
    idx = np.array([[0, 1], [2, -1], [3, 0], [0, 0], [1, 2]], dtype=np.int32)
    out = ops.dispatch(torch.tensor(idx, device="cuda"), E, C, return_ws=True)
    err = ops.read_error(out["ws"])
    h = H.host({k: v for k, v in out.items() if k != "ws"})
    assert err & 1
    valid = (idx >= 0) & (idx < E)
    # the valid choices are dispatched as if the invalid ones were absent
    a_valid = [(t, j) for t in range(idx.shape[0]) for j in range(2) if valid[t, j]]
    used = np.zeros(E, dtype=int)
    for t, j in a_valid:
        e = idx[t, j]
        want = used[e] if used[e] < C else -1
        assert h["slot"][t, j] == want
        used[e] += 1
    assert np.all(h["slot"][~valid] == -1) and np.all(h["kept"][~valid] == 0)
    ok = ops.dispatch(torch.tensor(np.clip(idx, 0, E - 1), device="cuda"), E, C, return_ws=True)
    assert ops.read_error(ok["ws"]) == 0


# ---------------------------------------------------------------------------------
# stand-alone entry points, degenerate capacities, determinism
# ---------------------------------------------------------------------------------

def test_combine_standalone_matches_oracle():
    ops = _ops()
    rng = np.random.default_rng(5)
    T, k, E, C, D = 300, 3, 6, 70, 64
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int64)
    d = om.dispatch(idx, E, C)
    gate = rng.random((T, k))
    eo = rng.standard_normal((E, C, D)).astype(np.float32)
    x = rng.standard_normal((T, D)).astype(np.float32)
    sh = rng.standard_normal((T, D)).astype(np.float32)
    t = lambda a, dt=torch.float32: torch.tensor(a, dtype=dt, device="cuda")
    y = ops.combine(t(eo), t(idx, torch.int32), t(d["slot"], torch.int32), t(gate), residual=t(x),
                    shared_out=t(sh))
    o = np.zeros((T, k, D))
    for tt in range(T):
        for j in range(k):
            if d["kept"][tt, j]:
                o[tt, j] = eo[idx[tt, j], d["slot"][tt, j]]
    want = om.combine(x, sh, o, gate.astype(np.float32), d["kept"], True)
    H.assert_close(y.cpu().numpy(), want, 1e-5, "combine")


@pytest.mark.parametrize("residual,shared", [(False, False), (True, True)])
def test_combine_standalone_bf16(residual, shared):
    """The bf16 combine on its own: y is the fp32 sum (x, shared, then the gated kept rows
    in choice order) rounded once to bf16, so it must lie within half a bf16 unit in the
    last place of the float64 sum, plus the fp32 rounding of that sum."""
    ops = _ops()
    rng = np.random.default_rng(7)
    T, k, E, C, D = 300, 8, 64, 30, 2048
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int64)
    d = om.dispatch(idx, E, C)
    gate = rng.random((T, k)).astype(np.float32)
    gate /= gate.sum(1, keepdims=True)
    bf = lambda a: om.bf16_round(a).astype(np.float32)
    eo = bf(rng.standard_normal((E, C, D)) * 0.1)
    x = bf(rng.standard_normal((T, D)))
    sh = bf(rng.standard_normal((T, D)) * 0.1)
    t = lambda a, dt=torch.bfloat16: torch.tensor(a, device="cuda").to(dt)
    y = ops.combine(t(eo), t(idx, torch.int32), t(d["slot"], torch.int32), t(gate, torch.float32),
                    residual=t(x) if residual else None, shared_out=t(sh) if shared else None)
    got = y.float().cpu().numpy().astype(np.float64)
    o = np.zeros((T, k, D))
    tt, jj = np.nonzero(d["kept"])
    o[tt, jj] = eo[idx[tt, jj], d["slot"][tt, jj]]
    want = om.combine(x, sh if shared else None, o, gate.astype(np.float64), d["kept"], residual)
    terms = np.abs(o * np.where(d["kept"], gate, 0.0)[:, :, None]).sum(1)
    terms = terms + (np.abs(x) if residual else 0.0) + (np.abs(sh) if shared else 0.0)
    bound = 0.5 * H.ulp(got, "bf16") + 16.0 * 2.0 ** -24 * terms
    err = np.abs(got - want)
    assert np.all(err <= bound), (float(np.max(err - bound)), int(np.sum(err > bound)))
    # fully dropped tokens with no other term: exactly zero
    if not residual and not shared:
        assert np.all(got[d["drops"] == k] == 0.0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_router_page_result_contract(dtype):
    """"Top-k MoE Router with Load Statistics", Examples 1-3, through ops.topk_router
    (moe_route with its load statistics, then moe_combine on the per-token expert
    outputs): the page's printed values, selected_experts as int64, every other result
    in x's dtype on x's device."""
    import json
    import os
    ops = _ops()
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "p2_router_examples.json")))["examples"]
    tol = 1e-6 if dtype == torch.float32 else 4e-3
    for e in ex:
        t = lambda a: torch.tensor(a, dtype=torch.float32, device="cuda").to(dtype)
        got = ops.topk_router(t(e["x"]), t(e["w_router"]), t(e["expert_outputs"]),
                              t(e["shared_output"]), e["k"])
        torch.cuda.synchronize()
        assert got["selected_experts"].dtype == torch.int64
        assert got["selected_experts"].cpu().tolist() == e["selected_experts"]
        for key in ("output", "selected_weights", "token_fraction", "probability_mass"):
            v = got[key]
            assert v.dtype == dtype and v.device.type == "cuda", key
            np.testing.assert_allclose(v.float().cpu().numpy(), np.array(e[key], dtype=np.float64),
                                       rtol=tol, atol=1e-6 if key == "probability_mass" else tol,
                                       err_msg=key)


def test_forward_load_statistics():
    """moe_forward's token_fraction and probability_mass are count / T and prob_sum / T
    of the same call."""
    w = SMALL[3]
    inp = make_inputs(w)
    out, _ = H.run_forward(w, inp)
    h = H.host(out)
    r, d = H.check_routing_dispatch(w, inp, h)
    H.assert_close(h["token_fraction"], r["count"] / w.T, 1e-6, "token_fraction")
    H.assert_close(h["probability_mass"], r["prob_sum"] / w.T, 1e-4, "probability_mass")


@pytest.mark.parametrize("D,dt", [(2, torch.float32), (7, torch.bfloat16), (1536, torch.bfloat16),
                                  (100, torch.float32)])
def test_combine_any_width(D, dt):
    """d_model that does not split into 16-byte pieces tiling the block (odd widths,
    1536 in bf16) runs the one-element-per-thread combine, same order, same result."""
    ops = _ops()
    rng = np.random.default_rng(D)
    T, k, E, C = 130, 3, 5, 60
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int64)
    d = om.dispatch(idx, E, C)
    gate = rng.random((T, k)).astype(np.float32)
    bf = (lambda a: om.bf16_round(a).astype(np.float32)) if dt == torch.bfloat16 else (lambda a: a.astype(np.float32))
    eo = bf(rng.standard_normal((E, C, D)))
    x = bf(rng.standard_normal((T, D)))
    t = lambda a, ty=dt: torch.tensor(a, device="cuda").to(ty)
    y = ops.combine(t(eo), t(idx, torch.int32), t(d["slot"], torch.int32), t(gate, torch.float32),
                    residual=t(x))
    o = np.zeros((T, k, D))
    tt, jj = np.nonzero(d["kept"])
    o[tt, jj] = eo[idx[tt, jj], d["slot"][tt, jj]]
    want = om.combine(x, None, o, gate.astype(np.float64), d["kept"], True)
    if dt == torch.bfloat16:
        want = om.bf16_round(want)
    H.assert_close(y.float().cpu().numpy(), want, 1e-2 if dt == torch.bfloat16 else 1e-5, "y")


def test_shared_expert_dense_entry_point():
    ops = _ops()
    w = SMALL[3]
    inp = make_inputs(w)
    g = H.gpu_inputs(inp)
    out = ops.expert_mlp(H.shared_dict(w, g), g["x"])
    torch.cuda.synchronize()
    want = om.shared_apply(H.oracle_shared(inp), to_numpy_f32(inp["x"]), bf16=True)
    H.assert_close(out["expert_out"].float().cpu().numpy(), want, 2e-2, "shared")


@pytest.mark.parametrize("cfg", [1, 3])
def test_zero_capacity_gives_residual_exactly(cfg):
    w = SMALL[cfg].scaled(cf=0.0, shared_F=0)
    inp = make_inputs(w)
    out, g = H.run_forward(w, inp)
    assert out["capacity"] == 0
    assert torch.equal(out["y"], g["x"])
    h = H.host(out)
    assert np.all(h["token_drops"] == w.k) and np.all(h["slot"] == -1)


def test_forward_is_deterministic():
    w = SMALL[3]
    inp = make_inputs(w)
    a, g = H.run_forward(w, inp)
    b, _ = H.run_forward(w, inp, g)
    for key in ("logits", "topk_gate", "prob_sum", "aux_loss", "y", "expert_out", "slot_assign"):
        ta, tb = a[key], b[key]
        if key == "expert_out":
            # rows past used[e] are unspecified
            used = a["expert_used"].cpu().numpy()
            for e in range(ta.shape[0]):
                assert torch.equal(ta[e, : used[e]], tb[e, : used[e]])
        else:
            assert torch.equal(ta, tb), key


def test_backward_is_deterministic():
    """Every reduction of the backward has a fixed order (no atomics): two calls give
    the same bits, for MLP experts with a shared expert, router weights and survivor
    renormalisation under the sigmoid router, with the aux and z-loss terms."""
    ops = _ops()
    w = BWD["swiglu_shared"]
    inp = make_inputs(w)
    g = H.gpu_inputs(inp)
    C = ops.capacity(w.T, w.k, w.E, w.cf)
    out = ops.forward(g["x"], H.experts_dict(w, g), k=w.k, capacity=C, w_router=g["w_router"],
                      shared=H.shared_dict(w, g), scoring="sigmoid", renormalize_kept=True,
                      z_loss=True)
    runs = []
    for _ in range(2):
        gr = ops.backward(g["dy"], g["x"], H.experts_dict(w, g), out, k=w.k, aux_grad_scale=0.5,
                          shared=H.shared_dict(w, g), w_router=g["w_router"], z_grad_scale=0.3)
        torch.cuda.synchronize()
        runs.append(gr)
    a, b = runs
    for key in ("dx", "dgate", "dlogits", "dw_router"):
        assert torch.equal(a[key], b[key]), key
    for key in a["dexperts"]:
        assert torch.equal(a["dexperts"][key], b["dexperts"][key]), key
    for key in a["dshared"]:
        assert torch.equal(a["dshared"][key], b["dshared"][key]), key
    # and the forward's z-loss
    out2 = ops.forward(g["x"], H.experts_dict(w, g), k=w.k, capacity=C, w_router=g["w_router"],
                       shared=H.shared_dict(w, g), scoring="sigmoid", renormalize_kept=True,
                       z_loss=True)
    torch.cuda.synchronize()
    assert torch.equal(out["z_loss"], out2["z_loss"])
    assert torch.equal(out["y"], out2["y"])
