"""Pins for the CPU oracle: each test ties it to something other than itself -- values
printed on the pages, closed forms, brute force on tiny inputs, textbook routines,
central finite differences -- so that a plausible slip in the oracle fails here.

The last group plants such slips in the oracle (monkeypatching it, on the CPU) and
checks that the pins catch them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle.moe_oracle as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------------
# Worked examples printed on the pages
# ---------------------------------------------------------------------------------

def check_p2_examples():
    """Top-k MoE Router with Load Statistics, Examples 1-3: routing from x w_router,
    gate-weighted sum of the given expert outputs plus the shared output, no residual,
    no capacity limit. Printed to 6 decimals."""
    for ex in _load("p2_router_examples.json")["examples"]:
        x = np.array(ex["x"], dtype=np.float64)
        w = np.array(ex["w_router"], dtype=np.float64)
        eo = np.array(ex["expert_outputs"], dtype=np.float64)
        sh = np.array(ex["shared_output"], dtype=np.float64)
        k = ex["k"]
        r = om.route(x @ w, k)
        T, E = r["p"].shape
        d = om.dispatch(r["idx"], E, T * k)
        o = np.stack([eo[np.arange(T), r["idx"][:, j]] for j in range(k)], axis=1)
        y = om.combine(x, sh, o, r["gate"], d["kept"], residual=False)
        assert r["idx"].tolist() == ex["selected_experts"]
        np.testing.assert_allclose(r["gate"], ex["selected_weights"], atol=1e-6)
        np.testing.assert_allclose(y, ex["output"], atol=1e-6)
        np.testing.assert_allclose(r["token_fraction"], ex["token_fraction"], atol=1e-6)
        np.testing.assert_allclose(r["probability_mass"], ex["probability_mass"], atol=5e-7)


def test_p2_examples():
    check_p2_examples()


def check_p3_tie_break():
    ref = _load("p3_reference.json")["tie_break"]
    r = om.route(np.array([ref["logits_row"]]), ref["k"])
    assert r["idx"][0].tolist() == ref["selected"]


def test_p3_tie_break():
    check_p3_tie_break()


def check_p3_capacity():
    """Module 7 REFERENCE capacity contract: 12 tokens x 4 experts, k=2, cf=1."""
    ref = _load("p3_reference.json")["capacity"]
    s = np.array(ref["logits"])
    T, E = s.shape
    r = om.route(s, 2)
    C = om.capacity(T, 2, E, 1.0)
    d = om.dispatch(r["idx"], E, C)
    assert C == ref["capacity_per_expert"] == 6
    assert r["count"].tolist() == ref["before_counts"]
    assert d["used"].tolist() == ref["after_counts"]
    assert int((~d["kept"]).sum()) == ref["dropped_assignments"]
    assert np.flatnonzero(d["drops"] == 2).tolist() == ref["fully_dropped_tokens"]
    # consequences of position priority spelled out: expert 0 keeps tokens 0..5
    assert d["overflow"].tolist() == [6, 0, 0, 0]
    assert d["drops"].tolist() == [0] * 6 + [1] * 6
    assert d["slot_assign"][0].tolist() == [0, 2, 4, 6, 8, 10]

    sec = _load("p3_reference.json")["capacity_second_case"]
    s2 = np.tile(sec["logits_row"], (sec["T"], 1))
    r2 = om.route(s2, sec["k"])
    C2 = om.capacity(sec["T"], sec["k"], 2, sec["capacity_factor"])
    d2 = om.dispatch(r2["idx"], 2, C2)
    assert C2 == 1
    assert d2["kept"][:, 0].tolist() == sec["kept"]
    assert np.flatnonzero(d2["drops"] == sec["k"]).tolist() == sec["fully_dropped_tokens"]


def test_p3_capacity():
    check_p3_capacity()


def check_p3_aux():
    """Module 7 REFERENCE losses: Switch aux of the 4x4 logits at k=1, and aux == 1 at
    uniform load (Sparse MoE Layer in NumPy, section 3, aux_uniform)."""
    ref = _load("p3_reference.json")["losses"]
    r = om.route(np.array(ref["aux_logits"]), 1)
    assert math.isclose(r["aux"], ref["switch_aux"], rel_tol=1e-12)
    # uniform load at k=2: a circulant of logits sends every expert exactly T*k/E
    # assignments and gives every expert the same mean probability.
    E, k = 4, 2
    base = np.array([3.0, 2.0, 0.5, -1.0])
    s = np.stack([np.roll(base, t) for t in range(E)] * 2)
    r2 = om.route(s, k)
    assert r2["count"].tolist() == [4, 4, 4, 4]
    assert math.isclose(r2["aux"], 1.0, rel_tol=1e-12)


def test_p3_aux():
    check_p3_aux()


# ---------------------------------------------------------------------------------
# Capacity: exact values, EP invariance, rejection rules
# ---------------------------------------------------------------------------------

def check_capacity():
    assert om.capacity(512, 2, 8, 1.25) == 160
    assert om.capacity(4096, 2, 16, 1.25) == 640
    assert om.capacity(16384, 8, 256, 1.0) == 512
    assert om.capacity(65536, 2, 64, 1.0) == 2048
    assert om.capacity(8192, 2, 32, 1.0) == 512
    assert om.capacity(10, 1, 4, 1.0) == 3          # ceil(2.5)
    assert om.capacity(7, 2, 4, 1.0) == 4           # ceil(3.5)
    assert om.capacity(8, 2, 4, 0.0) == 0           # no clamp
    assert om.capacity(3, 1, 3, 0.1) == 1           # ceil(0.1)
    # 0.1 is not exactly 1/10 as a double; the exact product 3*0.1 is just above 0.3,
    # and 10 * 0.1 (double) is just above 1, so its ceiling is 2
    assert om.capacity(10, 1, 1, 0.1) == 2
    # invariant to expert-parallel world size W (Sparse MoE Layer in NumPy, trap 2)
    for (T, k, E, cf) in [(16384, 8, 256, 1.0), (4096, 2, 16, 1.25), (96, 3, 8, 0.7)]:
        for W in (1, 2, 4, 8):
            if T % W == 0 and E % W == 0 and k <= E // W:
                assert om.capacity(T // W, k, E // W, cf) == om.capacity(T, k, E, cf)


def test_capacity():
    check_capacity()
    for bad in (-0.5, float("nan"), float("inf")):
        with pytest.raises(ValueError):
            om.capacity(8, 2, 4, bad)
    with pytest.raises(ValueError):
        om.capacity(8, 5, 4, 1.0)


def test_negative_inputs_rejected():
    """Module 7 negative tests: k > E and non-finite logits are rejected."""
    with pytest.raises(ValueError):
        om.route([[1.0, 2.0]], 3)
    with pytest.raises(ValueError):
        om.route([[1.0, np.nan]], 1)
    with pytest.raises(ValueError):
        om.dispatch(np.array([[0, 3]]), 3, 2)


# ---------------------------------------------------------------------------------
# Brute force over every 3x3 logit grid in {0, .25, .5}
# ---------------------------------------------------------------------------------

def _brute_topk(grids, k):
    """Rank by counting: rank(e) = #(strictly greater) + #(equal with lower index)."""
    N, T, E = grids.shape
    gt = (grids[:, :, None, :] > grids[:, :, :, None]).sum(-1)
    lower = np.arange(E)[None, :] < np.arange(E)[:, None]   # [e, e'] = e' < e
    eq = ((grids[:, :, None, :] == grids[:, :, :, None]) & lower[None, None]).sum(-1)
    rank = gt + eq
    idx = np.empty((N, T, k), dtype=np.int64)
    for j in range(k):
        idx[:, :, j] = np.argmax(rank == j, axis=-1)
    return idx


def _brute_slots(idx_flat):
    """slot_full[a] = #earlier assignments to the same expert."""
    N, A = idx_flat.shape
    eq = idx_flat[:, :, None] == idx_flat[:, None, :]
    earlier = np.tril(np.ones((A, A), dtype=bool), -1)       # [a, a'] = a' < a
    return (eq & earlier[None]).sum(-1)


def check_bruteforce(ks=(1, 2, 3), stride=1):
    vals = np.array([0.0, 0.25, 0.5])
    grids = np.array(list(itertools.product(vals, repeat=9))).reshape(-1, 3, 3)[::stride]
    T = E = 3
    for k in ks:
        bidx = _brute_topk(grids, k)
        bslot = _brute_slots(bidx.reshape(len(grids), -1))
        for n in range(len(grids)):
            r = om.route(grids[n], k)
            assert np.array_equal(r["idx"], bidx[n]), (n, k)
            for C in range(0, T * k + 1):
                d = om.dispatch(r["idx"], E, C)
                kept = bslot[n] < C
                assert np.array_equal(d["kept"].ravel(), kept)
                assert np.array_equal(d["slot"].ravel(), np.where(kept, bslot[n], -1))
                assert np.array_equal(d["used"], np.minimum(np.bincount(bidx[n].ravel(), minlength=E), C))


def test_bruteforce_3x3():
    check_bruteforce(ks=(1, 2, 3), stride=1)


# ---------------------------------------------------------------------------------
# Top-1 dispatch equals the exclusive-cumsum formulation; forward == dense reference
# ---------------------------------------------------------------------------------

def check_p4_cumsum():
    """32. Sparse MoE Token Dispatch & Combine, steps 2-6: for top-1, the position of a
    token in its expert's queue is the exclusive cumulative count of the one-hot
    assignment; dropped tokens get all-zero output (no residual)."""
    rng = np.random.default_rng(3)
    T, E, D, C = 40, 3, 4, 9
    expert_idx = rng.integers(0, E, size=T)
    onehot = np.eye(E)[expert_idx]
    pos = ((np.cumsum(onehot, axis=0) - onehot) * onehot).sum(1).astype(np.int64)
    keep = pos < C
    d = om.dispatch(expert_idx[:, None], E, C)
    assert np.array_equal(d["kept"][:, 0], keep)
    assert np.array_equal(d["slot"][:, 0], np.where(keep, pos, -1))
    # combine with the one-hot (T,E,C) tensor versus the oracle's sparse combine
    x = rng.standard_normal((T, D))
    W = rng.standard_normal((E, D, D))
    gate = rng.random(T)
    disp = np.zeros((T, E, C))
    kk = np.flatnonzero(keep)
    disp[kk, expert_idx[kk], pos[kk]] = 1.0
    ex_in = np.einsum("tec,td->ecd", disp, x)
    ex_out = np.einsum("ecd,edf->ecf", ex_in, W)
    y_ref = np.einsum("tec,ecd->td", disp * gate[:, None, None], ex_out)
    o = om.expert_outputs("linear", {"w_in": W}, x, expert_idx[:, None], d["kept"])
    y = om.combine(x, None, o, gate[:, None], d["kept"], residual=False)
    np.testing.assert_allclose(y, y_ref, atol=1e-12)
    assert np.all(y[~keep] == 0.0)


def test_p4_cumsum_top1():
    check_p4_cumsum()


def _tiny_weights(rng, kind, E, D, F, bias):
    w = {}
    if kind == "linear":
        w["w_in"] = rng.standard_normal((E, D, D)) * 0.5
    elif kind == "gelu":
        w["w_in"] = rng.standard_normal((E, D, F)) * 0.5
        w["w_out"] = rng.standard_normal((E, F, D)) * 0.5
        w["b_in"] = rng.standard_normal((E, F)) * 0.5 if bias else np.zeros((E, F))
        w["b_out"] = rng.standard_normal((E, D)) * 0.5 if bias else np.zeros((E, D))
    else:
        w["w_in"] = rng.standard_normal((E, D, F)) * 0.5
        w["w_up"] = rng.standard_normal((E, D, F)) * 0.5
        w["w_out"] = rng.standard_normal((E, F, D)) * 0.5
    return w


@pytest.mark.parametrize("kind", ["linear", "gelu", "swiglu"])
def test_sparse_equals_dense_reference(kind):
    """Sparse MoE Layer in NumPy, section 3: the sparse forward equals an independent
    dense reference that runs every expert on every token."""
    rng = np.random.default_rng(11)
    T, D, E, k, F = 24, 5, 4, 2, 7
    x = rng.standard_normal((T, D))
    s = np.round(rng.standard_normal((T, E)) * 4) / 4     # exact ties included
    w = _tiny_weights(rng, kind, E, D, F, True)
    shared = None
    if kind == "swiglu":
        shared = {"w_in": rng.standard_normal((D, F)), "w_up": rng.standard_normal((D, F)),
                  "w_out": rng.standard_normal((F, D))}
    for C in (0, 3, 6, 12, T * k):
        for residual in (True, False):
            f = om.forward(x, k, kind, w, logits=s, C=C, residual=residual, shared=shared)
            yd, _ = om.dense_forward(x, k, kind, w, logits=s, C=C, residual=residual, shared=shared)
            np.testing.assert_allclose(f["y"], yd, atol=1e-11, rtol=1e-11)


def test_p3_moe_invariants():
    """Module 7 EducationalMoE invariants: one expert at k=1 without capacity limit is
    the dense SwiGLU expert, and a shared expert adds its dense output."""
    rng = np.random.default_rng(60)
    h, i = 8, 12
    x = rng.standard_normal((16, h))
    w = {"w_in": rng.standard_normal((1, h, i)) / math.sqrt(h),
         "w_up": rng.standard_normal((1, h, i)) / math.sqrt(h),
         "w_out": rng.standard_normal((1, i, h)) / math.sqrt(i)}
    wr = rng.standard_normal((h, 1))
    dense = (scipy.special.expit(x @ w["w_in"][0]) * (x @ w["w_in"][0]) * (x @ w["w_up"][0])) @ w["w_out"][0]
    f = om.forward(x, 1, "swiglu", w, w_router=wr, C=16, residual=False)
    np.testing.assert_allclose(f["y"], dense, atol=1e-12)
    sh = {"w_in": rng.standard_normal((h, i)), "w_up": rng.standard_normal((h, i)),
          "w_out": rng.standard_normal((i, h))}
    dense_sh = (scipy.special.expit(x @ sh["w_in"]) * (x @ sh["w_in"]) * (x @ sh["w_up"])) @ sh["w_out"]
    f2 = om.forward(x, 1, "swiglu", w, w_router=wr, C=16, residual=False, shared=sh)
    np.testing.assert_allclose(f2["y"], dense + dense_sh, atol=1e-12)


# ---------------------------------------------------------------------------------
# Backward: central finite differences, closed form of the router chain
# ---------------------------------------------------------------------------------

def _fd_problem(seed=5, T=6, D=4, E=4, k=2, C=2):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    W = rng.standard_normal((E, D, D))
    # distinct logits with every gap >= 0.1, so +-1e-6 never flips the top-k set
    s = np.stack([rng.permutation(E) * 0.37 + rng.random() for _ in range(T)])
    dy = rng.standard_normal((T, D))
    return x, W, s, dy, k, C


def _loss(x, W, s, dy, k, C, residual, aux_scale, ref_idx=None, ref_kept=None):
    f = om.forward(x, k, "linear", {"w_in": W}, logits=s, C=C, residual=residual)
    if ref_idx is not None:
        assert np.array_equal(f["idx"], ref_idx) and np.array_equal(f["kept"], ref_kept)
    return float(np.sum(dy * f["y"]) + aux_scale * f["aux"])


def check_backward_fd(residual=True, aux_scale=0.0, C=2):
    x, W, s, dy, k, C = _fd_problem(C=C)
    f = om.forward(x, k, "linear", {"w_in": W}, logits=s, C=C, residual=residual)
    g = om.backward_linear(dy, x, W, s, f["idx"], f["gate"], f["kept"], f["slot"], f["count"],
                           residual=residual, aux_grad_scale=aux_scale)
    h = 1e-6
    args = dict(dy=dy, k=k, C=C, residual=residual, aux_scale=aux_scale,
                ref_idx=f["idx"], ref_kept=f["kept"])

    def fd(arr, name):
        out = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            a_p = arr.copy(); a_p[i] += h
            a_m = arr.copy(); a_m[i] -= h
            kw = {"x": x, "W": W, "s": s}
            kw[name] = a_p
            lp = _loss(kw["x"], kw["W"], kw["s"], **args)
            kw[name] = a_m
            lm = _loss(kw["x"], kw["W"], kw["s"], **args)
            out[i] = (lp - lm) / (2 * h)
        return out

    assert np.max(np.abs(fd(x, "x") - g["dx"])) < 1e-6
    assert np.max(np.abs(fd(W, "W") - g["dW"])) < 1e-6
    assert np.max(np.abs(fd(s, "s") - g["dlogits"])) < 1e-6
    assert (~f["kept"]).any() or C >= 12


@pytest.mark.parametrize("residual,aux_scale,C", [(True, 0.0, 2), (False, 0.0, 2),
                                                   (True, 1.0, 3), (True, 0.0, 12)])
def test_backward_finite_differences(residual, aux_scale, C):
    """Sparse MoE Layer in NumPy, section 3: backward equals central differences (bar
    1e-6; the page reaches about 4e-9), dropped assignments held constant."""
    check_backward_fd(residual, aux_scale, C)


def test_router_grad_closed_form():
    """The quotient rule followed by the softmax Jacobian collapses to
    ds[t, idx_tj] = g_tj (dgate_tj - sum_r g_tr dgate_tr) and 0 elsewhere; rows sum to
    zero; k = 1 gives zero (Module 7, B09: the single-choice gate has zero gradient)."""
    rng = np.random.default_rng(8)
    T, E = 20, 9
    for k in (1, 2, 4, 9):
        s = rng.standard_normal((T, E)) * 2
        r = om.route(s, k)
        dgate = rng.standard_normal((T, k))
        ds = om.router_grad(s, r["idx"], r["gate"], dgate)
        G = np.sum(r["gate"] * dgate, axis=1, keepdims=True)
        want = np.zeros((T, E))
        np.put_along_axis(want, r["idx"], r["gate"] * (dgate - G), axis=1)
        np.testing.assert_allclose(ds, want, atol=1e-13)
        np.testing.assert_allclose(ds.sum(1), 0.0, atol=1e-13)
        if k == 1:
            assert np.all(np.abs(ds) < 1e-15)


def test_aux_grad_fd():
    rng = np.random.default_rng(9)
    T, E, k = 7, 5, 2
    s = rng.standard_normal((T, E))
    r = om.route(s, k)
    g = om.aux_grad(s, r["count"], k)
    h = 1e-6
    fd = np.zeros_like(s)
    for i in np.ndindex(s.shape):
        sp = s.copy(); sp[i] += h
        sm = s.copy(); sm[i] -= h
        rp, rm = om.route(sp, k), om.route(sm, k)
        assert np.array_equal(rp["count"], r["count"]) and np.array_equal(rm["count"], r["count"])
        fd[i] = (rp["aux"] - rm["aux"]) / (2 * h)
    assert np.max(np.abs(fd - g)) < 1e-8


def test_activation_gradients():
    """gelu' and silu' against central differences of gelu / silu, and their values at
    0: both derivatives are 1/2 there (Phi(0) = sigma(0) = 1/2)."""
    z = np.linspace(-6, 6, 241)
    h = 1e-6
    np.testing.assert_allclose(om.gelu_grad(z), (om.gelu(z + h) - om.gelu(z - h)) / (2 * h), atol=1e-8)
    np.testing.assert_allclose(om.silu_grad(z), (om.silu(z + h) - om.silu(z - h)) / (2 * h), atol=1e-8)
    assert om.gelu_grad(np.array([0.0]))[0] == 0.5 and om.silu_grad(np.array([0.0]))[0] == 0.5


def _mlp_problem(kind, seed, T=7, D=4, E=3, k=2, F=5, with_shared=False, with_router=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, D))
    w = {"w_in": rng.standard_normal((E, D, D if kind == "linear" else F)) * 0.7}
    if kind == "gelu":
        w.update(b_in=rng.standard_normal((E, F)) * 0.5, w_out=rng.standard_normal((E, F, D)) * 0.7,
                 b_out=rng.standard_normal((E, D)) * 0.5)
    if kind == "swiglu":
        w.update(w_up=rng.standard_normal((E, D, F)) * 0.7, w_out=rng.standard_normal((E, F, D)) * 0.7)
    sh = None
    if with_shared:
        sh = {"w_in": rng.standard_normal((D, 3)) * 0.7, "w_up": rng.standard_normal((D, 3)) * 0.7,
              "w_out": rng.standard_normal((3, D)) * 0.7}
    wr = rng.standard_normal((D, E)) if with_router else None
    s = None if with_router else np.stack([rng.permutation(E) * 0.37 + rng.random() for _ in range(T)])
    dy = rng.standard_normal((T, D))
    return x, w, sh, wr, s, dy, k


@pytest.mark.parametrize("kind,shared,router,aux,residual", [
    ("gelu", False, False, 0.0, True), ("swiglu", False, False, 1.0, True),
    ("swiglu", True, False, 0.0, False), ("gelu", False, True, 1.0, True),
    ("swiglu", True, True, 0.5, True), ("linear", False, True, 0.0, True)])
def test_mlp_backward_finite_differences(kind, shared, router, aux, residual):
    """The whole-layer backward through GELU / SwiGLU experts, the shared expert and the
    router weights equals central differences of <dy, y> + aux_scale * aux with the top-k
    set and the kept mask constant (Sparse MoE Layer in NumPy, section 3 method)."""
    x, w, sh, wr, s, dy, k = _mlp_problem(kind, seed=11 + len(kind), with_shared=shared, with_router=router)
    C = 3
    f = om.forward(x, k, kind, w, logits=s, w_router=wr, C=C, residual=residual, shared=sh)
    g = om.backward(dy, x, kind, w, f["logits"], f["idx"], f["gate"], f["kept"], f["count"],
                    residual=residual, aux_grad_scale=aux, shared=sh, w_router=wr)
    assert (~f["kept"]).any()   # some assignments dropped
    h = 1e-6

    def loss(x_, w_, sh_, wr_, s_):
        ff = om.forward(x_, k, kind, w_, logits=s_, w_router=wr_, C=C, residual=residual, shared=sh_)
        assert np.array_equal(ff["idx"], f["idx"]) and np.array_equal(ff["kept"], f["kept"])
        return float(np.sum(dy * ff["y"]) + aux * ff["aux"])

    def fd(get, put):
        base = get()
        out = np.zeros_like(base)
        for i in np.ndindex(base.shape):
            a = base.copy(); a[i] += h; lp = put(a)
            a = base.copy(); a[i] -= h; lm = put(a)
            out[i] = (lp - lm) / (2 * h)
        return out

    np.testing.assert_allclose(fd(lambda: x, lambda a: loss(a, w, sh, wr, s)), g["dx"], atol=2e-6)
    for n, arr in w.items():
        def put(a, n=n):
            w2 = dict(w); w2[n] = a
            return loss(x, w2, sh, wr, s)
        np.testing.assert_allclose(fd(lambda arr=arr: arr, put), g["dexperts"][n], atol=2e-6)
    if sh is not None:
        for n, arr in sh.items():
            def put(a, n=n):
                s2 = dict(sh); s2[n] = a
                return loss(x, w, s2, wr, s)
            np.testing.assert_allclose(fd(lambda arr=arr: arr, put), g["dshared"][n][0] if g["dshared"][n].ndim == 3 else g["dshared"][n], atol=2e-6)
    if wr is not None:
        np.testing.assert_allclose(fd(lambda: wr, lambda a: loss(x, w, sh, a, s)), g["dw_router"], atol=2e-6)
    else:
        np.testing.assert_allclose(fd(lambda: s, lambda a: loss(x, w, sh, wr, a)), g["dlogits"], atol=2e-6)


# ---------------------------------------------------------------------------------
# P3 router variants: sigmoid scoring, selection bias, survivor renormalisation, z-loss
# ---------------------------------------------------------------------------------

def check_p3_sigmoid_router():
    """Module 7, the asserts after router_z_loss: the REFERENCE router entry (sigmoid
    scoring, top-4 of 8, with and without the selection bias; atol 1e-12 as printed) and
    the extreme-logit cases (finite log-space gates)."""
    ref = _load("p3_reference.json")["router"]
    s = np.array([ref["logits"]])
    base = om.route(s, 4, scoring="sigmoid")
    assert base["idx"][0].tolist() == ref["selected"]
    np.testing.assert_allclose(base["gate"][0], ref["gates"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(base["clean"][0], ref["scores"], rtol=0, atol=1e-15)
    biased = om.route(s, 4, scoring="sigmoid", selection_bias=np.array(ref["bias"]))
    assert biased["idx"][0].tolist() == ref["selected_with_bias"]
    np.testing.assert_allclose(biased["gate"][0], ref["gates_with_bias"], rtol=0, atol=1e-12)
    ext = om.route(np.array([[-1002.0, -1000.0, -1001.0]]), 2, scoring="sigmoid")
    assert ext["idx"].tolist() == [[1, 2]]
    assert np.all(np.isfinite(ext["gate"]))
    np.testing.assert_allclose(ext["gate"], [[1 / (1 + np.exp(-1)), 1 / (1 + np.exp(1))]],
                               rtol=0, atol=1e-15)
    ext4 = om.route(np.array([[-1002.0, -1000.0, -1001.0, -1003.0]]), 2, scoring="sigmoid")
    assert ext4["idx"].tolist() == [[1, 2]]


def test_p3_sigmoid_router():
    check_p3_sigmoid_router()


def check_p3_renormalise_survivors():
    """Module 7, REFERENCE capacity entry under its fifo_drop_then_renormalize_survivors
    policy: every token keeps at least one choice, so its renormalised gates sum to 1;
    and the all-same case (k = 1, cf = 0.5): tokens 1-3 fully dropped with zero gates."""
    ref = _load("p3_reference.json")["capacity"]
    assert ref["policy"] == "fifo_drop_then_renormalize_survivors"
    s = np.array(ref["logits"])
    r = om.route(s, 2)
    C = om.capacity(12, 2, 4, 1.0)
    d = om.dispatch(r["idx"], 4, C)
    g = om.renormalise_kept(r["gate"], d["kept"])
    assert C == ref["capacity_per_expert"]
    assert d["used"].tolist() == ref["after_counts"]
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(g[~d["kept"]] == 0.0)
    r1 = om.route(np.tile([9.0, 0.0], (4, 1)), 1)
    d1 = om.dispatch(r1["idx"], 2, om.capacity(4, 1, 2, 0.5))
    g1 = om.renormalise_kept(r1["gate"], d1["kept"])
    assert d1["kept"][:, 0].tolist() == [True, False, False, False]
    assert g1[0, 0] == 1.0 and np.all(g1[1:] == 0.0)


def test_p3_renormalise_survivors():
    check_p3_renormalise_survivors()


def check_p3_z_loss():
    """Module 7: router_z_loss on the REFERENCE aux logits (rel 1e-12), and squaring per
    token before the token mean (the two-token example and its wrong alternative)."""
    ref = _load("p3_reference.json")["losses"]
    z_ref = ref["z_loss"]
    s = np.array(ref["aux_logits"])
    assert math.isclose(om.z_loss(s), z_ref, rel_tol=1e-12)
    assert math.isclose(om.route(s, 1)["z_loss"], z_ref, rel_tol=1e-12)
    two = np.array([[0.0, 0.0], [2.0, 2.0]])
    want = (math.log(2) ** 2 + (2 + math.log(2)) ** 2) / 2
    assert math.isclose(om.z_loss(two), want, rel_tol=1e-12)
    assert not math.isclose(om.z_loss(two), (1 + math.log(2)) ** 2)


def test_p3_z_loss():
    check_p3_z_loss()


def test_z_loss_grad_fd():
    """The z-loss gradient against central differences, and its closed-form row sum
    (2/T) lse_t (the softmax row sums to 1)."""
    rng = np.random.default_rng(5)
    s = rng.standard_normal((6, 5)) * 2
    h = 1e-6
    fd = np.zeros_like(s)
    for i in np.ndindex(s.shape):
        a = s.copy(); a[i] += h; lp = om.z_loss(a)
        a = s.copy(); a[i] -= h; lm = om.z_loss(a)
        fd[i] = (lp - lm) / (2 * h)
    g = om.z_loss_grad(s)
    np.testing.assert_allclose(g, fd, atol=1e-8)
    lse = scipy.special.logsumexp(s, axis=1)
    np.testing.assert_allclose(g.sum(axis=1), 2.0 / s.shape[0] * lse, rtol=1e-12)


def check_sigmoid_router_grad():
    """Sigmoid-scored gates: router_grad against central differences of <w, gate>, the
    top-k set held fixed; with k = 1 the gate is the constant 1, so the gradient is 0
    (Module 7, the gradcheck and k = 1 asserts of the explicit router)."""
    rng = np.random.default_rng(9)
    T, E, k = 5, 6, 3
    s = np.stack([rng.permutation(E) * 0.41 + rng.standard_normal() for _ in range(T)])
    w = rng.standard_normal((T, k))
    r = om.route(s, k, scoring="sigmoid")
    g = om.router_grad(s, r["idx"], r["gate"], w, scoring="sigmoid")
    h = 1e-6
    fd = np.zeros_like(s)
    for i in np.ndindex(s.shape):
        a = s.copy(); a[i] += h; rp = om.route(a, k, scoring="sigmoid")
        a = s.copy(); a[i] -= h; rm = om.route(a, k, scoring="sigmoid")
        assert np.array_equal(rp["idx"], r["idx"]) and np.array_equal(rm["idx"], r["idx"])
        fd[i] = (np.sum(w * rp["gate"]) - np.sum(w * rm["gate"])) / (2 * h)
    np.testing.assert_allclose(g, fd, atol=1e-8)
    r1 = om.route(s, 1, scoring="sigmoid")
    assert np.all(r1["gate"] == 1.0)
    assert np.all(om.router_grad(s, r1["idx"], r1["gate"], w[:, :1], scoring="sigmoid") == 0.0)


def test_sigmoid_router_grad():
    check_sigmoid_router_grad()


@pytest.mark.parametrize("kind,scoring,renorm,zscale,bias", [
    ("gelu", "sigmoid", False, 0.0, False), ("swiglu", "softmax", True, 0.0, False),
    ("linear", "sigmoid", True, 0.7, True), ("gelu", "softmax", True, 0.3, True)])
def test_router_variants_backward_fd(kind, scoring, renorm, zscale, bias):
    """The whole-layer backward under P3's router variants against central differences
    of <dy, y> + 0.5 aux + zscale * z_loss, the top-k set and kept mask constant."""
    x, w, sh, wr, s, dy, k = _mlp_problem(kind, seed=23 + len(kind), with_shared=True)
    E = w["w_in"].shape[0]
    sb = np.array([0.05, -0.02, 0.03])[:E] if bias else None
    C, aux = 3, 0.5
    f = om.forward(x, k, kind, w, logits=s, C=C, shared=sh, scoring=scoring, selection_bias=sb,
                   renormalize=renorm)
    g = om.backward(dy, x, kind, w, f["logits"], f["idx"], f["gate"], f["kept"], f["count"],
                    aux_grad_scale=aux, shared=sh, scoring=scoring, renormalize=renorm,
                    z_grad_scale=zscale)
    assert (~f["kept"]).any()
    h = 1e-6

    def loss(x_, s_):
        ff = om.forward(x_, k, kind, w, logits=s_, C=C, shared=sh, scoring=scoring,
                        selection_bias=sb, renormalize=renorm)
        assert np.array_equal(ff["idx"], f["idx"]) and np.array_equal(ff["kept"], f["kept"])
        return float(np.sum(dy * ff["y"]) + aux * ff["aux"] + zscale * ff["z_loss"])

    for arr, want, put in ((s, g["dlogits"], lambda a: loss(x, a)),
                           (x, g["dx"], lambda a: loss(a, s))):
        fd = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            a = arr.copy(); a[i] += h; lp = put(a)
            a = arr.copy(); a[i] -= h; lm = put(a)
            fd[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(fd, want, atol=2e-6)


def test_general_backward_matches_linear_backward():
    """For single-linear experts the general backward reduces to backward_linear."""
    x, W, s, dy, k, C = _fd_problem(C=2)
    f = om.forward(x, k, "linear", {"w_in": W}, logits=s, C=C)
    a = om.backward_linear(dy, x, W, s, f["idx"], f["gate"], f["kept"], f["slot"], f["count"], aux_grad_scale=0.3)
    b = om.backward(dy, x, "linear", {"w_in": W}, s, f["idx"], f["gate"], f["kept"], f["count"], aux_grad_scale=0.3)
    for n_a, n_b in (("dx", "dx"), ("dgate", "dgate"), ("dlogits", "dlogits")):
        np.testing.assert_allclose(a[n_a], b[n_b], atol=1e-12)
    np.testing.assert_allclose(a["dW"], b["dexperts"]["w_in"], atol=1e-12)


# ---------------------------------------------------------------------------------
# Invariants and edge cases
# ---------------------------------------------------------------------------------

def test_invariants_random():
    rng = np.random.default_rng(2)
    for trial in range(20):
        T = int(rng.integers(1, 60)); E = int(rng.integers(1, 12)); k = int(rng.integers(1, E + 1))
        s = np.round(rng.standard_normal((T, E)) * 3) / 4
        r = om.route(s, k)
        C = int(rng.integers(0, T * k + 2))
        d = om.dispatch(r["idx"], E, C)
        np.testing.assert_allclose(r["gate"].sum(1), 1.0, atol=1e-12)
        for t in range(T):
            assert len(set(r["idx"][t].tolist())) == k
            sel = s[t, r["idx"][t]]
            assert np.all(np.diff(sel) <= 0)
            for j in range(k - 1):
                if sel[j] == sel[j + 1]:
                    assert r["idx"][t, j] < r["idx"][t, j + 1]
            # every unselected expert scores no higher than the last selected one
            rest = np.setdiff1d(np.arange(E), r["idx"][t])
            if rest.size:
                assert np.all(s[t, rest] <= sel[-1])
        assert r["count"].sum() == T * k
        assert np.array_equal(d["used"], np.minimum(r["count"], C))
        assert d["overflow"].sum() == d["drops"].sum()
        for e in range(E):
            a = d["slot_assign"][e, : d["used"][e]]
            assert np.all(a >= 0) and np.all(np.diff(a) > 0)
            assert np.all(d["slot_assign"][e, d["used"][e]:] == -1)
            tt, jj = a // k, a % k
            assert np.all(r["idx"][tt, jj] == e)
            assert np.array_equal(d["slot"][tt, jj], np.arange(d["used"][e]))


def test_edge_cases():
    """Sparse MoE Layer in NumPy, section 3 edge checks: k == E, capacity 0 (output
    exactly x), a single token, a single expert, no residual."""
    rng = np.random.default_rng(4)
    T, D, E = 9, 3, 4
    x = rng.standard_normal((T, D))
    W = rng.standard_normal((E, D, D))
    s = rng.standard_normal((T, E))
    f = om.forward(x, E, "linear", {"w_in": W}, logits=s, C=T, residual=True)
    assert f["kept"].all()
    dense = x + sum(f["gate"][:, j:j + 1] * np.einsum("td,tdf->tf", x, W[f["idx"][:, j]]) for j in range(E))
    np.testing.assert_allclose(f["y"], dense, atol=1e-12)
    f0 = om.forward(x, 2, "linear", {"w_in": W}, logits=s, cf=0.0, residual=True)
    assert f0["C"] == 0 and np.array_equal(f0["y"], x)
    f1 = om.forward(x[:1], 2, "linear", {"w_in": W}, logits=s[:1], cf=1.0)
    assert f1["C"] == 1 and f1["kept"].all()
    fe = om.forward(x, 1, "linear", {"w_in": W[:1]}, logits=s[:, :1], C=T, residual=False)
    np.testing.assert_allclose(fe["y"], x @ W[0], atol=1e-12)
    assert fe["aux"] == 1.0


def test_signed_zero_ties():
    """-0.0 and +0.0 tie, so the lower index wins whichever carries the sign."""
    r = om.route(np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]]), 1)
    assert r["idx"][:, 0].tolist() == [0, 0]


# ---------------------------------------------------------------------------------
# Textbook routines and the bf16 rounding
# ---------------------------------------------------------------------------------

def test_activations_against_library():
    z = np.linspace(-9, 9, 1001)
    np.testing.assert_allclose(om.gelu(z), z * scipy.stats.norm.cdf(z), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(om.silu(z), z * scipy.special.expit(z), rtol=1e-13, atol=1e-15)
    assert om.gelu(np.array([1.0]))[0] == pytest.approx(0.8413447460685429, rel=1e-15)
    assert om.silu(np.array([-800.0]))[0] == 0.0


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 8, 20000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0])])
    want = torch.tensor(v.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = om.bf16_round(v.astype(np.float32))
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------------
# Planted mistakes: each one must be caught by a pin above
# ---------------------------------------------------------------------------------

def _tie_to_higher(s, k):
    s = np.asarray(s, dtype=np.float64)
    T, E = s.shape
    return np.stack([np.lexsort((-np.arange(E), -s[t]))[:k] for t in range(T)])


def _dispatch_choice_major(idx, E, C):
    """Planted mistake: every token's first choice is served before any second choice
    (choice-major order instead of the flat token-then-choice order)."""
    T, k = idx.shape
    arrivals = np.zeros(E, dtype=np.int64)
    slot = np.full((T, k), -1, dtype=np.int64)
    for j in range(k):
        for t in range(T):
            e = idx[t, j]
            if arrivals[e] < C:
                slot[t, j] = arrivals[e]
            arrivals[e] += 1
    kept = slot >= 0
    used = np.minimum(arrivals, C)
    sa = np.full((E, C), -1, dtype=np.int64)
    return {"slot": slot, "kept": kept, "slot_assign": sa, "used": used,
            "overflow": arrivals - used, "drops": k - kept.sum(1)}


def _route_aux_over_T(logits, k):
    r = _ORIG_ROUTE(logits, k)
    T, E = r["p"].shape
    r["aux"] = float(E * np.sum(r["count"] / T * r["prob_sum"] / T))
    return r


def _route_no_renorm(logits, k):
    r = _ORIG_ROUTE(logits, k)
    r["gate"] = np.take_along_axis(r["p"], r["idx"], axis=1)
    return r


def _router_grad_no_centering(logits, idx, gate, dgate):
    p = om.softmax(logits)
    T, E = p.shape
    q = np.take_along_axis(p, idx, axis=1)
    S = np.sum(q, axis=1, keepdims=True)
    dq = dgate / S                       # quotient rule's second term dropped
    dp = np.zeros((T, E))
    for j in range(idx.shape[1]):
        np.add.at(dp, (np.arange(T), idx[:, j]), dq[:, j])
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def _capacity_floor(T, k, E, cf):
    return int(math.floor(cf * T * k / E))


def _route_gates_with_bias(logits, k, *, scoring="softmax", selection_bias=None):
    r = _ORIG_ROUTE(logits, k, scoring=scoring, selection_bias=selection_bias)
    if selection_bias is not None:       # the bias leaks into the mixture weights
        q = np.take_along_axis(r["clean"] + np.asarray(selection_bias)[None, :], r["idx"], axis=1)
        r["gate"] = q / q.sum(axis=1, keepdims=True)
    return r


def _z_loss_square_after_mean(logits):
    s = np.asarray(logits, dtype=np.float64)
    return float(np.mean(scipy.special.logsumexp(s, axis=1)) ** 2)


def _renorm_over_all_choices(gate, kept):
    g = np.where(kept, gate, 0.0)
    return g / np.sum(gate, axis=1, keepdims=True)


def _sigmoid_grad_no_derivative(logits, idx, gate, dgate, scoring="softmax"):
    if scoring != "sigmoid":
        return _ORIG_ROUTER_GRAD(logits, idx, gate, dgate, scoring)
    q = om.sigmoid(np.take_along_axis(logits, idx, axis=1))
    dq = (dgate - np.sum(gate * dgate, axis=1, keepdims=True)) / q.sum(axis=1, keepdims=True)
    ds = np.zeros(np.shape(logits))
    for j in range(idx.shape[1]):
        np.add.at(ds, (np.arange(idx.shape[0]), idx[:, j]), dq[:, j] * q[:, j])   # (1 - q) dropped
    return ds


def _sigmoid_flipped(s):
    return 1.0 / (1.0 + np.exp(np.asarray(s, dtype=np.float64)))


_ORIG_ROUTE = om.route
_ORIG_ROUTER_GRAD = om.router_grad

MUTATIONS = [
    ("top_k", _tie_to_higher, lambda: (check_p2_examples(), check_p3_tie_break())),
    ("dispatch", _dispatch_choice_major, lambda: check_bruteforce(ks=(2,), stride=7)),
    ("route", _route_aux_over_T, check_p3_aux),
    ("route", _route_no_renorm, check_p2_examples),
    ("router_grad", _router_grad_no_centering, lambda: check_backward_fd(True, 0.0, 2)),
    ("capacity", _capacity_floor, check_capacity),
    ("route", _route_gates_with_bias, check_p3_sigmoid_router),
    ("z_loss", _z_loss_square_after_mean, check_p3_z_loss),
    ("renormalise_kept", _renorm_over_all_choices, check_p3_renormalise_survivors),
    ("router_grad", _sigmoid_grad_no_derivative, check_sigmoid_router_grad),
    ("sigmoid", _sigmoid_flipped, check_p3_sigmoid_router),
]


@pytest.mark.parametrize("name,mutant,pin", MUTATIONS, ids=[m[1].__name__ for m in MUTATIONS])
def test_planted_mistakes_are_caught(monkeypatch, name, mutant, pin):
    monkeypatch.setattr(om, name, mutant)
    with pytest.raises(AssertionError):
        pin()
