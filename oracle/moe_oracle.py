"""Plain CPU oracle for the capacity-limited sparse MoE layer, forward and backward.

TEST INFRASTRUCTURE. This module is the slow, obviously-correct definition that the
HIP path is checked against. Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it. The
product path never calls it, and it imports nothing from the HIP package.

Everything is NumPy float64. Loops follow the pages where the pages loop (the
position-priority dispatch walks the assignments serially in token-then-choice
order). Library primitives (a sort, a matmul, ``exp``) are used as single steps;
nothing is blocked, fused or
reordered beyond what the definitions state.

Sources (page titles; sections named as on the pages):
  [P1] "Sparse MoE Layer in NumPy -- Token Drop, Exact Dispatch/Combine, Aux Loss &
       Backward" (ob1.it.com): section 1 (the seven traps), section 2 (top_k_gating,
       position_priority_dispatch, the forward/backward einsums), section 3.
  [P2] "Top-k MoE Router with Load Statistics" (tensortonic.com): the score, alpha,
       y, f_e and m_e equations; Requirements; Constraints.
  [P3] "Module 7. Mixture of Experts" (vladkulikov.com notebook): stable_softmax,
       _deterministic_top_k, route_logits, expert_capacity, dispatch_with_capacity,
       switch_auxiliary_loss, swiglu_expert, EducationalMoE.
  [P4] "32. Sparse MoE Token Dispatch & Combine (Capacity-Limited)": step-by-step
       approach, steps 2-6.
  [P5] "Mixture of Experts" (llm-atlas.app): the Expert and TopKMoE modules.

Readings where the pages are silent or disagree:
  * the top-k key is the fp32 logit, exact ties to the lower expert index (P2, P3);
  * -0.0 and +0.0 compare equal;
  * gates are renormalised over the k choices before any drop and never after (P1);
    P3's renormalisation of the survivors is a flag, off by default;
  * with sigmoid scoring (P3) the aux loss keeps the softmax probabilities for P_e
    and the counts of the selection actually made for f_e;
  * capacity is the exact ceil(T*k*cf/E) of the given double cf, with no clamp, so
    cf = 0 gives C = 0;
  * the aux loss uses f_e = count_e/(T*k) (P1 trap 6, P3), so it is 1 at uniform load;
  * GELU is the exact erf form (P5 uses F.gelu with its default);
  * bf16 configs round H and o to bf16 (round-to-nearest-even) after the activation
    and after the second GEMM; everything else is float64 here.

Parity pins live in tests/test_oracle_pins.py. Functions without an independent pin
say so in their docstring ("parity unpinned").
"""

from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "bf16_round",
    "softmax",
    "top_k",
    "route",
    "capacity",
    "dispatch",
    "gelu",
    "silu",
    "expert_apply",
    "expert_outputs",
    "combine",
    "forward",
    "dense_forward",
    "backward_linear",
    "backward",
    "gelu_grad",
    "silu_grad",
    "router_grad",
    "aux_grad",
    "sigmoid",
    "log_sigmoid",
    "renormalise_kept",
    "z_loss",
    "z_loss_grad",
]


# ----------------------------------------------------------------------------------
# Validation (P3: _finite_array / _positive_int / _bounded_real, and its negative tests)
# ----------------------------------------------------------------------------------

def _finite(name, a, ndim=None):
    a = np.asarray(a, dtype=np.float64)
    if ndim is not None and a.ndim != ndim:
        raise ValueError(f"{name} must have rank {ndim}, got shape {a.shape}")
    if a.size == 0:
        raise ValueError(f"{name} must be non-empty")
    if not np.all(np.isfinite(a)):
        raise ValueError(f"{name} must be finite")
    return a


def _check_k(k, E):
    if isinstance(k, bool) or not isinstance(k, (int, np.integer)):
        raise TypeError("k must be an integer")
    if not 1 <= int(k) <= E:
        raise ValueError(f"k must lie in [1, E={E}], got {k}")
    return int(k)


# ----------------------------------------------------------------------------------
# bf16 storage rounding
# ----------------------------------------------------------------------------------

def bf16_round(a):
    """Round to the nearest bf16 value, ties to even, returned as float64.

    The value is first rounded to float32 (NumPy's cast is round-to-nearest-even),
    then the low 16 bits of the float32 pattern are rounded away with the usual
    integer trick: add 0x7FFF plus the lowest kept bit, then truncate.
    """
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return bits.astype(np.uint32).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------------
# Routing: softmax, top-k, gates, load statistics, aux loss
# ----------------------------------------------------------------------------------

def softmax(s):
    """Row softmax with the row maximum subtracted first (P3 stable_softmax; P2
    requires the routing math in at least fp32; here it is float64)."""
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=1, keepdims=True)
    ex = np.exp(s - m)
    return ex / np.sum(ex, axis=1, keepdims=True)


def top_k(s, k):
    """The k experts of each row in descending score order; an exact tie goes to the
    lower expert index (P2: selection rule; P3: _deterministic_top_k; P1 trap 1).

    Each row is sorted lexicographically by the key (-score, expert index) and the
    first k entries are taken. -0.0 and +0.0 compare equal in the sort, so they tie.
    """
    s = np.asarray(s, dtype=np.float64)
    T, E = s.shape
    experts = np.arange(E)
    idx = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((experts, -s[t]))
        idx[t] = order[:k]
    return idx


def sigmoid(s):
    """Logistic function evaluated without overflow (P3 stable_sigmoid): 1/(1+e^-s) for
    s >= 0, e^s/(1+e^s) below."""
    s = np.asarray(s, dtype=np.float64)
    out = np.empty_like(s)
    pos = s >= 0.0
    out[pos] = 1.0 / (1.0 + np.exp(-s[pos]))
    ex = np.exp(s[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def log_sigmoid(s):
    """log(sigmoid(s)) = -log(1 + e^-s), finite for any finite s (P3 _log_sigmoid)."""
    return -np.logaddexp(0.0, -np.asarray(s, dtype=np.float64))


def route(logits, k, *, scoring="softmax", selection_bias=None):
    """Token-choice router with top-k selection, renormalised gates and pre-drop
    statistics.

    * p = softmax over all E experts (P1 section 2 top_k_gating; P5 TopKMoE).
    * clean scores: p for softmax scoring, sigmoid(s) for sigmoid scoring (P3
      route_logits, V3-style independent scores).
    * idx = top-k with lower-index tie-break (see ``top_k``) of the logits when no
      selection bias is given (both score functions are strictly increasing, so this
      is the ranking of the clean scores in exact arithmetic; P3 route_logits makes
      the same argument), else of clean + bias: the bias moves selection only (P3
      route_logits, selection_bias).
    * gates, from the clean scores of the selected experts only: softmax scoring,
      gate[t, j] = p[t, idx_tj] / sum_r p[t, idx_tr] (P1 top_k_gating; the softmax of
      the selected logits, P2 alpha equation); sigmoid scoring, the softmax over the
      selected experts of log sigmoid(s) (P3: normalised in log space), i.e.
      sigmoid(s_j) / sum_r sigmoid(s_r).
    * count[e] = number of (t, j) with idx = e, before any capacity drop;
      prob_sum[e] = sum_t p[t, e] (P2 f_e / m_e equations, P3 bincount).
    * aux = E * sum_e (count_e / (T*k)) * (prob_sum_e / T) (P1 trap 6; P3
      switch_auxiliary_loss).
    * z_loss = mean_t (logsumexp_e s[t, e])^2 (P3 router_z_loss, ST-MoE).
    """
    s = _finite("logits", logits, ndim=2)
    T, E = s.shape
    k = _check_k(k, E)
    if scoring not in ("softmax", "sigmoid"):
        raise ValueError("scoring must be 'softmax' or 'sigmoid'")
    p = softmax(s)
    clean = p if scoring == "softmax" else sigmoid(s)
    if selection_bias is None:
        idx = top_k(s, k)
    else:
        b = _finite("selection_bias", selection_bias, ndim=1)
        if b.shape != (E,):
            raise ValueError("selection_bias must have shape [E]")
        idx = top_k(clean + b[None, :], k)
    if scoring == "softmax":
        p_sel = np.take_along_axis(p, idx, axis=1)
        gate = p_sel / np.sum(p_sel, axis=1, keepdims=True)
    else:
        ls = log_sigmoid(np.take_along_axis(s, idx, axis=1))
        w = np.exp(ls - np.max(ls, axis=1, keepdims=True))
        gate = w / np.sum(w, axis=1, keepdims=True)
    count = np.bincount(idx.ravel(), minlength=E).astype(np.int64)
    prob_sum = np.sum(p, axis=0)
    f = count / (T * k)
    P = prob_sum / T
    aux = float(E * np.sum(f * P))
    return {
        "p": p,
        "clean": clean,
        "idx": idx,
        "gate": gate,
        "count": count,
        "prob_sum": prob_sum,
        "aux": aux,
        "z_loss": z_loss(s),
        "token_fraction": count / T,
        "probability_mass": P,
    }


def z_loss(logits):
    """Router z-loss: the token mean of the squared log-partition, mean_t lse_t^2 with
    lse_t = log sum_e exp(s[t, e]) (P3 router_z_loss; squared per token, then averaged)."""
    s = np.asarray(logits, dtype=np.float64)
    m = np.max(s, axis=1)
    lse = m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))
    return float(np.mean(lse ** 2))


def z_loss_grad(logits):
    """d z_loss / d s[t, e] = (2 / T) lse_t p[t, e], since d lse_t / d s[t, e] = p[t, e]."""
    s = np.asarray(logits, dtype=np.float64)
    T = s.shape[0]
    m = np.max(s, axis=1)
    lse = m + np.log(np.sum(np.exp(s - m[:, None]), axis=1))
    return (2.0 / T) * lse[:, None] * softmax(s)


# ----------------------------------------------------------------------------------
# Capacity and position-priority dispatch
# ----------------------------------------------------------------------------------

def capacity(T, k, E, cf):
    """C = ceil(T * k * cf / E) computed exactly on the given double cf (P1 trap 2;
    P3 expert_capacity). No clamp to 1: cf = 0 gives C = 0 (P1 section 3 edge check
    "capacity == 0")."""
    for name, v in (("T", T), ("k", k), ("E", E)):
        if isinstance(v, bool) or not isinstance(v, (int, np.integer)) or v < 1:
            raise ValueError(f"{name} must be a positive integer")
    if k > E:
        raise ValueError("k cannot exceed E")
    cf = float(cf)
    if not math.isfinite(cf) or cf < 0.0:
        raise ValueError("capacity_factor must be finite and >= 0")
    return int(math.ceil(Fraction(cf) * int(T) * int(k) / int(E)))


def dispatch(idx, E, C):
    """Position-priority slot assignment (P1 trap 3 and section 2; P3
    dispatch_with_capacity without survivor renormalisation; P4 steps 2-4).

    Definition: the assignments are ordered by their flat index a = t*k + j (earlier
    tokens first, then a token's choices in order). The slot of a is the number of
    earlier assignments to the same expert; a is kept iff that number is below C.

    Here the assignments are walked once in that order with one arrival counter per
    expert; the counter's value on arrival is the rank above. Every earlier arrival with
    a rank below C was itself kept, so the kept slots of an expert are 0..used-1.

    Returns slot [T,k] (-1 when dropped), kept [T,k] bool, slot_assign [E,C] holding
    the flat assignment a of each filled slot (-1 when empty), used [E],
    overflow [E] = arrivals - used, drops [T] = k - number kept.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    if np.any(idx < 0) or np.any(idx >= E):
        raise ValueError("expert index out of range")
    if C < 0:
        raise ValueError("capacity must be >= 0")
    flat = idx.reshape(-1)
    arrivals = np.zeros(E, dtype=np.int64)
    rank = np.empty(T * k, dtype=np.int64)
    slot_assign = np.full((E, C), -1, dtype=np.int64)
    for a in range(T * k):
        e = int(flat[a])
        rank[a] = arrivals[e]
        arrivals[e] += 1
        if rank[a] < C:
            slot_assign[e, rank[a]] = a
    keep = rank < C
    slot = np.where(keep, rank, -1).reshape(T, k)
    kept = keep.reshape(T, k)
    used = np.minimum(arrivals, C)
    return {
        "slot": slot,
        "kept": kept,
        "slot_assign": slot_assign,
        "used": used,
        "overflow": arrivals - used,
        "drops": (k - kept.sum(axis=1)).astype(np.int64),
    }


# ----------------------------------------------------------------------------------
# Experts
# ----------------------------------------------------------------------------------

_erf = np.vectorize(math.erf, otypes=[np.float64])


def gelu(z):
    """Exact GELU, z * Phi(z) = z/2 * (1 + erf(z / sqrt 2)) (P5 Expert uses F.gelu,
    whose default is this erf form)."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def silu(z):
    """SiLU, z * sigmoid(z), with the sigmoid evaluated in its overflow-free form
    (P3 swiglu_expert and stable_sigmoid)."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def expert_apply(kind, weights, e, xr, bf16=False):
    """Apply expert e to the rows xr [n, D].

    kind "linear": o = xr W_e (P1 section 2 forward einsum; weights W [E, D, D]).
    kind "gelu":   o = GELU(xr W1_e + b1_e) W2_e + b2_e (P5 Expert: fc1, gelu, fc2).
    kind "swiglu": o = (silu(xr Wg_e) * (xr Wu_e)) Wd_e (P3 swiglu_expert).

    ``weights`` maps w_in / w_up / w_out / b_in / b_out to arrays indexed [e, in, out]
    (or [e, out] for biases). With bf16=True the hidden activation and the output are
    rounded to bf16 where the layer stores them.
    """
    xr = _f64(xr)
    if kind == "linear":
        o = xr @ _f64(weights["w_in"][e])
    elif kind == "gelu":
        h = gelu(xr @ _f64(weights["w_in"][e]) + _f64(weights["b_in"][e]))
        if bf16:
            h = bf16_round(h)
        o = h @ _f64(weights["w_out"][e]) + _f64(weights["b_out"][e])
    elif kind == "swiglu":
        g = xr @ _f64(weights["w_in"][e])
        u = xr @ _f64(weights["w_up"][e])
        h = silu(g) * u
        if bf16:
            h = bf16_round(h)
        o = h @ _f64(weights["w_out"][e])
    else:
        raise ValueError(f"unknown expert kind {kind!r}")
    if bf16:
        o = bf16_round(o)
    return o


def expert_outputs(kind, weights, x, idx, kept, tokens=None, bf16=False):
    """Per-assignment expert outputs o[t, j] for the kept assignments of the given
    tokens (all tokens by default); dropped assignments get zeros. Rows are grouped by
    expert only so that each expert's weights are converted once (P3 EducationalMoE
    loops over experts the same way)."""
    x = np.asarray(x)
    idx = np.asarray(idx)
    T, k = idx.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    D_out = None
    out = {}
    sel_t, sel_j = [], []
    for t in tokens:
        for j in range(k):
            if kept[t, j]:
                sel_t.append(int(t))
                sel_j.append(j)
    sel_t = np.asarray(sel_t, dtype=np.int64)
    sel_j = np.asarray(sel_j, dtype=np.int64)
    experts = idx[sel_t, sel_j] if sel_t.size else np.zeros(0, dtype=np.int64)
    for e in np.unique(experts):
        rows = np.flatnonzero(experts == e)
        o = expert_apply(kind, weights, int(e), _f64(x[sel_t[rows]]), bf16=bf16)
        D_out = o.shape[1]
        for r, orow in zip(rows, o):
            out[(int(sel_t[r]), int(sel_j[r]))] = orow
    if D_out is None:
        D_out = np.asarray(x).shape[1]
    o_full = np.zeros((len(tokens), k, D_out))
    pos = {int(t): i for i, t in enumerate(tokens)}
    for (t, j), v in out.items():
        o_full[pos[t], j] = v
    return o_full


def shared_apply(shared, xr, bf16=False):
    """Always-on shared SwiGLU expert applied to every row, ungated (P2 y equation's
    shared term; P3 EducationalMoE shared loop)."""
    xr = _f64(xr)
    h = silu(xr @ _f64(shared["w_in"])) * (xr @ _f64(shared["w_up"]))
    if bf16:
        h = bf16_round(h)
    o = h @ _f64(shared["w_out"])
    if bf16:
        o = bf16_round(o)
    return o


def renormalise_kept(gate, kept):
    """Gates after P3's drop-then-renormalise-survivors policy (dispatch_with_capacity,
    renormalize_kept_gates): kept gates divided by the token's kept gate mass, dropped
    ones 0; a token with nothing kept keeps all zeros (no division by zero)."""
    g = np.where(np.asarray(kept, dtype=bool), _f64(gate), 0.0)
    mass = np.sum(g, axis=1, keepdims=True)
    return np.divide(g, mass, out=np.zeros_like(g), where=mass > 0.0)


def combine(x, shared_out, o, gate, kept, residual, renormalize=False):
    """y_t = r x_t + Sh_t + sum over kept j of gate_tj o_tj, j ascending (P1 trap 4 and
    section 2; P2 y equation; P4 step 6). A dropped assignment contributes nothing.
    With ``renormalize`` the kept gates are first renormalised over the survivors
    (``renormalise_kept``)."""
    o = _f64(o)
    T, k, D = o.shape
    g = renormalise_kept(gate, kept) if renormalize else np.where(kept, _f64(gate), 0.0)
    y = np.zeros((T, D))
    if residual:
        y = y + _f64(x)
    if shared_out is not None:
        y = y + _f64(shared_out)
    for j in range(k):
        w = np.where(kept[:, j], g[:, j], 0.0)
        y = y + w[:, None] * o[:, j, :]
    return y


def forward(x, k, kind, weights, *, logits=None, w_router=None, C=None, cf=None,
            residual=True, shared=None, bf16=False, tokens=None, scoring="softmax",
            selection_bias=None, renormalize=False):
    """The whole layer: router scores (if w_router is given), routing, capacity,
    dispatch, experts, combine, aux loss (P1 section 2 moe_forward; P3
    EducationalMoE.forward; P5 TopKMoE.forward). ``scoring``, ``selection_bias`` and
    ``renormalize`` select P3's router variants (see ``route`` and ``combine``).

    ``tokens`` restricts the expert/combine part to a subset of tokens (routing and
    dispatch always run over the whole batch, since slots depend on every earlier
    token). Returns a dict with the routing and dispatch results and y for the chosen
    tokens.
    """
    x = np.asarray(x)
    T = x.shape[0]
    if logits is None:
        if w_router is None:
            raise ValueError("need logits or w_router")
        logits = _f64(x) @ _f64(w_router)   # P2 score equation s = x^T w_e
    r = route(logits, k, scoring=scoring, selection_bias=selection_bias)
    E = r["p"].shape[1]
    if C is None:
        C = capacity(T, k, E, cf)
    d = dispatch(r["idx"], E, C)
    toks = np.arange(T) if tokens is None else np.asarray(tokens)
    o = expert_outputs(kind, weights, x, r["idx"], d["kept"], tokens=toks, bf16=bf16)
    sh = shared_apply(shared, np.asarray(x)[toks], bf16=bf16) if shared is not None else None
    y = combine(np.asarray(x)[toks], sh, o, r["gate"][toks], d["kept"][toks], residual,
                renormalize=renormalize)
    out = dict(r)
    out.update(d)
    out.update({"C": C, "logits": _f64(logits), "o": o, "shared_out": sh, "y": y,
                "tokens": toks})
    return out


def dense_forward(x, k, kind, weights, *, logits, C, residual=True, shared=None):
    """Independent dense reference (P1 section 3): run every expert on every token,
    then contract with the (T, E, C) combine tensor (P1 trap 5; P4 steps 4-6).

    combine[t, e, c] = gate_tj when token t's choice j went to expert e in slot c and
    was kept; 0 elsewhere. y = r x + sum_{e,c} combine[t,e,c] * Expert_e(x_t) + Sh.
    Only for tiny shapes: it materialises T x E x C and T x E x D.
    """
    x = _f64(x)
    r = route(logits, k)
    T, E = r["p"].shape
    d = dispatch(r["idx"], E, C)
    comb = np.zeros((T, E, C))
    for t in range(T):
        for j in range(k):
            if d["kept"][t, j]:
                comb[t, r["idx"][t, j], d["slot"][t, j]] = r["gate"][t, j]
    dense = np.stack([expert_apply(kind, weights, e, x) for e in range(E)], axis=1)
    y = np.einsum("tec,ted->td", comb, dense)
    if residual:
        y = y + x
    if shared is not None:
        y = y + shared_apply(shared, x)
    return y, comb


# ----------------------------------------------------------------------------------
# Backward (single-linear experts): P1 section 2 moe_backward and trap 7
# ----------------------------------------------------------------------------------

def router_grad(logits, idx, gate, dgate, scoring="softmax"):
    """Gradient of the loss through the renormalised gates back to the logits, with the
    top-k set held fixed (P1 trap 7: quotient rule, then the derivative of the scores).

    With q_j the clean score of the j-th choice and S_t = sum_r q_r, gate_j = q_j / S_t
    gives
        dq_j = (dgate_j - sum_r gate_r dgate_r) / S_t          (quotient rule)
    Softmax scoring, q = p[t, idx_tj]:
        dp[t, i] = sum_j [i == idx_tj] dq_j
        ds[t, i] = p_i (dp_i - sum_l p_l dp_l)                 (softmax Jacobian)
    Sigmoid scoring, q = sigmoid(s[t, idx_tj]) (P3's log-space normalisation is the
    same function): each score depends on its own logit only, so
        ds[t, idx_tj] = dq_j q_j (1 - q_j),  0 for experts not chosen.
    """
    s = np.asarray(logits, dtype=np.float64)
    T, E = s.shape
    k = idx.shape[1]
    if scoring == "sigmoid":
        q = sigmoid(np.take_along_axis(s, idx, axis=1))
        S = np.sum(q, axis=1, keepdims=True)
        G = np.sum(gate * dgate, axis=1, keepdims=True)
        dq = (dgate - G) / S
        ds = np.zeros((T, E))
        for j in range(k):
            np.add.at(ds, (np.arange(T), idx[:, j]), dq[:, j] * q[:, j] * (1.0 - q[:, j]))
        return ds
    p = softmax(s)
    q = np.take_along_axis(p, idx, axis=1)
    S = np.sum(q, axis=1, keepdims=True)
    G = np.sum(gate * dgate, axis=1, keepdims=True)
    dq = (dgate - G) / S
    dp = np.zeros((T, E))
    for j in range(k):
        np.add.at(dp, (np.arange(T), idx[:, j]), dq[:, j])
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def aux_grad(logits, count, k):
    """d aux / d logits with the counts held constant (they are piecewise constant in
    the logits): aux = E sum_e f_e P_e, P_e = mean_t p[t, e], f_e = count_e/(T k)
    (P1 section 3 checks this gradient by finite differences)."""
    p = softmax(logits)
    T, E = p.shape
    f = np.asarray(count, dtype=np.float64) / (T * k)
    return (E / T) * p * (f[None, :] - np.sum(p * f[None, :], axis=1, keepdims=True))


def backward_linear(dy, x, W, logits, idx, gate, kept, slot, count, *,
                    residual=True, aux_grad_scale=0.0):
    """Backward of y = r x + sum_kept gate * (x W_e) for single-linear experts, with the
    discrete choices (top-k set, kept mask) as constants (P1 section 2 moe_backward).

      dgate_a = kept_a <dy_t, x_t W_e>            (P1 dM einsum, restricted to kept)
      dW_e    = sum_{kept a -> e} gate_a x_t^T dy_t   (P1 dW einsum)
      dx_t    = r dy_t + sum_{kept a in t} gate_a dy_t W_e^T   (P1 dx einsum)
      dlogits = router_grad(dgate) + aux_grad_scale * aux_grad
    """
    dy = _f64(dy)
    x = _f64(x)
    T, k = idx.shape
    E = W.shape[0]
    D_in = x.shape[1]
    D_out = dy.shape[1]
    dgate = np.zeros((T, k))
    dW = np.zeros((E, D_in, D_out))
    dx = dy.copy() if residual else np.zeros((T, D_in))
    for e in range(E):
        tt, jj = np.nonzero((idx == e) & kept)
        if tt.size == 0:
            continue
        We = _f64(W[e])
        o = x[tt] @ We
        dgate[tt, jj] = np.sum(dy[tt] * o, axis=1)
        g = gate[tt, jj][:, None]
        dW[e] = x[tt].T @ (g * dy[tt])
        np.add.at(dx, tt, (g * dy[tt]) @ We.T)
    dlogits = router_grad(logits, idx, gate, dgate)
    if aux_grad_scale:
        dlogits = dlogits + aux_grad_scale * aux_grad(logits, count, k)
    return {"dgate": dgate, "dW": dW, "dx": dx, "dlogits": dlogits}


def gelu_grad(z):
    """d GELU / dz = Phi(z) + z phi(z) for the exact (erf) GELU, with Phi the standard
    normal CDF and phi its density (the derivative of z Phi(z))."""
    z = _f64(z)
    phi = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    Phi = 0.5 * (1.0 + np.vectorize(math.erf)(z / math.sqrt(2.0)))
    return Phi + z * phi


def silu_grad(z):
    """d silu / dz = sigma(z) (1 + z (1 - sigma(z))), the derivative of z sigma(z)."""
    z = _f64(z)
    sig = np.where(z >= 0, 1.0 / (1.0 + np.exp(-np.abs(z))), np.exp(-np.abs(z)) / (1.0 + np.exp(-np.abs(z))))
    return sig * (1.0 + z * (1.0 - sig))


def _mlp_backward(kind, w, e, xr, dO):
    """Backward of one expert applied to the rows xr with output gradient dO (already
    gated): returns (grads of its parameters, gradient of its input rows). The chain rule
    through o = act(xr W1 + b1) W2 + b2 (GELU), o = (silu(xr Wg) * (xr Wu)) Wd (SwiGLU),
    o = xr W (single linear); parameters indexed [e] in the layouts of expert_apply."""
    if kind == "linear":
        W = _f64(w["w_in"][e])
        return {"w_in": xr.T @ dO}, dO @ W.T
    if kind == "gelu":
        W1, W2 = _f64(w["w_in"][e]), _f64(w["w_out"][e])
        z = xr @ W1 + _f64(w["b_in"][e])
        h = gelu(z)
        dh = dO @ W2.T
        dz = dh * gelu_grad(z)
        g = {"w_in": xr.T @ dz, "b_in": dz.sum(axis=0), "w_out": h.T @ dO, "b_out": dO.sum(axis=0)}
        return g, dz @ W1.T
    if kind == "swiglu":
        Wg, Wu, Wd = _f64(w["w_in"][e]), _f64(w["w_up"][e]), _f64(w["w_out"][e])
        a = xr @ Wg
        u = xr @ Wu
        sa = silu(a)
        h = sa * u
        dh = dO @ Wd.T
        du = dh * sa
        da = dh * u * silu_grad(a)
        g = {"w_in": xr.T @ da, "w_up": xr.T @ du, "w_out": h.T @ dO}
        return g, da @ Wg.T + du @ Wu.T
    raise ValueError(f"unknown expert kind {kind!r}")


def backward(dy, x, kind, weights, logits, idx, gate, kept, count, *, residual=True,
             aux_grad_scale=0.0, shared=None, w_router=None, scoring="softmax",
             renormalize=False, z_grad_scale=0.0):
    """Backward of the whole layer for every expert kind, in float64, with the discrete
    choices (top-k set, kept mask) held constant (P1 section 2 moe_backward and trap 7,
    extended through the expert MLPs by the chain rule).

    For a kept assignment a = (t, j) to expert e the expert output o_a is scaled by
    gate_a, so its output gradient is gate_a dy_t and
      dgate_a = <dy_t, o_a>,
    the expert's parameter gradients sum over its kept rows, and its input gradient is
    added to dx_t. The shared SwiGLU expert (ungated, every token) contributes its own
    parameter gradients and adds its input gradient to dx. With ``w_router`` (logits =
    x W_r) the router weights get dW_r = x^T dlogits and dx gets dlogits W_r^T; without
    it the logits are an independent input and dx has no router term.

    P3's variants: ``scoring`` is the router's score function (see ``router_grad``);
    with ``renormalize`` the experts see the survivor-renormalised gates g'_a = gate_a /
    K_t (K_t the token's kept gate mass), so dgate' = <dy_t, o_a> is taken back to the
    pre-drop gates by the quotient rule, dgate_a = (dgate'_a - sum_kept g'_r dgate'_r) /
    K_t on kept a and 0 on dropped ones; ``z_grad_scale`` adds that multiple of the
    router z-loss gradient to dlogits.

    Returns dgate, dlogits, dx, a dict ``dexperts`` of [E, ...] gradients named like the
    weights (w_in, w_up, w_out, b_in, b_out as the kind has them), ``dshared`` (or None)
    and ``dw_router`` (or None).
    """
    dy = _f64(dy)
    x = _f64(x)
    T, k = idx.shape
    E = np.asarray(weights["w_in"]).shape[0]
    dgate = np.zeros((T, k))
    dx = dy.copy() if residual else np.zeros_like(x)
    names = {"linear": ["w_in"], "gelu": ["w_in", "b_in", "w_out", "b_out"],
             "swiglu": ["w_in", "w_up", "w_out"]}[kind]
    dexp = {n: np.zeros(np.asarray(weights[n]).shape) for n in names}
    kept = np.asarray(kept, dtype=bool)
    geff = renormalise_kept(gate, kept) if renormalize else np.where(kept, _f64(gate), 0.0)
    for e in range(E):
        tt, jj = np.nonzero((idx == e) & kept)
        if tt.size == 0:
            continue
        o = expert_apply(kind, weights, e, x[tt])
        dgate[tt, jj] = np.sum(dy[tt] * o, axis=1)
        dO = geff[tt, jj][:, None] * dy[tt]
        g, dxr = _mlp_backward(kind, weights, e, x[tt], dO)
        for n in names:
            dexp[n][e] = g[n]
        np.add.at(dx, tt, dxr)
    dshared = None
    if shared is not None:
        g, dxr = _mlp_backward("swiglu", {n: np.asarray(shared[n])[None] for n in ("w_in", "w_up", "w_out")},
                               0, x, dy)
        dshared = g
        dx = dx + dxr
    if renormalize:
        mass = np.sum(np.where(kept, _f64(gate), 0.0), axis=1, keepdims=True)
        Gp = np.sum(geff * dgate, axis=1, keepdims=True)
        dgate = np.where(kept & (mass > 0.0),
                         (dgate - Gp) / np.where(mass > 0.0, mass, 1.0), 0.0)
    dlogits = router_grad(logits, idx, gate, dgate, scoring)
    if aux_grad_scale:
        dlogits = dlogits + aux_grad_scale * aux_grad(logits, count, k)
    if z_grad_scale:
        dlogits = dlogits + z_grad_scale * z_loss_grad(logits)
    dw_router = None
    if w_router is not None:
        dw_router = x.T @ dlogits
        dx = dx + dlogits @ _f64(w_router).T
    return {"dgate": dgate, "dlogits": dlogits, "dx": dx, "dexperts": dexp,
            "dshared": dshared, "dw_router": dw_router}
