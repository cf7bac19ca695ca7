"""Thin torch binding over libmoe.so: argument marshalling only.

Each function here has the name of a C entry point without its ``moe_`` prefix. It
checks shapes and dtypes, allocates the outputs and the workspace with torch (device
memory), and enqueues the library call on torch's current stream. Every step of the
layer runs in the HIP kernels; nothing here computes.

Experts are passed as a dict: {"kind": "linear"|"gelu"|"swiglu", "w_in": [E,D,F],
"w_up": [E,D,F], "w_out": [E,F,D], "b_in": [E,F], "b_out": [E,D]} (absent keys = None),
all of one dtype (float32 or bfloat16) on the GPU. With "w_in_layout": "out_in", w_in and
w_up are given as [E,F,D] instead, with "w_out_layout": "out_in" w_out as [E,D,F] (bf16
forward only).
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib as L

_KIND = {"linear": L.MOE_EXPERT_LINEAR, "gelu": L.MOE_EXPERT_GELU_MLP,
         "swiglu": L.MOE_EXPERT_SWIGLU}
_SCORING = {"softmax": L.MOE_SCORE_SOFTMAX, "sigmoid": L.MOE_SCORE_SIGMOID}


def _router_opts(scoring, selection_bias, renormalize_kept, z_loss_out, token_fraction=None,
                 probability_mass=None):
    """moe_router_opts_t for the router variants and the optional load statistics;
    returns (struct, tensors to keep)."""
    bias = None
    if selection_bias is not None:
        bias = selection_bias.to(torch.float32).contiguous()
    o = L.RouterOpts(scoring=_SCORING[scoring], selection_bias=_p(bias),
                     renormalize_kept=1 if renormalize_kept else 0, z_loss=_p(z_loss_out),
                     token_fraction=_p(token_fraction), probability_mass=_p(probability_mass))
    return o, bias


def _dt(t):
    if t.dtype == torch.float32:
        return L.MOE_F32
    if t.dtype == torch.bfloat16:
        return L.MOE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _c(t):
    return None if t is None else t.contiguous()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def version():
    return L.lib().moe_version().decode()


def capacity(T, k, E, capacity_factor):
    c = L.lib().moe_capacity(int(T), int(k), int(E), float(capacity_factor))
    if c < 0:
        raise ValueError("invalid capacity arguments")
    return int(c)


_LAYOUT = {"in_out": L.MOE_LAYOUT_IN_OUT, "out_in": L.MOE_LAYOUT_OUT_IN}


def _experts_struct(ex):
    """moe_experts_t of an expert dict. ``ex["w_in_layout"]``: "in_out" (the default:
    w_in and w_up are [E, D, F]) or "out_in" ([E, F, D], a torch Linear weight per
    expert); ``ex["w_out_layout"]`` likewise for w_out ([E, F, D] or [E, D, F])."""
    w_in = _c(ex["w_in"])
    layout = ex.get("w_in_layout", "in_out")
    out_layout = ex.get("w_out_layout", "in_out")
    if layout not in _LAYOUT or out_layout not in _LAYOUT:
        raise ValueError(f"w_in_layout and w_out_layout must be one of {sorted(_LAYOUT)}")
    E = w_in.shape[0]
    D, F = (w_in.shape[2], w_in.shape[1]) if layout == "out_in" else (w_in.shape[1], w_in.shape[2])
    keep = {k: _c(ex.get(k)) for k in ("w_in", "w_up", "w_out", "b_in", "b_out")}
    s = L.Experts(kind=_KIND[ex["kind"]], dtype=_dt(w_in), num_experts=E, d_model=D, d_hidden=F,
                  w_in=_p(keep["w_in"]), w_up=_p(keep["w_up"]), w_out=_p(keep["w_out"]),
                  b_in=_p(keep["b_in"]), b_out=_p(keep["b_out"]), w_in_layout=_LAYOUT[layout],
                  w_out_layout=_LAYOUT[out_layout])
    return s, keep


def route(*, k, logits=None, x=None, w_router=None, scoring="softmax", selection_bias=None,
          z_loss=False):
    """moe_route. Either logits [T,E] fp32, or x [T,D] and w_router [D,E]. ``scoring``,
    ``selection_bias`` ([E]) and ``z_loss`` select the router variants. Besides the
    routing outputs, returns the router page's load statistics token_fraction
    (count / T) and probability_mass (prob_sum / T), both [E] fp32."""
    if w_router is not None:
        x = _c(x)
        w_router = _c(w_router)
        T, D = x.shape
        E = w_router.shape[1]
        dev = x.device
        logits = torch.empty(T, E, dtype=torch.float32, device=dev)
        xdt = _dt(x)
    else:
        logits = _c(logits)
        T, E = logits.shape
        D = 0
        dev = logits.device
        xdt = L.MOE_F32
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    gate = torch.empty(T, k, dtype=torch.float32, device=dev)
    count = torch.empty(E, dtype=torch.int32, device=dev)
    prob = torch.empty(E, dtype=torch.float32, device=dev)
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    zl = torch.empty(1, dtype=torch.float32, device=dev) if z_loss else None
    tf = torch.empty(E, dtype=torch.float32, device=dev)
    pm = torch.empty(E, dtype=torch.float32, device=dev)
    opts, bias = _router_opts(scoring, selection_bias, False, zl, tf, pm)
    ws = _ws(L.lib().moe_route_workspace_size(T, E), dev)
    st = L.lib().moe_route(_p(x) if w_router is not None else None, xdt, D, _p(w_router), _p(logits),
                           T, D, E, k, _p(idx), _p(gate), _p(count), _p(prob), _p(aux),
                           ctypes.byref(opts), _p(ws), ws.numel(), _stream())
    L.check("moe_route", st)
    del bias
    out = {"logits": logits, "topk_idx": idx, "topk_gate": gate, "expert_count": count,
           "prob_sum": prob, "aux_loss": aux, "token_fraction": tf, "probability_mass": pm}
    if z_loss:
        out["z_loss"] = zl
    return out


def dispatch(topk_idx, E, C, *, return_ws=False):
    """moe_dispatch: position-priority slots for topk_idx [T,k] int32."""
    idx = _c(topk_idx)
    if idx.dtype != torch.int32:
        idx = idx.to(torch.int32)
    T, k = idx.shape
    dev = idx.device
    slot = torch.empty(T, k, dtype=torch.int32, device=dev)
    kept = torch.empty(T, k, dtype=torch.uint8, device=dev)
    sa = torch.empty(E, max(C, 0), dtype=torch.int32, device=dev)
    used = torch.empty(E, dtype=torch.int32, device=dev)
    over = torch.empty(E, dtype=torch.int32, device=dev)
    drops = torch.empty(T, dtype=torch.int32, device=dev)
    ws = _ws(L.lib().moe_dispatch_workspace_size(T, k, E), dev)
    st = L.lib().moe_dispatch(_p(idx), T, k, E, C, _p(slot), _p(kept), _p(sa), _p(used), _p(over),
                              _p(drops), _p(ws), ws.numel(), _stream())
    L.check("moe_dispatch", st)
    out = {"slot": slot, "kept": kept, "slot_assign": sa, "expert_used": used,
           "expert_overflow": over, "token_drops": drops}
    if return_ws:
        out["ws"] = ws
    return out


def read_error(ws):
    return int(L.lib().moe_read_error(_p(ws), _stream()))


def expert_mlp(experts, x, *, k=1, C=0, slot_assign=None, expert_used=None, keep_hidden=False):
    """moe_expert_mlp. Routed: slot_assign [E,C] and expert_used [E]; dense (shared
    expert, E = 1): slot_assign None. Returns expert_out ([E,C,D] or [T,D]) and, with
    keep_hidden, the hidden activations."""
    s, keep = _experts_struct(experts)
    x = _c(x)
    T = x.shape[0]
    dev = x.device
    dense = slot_assign is None
    rows = T if dense else C
    E, D, F = s.num_experts, s.d_model, s.d_hidden
    out = torch.empty((T, D) if dense else (E, C, D), dtype=x.dtype, device=dev)
    hidden = None
    if keep_hidden and experts["kind"] != "linear":
        hidden = torch.empty((T, F) if dense else (E, C, F), dtype=x.dtype, device=dev)
    ws = _ws(L.lib().moe_expert_mlp_workspace_size(ctypes.byref(s), rows), dev)
    st = L.lib().moe_expert_mlp(ctypes.byref(s), _p(x), x.stride(0), T, k, C, _p(slot_assign),
                                _p(expert_used), _p(hidden), _p(out), _p(ws), ws.numel(),
                                _stream())
    L.check("moe_expert_mlp", st)
    return {"expert_out": out, "hidden": hidden}


def combine(expert_out, topk_idx, slot, topk_gate, *, residual=None, shared_out=None,
            renormalize_kept=False):
    """moe_combine: y = residual + shared + sum_kept gate * expert_out[idx, slot] (gates
    renormalised over the survivors with ``renormalize_kept``). With ``slot`` None,
    expert_out is [T, E, D], one output per token and expert, and every choice counts."""
    eo = _c(expert_out)
    T, k = topk_idx.shape
    if slot is None:
        _, E, D = eo.shape
        C = 0
    else:
        E, C, D = eo.shape
    ref = residual if residual is not None else eo
    y = torch.empty(T, D, dtype=eo.dtype, device=eo.device)
    st = L.lib().moe_combine(_dt(eo), _p(_c(residual)), _p(_c(shared_out)), _p(eo),
                             _p(_c(topk_idx)), _p(_c(slot)), _p(_c(topk_gate)), T, k, E, C, D,
                             1 if renormalize_kept else 0, _p(y), _stream())
    L.check("moe_combine", st)
    del ref
    return y


def topk_router(x, w_router, expert_outputs, shared_output, k):
    """The result contract of "Top-k MoE Router with Load Statistics": router scores
    x w_router, top-k by score (ties to the lower index) with softmax weights over the k
    chosen, y = shared_output + sum_j weight_j * expert_outputs[t, e_j], and the load
    statistics f (token_fraction) and m (probability_mass). The routing math is fp32 in
    moe_route; y is the fp32 combine of moe_combine in its dense mode. Returns the
    page's dictionary: selected_experts int64, every other result in x's dtype, all on
    x's device (dtype casts only; every value comes from the library)."""
    r = route(k=k, x=x, w_router=w_router)
    eo = _c(expert_outputs).to(x.dtype)
    y = combine(eo, r["topk_idx"], None, r["topk_gate"], shared_out=_c(shared_output).to(x.dtype))
    return {
        "output": y,
        "selected_experts": r["topk_idx"].to(torch.int64),
        "selected_weights": r["topk_gate"].to(x.dtype),
        "token_fraction": r["token_fraction"].to(x.dtype),
        "probability_mass": r["probability_mass"].to(x.dtype),
    }


def forward(x, experts, *, k, capacity, w_router=None, logits=None, shared=None,
            use_residual=True, keep_hidden=False, keep_shared_out=False, scoring="softmax",
            selection_bias=None, renormalize_kept=False, z_loss=False, _ws_cache=None):
    """moe_forward: the whole layer. Returns every output of the call (see moe.h);
    ``scoring``, ``selection_bias``, ``renormalize_kept`` and ``z_loss`` select the
    router variants."""
    x = _c(x)
    T, D = x.shape
    dev = x.device
    es, keep = _experts_struct(experts)
    E, F = es.num_experts, es.d_hidden
    C = int(capacity)
    if w_router is not None:
        w_router = _c(w_router)
        logits = torch.empty(T, E, dtype=torch.float32, device=dev)
    else:
        logits = _c(logits)
    shs, shkeep = (_experts_struct(shared) if shared is not None else (L.Experts(), {}))
    o = {
        "logits": logits,
        "topk_idx": torch.empty(T, k, dtype=torch.int32, device=dev),
        "topk_gate": torch.empty(T, k, dtype=torch.float32, device=dev),
        "expert_count": torch.empty(E, dtype=torch.int32, device=dev),
        "prob_sum": torch.empty(E, dtype=torch.float32, device=dev),
        "aux_loss": torch.empty(1, dtype=torch.float32, device=dev),
        "slot": torch.empty(T, k, dtype=torch.int32, device=dev),
        "kept": torch.empty(T, k, dtype=torch.uint8, device=dev),
        "slot_assign": torch.empty(E, C, dtype=torch.int32, device=dev),
        "expert_used": torch.empty(E, dtype=torch.int32, device=dev),
        "expert_overflow": torch.empty(E, dtype=torch.int32, device=dev),
        "token_drops": torch.empty(T, dtype=torch.int32, device=dev),
        "expert_out": torch.empty(E, C, D, dtype=x.dtype, device=dev),
        "y": torch.empty(T, D, dtype=x.dtype, device=dev),
        "hidden": (torch.empty(E, C, F, dtype=x.dtype, device=dev)
                   if keep_hidden and experts["kind"] != "linear" else None),
        "shared_out": (torch.empty(T, D, dtype=x.dtype, device=dev)
                       if keep_shared_out and shared is not None else None),
        "capacity": C,
        "z_loss": torch.empty(1, dtype=torch.float32, device=dev) if z_loss else None,
        "token_fraction": torch.empty(E, dtype=torch.float32, device=dev),
        "probability_mass": torch.empty(E, dtype=torch.float32, device=dev),
        "router": {"scoring": scoring, "renormalize_kept": bool(renormalize_kept)},
    }
    ropts, bias = _router_opts(scoring, selection_bias, renormalize_kept, o["z_loss"],
                               o["token_fraction"], o["probability_mass"])
    a = L.ForwardArgs(
        x=_p(x), ldx=x.stride(0), T=T, w_router=_p(w_router), logits=_p(logits), experts=es,
        shared=shs, k=k, capacity=C, use_residual=1 if use_residual else 0,
        topk_idx=_p(o["topk_idx"]), topk_gate=_p(o["topk_gate"]),
        expert_count=_p(o["expert_count"]), prob_sum=_p(o["prob_sum"]),
        aux_loss=_p(o["aux_loss"]), slot=_p(o["slot"]), kept=_p(o["kept"]),
        slot_assign=_p(o["slot_assign"]), expert_used=_p(o["expert_used"]),
        expert_overflow=_p(o["expert_overflow"]), token_drops=_p(o["token_drops"]),
        hidden_cache=_p(o["hidden"]), expert_out=_p(o["expert_out"]),
        shared_out=_p(o["shared_out"]), y=_p(o["y"]), router=ropts)
    need = L.lib().moe_forward_workspace_size(ctypes.byref(a))
    if _ws_cache is not None and _ws_cache.numel() >= need:
        ws = _ws_cache
    else:
        ws = _ws(need, dev)
    st = L.lib().moe_forward(ctypes.byref(a), _p(ws), ws.numel(), _stream())
    L.check("moe_forward", st)
    o["ws"] = ws
    # everything a repeat call needs, kept alive together
    o["_call"] = PreparedCall("moe_forward", a, ws, (x, w_router, keep, shkeep, bias))
    return o


class PreparedCall:
    """A prepared library call (moe_forward or moe_backward): the argument struct and
    workspace of an earlier call, so that the same layer can be re-run on the same
    buffers without re-marshalling."""

    def __init__(self, fn_name, args, ws, keepalive):
        self.args = args
        self.ws = ws
        self._keep = keepalive
        self._name = fn_name
        self._fn = getattr(L.lib(), fn_name)
        self._ref = ctypes.byref(self.args)
        self._ws_p = _p(ws)
        self._ws_n = ws.numel()

    def __call__(self, stream=None):
        s = ctypes.c_void_p(stream) if stream is not None else _stream()
        st = self._fn(self._ref, self._ws_p, self._ws_n, s)
        if st != L.MOE_OK:
            L.check(self._name, st)


def backward(dy, x, experts, fwd, *, k, use_residual=True, aux_grad_scale=0.0, shared=None,
             w_router=None, z_grad_scale=0.0):
    """moe_backward for fp32 experts of any kind. ``fwd`` is the dict returned by
    forward(). ``shared``: the shared SwiGLU expert of the forward; ``w_router``: the
    router weights, for dw_router and the router term of dx. The router variant
    (scoring, survivor renormalisation) is the forward's; ``z_grad_scale`` weights the
    z-loss gradient in dlogits.

    Returns dx, dgate, dlogits, ``dexperts`` (gradients named like the expert weights),
    ``dW`` (= dexperts["w_in"]), ``dshared`` (or None) and ``dw_router`` (or None)."""
    dy = _c(dy)
    x = _c(x)
    T, D = x.shape
    dev = x.device
    es, keep = _experts_struct(experts)
    E, F = es.num_experts, es.d_hidden
    C = int(fwd["capacity"])
    kind = experts["kind"]

    def new(*shape):
        return torch.empty(*shape, dtype=x.dtype, device=dev)

    dexp = {"w_in": new(E, D, F)}
    if kind == "swiglu":
        dexp["w_up"] = new(E, D, F)
    if kind != "linear":
        dexp["w_out"] = new(E, F, D)
    if kind == "gelu":
        if experts.get("b_in") is not None:
            dexp["b_in"] = new(E, F)
        if experts.get("b_out") is not None:
            dexp["b_out"] = new(E, D)
    shs, shkeep = (_experts_struct(shared) if shared is not None else (L.Experts(), {}))
    dsh = None
    if shared is not None:
        Fs = shs.d_hidden
        dsh = {"w_in": new(D, Fs), "w_up": new(D, Fs), "w_out": new(Fs, D)}
    dwr = None
    if w_router is not None:
        w_router = _c(w_router)
        dwr = torch.empty(D, E, dtype=torch.float32, device=dev)
    out = {
        "dx": new(T, D),
        "dgate": torch.empty(T, k, dtype=torch.float32, device=dev),
        "dlogits": torch.empty(T, E, dtype=torch.float32, device=dev),
        "dexperts": dexp,
        "dW": dexp["w_in"],
        "dshared": dsh,
        "dw_router": dwr,
    }
    a = L.BackwardArgs(
        dy=_p(dy), x=_p(x), ld=x.stride(0), T=T, logits=_p(fwd["logits"]), experts=es, k=k,
        capacity=C, use_residual=1 if use_residual else 0, aux_grad_scale=float(aux_grad_scale),
        topk_idx=_p(fwd["topk_idx"]), topk_gate=_p(fwd["topk_gate"]),
        expert_count=_p(fwd["expert_count"]), slot=_p(fwd["slot"]),
        slot_assign=_p(fwd["slot_assign"]), expert_used=_p(fwd["expert_used"]),
        expert_out=_p(fwd["expert_out"]), dx=_p(out["dx"]), dW=_p(dexp["w_in"]),
        dgate=_p(out["dgate"]), dlogits=_p(out["dlogits"]),
        dW_up=_p(dexp.get("w_up")), dW_out=_p(dexp.get("w_out")), db_in=_p(dexp.get("b_in")),
        db_out=_p(dexp.get("b_out")), shared=shs,
        dshared_w_in=_p(dsh["w_in"]) if dsh else None,
        dshared_w_up=_p(dsh["w_up"]) if dsh else None,
        dshared_w_out=_p(dsh["w_out"]) if dsh else None,
        w_router=_p(w_router), dw_router=_p(dwr),
        router=L.RouterOpts(scoring=_SCORING[fwd.get("router", {}).get("scoring", "softmax")],
                            renormalize_kept=1 if fwd.get("router", {}).get("renormalize_kept") else 0),
        z_grad_scale=float(z_grad_scale))
    ws = _ws(L.lib().moe_backward_workspace_size(ctypes.byref(a)), dev)
    st = L.lib().moe_backward(ctypes.byref(a), _p(ws), ws.numel(), _stream())
    L.check("moe_backward", st)
    out["_call"] = PreparedCall("moe_backward", a, ws,
                                (dy, x, w_router, keep, shkeep, fwd, out.copy()))
    return out


def profile_enable(on=True):
    L.lib().moe_profile_enable(1 if on else 0)


def profile_read(max_entries=64):
    """Per-kernel launch counts and summed milliseconds since the last read."""
    stride = 64
    names = ctypes.create_string_buffer(stride * max_entries)
    counts = (ctypes.c_int32 * max_entries)()
    ms = (ctypes.c_double * max_entries)()
    n = L.lib().moe_profile_read(names, stride, counts, ms, max_entries)
    out = {}
    for i in range(n):
        nm = names.raw[i * stride:(i + 1) * stride].split(b"\0", 1)[0].decode()
        out[nm] = (int(counts[i]), float(ms[i]))
    return out
