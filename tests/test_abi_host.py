"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every symbol
the header declares, computes the capacity exactly, and rejects bad arguments before
launching anything."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle.moe_oracle as om
from sparse_mixture_experts_stable_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", src)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    lib = L.lib()
    decl = declared_functions()
    assert len(decl) >= 17
    for name in decl:
        assert hasattr(lib, name), name
    assert sorted(L.EXPORTED) == decl


def test_version_and_status_strings():
    lib = L.lib()
    assert lib.moe_version().decode().startswith("moe-gfx950")
    assert lib.moe_status_string(L.MOE_ERR_WORKSPACE) == b"MOE_ERR_WORKSPACE"


def test_capacity_matches_oracle():
    lib = L.lib()
    rng = np.random.default_rng(0)
    for _ in range(5000):
        T = int(rng.integers(1, 10 ** 7)); E = int(rng.integers(1, 1025)); k = int(rng.integers(1, E + 1))
        cf = float(rng.choice([rng.random() * 3, round(rng.random() * 4, 2), 1e-300, 0.1, 1 / 3, 0.0]))
        want = om.capacity(T, k, E, cf)
        if want > 2 ** 31 - 1:
            want = -1
        assert lib.moe_capacity(T, k, E, cf) == want, (T, k, E, cf)
    for bad in [(8, 2, 4, -0.5), (8, 2, 4, float("nan")), (8, 2, 4, float("inf")), (8, 5, 4, 1.0),
                (0, 1, 4, 1.0)]:
        assert lib.moe_capacity(*bad) == -1


def _null():
    return None


def test_route_rejects_bad_arguments():
    lib = L.lib()
    ws = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first
    p = ctypes.c_void_p(1 << 21)
    common = dict(x=None, dt=L.MOE_F32, ldx=0, w=None, logits=p)

    def call(T, E, k, ws_bytes=1 << 30, idx=p, opts=None):
        return lib.moe_route(common["x"], common["dt"], common["ldx"], common["w"], common["logits"],
                             T, 0, E, k, idx, p, p, p, p, opts, ws, ws_bytes, None)
    assert call(8, 4, 0) == L.MOE_ERR_INVALID_ARG
    assert call(8, 4, 2, opts=ctypes.byref(L.RouterOpts(scoring=2))) == L.MOE_ERR_INVALID_ARG
    assert call(8, 4, 5) == L.MOE_ERR_INVALID_ARG
    assert call(0, 4, 1) == L.MOE_ERR_INVALID_ARG
    assert call(8, 2000, 1) == L.MOE_ERR_INVALID_ARG
    assert call(8, 4, 2, idx=None) == L.MOE_ERR_INVALID_ARG
    assert call(8, 4, 2, ws_bytes=16) == L.MOE_ERR_WORKSPACE


def test_dispatch_and_forward_reject_bad_arguments():
    lib = L.lib()
    p = ctypes.c_void_p(1 << 21)
    assert lib.moe_dispatch(p, 8, 2, 4, -1, p, p, p, p, p, p, p, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(p, 8, 2, 4, 4, p, p, None, p, p, p, p, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch(p, 8, 2, 4, 4, p, p, p, p, p, p, p, 8, None) == L.MOE_ERR_WORKSPACE
    ex = L.Experts(kind=L.MOE_EXPERT_SWIGLU, dtype=L.MOE_BF16, num_experts=4, d_model=100,
                   d_hidden=64, w_in=p, w_up=p, w_out=p)
    a = L.ForwardArgs(x=p, ldx=100, T=8, logits=p, experts=ex, k=2, capacity=4)
    assert lib.moe_forward(ctypes.byref(a), p, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED
    ex.d_model = 128
    a = L.ForwardArgs(x=p, ldx=128, T=8, logits=p, experts=ex, k=5, capacity=4)
    assert lib.moe_forward(ctypes.byref(a), p, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    bex = L.Experts(kind=L.MOE_EXPERT_SWIGLU, dtype=L.MOE_BF16, num_experts=4, d_model=128,
                    d_hidden=128, w_in=p, w_up=p, w_out=p)
    b = L.BackwardArgs(dy=p, x=p, ld=128, T=8, logits=p, experts=bex, k=2, capacity=4)
    assert lib.moe_backward(ctypes.byref(b), p, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED
    # fp32 MLP backward: every gradient the kind has must be given
    fex = L.Experts(kind=L.MOE_EXPERT_SWIGLU, dtype=L.MOE_F32, num_experts=4, d_model=128,
                    d_hidden=64, w_in=p, w_up=p, w_out=p)
    full = dict(dy=p, x=p, ld=128, T=8, logits=p, experts=fex, k=2, capacity=4, topk_idx=p,
                topk_gate=p, expert_count=p, slot=p, slot_assign=p, expert_used=p,
                expert_out=p, dx=p, dW=p, dgate=p, dlogits=p, dW_up=p, dW_out=p)
    for drop in ("dW_up", "dW_out", "dW"):
        kw = dict(full)
        kw[drop] = None
        b = L.BackwardArgs(**kw)
        assert lib.moe_backward(ctypes.byref(b), p, 1 << 30, None) == L.MOE_ERR_INVALID_ARG, drop
    b = L.BackwardArgs(**full)
    assert lib.moe_backward(ctypes.byref(b), p, 1, None) == L.MOE_ERR_WORKSPACE
    # router weights need their gradient, and E a multiple of 4
    b = L.BackwardArgs(**dict(full, w_router=p))
    assert lib.moe_backward(ctypes.byref(b), p, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    fex3 = L.Experts(kind=L.MOE_EXPERT_SWIGLU, dtype=L.MOE_F32, num_experts=3, d_model=128,
                     d_hidden=64, w_in=p, w_up=p, w_out=p)
    b = L.BackwardArgs(**dict(full, experts=fex3, w_router=p, dw_router=p))
    assert lib.moe_backward(ctypes.byref(b), p, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED
    # GELU biases need their gradients; the shared expert needs all three
    gex = L.Experts(kind=L.MOE_EXPERT_GELU_MLP, dtype=L.MOE_F32, num_experts=4, d_model=128,
                    d_hidden=64, w_in=p, w_out=p, b_in=p, b_out=p)
    b = L.BackwardArgs(**dict(full, experts=gex, db_in=p))
    assert lib.moe_backward(ctypes.byref(b), p, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    sh = L.Experts(kind=L.MOE_EXPERT_SWIGLU, dtype=L.MOE_F32, num_experts=1, d_model=128,
                   d_hidden=64, w_in=p, w_up=p, w_out=p)
    b = L.BackwardArgs(**dict(full, shared=sh, dshared_w_in=p, dshared_w_up=p))
    assert lib.moe_backward(ctypes.byref(b), p, 1 << 30, None) == L.MOE_ERR_INVALID_ARG


def test_workspace_sizes_positive():
    lib = L.lib()
    assert lib.moe_route_workspace_size(16384, 256) > 16384 // 16 * 256 * 4
    assert lib.moe_dispatch_workspace_size(16384, 8, 256) > 0


def test_missing_library_fails_loudly():
    """With libmoe.so absent, the binding raises ImportError at the first call: there is
    no fallback (CPU or otherwise) behind the Python names."""
    import subprocess
    import sys
    code = (
        "import sparse_mixture_experts_stable_amd._lib as L\n"
        "L.LIB_PATH = '/nonexistent/libmoe.so'\n"
        "from sparse_mixture_experts_stable_amd import ops\n"
        "try:\n"
        "    ops.capacity(16, 2, 4, 1.0)\n"
        "    print('no error')\n"
        "except ImportError as e:\n"
        "    print('ImportError:', e)\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("ImportError:"), r.stdout


def test_package_does_not_use_the_oracle():
    """The product package neither imports nor names the oracle (the oracle is test
    infrastructure only)."""
    pkg = os.path.join(ROOT, "sparse_mixture_experts_stable_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", src), os.path.join(dirpath, f)


def test_weight_layout_validation():
    """w_in_layout: values other than IN_OUT / OUT_IN are invalid; OUT_IN is taken by
    bf16 experts in the forward only, with the shared expert in the same layout."""
    lib = L.lib()
    p = ctypes.c_void_p(1 << 21)
    mk = lambda dt, lay, kind=L.MOE_EXPERT_SWIGLU, E=4: L.Experts(
        kind=kind, dtype=dt, num_experts=E, d_model=128, d_hidden=128, w_in=p, w_up=p, w_out=p,
        w_in_layout=lay)
    outs = {f: p for f in ("topk_idx", "topk_gate", "expert_count", "prob_sum", "aux_loss", "slot",
                           "kept", "slot_assign", "expert_used", "expert_overflow", "token_drops",
                           "expert_out", "y")}
    fwd = lambda ex, sh=L.Experts(): L.ForwardArgs(x=p, ldx=128, T=8, logits=p, experts=ex,
                                                   shared=sh, k=2, capacity=4, **outs)
    assert lib.moe_forward(ctypes.byref(fwd(mk(L.MOE_BF16, 7))), p, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(ctypes.byref(fwd(mk(L.MOE_F32, L.MOE_LAYOUT_OUT_IN))), p, 1 << 30,
                           None) == L.MOE_ERR_UNSUPPORTED
    mixed = fwd(mk(L.MOE_BF16, L.MOE_LAYOUT_OUT_IN), mk(L.MOE_BF16, L.MOE_LAYOUT_IN_OUT, E=1))
    assert lib.moe_forward(ctypes.byref(mixed), p, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED
    b = L.BackwardArgs(dy=p, x=p, ld=128, T=8, logits=p, experts=mk(L.MOE_F32, L.MOE_LAYOUT_OUT_IN),
                       k=2, capacity=4)
    assert lib.moe_backward(ctypes.byref(b), p, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED


def test_w_out_layout_validation():
    """w_out_layout: values other than IN_OUT / OUT_IN are invalid; OUT_IN needs bf16
    experts (forward only) and the shared expert in the same layout."""
    lib = L.lib()
    p = ctypes.c_void_p(1 << 21)
    mk = lambda dt, lay, E=4: L.Experts(
        kind=L.MOE_EXPERT_SWIGLU, dtype=dt, num_experts=E, d_model=128, d_hidden=128, w_in=p,
        w_up=p, w_out=p, w_out_layout=lay)
    outs = {f: p for f in ("topk_idx", "topk_gate", "expert_count", "prob_sum", "aux_loss", "slot",
                           "kept", "slot_assign", "expert_used", "expert_overflow", "token_drops",
                           "expert_out", "y")}
    fwd = lambda ex, sh=L.Experts(): L.ForwardArgs(x=p, ldx=128, T=8, logits=p, experts=ex,
                                                   shared=sh, k=2, capacity=4, **outs)
    assert lib.moe_forward(ctypes.byref(fwd(mk(L.MOE_BF16, 3))), p, 1 << 30, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_forward(ctypes.byref(fwd(mk(L.MOE_F32, L.MOE_LAYOUT_OUT_IN))), p, 1 << 30,
                           None) == L.MOE_ERR_UNSUPPORTED
    mixed = fwd(mk(L.MOE_BF16, L.MOE_LAYOUT_OUT_IN), mk(L.MOE_BF16, L.MOE_LAYOUT_IN_OUT, E=1))
    assert lib.moe_forward(ctypes.byref(mixed), p, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED
    b = L.BackwardArgs(dy=p, x=p, ld=128, T=8, logits=p, experts=mk(L.MOE_F32, L.MOE_LAYOUT_OUT_IN),
                       k=2, capacity=4)
    assert lib.moe_backward(ctypes.byref(b), p, 1 << 30, None) == L.MOE_ERR_UNSUPPORTED


def test_bf16_shapes_past_32bit_row_offsets_are_rejected():
    """The bf16 tile loader addresses rows with 32-bit byte offsets from each group's
    base; shapes whose rows start 4 GiB or more from it (x of 2^20 tokens at d_model
    2048, a dense shared hidden of 2^22 rows at width 512) are refused before any launch,
    and the largest shapes below the limit pass validation (the workspace check that
    follows fails instead, so nothing runs)."""
    lib = L.lib()
    p = ctypes.c_void_p(1 << 21)
    outs = {f: p for f in ("topk_idx", "topk_gate", "expert_count", "prob_sum", "aux_loss", "slot",
                           "kept", "slot_assign", "expert_used", "expert_overflow", "token_drops",
                           "expert_out", "y")}
    ex = L.Experts(kind=L.MOE_EXPERT_SWIGLU, dtype=L.MOE_BF16, num_experts=8, d_model=2048,
                   d_hidden=512, w_in=p, w_up=p, w_out=p)
    big = L.ForwardArgs(x=p, ldx=2048, T=1 << 20, w_router=p, logits=p, experts=ex, k=1,
                        capacity=1024, **outs)
    assert lib.moe_forward(ctypes.byref(big), p, 1 << 62, None) == L.MOE_ERR_UNSUPPORTED
    ok = L.ForwardArgs(x=p, ldx=2048, T=(1 << 20) - 1, w_router=p, logits=p, experts=ex, k=1,
                       capacity=1024, **outs)
    assert lib.moe_forward(ctypes.byref(ok), p, 1, None) == L.MOE_ERR_WORKSPACE
    # the shared expert's hidden activation, [T, 512] bf16, over 2^22 rows
    sh = L.Experts(kind=L.MOE_EXPERT_SWIGLU, dtype=L.MOE_BF16, num_experts=1, d_model=64,
                   d_hidden=512, w_in=p, w_up=p, w_out=p)
    ex64 = L.Experts(kind=L.MOE_EXPERT_SWIGLU, dtype=L.MOE_BF16, num_experts=8, d_model=64,
                     d_hidden=64, w_in=p, w_up=p, w_out=p)
    a = L.ForwardArgs(x=p, ldx=64, T=1 << 22, w_router=p, logits=p, experts=ex64, shared=sh, k=1,
                      capacity=1024, **outs)
    assert lib.moe_forward(ctypes.byref(a), p, 1 << 62, None) == L.MOE_ERR_UNSUPPORTED
    # moe_route's router GEMM on bf16 x
    assert lib.moe_route(p, L.MOE_BF16, 2048, p, p, 1 << 20, 2048, 8, 1, p, p, p, p, p, None, p,
                         1 << 62, None) == L.MOE_ERR_UNSUPPORTED
    # moe_expert_mlp, routed and dense
    assert lib.moe_expert_mlp(ctypes.byref(ex), p, 2048, 1 << 20, 1, 1024, p, p, p, p, p, 1 << 62,
                              None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_mlp(ctypes.byref(sh), p, 64, 1 << 22, 1, 0, None, None, p, p, p, 1 << 62,
                              None) == L.MOE_ERR_UNSUPPORTED
