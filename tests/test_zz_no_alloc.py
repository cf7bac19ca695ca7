"""moe_forward_noalloc (the forward with its workspace in the library's own device array,
for callers that cannot allocate) against moe_forward on the same inputs: every output
bit for bit (the same kernels in the same order), on two calls in a row, the second with
a smaller batch, each call through the C ABI."""

import ctypes

import numpy as np
import pytest
import torch

from tests import _harness as H
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

SCRATCH_MAX = 32 << 20   # bytes, the array's size as the header states it

OUTS = ("topk_idx", "topk_gate", "expert_count", "prob_sum", "aux_loss", "slot", "kept",
        "slot_assign", "expert_used", "expert_overflow", "token_drops", "expert_out",
        "shared_out", "y", "token_fraction", "probability_mass")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _noalloc(L):
    return L.lib().moe_forward_noalloc


def _run_both(w):
    from sparse_mixture_experts_stable_amd import _lib as L
    from sparse_mixture_experts_stable_amd import ops
    inp = make_inputs(w)
    ref, g = H.run_forward(w, inp, keep_hidden=True)
    a = ref["_call"].args
    b = L.ForwardArgs.from_buffer_copy(a)
    got = {}
    for key in OUTS:
        t = ref.get(key)
        if t is None:
            continue
        got[key] = torch.full_like(t, 7) if t.dtype != torch.uint8 else torch.full_like(t, 3)
        setattr(b, key, ctypes.c_void_p(got[key].data_ptr()))
    got["hidden"] = torch.empty_like(ref["hidden"])
    b.hidden_cache = ctypes.c_void_p(got["hidden"].data_ptr())
    b.router.token_fraction = ctypes.c_void_p(got["token_fraction"].data_ptr())
    b.router.probability_mass = ctypes.c_void_p(got["probability_mass"].data_ptr())
    lg = torch.empty_like(ref["logits"])
    b.logits = ctypes.c_void_p(lg.data_ptr())
    st = _noalloc(L)(ctypes.byref(b), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == L.MOE_OK, L.lib().moe_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(lg, ref["logits"])
    used = ref["expert_used"].cpu().numpy()
    for key, t in got.items():
        if key in ("expert_out", "hidden"):
            for e in range(t.shape[0]):
                assert torch.equal(t[e, : used[e]], ref[key][e, : used[e]]), (key, e)
        else:
            assert torch.equal(t, ref[key]), key
    return ref, got


def test_noalloc_forward_matches_forward_twice():
    big = WORKLOADS[3].scaled(T=4096, D=512, E=32, F=512, shared_F=512)   # 256x256 tiles
    small = WORKLOADS[3].scaled(T=600, D=256, E=16, F=128, shared_F=128)
    _run_both(big)
    _run_both(small)


def test_noalloc_forward_rejects_oversized_workspace():
    """The shared expert's hidden activation of 40,000 tokens at width 512 (39 MiB of bf16)
    does not fit the array: MOE_ERR_WORKSPACE, nothing launched."""
    from sparse_mixture_experts_stable_amd import _lib as L
    p = ctypes.c_void_p(1 << 21)
    ex = L.Experts(kind=L.MOE_EXPERT_SWIGLU, dtype=L.MOE_BF16, num_experts=8, d_model=256,
                   d_hidden=128, w_in=p, w_up=p, w_out=p)
    sh = L.Experts(kind=L.MOE_EXPERT_SWIGLU, dtype=L.MOE_BF16, num_experts=1, d_model=256,
                   d_hidden=512, w_in=p, w_up=p, w_out=p)
    outs = {f: p for f in OUTS[:-2] + ("hidden_cache",)}
    a = L.ForwardArgs(x=p, ldx=256, T=40000, w_router=p, logits=p, experts=ex, shared=sh, k=2,
                      capacity=10000, **outs)
    assert L.lib().moe_forward_workspace_size(ctypes.byref(a)) > SCRATCH_MAX
    assert _noalloc(L)(ctypes.byref(a), None) == L.MOE_ERR_WORKSPACE
    # hidden_cache and shared_out are required outputs here
    a.hidden_cache = None
    assert _noalloc(L)(ctypes.byref(a), None) == L.MOE_ERR_INVALID_ARG
