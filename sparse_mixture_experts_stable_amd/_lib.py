"""ctypes loader for libmoe.so and mirrors of the C structs in include/moe.h.

Loading fails loudly when the library has not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_EXPERT_LINEAR, MOE_EXPERT_GELU_MLP, MOE_EXPERT_SWIGLU = 0, 1, 2
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_LAYOUT_IN_OUT, MOE_LAYOUT_OUT_IN = 0, 1

EXPORTED = [
    "moe_version", "moe_status_string", "moe_capacity",
    "moe_route_workspace_size", "moe_route",
    "moe_dispatch_workspace_size", "moe_dispatch",
    "moe_expert_mlp_workspace_size", "moe_expert_mlp",
    "moe_combine",
    "moe_forward_workspace_size", "moe_forward", "moe_forward_noalloc",
    "moe_backward_workspace_size", "moe_backward",
    "moe_read_error", "moe_profile_enable", "moe_profile_read",
]


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


vp = ctypes.c_void_p
i32 = ctypes.c_int32
i64 = ctypes.c_int64
f32 = ctypes.c_float
sz = ctypes.c_size_t


class Experts(ctypes.Structure):
    _fields_ = [("kind", i32), ("dtype", i32), ("num_experts", i32), ("d_model", i32),
                ("d_hidden", i32), ("w_in", vp), ("w_up", vp), ("w_out", vp), ("b_in", vp),
                ("b_out", vp), ("w_in_layout", i32), ("w_out_layout", i32)]


class RouterOpts(ctypes.Structure):
    _fields_ = [("scoring", i32), ("selection_bias", vp), ("renormalize_kept", i32),
                ("z_loss", vp), ("token_fraction", vp), ("probability_mass", vp)]


class ForwardArgs(ctypes.Structure):
    _fields_ = [("x", vp), ("ldx", i64), ("T", i32), ("w_router", vp), ("logits", vp),
                ("experts", Experts), ("shared", Experts), ("k", i32), ("capacity", i32),
                ("use_residual", i32), ("topk_idx", vp), ("topk_gate", vp),
                ("expert_count", vp), ("prob_sum", vp), ("aux_loss", vp), ("slot", vp),
                ("kept", vp), ("slot_assign", vp), ("expert_used", vp),
                ("expert_overflow", vp), ("token_drops", vp), ("hidden_cache", vp),
                ("expert_out", vp), ("shared_out", vp), ("y", vp), ("router", RouterOpts)]


class BackwardArgs(ctypes.Structure):
    _fields_ = [("dy", vp), ("x", vp), ("ld", i64), ("T", i32), ("logits", vp),
                ("experts", Experts), ("k", i32), ("capacity", i32), ("use_residual", i32),
                ("aux_grad_scale", f32), ("topk_idx", vp), ("topk_gate", vp),
                ("expert_count", vp), ("slot", vp), ("slot_assign", vp), ("expert_used", vp),
                ("expert_out", vp), ("dx", vp), ("dW", vp), ("dgate", vp), ("dlogits", vp),
                ("dW_up", vp), ("dW_out", vp), ("db_in", vp), ("db_out", vp),
                ("shared", Experts), ("dshared_w_in", vp), ("dshared_w_up", vp),
                ("dshared_w_out", vp), ("w_router", vp), ("dw_router", vp),
                ("router", RouterOpts), ("z_grad_scale", f32)]


_lib = None


def _declare(L):
    P = ctypes.POINTER
    L.moe_version.restype = ctypes.c_char_p
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_status_string.argtypes = [i32]
    L.moe_capacity.restype = i64
    L.moe_capacity.argtypes = [i64, i32, i32, ctypes.c_double]
    L.moe_route_workspace_size.restype = sz
    L.moe_route_workspace_size.argtypes = [i32, i32]
    L.moe_route.restype = i32
    L.moe_route.argtypes = [vp, i32, i64, vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                            P(RouterOpts), vp, sz, vp]
    L.moe_dispatch_workspace_size.restype = sz
    L.moe_dispatch_workspace_size.argtypes = [i32, i32, i32]
    L.moe_dispatch.restype = i32
    L.moe_dispatch.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_expert_mlp_workspace_size.restype = sz
    L.moe_expert_mlp_workspace_size.argtypes = [P(Experts), i32]
    L.moe_expert_mlp.restype = i32
    L.moe_expert_mlp.argtypes = [P(Experts), vp, i64, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.moe_combine.restype = i32
    L.moe_combine.argtypes = [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp]
    L.moe_forward_workspace_size.restype = sz
    L.moe_forward_workspace_size.argtypes = [P(ForwardArgs)]
    L.moe_forward.restype = i32
    L.moe_forward.argtypes = [P(ForwardArgs), vp, sz, vp]
    L.moe_forward_noalloc.restype = i32
    L.moe_forward_noalloc.argtypes = [P(ForwardArgs), vp]
    L.moe_backward_workspace_size.restype = sz
    L.moe_backward_workspace_size.argtypes = [P(BackwardArgs)]
    L.moe_backward.restype = i32
    L.moe_backward.argtypes = [P(BackwardArgs), vp, sz, vp]
    L.moe_read_error.restype = i32
    L.moe_read_error.argtypes = [vp, vp]
    L.moe_profile_enable.restype = None
    L.moe_profile_enable.argtypes = [i32]
    L.moe_profile_read.restype = i32
    L.moe_profile_read.argtypes = [ctypes.c_char_p, i32, P(i32), P(ctypes.c_double), i32]


def lib():
    """The loaded libmoe.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m sparse_mixture_experts_stable_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


def check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status, lib().moe_status_string(status).decode())
