"""MI355X-native capacity-limited sparse MoE layer (gfx950 HIP kernels behind a C ABI).

The torch-level binding is ``sparse_mixture_experts_stable_amd.ops``; the library loads
on first use and raises if it has not been built
(``python -m sparse_mixture_experts_stable_amd.build``).
"""
