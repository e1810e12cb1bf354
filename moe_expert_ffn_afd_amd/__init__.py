"""FFN (expert) side of an attention-FFN-disaggregated MoE layer on MI355X.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``); ``afd`` is its thin ctypes binding and ``inputs`` the seeded
synthetic workload generator.  Importing the package loads nothing native;
``moe_expert_ffn_afd_amd.afd`` loads the library on first use and raises if it
is missing.
"""
__all__ = ["afd", "inputs"]
