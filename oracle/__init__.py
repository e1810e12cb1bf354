"""fp64 CPU oracle of the FFN-side MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls anything here.
"""
from .oracle import build, dispatch, forward, e4m3_decode, bf16_decode, library_path  # noqa: F401
