"""The C-ABI library on the CPU: it loads, exports every symbol include/afd_ffn.h
declares, binds to torch's HIP runtime only, and rejects bad arguments on the
host before any GPU work (no compute call is made here)."""
import ctypes
import os
import re

import pytest
import torch  # noqa: F401  (before the library: one HIP runtime)

from moe_expert_ffn_afd_amd import afd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "afd_ffn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(afd_ffn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return afd.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("afd_ffn_create", "afd_ffn_forward", "afd_ffn_destroy"):
        assert required in names
    assert set(names) == set(afd.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_single_hip_runtime(lib):
    maps = open("/proc/self/maps").read().split("\n")
    hip = sorted(set(m.split()[-1] for m in maps if "libamdhip64" in m))
    assert len(hip) == 1, hip
    assert os.path.dirname(torch.__file__) in hip[0]


def _cfg(**kw):
    base = dict(hidden=256, inter=512, num_experts=8, top_k=2, max_tokens=64, shared_inter=0,
                dtype=afd.AFD_DTYPE_BF16, device=0, w_gate=0x1000, w_up=0x2000, w_down=0x3000)
    base.update(kw)
    return afd.afd_ffn_config(**base)


def test_validate_config_accepts_good(lib):
    afd.afd_ffn_validate_config(_cfg())
    afd.afd_ffn_validate_config(_cfg(dtype=afd.AFD_DTYPE_F32, w_gate=0x1004))  # fp32: 4-byte alignment
    # (2^17 - 4096) * 8 rows of 1024 bf16 = 1.94 GiB: still within 32-bit offsets
    afd.afd_ffn_validate_config(_cfg(max_tokens=(1 << 17) - 4096, top_k=8, hidden=1024, inter=1024))
    afd.afd_ffn_validate_config(_cfg(dtype=afd.AFD_DTYPE_FP8_BLOCK, s_gate=8, s_up=8, s_down=8))
    afd.afd_ffn_validate_config(_cfg(shared_inter=512, sh_gate=0x4000, sh_up=0x5000, sh_down=0x6000))
    # a shared expert of another width than the routed ones: parts of width inter
    for si in (128, 768, 2048, 16 * 512):
        afd.afd_ffn_validate_config(_cfg(shared_inter=si, sh_gate=0x4000, sh_up=0x5000, sh_down=0x6000))


@pytest.mark.parametrize("bad, status", [
    (dict(hidden=0), afd.AFD_ERR_INVALID_ARG),
    (dict(inter=-128), afd.AFD_ERR_INVALID_ARG),
    (dict(top_k=0), afd.AFD_ERR_INVALID_ARG),
    (dict(max_tokens=0), afd.AFD_ERR_INVALID_ARG),
    (dict(hidden=200), afd.AFD_ERR_UNSUPPORTED),
    (dict(inter=96), afd.AFD_ERR_UNSUPPORTED),
    (dict(num_experts=513), afd.AFD_ERR_UNSUPPORTED),
    (dict(top_k=33), afd.AFD_ERR_UNSUPPORTED),
    (dict(dtype=7), afd.AFD_ERR_UNSUPPORTED),
    (dict(max_tokens=1 << 24, top_k=8), afd.AFD_ERR_UNSUPPORTED),
    (dict(w_up=0), afd.AFD_ERR_INVALID_ARG),
    (dict(dtype=afd.AFD_DTYPE_FP8_BLOCK), afd.AFD_ERR_INVALID_ARG),          # scales missing
    (dict(s_gate=8, s_up=8, s_down=8), afd.AFD_ERR_INVALID_ARG),              # scales with bf16
    (dict(shared_inter=200, sh_gate=0x4000, sh_up=0x5000, sh_down=0x6000), afd.AFD_ERR_UNSUPPORTED),  # not x128
    (dict(shared_inter=17 * 512, sh_gate=0x4000, sh_up=0x5000, sh_down=0x6000), afd.AFD_ERR_UNSUPPORTED),  # > 16 I
    (dict(shared_inter=512), afd.AFD_ERR_INVALID_ARG),                        # shared weights missing
    (dict(device=-1), afd.AFD_ERR_INVALID_ARG),
    (dict(w_gate=0x1008), afd.AFD_ERR_INVALID_ARG),                          # bf16 weights need 16 bytes
    (dict(dtype=afd.AFD_DTYPE_FP8_BLOCK, s_gate=8, s_up=8, s_down=6), afd.AFD_ERR_INVALID_ARG),  # scales 4
    (dict(dtype=afd.AFD_DTYPE_F32, w_down=0x3002), afd.AFD_ERR_INVALID_ARG),  # fp32 weights need 4
    # activation rows beyond 32-bit buffer offsets: 2^20 * 8 rows of 512 bf16
    (dict(max_tokens=1 << 20, top_k=8), afd.AFD_ERR_UNSUPPORTED),
    # hidden rows alone: 2^18 tokens of 4096 bf16 = 2 GiB
    (dict(max_tokens=1 << 18, top_k=1, hidden=4096, inter=128), afd.AFD_ERR_UNSUPPORTED),
])
def test_validate_config_rejects(lib, bad, status):
    with pytest.raises(afd.AfdError) as ei:
        afd.afd_ffn_validate_config(_cfg(**bad))
    assert ei.value.status == status
    assert afd.afd_ffn_last_error()


def test_null_arguments_rejected_on_host(lib):
    assert lib.afd_ffn_validate_config(None) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_create(ctypes.byref(_cfg()), None) == afd.AFD_ERR_INVALID_ARG
    h = ctypes.c_void_p(0)
    assert lib.afd_ffn_create(ctypes.byref(_cfg(hidden=100)), ctypes.byref(h)) == afd.AFD_ERR_UNSUPPORTED
    assert h.value is None
    assert lib.afd_ffn_forward(None, 4, None, None, None, None, None, None) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_clone(None, ctypes.byref(h)) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_debug_dispatch(None, None, None, None, None, None) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_set_timing(None, 1) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_set_timing_stages(None, 4) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_set_concurrency(None, 2) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_set_canaries(None, 65536) == afd.AFD_ERR_INVALID_ARG
    n = ctypes.c_int64(-1)
    assert lib.afd_ffn_check_canaries(None, ctypes.byref(n), None) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_debug_poke_canary(None, 0, 0) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_destroy(None) == afd.AFD_OK
    # measurement helpers: argument errors come back before any device call
    t, c = ctypes.c_double(0.0), ctypes.c_double(0.0)
    assert lib.afd_ffn_mfma_peak(1, 0, 100, None, ctypes.byref(c)) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_mfma_peak(0, 0, 100, ctypes.byref(t), ctypes.byref(c)) == afd.AFD_ERR_UNSUPPORTED  # fp32
    assert lib.afd_ffn_mfma_lds_peak(0, 90, 5, ctypes.byref(t), ctypes.byref(c)) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_mfma_lds_peak(0, 2, 6, ctypes.byref(t), ctypes.byref(c)) == afd.AFD_ERR_INVALID_ARG
    assert lib.afd_ffn_mfma_lds_peak(0, 90, 0, None, ctypes.byref(c)) == afd.AFD_ERR_INVALID_ARG


def test_status_strings(lib):
    for st in range(6):
        assert afd.afd_ffn_status_string(st)
    assert "unknown" in afd.afd_ffn_status_string(99)


def test_c_program_is_built_and_links():
    """The plain-C user of the ABI (tests/c_abi/abi_forward, run on the GPU by
    test_gpu_c_abi.py) is built and every library it needs resolves."""
    import subprocess

    binary = os.path.join(ROOT, "tests", "c_abi", "abi_forward")
    assert os.path.exists(binary), "run the build step (it builds tests/c_abi/abi_forward)"
    r = subprocess.run(["ldd", binary], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "not found" not in r.stdout, r.stdout
    for lib in ("libafd_ffn.so", "libafd_oracle.so", "libamdhip64"):
        assert lib in r.stdout, lib
