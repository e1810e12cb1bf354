"""ctypes front end of the C oracle (afd_oracle.c) -- TEST INFRASTRUCTURE ONLY.

The arithmetic lives in afd_oracle.c (plain C, fp64, pthreads).  This module
only compiles it with gcc, marshals numpy arrays into its problem struct and
returns fp64 numpy results.  Dispatch follows the definition of the
expert-major permutation; the forward follows the SwiGLU MoE layer described
in the header comment of afd_oracle.c.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "afd_oracle.c")
_LIB = os.path.join(_HERE, "libafd_oracle.so")
_lock = threading.Lock()
_lib = None

DTYPES = {"f32": 0, "bf16": 1, "fp8": 2, "w8a8": 3}


def library_path() -> str:
    return _LIB


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-pthread",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("T", "H", "I", "E", "K", "shared_inter", "dtype")] + [
        ("hidden", ctypes.c_void_p), ("hidden_scales", ctypes.c_void_p),
        ("ids", ctypes.c_void_p), ("weights", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
        ("sh_gate", ctypes.c_void_p), ("sh_up", ctypes.c_void_p), ("sh_down", ctypes.c_void_p),
        ("sh_s_gate", ctypes.c_void_p), ("sh_s_up", ctypes.c_void_p), ("sh_s_down", ctypes.c_void_p),
    ]


def load(path: str | None = None):
    """Load (building first if needed) the oracle library."""
    global _lib
    with _lock:
        if path is not None:
            lib = ctypes.CDLL(path)
        else:
            if _lib is not None:
                return _lib
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
        lib.afd_oracle_dispatch.restype = ctypes.c_int
        lib.afd_oracle_dispatch.argtypes = [ctypes.c_int32] * 3 + [ctypes.c_void_p] * 5
        lib.afd_oracle_forward.restype = ctypes.c_int
        lib.afd_oracle_forward.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int32, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int32]
        lib.afd_oracle_bf16_to_f64.restype = ctypes.c_double
        lib.afd_oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.afd_oracle_e4m3_to_f64.restype = ctypes.c_double
        lib.afd_oracle_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        lib.afd_oracle_i8_to_f64.restype = ctypes.c_double
        lib.afd_oracle_i8_to_f64.argtypes = [ctypes.c_uint8]
        if path is None:
            _lib = lib
        return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def dispatch(ids: np.ndarray, num_experts: int, lib=None) -> dict:
    """counts [E], offsets [E+1], sorted_assign [N], row_of [T,K] (all int32)."""
    lib = lib or load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, K = ids.shape
    counts = np.zeros(num_experts, np.int32)
    offsets = np.zeros(num_experts + 1, np.int32)
    sorted_assign = np.full(max(T * K, 1), -7, np.int32)
    row_of = np.zeros((T, K), np.int32)
    rc = lib.afd_oracle_dispatch(T, K, num_experts, _ptr(ids), _ptr(counts), _ptr(offsets),
                                 _ptr(sorted_assign), _ptr(row_of))
    if rc != 0:
        raise ValueError("oracle dispatch rejected the routing (rc=%d)" % rc)
    n = int(offsets[-1])
    return {"counts": counts, "offsets": offsets, "sorted_assign": sorted_assign[:n].copy(),
            "row_of": row_of}


def e4m3_decode(code: int, lib=None) -> float:
    return (lib or load()).afd_oracle_e4m3_to_f64(int(code))


def i8_decode(raw: int, lib=None) -> float:
    """Value of an int8 code given as its raw byte 0..255."""
    return (lib or load()).afd_oracle_i8_to_f64(int(raw))


def bf16_decode(bits: int, lib=None) -> float:
    return (lib or load()).afd_oracle_bf16_to_f64(int(bits))


def _as_raw(a, dtype: str):
    """numpy view of an input in the oracle's raw element type."""
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor: take its host bytes
        import torch
        t = a.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16 or t.dtype == torch.float16:
            t = t.view(torch.int16)
        elif t.dtype == torch.float8_e4m3fn or t.dtype == torch.int8:
            t = t.view(torch.uint8)
        a = t.numpy()
    want = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8, "w8a8": np.uint8}[dtype]
    a = np.ascontiguousarray(a)
    if a.dtype != want:
        a = a.view(want) if a.dtype.itemsize == np.dtype(want).itemsize else a.astype(want)
    return a


def _f32(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu().float().contiguous().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def forward(p: dict, tokens=None, nthreads: int = 0, lib=None) -> np.ndarray:
    """fp64 outputs [len(tokens), H] for the problem dict ``p``.

    ``p`` holds: dtype ('f32'|'bf16'|'fp8'|'w8a8'), hidden [T,H], hidden_scales
    (fp8 [T,H/128], w8a8 [T]), ids [T,K] int32, weights [T,K] fp32, w_gate/w_up
    [E,H,I], w_down [E,I,H], s_gate/s_up/s_down (fp8 block grids, w8a8
    [E,I], [E,I], [E,H] per output column), optionally sh_gate/sh_up/sh_down
    (+ sh_s_*).
    Arrays may be numpy or torch (any device; copied to host).
    """
    lib = lib or load()
    dt = p["dtype"]
    hidden = _as_raw(p["hidden"], dt)
    T, H = hidden.shape
    ids = np.ascontiguousarray(_as_raw_int(p["ids"]))
    K = ids.shape[1]
    wts = _f32(p["weights"])
    wg, wu, wd = (_as_raw(p[n], dt) for n in ("w_gate", "w_up", "w_down"))
    E, _, I = wg.shape
    keep = [hidden, ids, wts, wg, wu, wd]
    prob = _Problem(T=T, H=H, I=I, E=E, K=K, shared_inter=0, dtype=DTYPES[dt])
    prob.hidden, prob.ids, prob.weights = _ptr(hidden), _ptr(ids), _ptr(wts)
    prob.w_gate, prob.w_up, prob.w_down = _ptr(wg), _ptr(wu), _ptr(wd)
    if dt in ("fp8", "w8a8"):
        hs, sg, su, sd = (_f32(p[n]) for n in ("hidden_scales", "s_gate", "s_up", "s_down"))
        keep += [hs, sg, su, sd]
        prob.hidden_scales, prob.s_gate, prob.s_up, prob.s_down = _ptr(hs), _ptr(sg), _ptr(su), _ptr(sd)
    if p.get("sh_gate") is not None:
        shg, shu, shd = (_as_raw(p[n], dt) for n in ("sh_gate", "sh_up", "sh_down"))
        keep += [shg, shu, shd]
        prob.shared_inter = shg.shape[1]
        prob.sh_gate, prob.sh_up, prob.sh_down = _ptr(shg), _ptr(shu), _ptr(shd)
        if dt in ("fp8", "w8a8"):
            ssg, ssu, ssd = (_f32(p[n]) for n in ("sh_s_gate", "sh_s_up", "sh_s_down"))
            keep += [ssg, ssu, ssd]
            prob.sh_s_gate, prob.sh_s_up, prob.sh_s_down = _ptr(ssg), _ptr(ssu), _ptr(ssd)
    tok = np.arange(T, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    out = np.zeros((max(len(tok), 1), H), np.float64)
    rc = lib.afd_oracle_forward(ctypes.byref(prob), len(tok), _ptr(tok), _ptr(out), int(nthreads))
    if rc != 0:
        raise ValueError("oracle forward rejected the problem (rc=%d)" % rc)
    del keep
    return out[:len(tok)]


def _as_raw_int(a):
    if hasattr(a, "detach"):
        a = a.detach().cpu().contiguous().numpy()
    return np.asarray(a, dtype=np.int32)
