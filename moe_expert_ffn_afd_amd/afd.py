"""ctypes binding of libafd_ffn.so (include/afd_ffn.h), same names as the C ABI.

Argument marshalling only: torch tensors supply device pointers
(``data_ptr()``) and ``torch.cuda.current_stream()`` supplies the stream; every
step of the layer runs in the library's HIP kernels.  The library must have
been built (``python -m moe_expert_ffn_afd_amd.build``); loading raises if it
is missing -- there is no fallback.

torch is imported before the library is loaded so that the library binds to
torch's HIP runtime (one runtime per process).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading the library: one HIP runtime)

# AFD_FFN_LIB may name another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("AFD_FFN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libafd_ffn.so")

AFD_OK, AFD_ERR_INVALID_ARG, AFD_ERR_UNSUPPORTED, AFD_ERR_OUT_OF_MEMORY, AFD_ERR_HIP, AFD_ERR_BAD_ROUTING = range(6)
AFD_DTYPE_F32, AFD_DTYPE_BF16, AFD_DTYPE_FP8_BLOCK, AFD_DTYPE_W8A8 = 0, 1, 2, 3
AFD_NUM_STAGES = 5
STAGE_NAMES = ("dispatch_count_scan", "dispatch_scatter", "gemm_gate_up_swiglu", "gemm_down", "combine")
DTYPE_CODES = {"f32": AFD_DTYPE_F32, "bf16": AFD_DTYPE_BF16, "fp8": AFD_DTYPE_FP8_BLOCK, "w8a8": AFD_DTYPE_W8A8}

EXPORTS = ("afd_ffn_validate_config", "afd_ffn_create", "afd_ffn_clone", "afd_ffn_forward",
           "afd_ffn_forward_noalloc",
           "afd_ffn_destroy", "afd_ffn_status_string", "afd_ffn_last_error", "afd_ffn_debug_dispatch",
           "afd_ffn_routing_errors", "afd_ffn_set_timing", "afd_ffn_set_timing_stages", "afd_ffn_get_timing",
           "afd_ffn_set_concurrency", "afd_ffn_set_fused", "afd_ffn_fused_errors", "afd_ffn_mfma_peak",
           "afd_ffn_mfma_lds_peak", "afd_ffn_set_canaries", "afd_ffn_check_canaries", "afd_ffn_debug_poke_canary")


class afd_ffn_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("hidden", "inter", "num_experts", "top_k", "max_tokens",
                                              "shared_inter", "dtype", "device")] + \
               [(n, ctypes.c_void_p) for n in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                                               "sh_gate", "sh_up", "sh_down", "sh_s_gate", "sh_s_up",
                                               "sh_s_down")]


class AfdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_status_name(status), message))
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libafd_ffn.so is not built (%s); run python -m moe_expert_ffn_afd_amd.build" % path)
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.afd_ffn_validate_config.argtypes = [ctypes.POINTER(afd_ffn_config)]
    lib.afd_ffn_create.argtypes = [ctypes.POINTER(afd_ffn_config), ctypes.POINTER(vp)]
    lib.afd_ffn_clone.argtypes = [vp, ctypes.POINTER(vp)]
    lib.afd_ffn_forward.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
    lib.afd_ffn_forward_noalloc.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp]
    lib.afd_ffn_destroy.argtypes = [vp]
    lib.afd_ffn_status_string.argtypes = [ctypes.c_int]
    lib.afd_ffn_status_string.restype = ctypes.c_char_p
    lib.afd_ffn_last_error.argtypes = []
    lib.afd_ffn_last_error.restype = ctypes.c_char_p
    lib.afd_ffn_debug_dispatch.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.afd_ffn_routing_errors.argtypes = [vp, ctypes.POINTER(i32), vp]
    lib.afd_ffn_set_timing.argtypes = [vp, i32]
    lib.afd_ffn_set_timing_stages.argtypes = [vp, ctypes.c_uint32]
    lib.afd_ffn_set_concurrency.argtypes = [vp, i32]
    lib.afd_ffn_set_fused.argtypes = [vp, i32]
    lib.afd_ffn_mfma_peak.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    lib.afd_ffn_mfma_lds_peak.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_double)]
    lib.afd_ffn_fused_errors.argtypes = [vp, ctypes.POINTER(i32), vp]
    lib.afd_ffn_get_timing.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    lib.afd_ffn_set_canaries.argtypes = [vp, ctypes.c_int64]
    lib.afd_ffn_check_canaries.argtypes = [vp, ctypes.POINTER(ctypes.c_int64), vp]
    lib.afd_ffn_debug_poke_canary.argtypes = [vp, i32, ctypes.c_int64]
    for name in EXPORTS:
        if name not in ("afd_ffn_status_string", "afd_ffn_last_error"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _status_name(st: int) -> str:
    try:
        return load().afd_ffn_status_string(st).decode()
    except Exception:
        return "status %d" % st


def _check(st: int):
    if st != AFD_OK:
        raise AfdError(st, load().afd_ffn_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def make_config(p: dict, max_tokens: int, device: int = 0) -> afd_ffn_config:
    """Config struct from a problem dict of device tensors (see inputs.make_problem)."""
    H, I, E, K = p["H"], p["I"], p["E"], p["K"]
    c = afd_ffn_config(hidden=H, inter=I, num_experts=E, top_k=K, max_tokens=max_tokens,
                       shared_inter=p["sh_gate"].shape[1] if p.get("sh_gate") is not None else 0,
                       dtype=DTYPE_CODES[p["dtype"]], device=device)
    for name in ("w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down", "sh_gate", "sh_up", "sh_down",
                 "sh_s_gate", "sh_s_up", "sh_s_down"):
        t = p.get(name)
        setattr(c, name, None if t is None else t.data_ptr())
    return c


def afd_ffn_validate_config(cfg: afd_ffn_config) -> None:
    _check(load().afd_ffn_validate_config(ctypes.byref(cfg)))


def afd_ffn_create(cfg: afd_ffn_config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load().afd_ffn_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def afd_ffn_clone(handle) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load().afd_ffn_clone(handle, ctypes.byref(h)))
    return h


def afd_ffn_forward(handle, num_tokens: int, hidden, hidden_scales, topk_ids, topk_weights, out,
                    stream=None) -> None:
    _check(load().afd_ffn_forward(handle, int(num_tokens), _ptr(hidden), _ptr(hidden_scales), _ptr(topk_ids),
                                  _ptr(topk_weights), _ptr(out), _stream(stream)))


def afd_ffn_forward_noalloc(handle, num_tokens: int, hidden, hidden_scales, topk_ids, topk_weights, out,
                            stream=None) -> None:
    """The forward on the library's static device scratch (allocates nothing)."""
    _check(load().afd_ffn_forward_noalloc(handle, int(num_tokens), _ptr(hidden), _ptr(hidden_scales),
                                          _ptr(topk_ids), _ptr(topk_weights), _ptr(out), _stream(stream)))


def afd_ffn_destroy(handle) -> None:
    _check(load().afd_ffn_destroy(handle))


def afd_ffn_status_string(status: int) -> str:
    return load().afd_ffn_status_string(status).decode()


def afd_ffn_last_error() -> str:
    return load().afd_ffn_last_error().decode()


def afd_ffn_debug_dispatch(handle, counts, offsets, sorted_assign, row_of, stream=None) -> None:
    _check(load().afd_ffn_debug_dispatch(handle, _ptr(counts), _ptr(offsets), _ptr(sorted_assign), _ptr(row_of),
                                         _stream(stream)))


def afd_ffn_routing_errors(handle, stream=None) -> int:
    n = ctypes.c_int32(0)
    st = load().afd_ffn_routing_errors(handle, ctypes.byref(n), _stream(stream))
    if st not in (AFD_OK, AFD_ERR_BAD_ROUTING):
        _check(st)
    return int(n.value)


def afd_ffn_set_concurrency(handle, streams: int) -> None:
    _check(load().afd_ffn_set_concurrency(handle, int(streams)))


def afd_ffn_set_fused(handle, enable: bool) -> None:
    _check(load().afd_ffn_set_fused(handle, 1 if enable else 0))


def afd_ffn_fused_errors(handle, stream=None) -> int:
    """Timed-out grid-barrier waits of fused forwards since the last query."""
    n = ctypes.c_int32(0)
    st = load().afd_ffn_fused_errors(handle, ctypes.byref(n), _stream(stream))
    if st not in (AFD_OK, AFD_ERR_HIP):
        _check(st)
    return int(n.value)


def afd_ffn_set_canaries(handle, guard_bytes: int) -> None:
    """Re-allocate the handle's workspace with canary bands of guard_bytes (0: none)."""
    _check(load().afd_ffn_set_canaries(handle, int(guard_bytes)))


def afd_ffn_check_canaries(handle, stream=None) -> int:
    """Workspace guard-band bytes that lost the canary (0 when every band is intact)."""
    n = ctypes.c_int64(0)
    st = load().afd_ffn_check_canaries(handle, ctypes.byref(n), _stream(stream))
    if st not in (AFD_OK, AFD_ERR_HIP) or (st == AFD_ERR_HIP and n.value == 0):
        _check(st)
    return int(n.value)


def afd_ffn_debug_poke_canary(handle, band: int, offset: int) -> None:
    """Overwrite one byte of a guard band (a positive control of the canary check)."""
    _check(load().afd_ffn_debug_poke_canary(handle, int(band), int(offset)))


def afd_ffn_mfma_lds_peak(lds_reads: int, device: int = 0, iters: int = 90000):
    """(TFLOP/s, shader GHz) of the LDS-tiled bf16 GEMM's MFMA loop with (6) or without (0)
    its LDS fragment reads, no memory traffic."""
    t, c = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check(load().afd_ffn_mfma_lds_peak(int(device), int(iters), int(lds_reads), ctypes.byref(t), ctypes.byref(c)))
    return t.value, c.value


def afd_ffn_mfma_peak(dtype: str, device: int = 0, iters: int = 200000):
    """(TFLOP/s, shader GHz) of MFMA chains with no memory traffic ('bf16', 'fp8', 'w8a8')."""
    t, c = ctypes.c_double(0.0), ctypes.c_double(0.0)
    _check(load().afd_ffn_mfma_peak(DTYPE_CODES[dtype], int(device), int(iters), ctypes.byref(t), ctypes.byref(c)))
    return t.value, c.value


def afd_ffn_set_timing(handle, enable: bool) -> None:
    _check(load().afd_ffn_set_timing(handle, 1 if enable else 0))


def afd_ffn_set_timing_stages(handle, stages) -> None:
    """Time only the given stage indices (0..AFD_NUM_STAGES-1) of later forwards."""
    mask = 0
    for st in stages:
        mask |= 1 << int(st)
    _check(load().afd_ffn_set_timing_stages(handle, mask))


def afd_ffn_get_timing(handle):
    """(per-stage summed ms list, number of forwards) since the last query."""
    ms = (ctypes.c_float * AFD_NUM_STAGES)()
    n = ctypes.c_int32(0)
    _check(load().afd_ffn_get_timing(handle, ms, ctypes.byref(n)))
    return list(ms), int(n.value)


def _check_inputs(layer, T, hidden, hidden_scales, ids, weights, out):
    """Host-side shape/dtype/device checks of the tensors behind the raw pointers."""
    esz = {"f32": 4, "bf16": 2, "fp8": 1, "w8a8": 1}[layer.dtype]
    H, K = layer.H, layer.K
    def need(ok, what):
        if not ok:
            raise ValueError("afd_ffn_forward: " + what)
    need(0 <= T <= layer.max_tokens, "T=%d outside [0, %d]" % (T, layer.max_tokens))
    for name, t, shape, size in (("hidden", hidden, (T, H), esz), ("topk_ids", ids, (T, K), 4),
                                 ("topk_weights", weights, (T, K), 4), ("out", out, (T, H), 4 if esz == 4 else 2)):
        need(t.is_cuda, name + " must be a device tensor")
        need(tuple(t.shape) == shape, "%s shape %s != %s" % (name, tuple(t.shape), shape))
        need(t.is_contiguous() and t.element_size() == size, name + " must be contiguous with %d-byte elements" % size)
    need(ids.dtype == torch.int32 and weights.dtype == torch.float32, "ids int32 and weights float32")
    if layer.dtype in ("fp8", "w8a8"):
        shape = (T, H // 128) if layer.dtype == "fp8" else (T,)
        need(hidden_scales is not None and tuple(hidden_scales.shape) == shape and
             hidden_scales.dtype == torch.float32 and hidden_scales.is_contiguous(),
             "hidden_scales %s fp32" % ("[T, H/128]" if layer.dtype == "fp8" else "[T]"))
    else:
        need(hidden_scales is None, "hidden_scales only for fp8 and w8a8")


class Layer:
    """Owning wrapper: create from a problem dict, forward into an output tensor."""

    def __init__(self, p: dict, max_tokens: int | None = None, device: int = 0, handle=None):
        self.dtype = p["dtype"]
        self.H = p["H"]
        self.K = p["K"]
        self.E = p["E"]
        self.max_tokens = max_tokens or p["T"]
        self.handle = handle if handle is not None else afd_ffn_create(make_config(p, self.max_tokens, device))

    def clone(self) -> "Layer":
        other = object.__new__(Layer)
        other.__dict__.update(self.__dict__)
        other.handle = afd_ffn_clone(self.handle)
        return other

    def set_concurrency(self, streams: int) -> None:
        """Forwards run at once on other streams (this handle and its clones)."""
        afd_ffn_set_concurrency(self.handle, streams)

    def set_fused(self, enable: bool) -> None:
        """Later forwards as one persistent launch (block-FP8 and W8A8 layers)."""
        afd_ffn_set_fused(self.handle, enable)

    def set_canaries(self, guard_bytes: int = 1 << 16) -> None:
        """Canary bands of guard_bytes around every workspace buffer (0: none)."""
        afd_ffn_set_canaries(self.handle, guard_bytes)

    def check_canaries(self, stream=None) -> int:
        """Bytes of the workspace's canary bands that were overwritten."""
        return afd_ffn_check_canaries(self.handle, stream)

    def out_like(self, T: int, device="cuda"):
        dt = torch.float32 if self.dtype == "f32" else torch.bfloat16
        return torch.empty((T, self.H), dtype=dt, device=device)

    def forward(self, hidden, hidden_scales, ids, weights, out=None, stream=None):
        T = hidden.shape[0]
        if out is None:
            out = self.out_like(T, hidden.device)
        _check_inputs(self, T, hidden, hidden_scales, ids, weights, out)
        afd_ffn_forward(self.handle, T, hidden, hidden_scales, ids, weights, out, stream)
        return out

    def dispatch(self, T: int, stream=None) -> dict:
        dev = torch.device("cuda")
        counts = torch.empty(self.E, dtype=torch.int32, device=dev)
        offsets = torch.empty(self.E + 1, dtype=torch.int32, device=dev)
        sa = torch.full((max(T * self.K, 1),), -7, dtype=torch.int32, device=dev)
        row_of = torch.empty((max(T, 1), self.K), dtype=torch.int32, device=dev)
        afd_ffn_debug_dispatch(self.handle, counts, offsets, sa, row_of, stream)
        torch.cuda.synchronize()
        n = int(offsets[-1].item())
        return {"counts": counts.cpu().numpy(), "offsets": offsets.cpu().numpy(),
                "sorted_assign": sa[:n].cpu().numpy(), "row_of": row_of[:T].cpu().numpy()}

    def close(self):
        if self.handle is not None:
            afd_ffn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
