"""Build the HIP library libafd_ffn.so in-tree for gfx950.

Every ``csrc/*.hip`` file is compiled with hipcc (device code for gfx950
only) and the objects are linked against the HIP runtime that torch ships,
so that one HIP runtime serves both torch's allocations/streams and this
library in a process that imported torch first.

    python -m moe_expert_ffn_afd_amd.build
"""
from __future__ import annotations

import concurrent.futures
import glob
import importlib.util
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libafd_ffn.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def torch_lib_dir() -> str:
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.origin:
        raise RuntimeError("torch is not importable: its HIP runtime is needed to link")
    return os.path.join(os.path.dirname(spec.origin), "lib")


def _compile(src: str, extra=(), build_dir=BUILD) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + HIP_FLAGS + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False, extra_flags=(), out: str = OUT) -> str:
    """Compile and link; `extra_flags` (e.g. -D tuning macros) and `out` allow
    building variants side by side."""
    build_dir = BUILD if out == OUT else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra_flags, build_dir), srcs))
    tl = torch_lib_dir()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["g++", "-shared", "-o", tmp] + objs + ["-L" + tl, "-l:libamdhip64.so", "-Wl,-rpath," + tl,
                                                 "-Wl,--no-undefined"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
