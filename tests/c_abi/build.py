"""Build tests/c_abi/abi_forward: the C ABI called from plain C (no Python in
the process), linked against the layer library, the fp64 oracle it is checked
against, and the system HIP runtime (the library resolves the same one when
no other is loaded).  Test infrastructure: run by the build step, executed
by tests/test_gpu_c_abi.py."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_forward.c")
OUT = os.path.join(HERE, "abi_forward")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"), SRC, "-o", tmp,
           "-L" + os.path.join(ROOT, "moe_expert_ffn_afd_amd"), "-l:libafd_ffn.so",
           "-L" + os.path.join(ROOT, "oracle"), "-l:libafd_oracle.so",
           "-L" + os.path.join(ROCM, "lib"), "-l:libamdhip64.so", "-lm",
           "-Wl,-rpath,$ORIGIN/../../moe_expert_ffn_afd_amd:$ORIGIN/../../oracle:" + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the C ABI test failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
