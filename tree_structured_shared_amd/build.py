"""Build the tree-attention HIP library in-tree (gfx950).

    python -m tree_structured_shared_amd.build

compiles csrc/*.cpp and csrc/*.hip with hipcc into
tree_structured_shared_amd/libtree_attn.so. hipcc cross-compiles, so this
also runs on a machine without a GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtree_attn.so")
SOURCES = ["planner.cpp", "capi.cpp", "kernels.hip"]
ARCH = os.environ.get("TREE_ATTN_ARCH", "gfx950")

# Packed-FP32 instructions are kept out of every device build.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# The host-sanitized build (CPU tests of the planner and the C ABI): address
# and undefined-behaviour sanitizers on the host code only, each flag scoped
# to the host compile; device code is built as usual. The library links the
# shared sanitizer runtime, which the process that loads it preloads.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-shared-libasan", "-g"]


def asan_runtime():
    """Path of the shared address-sanitizer runtime of the compiler that
    builds the library (for LD_PRELOAD), or None."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def hipcc_cmd(out=LIB, extra=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    return ([hipcc, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]
            + DEVICE_FLAGS + list(extra)
            + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out])


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    tmp = out + ".tmp"
    cmd = hipcc_cmd(tmp, SANITIZE_FLAGS if sanitize else ())
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(x for x in (res.stdout + res.stderr).splitlines() if noise not in x)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + msgs)
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
