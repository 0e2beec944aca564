"""Build the gfx950 shuffle library in-tree: combine_shuffling_amd/libmoeshuffle.so.

Run ``python -m combine_shuffling_amd.build`` (or ``__graft_entry__.build()``).
Cross-compiles with hipcc; no GPU is needed to build.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoeshuffle.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ("route_plan.hip", "move.hip", "pipeline.hip", "moe_api.cpp")

# -packed-fp32-ops: no packed fp32 instructions in device code.
HIP_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: install ROCm or put hipcc on PATH")
    return path


def build(verbose: bool = False, extra_flags=(), out: str | None = None) -> str:
    """Compile every source into ``out`` (default LIB_PATH; always recompiles).

    extra_flags: more hipcc flags (for instance -save-temps to keep the
    gfx950 assembly).
    """
    out = LIB_PATH if out is None else out
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "is not a recognized feature for this target")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)
    return out


C_TESTS = os.path.join(ROOT, "tests", "c")


def build_c_tests() -> list:
    """Compile the plain-C users of the ABI (tests/c/*.c) against the built
    library with gcc, into tests/c/build/.  abi_gpu also links the HIP C
    runtime.  The binaries find the library through an $ORIGIN-relative
    rpath, so the tree can move."""
    out_dir = os.path.join(C_TESTS, "build")
    os.makedirs(out_dir, exist_ok=True)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    rpath = "-Wl,-rpath,$ORIGIN/../../../combine_shuffling_amd"
    common = ["gcc", "-O2", "-std=c11", "-Wall", "-Werror", f"-I{INCLUDE}"]
    link = [f"-L{PKG}", "-lmoeshuffle", rpath]
    built = []
    for name, extra in (("abi_host", []),
                        ("abi_gpu", ["-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
                                     f"-L{rocm}/lib", "-lamdhip64", f"-Wl,-rpath,{rocm}/lib"])):
        dst = os.path.join(out_dir, name)
        cmd = [*common, os.path.join(C_TESTS, name + ".c"), "-o", dst, *link, *extra]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"gcc failed for {name}:\n{res.stdout}{res.stderr}")
        built.append(dst)
    return built


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print("\n".join(build_c_tests()))
