"""Build libmoe355.so in-tree with hipcc for gfx950.

Each .hip file compiles to its own object (route and router keep
-ffp-contract=off so the pinned sigmoid and the bias update are exactly the
written operation sequences), then one shared library is linked.  Run as ``python -m token_routing_expert_amd.build``.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe355.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["route.hip", "router.hip", "permute.hip", "grouped_gemm.hip", "grouped_gemm_bwd.hip",
           "grouped_wgrad.hip", "dense_splitk.hip",
           "combine.hip", "backward.hip"]
COMMON = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
    # Packed fp32 VALU forms stay off; the compiler emits scalar fp32 instead.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-Wall", "-Wno-unused-function",
]
PER_FILE = {"route.hip": ["-ffp-contract=off"], "router.hip": ["-ffp-contract=off"]}


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, src.replace(".hip", ".o"))
    cmd = [HIPCC, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    _check_no_missing_kernels(LIB + ".tmp")
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _check_no_missing_kernels(path: str) -> None:
    """Fail if the library references a symbol of its own namespace that it
    does not define: the host side of a kernel can be left out without a
    compile error, and the library would then fail to load."""
    nm = "/opt/rocm/llvm/bin/llvm-nm" if os.path.exists("/opt/rocm/llvm/bin/llvm-nm") else "nm"
    out = subprocess.run([nm, "-D", "--undefined-only", path], capture_output=True, text=True,
                         check=True).stdout
    missing = [line.split()[-1] for line in out.splitlines() if "_ZN3moe" in line]
    if missing:
        raise RuntimeError(f"{path}: undefined library symbols (kernel host stubs missing): {missing[:4]}")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
