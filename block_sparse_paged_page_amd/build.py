"""Build libkap.so (HIP, gfx950) in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction
selection turned off, and linked into one shared library exporting the C ABI
of include/kap.h.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkap.so")
SOURCES = ["kap_api.hip", "attn.hip", "score.hip", "select.hip", "compact.hip", "proxy.hip",
           "kvcopy.hip", "diag.hip"]
HOST_SOURCES = ["host_route.cpp"]  # host-only C++ (CPU-offloaded routing)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden", "-pthread",
              "-I", os.path.join(os.path.dirname(HERE), "include")]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden",
]


def build(verbose: bool = False, jobs: int = 6) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for src in HOST_SOURCES:
        obj = os.path.join(objdir, src.replace(".cpp", ".o"))
        objs.append(obj)
        cmd = [CXX] + HOST_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    for p in procs:
        _wait(p)
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-pthread", "-o", LIB + ".tmp"] + objs
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def _wait(entry):
    src, p = entry
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    noise = "is not a recognized feature for this target"
    lines = [ln for ln in text.splitlines() if noise not in ln]
    if lines:
        print("\n".join(lines), flush=True)
    if p.returncode != 0:
        raise RuntimeError(f"compiler failed on {src}")


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
