"""Build libpa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python paged_kv_attention_07_amd/build.py [--verbose]

The library lands next to this file; the Python binding loads it from there.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libpa.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpa.so)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        # packed fp32 arithmetic is kept off: hipcc would otherwise form
        # v_pk_{add,mul,fma}_f32 from ordinary float code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Per-source flags.  The attention-tile translation units hold only kernels
# and their launchers, and no NaN appears in their arithmetic (masked scores
# are -inf, never NaN, and no code there tests for NaN): there the row max
# can skip the NaN-quieting copies that IEEE max needs on operands the
# compiler cannot prove quiet (a matrix-core result, a lane-swap result).
SOURCE_FLAGS = {
    "pa_prefill.hip": ["-fno-honor-nans"],
    "pa_fused.hip": ["-fno-honor-nans"],
}


def host_sources():
    """Plain C++ (host-only) sources, compiled with the host compiler."""
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")))


def host_flags():
    return ["-O2", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def build(verbose: bool = False, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile every source into one shared library; returns its path."""
    objs = []
    build_dir = os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    procs = []
    for src in sources():
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [cc, *compile_flags(), *SOURCE_FLAGS.get(os.path.basename(src), []), *extra_flags,
               "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT), src))
        objs.append(obj)
    cxx = shutil.which("g++") or "c++"
    for src in host_sources():
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [cxx, *host_flags(), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT), src))
        objs.append(obj)
    failed = []
    for p, src in procs:
        text = p.communicate()[0].decode(errors="replace")
        if verbose or p.returncode:
            lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l
                     and "is not a recognized feature" not in l]
            if lines:
                print("\n".join(lines), flush=True)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError("compilation failed for: " + ", ".join(os.path.basename(f) for f in failed))
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
