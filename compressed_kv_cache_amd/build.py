"""Build libgva.so (HIP for gfx950) in-tree with hipcc.

Usage: python compressed_kv_cache_amd/build.py [--verbose]
(run by path: importing the package loads the library this script builds)
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libgva.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["gva_api.cpp", "gva_prologue.hip", "gva_decode_ref.hip",
           "gva_decode_mfma.hip", "gva_decode_rope.hip", "gva_prefill.hip",
           "gva_probe.hip", "gva_noalloc.hip"]

# Packed fp32 instructions are switched off for all device code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function"]


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"),
                 "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libgva)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}")
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if verbose and msg.strip():
        print(msg)


def build(verbose=False, jobs=8):
    """Compile every source to an object under _build/ and link libgva.so."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, *lang, "-c",
               os.path.join(CSRC, src), "-o", obj]
        objs.append(obj)
        procs.append(cmd)
    # compile in parallel
    running = []
    for cmd in procs:
        if verbose:
            print(" ".join(cmd), flush=True)
        running.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                              stderr=subprocess.STDOUT, text=True)))
    failed = False
    for cmd, p in running:
        out, _ = p.communicate()
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in out.splitlines() if noise not in l)
        if p.returncode != 0:
            failed = True
            sys.stderr.write(msg + "\n")
        elif verbose and msg.strip():
            print(msg)
    if failed:
        raise RuntimeError("libgva compilation failed")
    tmp = LIB + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
