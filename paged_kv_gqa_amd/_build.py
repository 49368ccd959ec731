"""Build libpkv.so in-tree with hipcc for gfx950 (no JIT, no site-packages install).

    python paged_kv_gqa_amd/_build.py

(Run as a file: importing it through the package would load the package, which needs
the library.)
"""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpkv.so")
# Read-bandwidth probes for the bench's roofline (measurement only, a library of its own).
PROBE_SRC = "read_probe.hip"
PROBE_LIB = os.path.join(PKG, "libpkv_probe.so")

SOURCES = ["planner.cpp", "api.cpp", "validate.cpp", "decode_partial.hip", "combine.hip", "plan_device.hip",
           "block_sparse.hip", "kv_append.hip", "prefill.hip", "noalloc.hip"]
HEADERS = ["planner.hpp", "kernels.hpp", "status.hpp", "validate.hpp"]

# Packed-fp32 VALU forms are kept out of the generated code on purpose.
HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose=False):
    """Compile every source and link libpkv.so (and the bench's libpkv_probe.so);
    always recompiles."""
    os.makedirs(OBJ, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc()] + HIPCC_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        _run(cmd, verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB)
    probe_obj = os.path.join(OBJ, "read_probe.o")
    _run([hipcc()] + HIPCC_FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, PROBE_SRC), "-o", probe_obj],
         verbose)
    tmp = PROBE_LIB + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", probe_obj, "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError("build failed: %s\n%s" % (" ".join(cmd), out))
    if verbose and out.strip():
        print(out)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
