"""Build libvbprop.so (HIP, gfx950) in-tree with hipcc.

Each source is compiled to an object in parallel (under _build/), then the
objects are linked into the shared library.  The measurement probes (an
MFMA-only loop and HBM read / write streams) are a separate library,
libvbprobe.so, loaded only by the benchmark.

Usage: python -m linear_bound_propagation_amd.build [-v]
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libvbprop.so")
PROBE_LIB = os.path.join(HERE, "libvbprobe.so")

SOURCES = ["vb_gemm.hip", "vb_ibp_narrow.hip", "vb_kernels.hip", "vb_scratch.hip", "vb_api.cpp"]
PROBE_SOURCES = ["vb_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU instructions stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the GEMM epilogues index the MFMA accumulators by unrolled loop counters;
    # a partially unrolled loop would move the accumulators to scratch memory
    "-mllvm", "-pragma-unroll-threshold=200000",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _filter(text: str) -> str:
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops' is not a recognized feature" not in l)


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = _filter(res.stdout + res.stderr)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
    if verbose and out.strip():
        print(out)


def _link(sources, lib, verbose):
    os.makedirs(OBJ, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + ".o") for s in sources]
    cmds = [[hipcc()] + HIPCC_FLAGS + inc + ["-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(sources, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = lib + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    with ThreadPoolExecutor(max_workers=2) as ex:
        a = ex.submit(_link, SOURCES, LIB, verbose)
        b = ex.submit(_link, PROBE_SOURCES, PROBE_LIB, verbose)
        a.result()
        b.result()
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
