"""Compile the gfx950 HIP sources into in-tree shared libraries.

libdsi.so is the indexer library (include/dsi.h); libdsi_ceiling.so holds the
measurement kernels the benchmark reads rooflines against (include/dsi_ceiling.h);
libdsi_probe.so runs the kernels' device converters over whole input ranges for the
tests (include/dsi_probe.h).
Each source compiles to its own object under _build/ (in parallel), then one
hipcc link per library.  Packed FP32 ops are disabled for every device
compilation.
"""
import concurrent.futures
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdsi.so")
LIB_CEILING = os.path.join(HERE, "libdsi_ceiling.so")
LIB_PROBE = os.path.join(HERE, "libdsi_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["quant.hip", "prefill.hip", "gather_logits.hip", "topk.hip", "index.hip", "prefill_gather.hip", "q_prep.hip", "cp_merge.hip", "status.cpp"]
CEILING_SOURCES = ["ceiling.hip"]
PROBE_SOURCES = ["probe.hip"]

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
    if msgs:
        print(msgs)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CEILING_SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in CEILING_SOURCES], LIB_CEILING, verbose)
    _link([objs[s] for s in PROBE_SOURCES], LIB_PROBE, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
