"""Build libtv.so (the HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtv.so")
PROBE_SRC = os.path.join(HERE, "probe", "tv_probe.hip")
PROBE_LIB = os.path.join(HERE, "libtv_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in architectural VGPRs: with the default AGPR form the
    # loop-carried attention accumulators are copied between the two register
    # files on every iteration
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Extra flags per source.  The attention kernels compare MFMA results that are
# never NaN: without NaN semantics a max is one v_max3 instead of a quieting
# v_max per operand.
FILE_FLAGS = {
    "tv_attention.hip": ["-fno-honor-nans"],
}


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link them into token_tree_verification_amd/libtv.so."""
    import tempfile
    from concurrent.futures import ThreadPoolExecutor

    tmp = LIB + f".tmp{os.getpid()}"
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="tv_build_") as d:
        def compile_one(src):
            obj = os.path.join(d, os.path.basename(src) + ".o")
            cmd = ["hipcc", *compile_flags, *FILE_FLAGS.get(os.path.basename(src), []), "-I", INCLUDE, "-I", CSRC,
                   "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            return obj, subprocess.run(cmd, capture_output=True, text=True)

        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(compile_one, sources()))
        objs = []
        for obj, res in results:
            err = "\n".join(l for l in (res.stderr or "").splitlines() if "packed-fp32-ops" not in l)
            if res.returncode != 0:
                raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
            objs.append(obj)
        cmd = ["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc link failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


def build_probe(verbose: bool = False) -> str:
    """Compile the measurement probes (plain streaming-read and MFMA-loop
    kernels) into token_tree_verification_amd/libtv_probe.so."""
    tmp = PROBE_LIB + f".tmp{os.getpid()}"
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", INCLUDE, PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        err = "\n".join(l for l in (res.stderr or "").splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose=True))
