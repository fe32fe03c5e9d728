"""Static checks on the gfx950 code of every libtv kernel and of the
measurement probes (CPU only; hipcc cross-compiles):

* no kernel reads the dispatch packet (it lives in host memory; a compiler
  that promotes dynamically indexed private arrays to LDS reads the
  workgroup size from it, costing microseconds per launch);
* no kernel spills to scratch;
* no scalar-cache store, atomic or write-back anywhere.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "token_tree_verification_amd", "csrc")


def _asm(src, d):
    from token_tree_verification_amd import build as tvbuild
    flags = [f for f in tvbuild.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    out = os.path.join(d, os.path.basename(src) + ".s")
    subprocess.check_call(["hipcc", *flags, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--offload-device-only",
                           "-S", "-o", out, src], stderr=subprocess.DEVNULL)
    return open(out).read()


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_kernel_resources():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    srcs.append(os.path.join(ROOT, "token_tree_verification_amd", "probe", "tv_probe.hip"))
    with tempfile.TemporaryDirectory() as d:
        for src in srcs:
            text = _asm(src, d)
            assert not re.search(r"^\s+s_(store|atomic|buffer_store|buffer_atomic|scratch_store|dcache_wb)", text,
                                 re.M), f"scalar-cache write in {src}"
            for name, body in re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
                assert re.search(r"\.amdhsa_user_sgpr_dispatch_ptr 0", body), f"{name} reads the dispatch packet"
                assert re.search(r"\.amdhsa_private_segment_fixed_size 0\b", body), f"{name} uses scratch"
