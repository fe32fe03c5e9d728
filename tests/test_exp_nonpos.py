"""Accuracy of the library's fp64 exp for non-positive arguments (the
residual and draw passes of the accept walk use it), checked on the CPU
against the C library's exp."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_exp_nonpos_relative_error():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "expcheck")
        subprocess.check_call(["hipcc", "-O2", "-w", "-I", os.path.join(ROOT, "token_tree_verification_amd", "csrc"),
                               "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "exp_nonpos_check.cpp"), "-o",
                               exe], stderr=subprocess.DEVNULL)
        worst = float(subprocess.check_output([exe], text=True).split()[0])
    assert worst < 1e-14
