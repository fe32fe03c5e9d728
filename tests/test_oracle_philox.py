"""Pins of the oracle's Philox-4x32-10 (written from Salmon et al., SC'11)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")
def test_matches_rocrand_philox_engine():
    """rocRAND's Philox-4x32-10 engine (a library routine, run host-side)
    must give the same 128-bit block for the same key and counter."""
    rng = np.random.default_rng(0)
    n = 4000
    seeds = rng.integers(0, 2 ** 63, size=n, dtype=np.uint64)
    seeds[:4] = [0, 1, 2 ** 32, 2 ** 63 - 1]
    node = rng.integers(0, 2 ** 32, size=n, dtype=np.uint64).astype(np.uint32)
    # rocRAND's 64-bit offset holds 4 * ((seq << 32) | node), so seq < 2^30 here
    seq = rng.integers(0, 2 ** 30, size=n, dtype=np.uint64).astype(np.uint32)
    purpose = rng.integers(0, 3, size=n).astype(np.uint32)
    node[:100] = np.arange(100)
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "ref")
        subprocess.check_call(["hipcc", "-O1", "-w", os.path.join(HERE, "philox_rocrand_ref.cpp"), "-o", exe],
                              stderr=subprocess.DEVNULL)
        text = "".join(f"{int(s)} {int(a)} {int(b)} {int(c)}\n" for s, a, b, c in zip(seeds, node, seq, purpose))
        res = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(x) for x in l.split()] for l in res.strip().splitlines()], dtype=np.uint32)
    ctr = np.stack([node, seq, purpose, np.zeros(n, np.uint32)], 1)
    key = np.stack([(seeds & 0xFFFFFFFF).astype(np.uint32), (seeds >> np.uint64(32)).astype(np.uint32)], 1)
    got = oracle.philox4x32_10(ctr, key)
    assert np.array_equal(got, ref)
    # uniform = first word >> 8, scaled by 2^-24
    u = oracle.uniforms(int(seeds[5]), [[node[5], seq[5], purpose[5]]])[0]
    assert u == (int(ref[5, 0]) >> 8) / 2 ** 24


def test_uniformity_chi_square():
    n = 1 << 20
    idx = np.arange(n, dtype=np.uint32)
    triples = np.stack([idx % 64, idx // 64, np.zeros(n, np.uint32)], 1)
    u = oracle.uniforms(12345, triples)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))  # 24-bit grid
    counts = np.bincount(np.floor(u * 1024).astype(int), minlength=1024)
    e = n / 1024
    chi2 = ((counts - e) ** 2 / e).sum()
    assert chi2 < 1168.0  # 1023 dof, p > 0.001
    # serial pairs (u_i, u_{i+1}) over a 32x32 grid
    a = np.floor(u[0::2] * 32).astype(int) * 32 + np.floor(u[1::2] * 32).astype(int)
    c2 = np.bincount(a, minlength=1024)
    e2 = (n // 2) / 1024
    assert ((c2 - e2) ** 2 / e2).sum() < 1168.0


def test_distinct_purposes_and_sequences_decorrelate():
    base = oracle.uniforms(7, [[i, 0, 0] for i in range(4096)])
    other = [oracle.uniforms(7, [[i, 0, 1] for i in range(4096)]),
             oracle.uniforms(7, [[i, 1, 0] for i in range(4096)]),
             oracle.uniforms(8, [[i, 0, 0] for i in range(4096)])]
    for o in other:
        assert abs(np.corrcoef(base, o)[0, 1]) < 0.06
        assert not np.array_equal(base, o)
