"""The allocation-free accept call (static per-GPU scratch) against the call
with a caller workspace, through the C ABI: bit-identical outputs on two calls
in a row, the second on a smaller input, in greedy, sampling and
without-replacement modes; shapes beyond the scratch are refused up front."""
import ctypes

import numpy as np
import pytest
import torch

from workloads import CONFIGS, Workload, accept_inputs

pytestmark = pytest.mark.gpu

P = ctypes.c_void_p


@pytest.fixture(scope="module")
def lib():
    import token_tree_verification_amd as tv
    lib = tv.library()
    lib.tv_spec_accept_noalloc.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                           ctypes.c_float, ctypes.c_int, P, P, P, P]
    lib.tv_spec_accept_noalloc.restype = ctypes.c_int
    return lib


def _ptr(t):
    return None if t is None else P(t.data_ptr())


def _outputs(B, N, dev):
    return (torch.full((B,), -9, dtype=torch.int32, device=dev), torch.full((B, N), -9, dtype=torch.int32, device=dev),
            torch.full((B, N), -9, dtype=torch.int32, device=dev))


def _call(lib, fn, q, p, draft, parent, seed, T, flags, ws=None):
    B, N, V = q.shape
    dev = q.device
    outs = _outputs(B, N, dev)
    stream = P(torch.cuda.current_stream(dev).cuda_stream)
    common = (_ptr(q), _ptr(p), _ptr(draft), _ptr(parent), None, B, N, V, seed, T, flags, *(_ptr(o) for o in outs))
    if fn == "noalloc":
        rc = lib.tv_spec_accept_noalloc(*common, stream)
    else:
        rc = lib.tv_spec_accept_ex(*common, _ptr(ws), ws.numel(), stream)
    assert rc == 0, rc
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def test_noalloc_matches_workspace_call(lib):
    import token_tree_verification_amd as tv
    dev = torch.device("cuda:0")
    big = CONFIGS["c3"]
    small = Workload("small", B=3, N=17, Hq=1, Hkv=1, D=128, L=1, V=5003, sigma_q=3.0, sigma_n=1.0,
                     temperatures=(0.8,), tree="random", max_depth=5, data_seed=31)
    for flags in (0, 1, 2):  # sampling, greedy, siblings without replacement
        for w in (big, small):  # two calls in a row, the second smaller
            q, p, draft, parent = accept_inputs(w, device=dev)
            ws = torch.zeros(tv.accept_workspace_bytes(w.B, w.N, w.V, flags & 1), dtype=torch.uint8, device=dev)
            for seed in (0, 7):
                want = _call(lib, "ex", q, p, draft, parent, seed, 0.8, flags, ws)
                got = _call(lib, "noalloc", q, p, draft, parent, seed, 0.8, flags)
                for a, b in zip(want, got):
                    assert np.array_equal(a, b), (flags, w.name, seed)
                assert (got[0] >= 0).all()


def test_noalloc_refuses_shapes_beyond_its_scratch(lib):
    """256 sequences of 256-node trees in sampling mode plan 8.1 MiB of team
    statistics and walk records, more than the 4 MiB scratch: refused before
    anything is enqueued; the same shape in greedy mode fits and runs."""
    import token_tree_verification_amd as tv
    B, N, V = 256, 256, 1000
    assert tv.accept_workspace_bytes(B, N, V, False) > 4 << 20
    assert tv.accept_workspace_bytes(B, N, V, True) <= 4 << 20
    x = torch.zeros(16, dtype=torch.float32, device="cuda:0")
    rc = lib.tv_spec_accept_noalloc(_ptr(x), _ptr(x), _ptr(x), _ptr(x), None, B, N, V, 0, 1.0, 0,
                                    _ptr(x), _ptr(x), _ptr(x), None)
    assert rc == -6
    assert "scratch" in lib.tv_status_string(-6).decode()
    w = Workload("fits", B=B, N=N, Hq=1, Hkv=1, D=128, L=1, V=V, sigma_q=3.0, sigma_n=1.0, temperatures=(1.0,),
                 tree="random", max_depth=9, data_seed=3)
    q, p, draft, parent = accept_inputs(w, device="cuda:0")
    ws = torch.zeros(tv.accept_workspace_bytes(B, N, V, True), dtype=torch.uint8, device="cuda:0")
    want = _call(lib, "ex", q, None, draft, parent, 0, 1.0, 1, ws)
    got = _call(lib, "noalloc", q, None, draft, parent, 0, 1.0, 1)
    for a, b in zip(want, got):
        assert np.array_equal(a, b)


_FIRST_CALL_CAPTURED = r'''
import ctypes, sys
import numpy as np
import torch
sys.path[:0] = [ROOT, ROOT + "/tests"]
import token_tree_verification_amd as tv
from workloads import CONFIGS, accept_inputs
P = ctypes.c_void_p
lib = tv.library()
lib.tv_spec_accept_noalloc.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                       ctypes.c_float, ctypes.c_int, P, P, P, P]
lib.tv_spec_accept_noalloc.restype = ctypes.c_int
dev = torch.device("cuda:0")
w = CONFIGS["c3"]
s = torch.cuda.Stream(dev)
with torch.cuda.stream(s):
    batches = [accept_inputs(w, device=dev, seed=seed) for seed in (101, 102, 103)]
    q, p, draft, parent = (t.clone() for t in batches[0])
    outs = [torch.full((w.B,), -9, dtype=torch.int32, device=dev),
            torch.full((w.B, w.N), -9, dtype=torch.int32, device=dev),
            torch.full((w.B, w.N), -9, dtype=torch.int32, device=dev)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):  # the process's first call of the entry point
        rc = lib.tv_spec_accept_noalloc(P(q.data_ptr()), P(p.data_ptr()), P(draft.data_ptr()), P(parent.data_ptr()),
                                        None, w.B, w.N, w.V, 7, 0.7, 0, *(P(o.data_ptr()) for o in outs),
                                        P(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, rc
    for rep in range(6):
        for dst, src in zip((q, p, draft, parent), batches[rep % 3]):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        got = [o.cpu().numpy().copy() for o in outs]
        a, n, t = tv.spec_accept(q, p, draft, parent, seed=7, temperature=0.7)
        torch.cuda.synchronize()
        for x, y in zip(got, (a, n, t)):
            assert np.array_equal(x, y.cpu().numpy()), f"replay {rep} differs from the workspace call"
print("first-call-captured ok")
'''


@pytest.mark.timeout(300)
def test_noalloc_first_call_captured_in_a_graph():
    """In a fresh process the first call of the entry point (which puts the
    scratch's control words in order) is captured into a HIP graph; replays
    with new inputs in the same buffers match the workspace call every time."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = f"ROOT = {root!r}\n" + _FIRST_CALL_CAPTURED
    res = subprocess.run([sys.executable, "-u", "-c", code], capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "first-call-captured ok" in res.stdout
