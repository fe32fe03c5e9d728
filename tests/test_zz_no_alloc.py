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
