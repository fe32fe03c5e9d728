"""The C ABI library loads and exports every symbol include/tv.h declares;
host-side argument checks return their documented status without any device
work (CPU only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import token_tree_verification_amd as tv
    if not os.path.exists(tv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return tv.library()


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("tv_build_tree_mask", "tv_tree_attention", "tv_spec_accept", "tv_tree_attention_workspace",
              "tv_spec_accept_workspace", "tv_status_string", "tv_version", "tv_philox_uniforms",
              "tv_build_tree_mask_ex", "tv_tree_attention_ex", "tv_spec_accept_ex", "tv_spec_accept_plan",
              "tv_set_wait_limit"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert lib.tv_status_string(s)
    assert lib.tv_version() >= 100


def test_workspace_queries(lib):
    assert lib.tv_tree_attention_workspace(1, 6, 32, 8, 128, 4096) > 0
    assert lib.tv_tree_attention_workspace(64, 64, 64, 8, 128, 8192) == 0  # one split: no partials
    assert lib.tv_tree_attention_workspace(1, 6, 32, 8, 64, 4096) == 0     # unsupported head dim
    # the accept plan depends on the device's resident capacity: invalid shapes give 0 anywhere
    assert lib.tv_spec_accept_workspace(0, 6, 128256, 1) == 0
    assert lib.tv_spec_accept_workspace(1, 257, 128256, 0) == 0
    assert lib.tv_spec_accept_workspace(1, 6, 0, 0) == 0


def _attn(lib, **kw):
    a = dict(Q=1, Kc=1, Vc=1, Kt=1, Vt=1, anc=1, out=1, B=1, N=6, Hq=32, Hkv=8, D=128, L=16, scale=0.088,
             ws=None, wsb=0)
    a.update(kw)
    P = lambda v: ctypes.c_void_p(v) if v else None
    return lib.tv_tree_attention(P(a["Q"]), P(a["Kc"]), P(a["Vc"]), P(a["Kt"]), P(a["Vt"]), P(a["anc"]), P(a["out"]),
                                 a["B"], a["N"], a["Hq"], a["Hkv"], a["D"], a["L"], a["scale"], P(a["ws"]), a["wsb"],
                                 None)


def test_attention_host_validation(lib):
    assert _attn(lib, B=-1) == -1
    assert _attn(lib, N=0) == -1
    assert _attn(lib, Hq=30, Hkv=8) == -1
    assert _attn(lib, L=-2) == -1
    assert _attn(lib, N=257) == -2
    assert _attn(lib, D=64) == -2
    assert _attn(lib, scale=float("nan")) == -1
    assert _attn(lib, B=0) == 0
    assert _attn(lib, Q=0) == -1
    assert _attn(lib, Kc=0) == -1
    assert _attn(lib, Q=8) == -1  # misaligned pointer
    assert _attn(lib, L=4096, Q=256, Kc=256, Vc=256, Kt=256, Vt=256, anc=256, out=256) == -4  # no workspace


def _acc(lib, **kw):
    a = dict(q=256, p=256, d=256, par=256, B=1, N=6, V=100, seed=0, T=1.0, greedy=0, al=256, an=256, ot=256,
             ws=None, wsb=0)
    a.update(kw)
    P = lambda v: ctypes.c_void_p(v) if v else None
    return lib.tv_spec_accept(P(a["q"]), P(a["p"]), P(a["d"]), P(a["par"]), a["B"], a["N"], a["V"], a["seed"], a["T"],
                              a["greedy"], P(a["al"]), P(a["an"]), P(a["ot"]), P(a["ws"]), a["wsb"], None)


def test_accept_host_validation(lib):
    assert _acc(lib, B=-1) == -1
    assert _acc(lib, V=0) == -1
    assert _acc(lib, N=257) == -2
    assert _acc(lib, T=0.0) == -1
    assert _acc(lib, T=float("nan")) == -1
    assert _acc(lib, T=float("inf")) == -1
    assert _acc(lib, p=0) == -1
    assert _acc(lib, B=0) == 0
    assert _acc(lib) == -4  # no workspace
    # greedy ignores temperature and p
    assert _acc(lib, greedy=1, T=0.0, p=0) == -4


def test_accept_ex_host_validation(lib):
    P = ctypes.c_void_p
    lib.tv_spec_accept_ex.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                      ctypes.c_float, ctypes.c_int, P, P, P, P, ctypes.c_size_t, P]
    call = lambda flags, sn=None: lib.tv_spec_accept_ex(P(256), P(256), P(256), P(256), sn, 1, 6, 100, 0, 1.0, flags,
                                                        P(256), P(256), P(256), None, 0, None)
    assert call(4) == -1          # unknown flag
    assert call(3) == -4          # greedy | without replacement: valid, no workspace
    assert call(2, P(256)) == -4  # ragged, without replacement
    lib.tv_set_wait_limit.argtypes = [ctypes.c_uint32]
    lib.tv_set_wait_limit.restype = ctypes.c_uint32
    prev = lib.tv_set_wait_limit(5)
    assert lib.tv_set_wait_limit(0xFFFFFFFF) == 5
    assert lib.tv_set_wait_limit(0xFFFFFFFF) == prev


def test_mask_host_validation(lib):
    P = ctypes.c_void_p
    assert lib.tv_build_tree_mask(P(256), 1, 0, P(256), P(256), None, None) == -1
    assert lib.tv_build_tree_mask(P(256), 1, 257, P(256), P(256), None, None) == -2
    assert lib.tv_build_tree_mask(None, 1, 4, P(256), P(256), None, None) == -1
    assert lib.tv_build_tree_mask(P(256), 0, 4, P(256), P(256), None, None) == 0


def test_python_binding_rejects_host_tensors():
    import torch
    import token_tree_verification_amd as tv
    with pytest.raises(ValueError):
        tv.build_tree_mask(torch.zeros((1, 3), dtype=torch.int32))
    with pytest.raises(TypeError):
        tv.build_tree_mask(torch.zeros((1, 3), dtype=torch.int64))


PROBE_HEADER = os.path.join(ROOT, "include", "tv_probe.h")


@pytest.fixture(scope="module")
def probe():
    path = os.path.join(ROOT, "token_tree_verification_amd", "libtv_probe.so")
    if not os.path.exists(path):
        from token_tree_verification_amd import build as tvbuild
        tvbuild.build_probe()
    return ctypes.CDLL(path)


def test_probe_library_exports_its_header(probe):
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(tv_probe_[a-z_0-9]+)\s*\(", text)))
    assert names == ["tv_probe_mfma_loop", "tv_probe_mfma_loop_flops", "tv_probe_stream_read"]
    for name in names:
        assert hasattr(probe, name), name


def test_probe_host_checks(probe):
    probe.tv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_void_p]
    probe.tv_probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe.tv_probe_mfma_loop_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    probe.tv_probe_mfma_loop_flops.restype = ctypes.c_double
    for nt in (0, 1):
        assert probe.tv_probe_stream_read(None, 1 << 20, nt, 16, 8, None) == -1    # null source
        assert probe.tv_probe_stream_read(16, 8, nt, 16, 8, None) == -1            # fewer than 16 bytes
        assert probe.tv_probe_stream_read(24, 1 << 20, nt, 16, 8, None) == -1      # misaligned source
        assert probe.tv_probe_stream_read(16, 1 << 20, nt, 16, 0, None) == -1      # no workgroups
    for rnd in (0, 1):
        assert probe.tv_probe_mfma_loop(0, 8, rnd, 16, None) == -1
        assert probe.tv_probe_mfma_loop(8, 0, rnd, 16, None) == -1
        assert probe.tv_probe_mfma_loop(8, 8, rnd, None, None) == -1
    # 32 x 32 x 16 multiply-adds per MFMA, four chains, four waves per workgroup
    assert probe.tv_probe_mfma_loop_flops(3, 5) == 2 * 32 * 32 * 16 * 4 * 5 * 4 * 3
