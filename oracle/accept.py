"""ctypes front end of the C accept/reject oracle (test infrastructure only).

The arithmetic lives in ``oracle/csrc/accept_oracle.c`` (plain C, fp64); this
module only builds it with gcc when needed and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csrc", "accept_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build_liboracle(force: bool = False) -> str:
    """Compile the C oracle with gcc into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build_liboracle())
        P = ctypes.c_void_p
        lib.orc_philox4x32_10.argtypes = [P, P, P]
        lib.orc_philox4x32_10.restype = None
        lib.orc_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        lib.orc_uniform.restype = ctypes.c_double
        lib.orc_philox_batch.argtypes = [P, P, ctypes.c_int64, P]
        lib.orc_philox_batch.restype = None
        lib.orc_uniform_batch.argtypes = [ctypes.c_uint64, P, ctypes.c_int64, P]
        lib.orc_uniform_batch.restype = None
        lib.orc_spec_accept.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                        ctypes.c_double, ctypes.c_int, ctypes.c_int, P, P, P, P, P]
        lib.orc_spec_accept.restype = ctypes.c_int
        lib.orc_spec_accept_ex.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                           ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint32,
                                           P, P, P, P, P]
        lib.orc_spec_accept_ex.restype = ctypes.c_int
        lib.orc_lossless_trials.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_uint64,
                                            ctypes.c_int64, ctypes.c_int, ctypes.c_int, P, P, P, P]
        lib.orc_lossless_trials.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def philox4x32_10(counters, keys):
    """Raw Philox-4x32-10 blocks.  counters uint32 [n,4], keys uint32 [n,2] -> uint32 [n,4]."""
    c = np.ascontiguousarray(counters, dtype=np.uint32).reshape(-1, 4)
    k = np.ascontiguousarray(keys, dtype=np.uint32).reshape(-1, 2)
    out = np.empty_like(c)
    _load().orc_philox_batch(_ptr(c), _ptr(k), c.shape[0], _ptr(out))
    return out


def uniform(seed: int, node: int, seq: int, purpose: int) -> float:
    return _load().orc_uniform(seed, node, seq, purpose)


def uniforms(seed: int, triples) -> np.ndarray:
    """U(seed, node, seq, purpose) for each row (node, seq, purpose) of ``triples``."""
    t = np.ascontiguousarray(triples, dtype=np.uint32).reshape(-1, 3)
    out = np.empty(t.shape[0], dtype=np.float64)
    _load().orc_uniform_batch(seed, _ptr(t), t.shape[0], _ptr(out))
    return out


def spec_accept(q_logits, p_logits, draft, parent, seed=0, temperature=1.0, greedy=False, variant=0,
                seq_nodes=None, wor=False, seq_offset=0):
    """Accept/reject walk for every sequence.

    q_logits, p_logits: float32 [B,N,V] (p may be None when greedy); draft,
    parent: int32 [B,N].  seq_nodes: optional int [B], nodes of each sequence
    (the others are padding).  wor: siblings drawn without replacement from
    the draft row of their parent (p row u belongs to node u's children).
    seq_offset: Philox sequence counter of batch entry 0.  Returns
    dict(accept_len [B], accepted_nodes [B,N], out_tokens [B,N], flags [B],
    margin [B]).
    """
    q = np.ascontiguousarray(q_logits, dtype=np.float32)
    B, N, V = q.shape
    p = None if p_logits is None else np.ascontiguousarray(p_logits, dtype=np.float32)
    d = np.ascontiguousarray(draft, dtype=np.int32)
    par = np.ascontiguousarray(parent, dtype=np.int32)
    sn = None if seq_nodes is None else np.ascontiguousarray(seq_nodes, dtype=np.int32)
    acc_len = np.zeros(B, np.int32)
    acc_nodes = np.zeros((B, N), np.int32)
    toks = np.zeros((B, N), np.int32)
    flags = np.zeros(B, np.int32)
    margin = np.zeros(B, np.float64)
    rc = _load().orc_spec_accept_ex(_ptr(q), _ptr(p), _ptr(d), _ptr(par), _ptr(sn), B, N, V, int(seed),
                                    float(temperature), int(bool(greedy)), int(variant), int(bool(wor)),
                                    int(seq_offset) & 0xFFFFFFFF, _ptr(acc_len), _ptr(acc_nodes), _ptr(toks),
                                    _ptr(flags), _ptr(margin))
    if rc != 0:
        raise ValueError(f"oracle spec_accept rejected its input (status {rc})")
    return dict(accept_len=acc_len, accepted_nodes=acc_nodes, out_tokens=toks, flags=flags, margin=margin)


def lossless_trials(q_logits, p_logits, parent, temperature, seed0, ntrials, variant=0, draft_mode=0):
    """Run the walk for ``ntrials`` consecutive Philox seeds on one sequence with
    freshly drawn drafts (draft_mode 0: x_c ~ P_p(c); 1: argmax p_c; 2: the
    children of u drawn from P_p(u) without replacement, walked in that mode;
    3: drawn from P_p(u) with replacement, walked in the without-replacement
    mode)."""
    q = np.ascontiguousarray(q_logits, dtype=np.float32)
    N, V = q.shape
    p = np.ascontiguousarray(p_logits, dtype=np.float32)
    par = np.ascontiguousarray(parent, dtype=np.int32)
    drafts = np.zeros((ntrials, N), np.int32)
    acc_len = np.zeros(ntrials, np.int32)
    acc = np.zeros((ntrials, N), np.int32)
    toks = np.zeros((ntrials, N), np.int32)
    rc = _load().orc_lossless_trials(_ptr(q), _ptr(p), _ptr(par), N, V, float(temperature), int(seed0),
                                     int(ntrials), int(variant), int(draft_mode), _ptr(drafts), _ptr(acc_len),
                                     _ptr(acc), _ptr(toks))
    if rc != 0:
        raise ValueError(f"oracle lossless_trials rejected its input (status {rc})")
    return dict(drafts=drafts, accept_len=acc_len, accepted=acc, tokens=toks)
