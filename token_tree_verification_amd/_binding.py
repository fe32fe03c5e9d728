"""ctypes binding of libtv.so: argument checking and marshalling only.

Every step of the verification path runs in the HIP kernels behind the C ABI
declared in include/tv.h; this module checks tensor shapes, dtypes and
devices, allocates outputs and workspaces with torch (device memory only),
and passes raw pointers plus the current HIP stream.  There is no CPU
fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtv.so")

TV_OK = 0
_lib = None


class TVError(RuntimeError):
    def __init__(self, func: str, status: int):
        msg = _load().tv_status_string(status).decode()
        super().__init__(f"{func} failed with status {status}: {msg}")
        self.status = status


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libtv.so is not built ({LIB_PATH}); run __graft_entry__.build() "
                           "or python token_tree_verification_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, U64, SZ, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_float
    lib.tv_status_string.argtypes = [I]
    lib.tv_status_string.restype = ctypes.c_char_p
    lib.tv_version.argtypes = []
    lib.tv_version.restype = I
    lib.tv_build_tree_mask.argtypes = [P, I, I, P, P, P, P]
    lib.tv_build_tree_mask.restype = I
    lib.tv_build_tree_mask_ex.argtypes = [P, P, I, I, P, P, P, P]
    lib.tv_build_tree_mask_ex.restype = I
    lib.tv_tree_attention_workspace.argtypes = [I, I, I, I, I, I]
    lib.tv_tree_attention_workspace.restype = SZ
    lib.tv_tree_attention.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, SZ, P]
    lib.tv_tree_attention.restype = I
    lib.tv_tree_attention_ex.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, F, P, SZ, P]
    lib.tv_tree_attention_ex.restype = I
    lib.tv_spec_accept_workspace.argtypes = [I, I, I, I]
    lib.tv_spec_accept_workspace.restype = SZ
    lib.tv_spec_accept.argtypes = [P, P, P, P, I, I, I, U64, F, I, P, P, P, P, SZ, P]
    lib.tv_spec_accept.restype = I
    lib.tv_spec_accept_ex.argtypes = [P, P, P, P, P, I, I, I, U64, F, I, P, P, P, P, SZ, P]
    lib.tv_spec_accept_ex.restype = I
    lib.tv_spec_accept_plan.argtypes = [I, I, I, I, P, P, P]
    lib.tv_spec_accept_plan.restype = I
    lib.tv_set_wait_limit.argtypes = [ctypes.c_uint32]
    lib.tv_set_wait_limit.restype = ctypes.c_uint32
    lib.tv_commit_kv.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, P]
    lib.tv_commit_kv.restype = I
    lib.tv_tree_expand.argtypes = [P, P, P, I, I, I, I, F, P, P, P, I, I, P, I, P]
    lib.tv_tree_expand.restype = I
    lib.tv_tree_select.argtypes = [P, P, P, I, I, I, I, P, P, P, P, P]
    lib.tv_tree_select.restype = I
    lib.tv_philox_uniforms.argtypes = [U64, P, I, P, P, P]
    lib.tv_philox_uniforms.restype = I
    _lib = lib
    return lib


def library():
    """The loaded ctypes handle of libtv.so (raises if it is not built)."""
    return _load()


def _check(func, status):
    if status != TV_OK:
        raise TVError(func, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: int, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    """Caller-supplied workspace, or a fresh zero-filled one (the accept call
    keeps its control words in the workspace and needs them zero at first use)."""
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.device != device or workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace must hold {nbytes} bytes on {device}")
        return workspace
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


TV_MAX_NODES = 256
ACCEPT_GREEDY = 1
ACCEPT_SIBLINGS_WOR = 2
WAIT_DEFAULT = 0xFFFFFFFF


def mask_words(N: int) -> int:
    return (N + 63) // 64


def _seq_array(t: Optional[torch.Tensor], name: str, B: int, dev):
    if t is None:
        return None
    _need(t, name, torch.int32, 1, dev)
    if t.shape[0] != B:
        raise ValueError(f"{name} must be [B]")
    return t


def build_tree_mask(parent: torch.Tensor, seq_nodes: Optional[torch.Tensor] = None):
    """parent int32 [B,N] (seq_nodes: optional int32 [B] nodes per sequence) ->
    (anc_mask int64 [B,N,W] holding the uint64 ancestor words, W = ceil(N/64),
    depth int32 [B,N], seq_status int32 [B])."""
    _need(parent, "parent", torch.int32, 2)
    B, N = parent.shape
    dev = parent.device
    sn = _seq_array(seq_nodes, "seq_nodes", B, dev)
    anc = torch.empty((B, N, mask_words(N)), dtype=torch.int64, device=dev)
    depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check("tv_build_tree_mask_ex",
           _load().tv_build_tree_mask_ex(_ptr(parent), _ptr(sn), B, N, _ptr(anc), _ptr(depth), _ptr(status),
                                         _stream(dev)))
    return anc, depth, status


def attention_workspace_bytes(B, N, Hq, Hkv, D, L) -> int:
    return int(_load().tv_tree_attention_workspace(B, N, Hq, Hkv, D, L))


def tree_attention(Q, K_cache, V_cache, K_tree, V_tree, anc_mask, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                   seq_nodes: Optional[torch.Tensor] = None, seq_len: Optional[torch.Tensor] = None):
    """Q bf16 [B,N,Hq,D]; K/V_cache bf16 [B,Hkv,L,D]; K/V_tree bf16 [B,N,Hkv,D];
    anc_mask int64 [B,N,W] (or [B,N] when N <= 64); optional seq_nodes,
    seq_len int32 [B] for ragged batches -> out fp32 [B,N,Hq,D]."""
    _need(Q, "Q", torch.bfloat16, 4)
    dev = Q.device
    B, N, Hq, D = Q.shape
    for name, t in (("K_cache", K_cache), ("V_cache", V_cache), ("K_tree", K_tree), ("V_tree", V_tree)):
        _need(t, name, torch.bfloat16, 4, dev)
    if anc_mask.dim() == 2:
        anc_mask = anc_mask.unsqueeze(-1)
    _need(anc_mask, "anc_mask", torch.int64, 3, dev)
    Hkv, L = K_cache.shape[1], K_cache.shape[2]
    if tuple(K_cache.shape) != (B, Hkv, L, D) or tuple(V_cache.shape) != (B, Hkv, L, D):
        raise ValueError("K_cache/V_cache must be [B,Hkv,L,D]")
    if tuple(K_tree.shape) != (B, N, Hkv, D) or tuple(V_tree.shape) != (B, N, Hkv, D):
        raise ValueError("K_tree/V_tree must be [B,N,Hkv,D]")
    if tuple(anc_mask.shape) != (B, N, mask_words(N)):
        raise ValueError("anc_mask must be [B,N,ceil(N/64)]")
    sn = _seq_array(seq_nodes, "seq_nodes", B, dev)
    sl = _seq_array(seq_len, "seq_len", B, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", torch.float32, 4, dev)
        if tuple(out.shape) != (B, N, Hq, D):
            raise ValueError("out must be [B,N,Hq,D]")
    ws = _workspace(attention_workspace_bytes(B, N, Hq, Hkv, D, L), dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("tv_tree_attention_ex",
           _load().tv_tree_attention_ex(_ptr(Q), _ptr(K_cache), _ptr(V_cache), _ptr(K_tree), _ptr(V_tree),
                                        _ptr(anc_mask), _ptr(out), _ptr(sn), _ptr(sl), B, N, Hq, Hkv, D, L,
                                        float(scale), _ptr(ws), nbytes, _stream(dev)))
    return out


def accept_workspace_bytes(B, N, V, greedy) -> int:
    return int(_load().tv_spec_accept_workspace(B, N, V, int(bool(greedy))))


def accept_plan(B, N, V, greedy):
    """(team size, teams, slice length) that the accept call plans on the current device."""
    w, t, sl = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check("tv_spec_accept_plan", _load().tv_spec_accept_plan(B, N, V, int(bool(greedy)), ctypes.byref(w),
                                                               ctypes.byref(t), ctypes.byref(sl)))
    return w.value, t.value, sl.value


def set_wait_limit(polls: int) -> int:
    """Polls each team wait of later accept calls makes (WAIT_DEFAULT restores
    the default); returns the previous setting.  For tests and diagnostics."""
    return int(_load().tv_set_wait_limit(int(polls) & 0xFFFFFFFF))


def spec_accept(q_logits, p_logits, draft_tokens, parent, seed: int = 0, temperature: float = 1.0,
                greedy: bool = False, workspace: Optional[torch.Tensor] = None, outputs=None,
                seq_nodes: Optional[torch.Tensor] = None, wor: bool = False):
    """q_logits/p_logits fp32 [B,N,V] (p may be None when greedy); draft_tokens,
    parent int32 [B,N]; optional seq_nodes int32 [B]; wor: siblings drawn
    without replacement (p row u is the draft row at node u) ->
    (accept_len int32 [B], accepted_nodes int32 [B,N], out_tokens int32 [B,N])."""
    _need(q_logits, "q_logits", torch.float32, 3)
    dev = q_logits.device
    B, N, V = q_logits.shape
    if not greedy or p_logits is not None:
        _need(p_logits, "p_logits", torch.float32, 3, dev)
        if tuple(p_logits.shape) != (B, N, V):
            raise ValueError("p_logits must be [B,N,V]")
    _need(draft_tokens, "draft_tokens", torch.int32, 2, dev)
    _need(parent, "parent", torch.int32, 2, dev)
    if tuple(draft_tokens.shape) != (B, N) or tuple(parent.shape) != (B, N):
        raise ValueError("draft_tokens and parent must be [B,N]")
    sn = _seq_array(seq_nodes, "seq_nodes", B, dev)
    if outputs is None:
        acc_len = torch.empty((B,), dtype=torch.int32, device=dev)
        acc_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
        toks = torch.empty((B, N), dtype=torch.int32, device=dev)
    else:
        acc_len, acc_nodes, toks = outputs
    flags = (ACCEPT_GREEDY if greedy else 0) | (ACCEPT_SIBLINGS_WOR if wor else 0)
    ws = _workspace(accept_workspace_bytes(B, N, V, greedy), dev, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("tv_spec_accept_ex",
           _load().tv_spec_accept_ex(_ptr(q_logits), _ptr(p_logits), _ptr(draft_tokens), _ptr(parent), _ptr(sn), B,
                                     N, V, int(seed) & 0xFFFFFFFFFFFFFFFF, float(temperature), flags, _ptr(acc_len),
                                     _ptr(acc_nodes), _ptr(toks), _ptr(ws), nbytes, _stream(dev)))
    return acc_len, acc_nodes, toks


def commit_kv(K_tree, V_tree, accept_len, accepted_nodes, cache_len, K_cache, V_cache):
    """Append each sequence's root and accepted path (K/V_tree bf16 [B,N,Hkv,D])
    to K/V_cache bf16 [B,Hkv,L,D] in place at its committed length
    (cache_len int32 [B]) -> (new_cache_len int32 [B], seq_status int32 [B])."""
    _need(K_tree, "K_tree", torch.bfloat16, 4)
    dev = K_tree.device
    B, N, Hkv, D = K_tree.shape
    _need(V_tree, "V_tree", torch.bfloat16, 4, dev)
    for name, t in (("K_cache", K_cache), ("V_cache", V_cache)):
        _need(t, name, torch.bfloat16, 4, dev)
    L = K_cache.shape[2]
    if tuple(V_tree.shape) != (B, N, Hkv, D) or tuple(K_cache.shape) != (B, Hkv, L, D) or \
            tuple(V_cache.shape) != (B, Hkv, L, D):
        raise ValueError("K/V_tree must be [B,N,Hkv,D] and K/V_cache [B,Hkv,L,D]")
    _need(accept_len, "accept_len", torch.int32, 1, dev)
    _need(accepted_nodes, "accepted_nodes", torch.int32, 2, dev)
    _need(cache_len, "cache_len", torch.int32, 1, dev)
    if accept_len.shape[0] != B or tuple(accepted_nodes.shape) != (B, N) or cache_len.shape[0] != B:
        raise ValueError("accept_len, cache_len must be [B] and accepted_nodes [B,N]")
    new_len = torch.empty((B,), dtype=torch.int32, device=dev)
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    _check("tv_commit_kv",
           _load().tv_commit_kv(_ptr(K_tree), _ptr(V_tree), _ptr(accept_len), _ptr(accepted_nodes), _ptr(cache_len),
                                _ptr(K_cache), _ptr(V_cache), _ptr(new_len), _ptr(status), B, N, Hkv, D, L,
                                _stream(dev)))
    return new_len, status


def tree_pool(B: int, P: int, device):
    """An empty node pool for dynamic tree construction: (value fp32 [B,P],
    parent int32 [B,P], token int32 [B,P])."""
    return (torch.full((B, P), float("-inf"), dtype=torch.float32, device=device),
            torch.full((B, P), -1, dtype=torch.int32, device=device),
            torch.full((B, P), -1, dtype=torch.int32, device=device))


def tree_expand(draft_logits, frontier, pool, pool_base: int, topk: int, n_next: int, temperature: float = 1.0,
                root_token: Optional[torch.Tensor] = None):
    """One expansion step (frontier None: the root).  draft_logits fp32 [B,F,V];
    pool from tree_pool(), updated in place -> next frontier int32 [B,n_next]."""
    _need(draft_logits, "draft_logits", torch.float32, 3)
    dev = draft_logits.device
    B, F, V = draft_logits.shape
    if frontier is not None:
        _need(frontier, "frontier", torch.int32, 2, dev)
        if tuple(frontier.shape) != (B, F):
            raise ValueError("frontier must be [B,F]")
    score, parent, token = pool
    Pn = score.shape[1]
    for name, t, dt in (("pool value", score, torch.float32), ("pool parent", parent, torch.int32),
                        ("pool token", token, torch.int32)):
        _need(t, name, dt, 2, dev)
        if tuple(t.shape) != (B, Pn):
            raise ValueError("pool arrays must be [B,P]")
    rt = _seq_array(root_token, "root_token", B, dev)
    nxt = torch.empty((B, n_next), dtype=torch.int32, device=dev)
    _check("tv_tree_expand",
           _load().tv_tree_expand(_ptr(draft_logits), _ptr(frontier), _ptr(rt), B, F, V, int(topk), float(temperature),
                                  _ptr(score), _ptr(parent), _ptr(token), Pn, int(pool_base),
                                  _ptr(nxt) if n_next else None, int(n_next), _stream(dev)))
    return nxt


def tree_select(pool, pool_count: int, M: int):
    """The root plus the M - 1 most valuable pool nodes, renumbered ->
    (parent int32 [B,M], tokens int32 [B,M], pool_index int32 [B,M],
    seq_nodes int32 [B])."""
    score, parent, token = pool
    dev = score.device
    B, Pn = score.shape
    outs = [torch.empty((B, M), dtype=torch.int32, device=dev) for _ in range(3)]
    nodes = torch.empty((B,), dtype=torch.int32, device=dev)
    _check("tv_tree_select",
           _load().tv_tree_select(_ptr(score), _ptr(parent), _ptr(token), B, Pn, int(pool_count), int(M),
                                  *(_ptr(o) for o in outs), _ptr(nodes), _stream(dev)))
    return outs[0], outs[1], outs[2], nodes


def philox_uniforms(seed: int, triples: torch.Tensor):
    """triples int32 [n,3] (node, sequence, purpose) on the device ->
    (uniforms fp32 [n], raw Philox blocks int32 [n,4] holding uint32 bits)."""
    _need(triples, "triples", torch.int32, 2)
    n = triples.shape[0]
    dev = triples.device
    u = torch.empty((n,), dtype=torch.float32, device=dev)
    raw = torch.empty((n, 4), dtype=torch.int32, device=dev)
    _check("tv_philox_uniforms",
           _load().tv_philox_uniforms(int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(triples), n, _ptr(u), _ptr(raw),
                                      _stream(dev)))
    return u, raw
