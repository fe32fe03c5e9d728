"""Seeded synthetic workloads for token-tree verification.

This module only draws random inputs (trees, bf16 attention tensors, fp32
logits, draft tokens).  It holds none of the verification arithmetic: the
tree mask, attention and accept/reject rule live in ``oracle/`` (CPU
reference) and in the HIP library, which share no code.  Both sides receive
the exact tensors produced here.

Shapes follow the pages' workloads: EAGLE's static draft tree of 60 nodes,
depth 6, at most 10 nodes per level (EAGLE explainer, section on static-tree
parallel verification); a K-token draft chain verified with K+1 target
distributions (speculative-decoding survey explainer, formal definition,
verification phase); EAGLE-2 style per-sequence dynamic trees (EAGLE-3
explainer, comparison with EAGLE-2); Vicuna/LLaMA/Qwen-sized heads and
vocabularies.  No benchmark dataset is used.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

# Static 60-node tree (root + 59 drafts), depth 6, level widths
# [1, 10, 10, 10, 10, 10, 9].  Nodes are numbered breadth first.  Level 1 hangs
# off the root; each deeper level gives 4 children to the previous level's
# first node, 3 to the second, 2 to the third and 1 to the fourth.
STATIC_TREE_60 = [
    -1,
    0, 0, 0, 0, 0, 0, 0, 0, 0, 0,
    1, 1, 1, 1, 2, 2, 2, 3, 3, 4,
    11, 11, 11, 11, 12, 12, 12, 13, 13, 14,
    21, 21, 21, 21, 22, 22, 22, 23, 23, 24,
    31, 31, 31, 31, 32, 32, 32, 33, 33, 34,
    41, 41, 41, 41, 42, 42, 42, 43, 43,
]


def static_tree_60() -> np.ndarray:
    return np.asarray(STATIC_TREE_60, dtype=np.int32)


def chain(n: int) -> np.ndarray:
    """Linear draft chain: root plus n-1 drafts, parent[i] = i-1."""
    return np.arange(-1, n - 1, dtype=np.int32)


def random_tree(n: int, max_depth: int, seed: int) -> np.ndarray:
    """EAGLE-2 style dynamic topology: each node's parent is drawn uniformly
    from the earlier nodes whose depth is below ``max_depth``."""
    rng = np.random.default_rng(seed)
    parent = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int32)
    for i in range(1, n):
        cand = np.nonzero(depth[:i] < max_depth)[0]
        p = int(cand[rng.integers(0, cand.size)])
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    L: int
    V: int
    sigma_q: float
    sigma_n: float
    temperatures: tuple  # sampling temperatures measured; 0.0 stands for greedy
    tree: str            # "static60" | "chain" | "random"
    max_depth: int = 8
    data_seed: int = 0
    philox_seed: int = 0

    def parents(self) -> np.ndarray:
        if self.tree == "static60":
            assert self.N == 60
            return np.tile(static_tree_60(), (self.B, 1))
        if self.tree == "chain":
            return np.tile(chain(self.N), (self.B, 1))
        if self.tree == "random":
            return np.stack([random_tree(self.N, self.max_depth, 2000 + b) for b in range(self.B)])
        raise ValueError(self.tree)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def describe(self) -> str:
        return (f"{self.name}: B={self.B} N={self.N} Hq/Hkv={self.Hq}/{self.Hkv} D={self.D} "
                f"L={self.L} V={self.V} tree={self.tree}")


# The five benchmark workloads.  temperature 0.0 = greedy mode.
CONFIGS = {
    "c1": Workload("c1", B=1, N=60, Hq=32, Hkv=32, D=128, L=512, V=32000, sigma_q=3.0, sigma_n=1.0,
                   temperatures=(1.0,), tree="static60", data_seed=1001),
    "c2": Workload("c2", B=1, N=6, Hq=32, Hkv=8, D=128, L=4096, V=128256, sigma_q=3.0, sigma_n=1.5,
                   temperatures=(0.0, 1.0), tree="chain", data_seed=1002),
    "c3": Workload("c3", B=16, N=60, Hq=40, Hkv=40, D=128, L=2048, V=32000, sigma_q=3.0, sigma_n=1.0,
                   temperatures=(0.7,), tree="static60", data_seed=1003),
    "c4": Workload("c4", B=64, N=64, Hq=64, Hkv=8, D=128, L=8192, V=128256, sigma_q=3.0, sigma_n=2.0,
                   temperatures=(1.0,), tree="random", max_depth=8, data_seed=1004),
    "c5": Workload("c5", B=8, N=60, Hq=32, Hkv=8, D=128, L=32768, V=152064, sigma_q=4.0, sigma_n=1.0,
                   temperatures=(0.0, 0.7), tree="static60", data_seed=1005),
}

CONFIG_TEXT = {
    "c1": "single sequence, static 60-node tree, MHA 32x128, KV 512, vocab 32000",
    "c2": "batch 1 chain K=5, GQA 32/8x128, KV 4096, vocab 128256",
    "c3": "batch 16 static 60-node trees, MHA 40x128, KV 2048, vocab 32000",
    "c4": "batch 64 dynamic 64-node trees, GQA 64/8x128, KV 8192, vocab 128256",
    "c5": "batch 8 static 60-node trees, GQA 32/8x128, KV 32768, vocab 152064",
}


def _generator(device, seed: int, stream: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(stream))
    return g


def _randn(shape, device, seed, stream, scale=1.0):
    import torch
    t = torch.randn(shape, generator=_generator(device, seed, stream), device=device, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t


def attention_inputs(w: Workload, device="cpu", seed: Optional[int] = None, L: Optional[int] = None):
    """bf16 tensors ~N(0,1) (round to nearest even), layouts:
    Q [B,N,Hq,D], K/V cache [B,Hkv,L,D] (head-major), K/V tree [B,N,Hkv,D]."""
    import torch
    s = w.data_seed if seed is None else seed
    L = w.L if L is None else L
    bf = torch.bfloat16
    Q = _randn((w.B, w.N, w.Hq, w.D), device, s, 1).to(bf)
    Kc = _randn((w.B, w.Hkv, L, w.D), device, s, 2).to(bf)
    Vc = _randn((w.B, w.Hkv, L, w.D), device, s, 3).to(bf)
    Kt = _randn((w.B, w.N, w.Hkv, w.D), device, s, 4).to(bf)
    Vt = _randn((w.B, w.N, w.Hkv, w.D), device, s, 5).to(bf)
    return Q, Kc, Vc, Kt, Vt


def accept_inputs(w: Workload, device="cpu", seed: Optional[int] = None, parent: Optional[np.ndarray] = None):
    """Target logits q ~ N(0, sigma_q^2) fp32 [B,N,V]; draft logits for node c are a
    noisy copy of the target row at c's parent, p[c] = q[parent(c)] + N(0, sigma_n^2);
    the draft token of c is the argmax of p[c]; p row 0 is zero (unused)."""
    import torch
    s = w.data_seed if seed is None else seed
    par = w.parents() if parent is None else parent
    par_t = torch.as_tensor(par, dtype=torch.int64, device=device)
    q = _randn((w.B, w.N, w.V), device, s, 6, w.sigma_q)
    p = torch.empty_like(q)
    noise_gen = _generator(device, s, 7)
    for b in range(w.B):
        idx = par_t[b].clamp(min=0)
        p[b] = q[b].index_select(0, idx)
        p[b].add_(torch.randn((w.N, w.V), generator=noise_gen, device=device, dtype=torch.float32),
                  alpha=w.sigma_n)
    p[:, 0, :] = 0.0
    draft = p.argmax(dim=-1).to(torch.int32)
    draft[:, 0] = 0
    parent_t = torch.as_tensor(par, dtype=torch.int32, device=device)
    return q, p, draft, parent_t


def bf16_to_f64(t) -> np.ndarray:
    """Exact widening of a bf16 torch tensor to a float64 numpy array."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def tiny_workloads() -> List[Workload]:
    """Small shapes that still span several tiles and leave ragged tails."""
    return [
        Workload("t_chain", B=2, N=6, Hq=4, Hkv=2, D=128, L=100, V=1000, sigma_q=3.0, sigma_n=1.0,
                 temperatures=(0.0, 1.0), tree="chain", data_seed=11),
        Workload("t_static", B=2, N=60, Hq=2, Hkv=2, D=128, L=300, V=3000, sigma_q=3.0, sigma_n=1.0,
                 temperatures=(0.0, 0.7), tree="static60", data_seed=12),
        Workload("t_random", B=3, N=64, Hq=8, Hkv=1, D=128, L=257, V=5003, sigma_q=3.0, sigma_n=2.0,
                 temperatures=(0.0, 1.0), tree="random", data_seed=13),
        Workload("t_nocache", B=2, N=17, Hq=4, Hkv=4, D=128, L=0, V=777, sigma_q=3.0, sigma_n=1.0,
                 temperatures=(0.0, 1.3), tree="random", max_depth=5, data_seed=14),
    ]
