"""Host-side helpers of the GPU parity tests: the oracle run over many
sequences or seeds on host threads (its arithmetic unchanged; ctypes and
numpy release the GIL), with progress lines so that long comparisons report
as they go."""
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from workloads import bf16_to_f64


def workers():
    return max(1, min(16, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), os.cpu_count() or 1))


def say(msg):
    sys.__stderr__.write(f"    {msg}\n")
    sys.__stderr__.flush()


def oracle_attention(Q, Kc, Vc, Kt, Vt, par, seq_nodes=None, seq_len=None, label=""):
    """The fp64 oracle over every (sequence, head), one sequence per task."""
    import torch
    t0 = time.time()
    host = [t.detach().to("cpu") for t in (Q, Kc, Vc, Kt, Vt)]
    B, N, Hq, D = Q.shape
    out = np.empty((B, N, Hq, D))

    def one(b):
        sl = [bf16_to_f64(t[b:b + 1]) for t in host]
        kw = {}
        if seq_nodes is not None:
            kw["seq_nodes"] = np.asarray(seq_nodes)[b:b + 1]
        if seq_len is not None:
            kw["seq_len"] = np.asarray(seq_len)[b:b + 1]
        return b, oracle.tree_attention(*sl, par[b:b + 1], **kw)[0]

    done = 0
    with ThreadPoolExecutor(workers()) as ex:
        for b, o in ex.map(one, range(B)):
            out[b] = o
            done += 1
            if done % 16 == 0 or done == B:
                say(f"{label} oracle attention {done}/{B} sequences, {time.time() - t0:.1f} s")
    del torch
    return out


def oracle_accept_seeds(q, p, draft, parent, seeds, temperature, label="", **kw):
    """oracle.spec_accept for each seed (whole batch per task)."""
    t0 = time.time()
    res = {}

    def one(seed):
        return seed, oracle.spec_accept(q, p, draft, parent, seed=seed, temperature=temperature, **kw)

    with ThreadPoolExecutor(workers()) as ex:
        for i, (seed, r) in enumerate(ex.map(one, seeds)):
            res[seed] = r
            if (i + 1) % max(1, len(seeds) // 8) == 0:
                say(f"{label} oracle walks {i + 1}/{len(seeds)} seeds, {time.time() - t0:.1f} s")
    return res


def oracle_accept_chunks(q, p, draft, parent, seed, temperature, chunk=64, label="", **kw):
    """oracle.spec_accept over a large batch in chunks of sequences (each chunk
    keeps its sequences' Philox numbers through seq_offset)."""
    B = q.shape[0]
    seq_nodes = kw.pop("seq_nodes", None)

    def one(b0):
        b1 = min(B, b0 + chunk)
        extra = dict(kw)
        if seq_nodes is not None:
            extra["seq_nodes"] = np.asarray(seq_nodes)[b0:b1]
        return b0, oracle.spec_accept(q[b0:b1], None if p is None else p[b0:b1], draft[b0:b1], parent[b0:b1],
                                      seed=seed, temperature=temperature, seq_offset=b0, **extra)

    out = None
    t0 = time.time()
    with ThreadPoolExecutor(workers()) as ex:
        for b0, r in ex.map(one, range(0, B, chunk)):
            if out is None:
                out = {k: np.empty((B,) + v.shape[1:], v.dtype) for k, v in r.items()}
            for k, v in r.items():
                out[k][b0:b0 + v.shape[0]] = v
    say(f"{label} oracle walks over {B} sequences, {time.time() - t0:.1f} s")
    return out
