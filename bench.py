#!/usr/bin/env python3
"""Benchmark of one token-tree verification step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
tree mask -> ancestor-masked tree attention -> accept/reject walk.  The
headline workload is the largest of the five benchmark workloads that fits
one GPU: "batch 64 dynamic 64-node trees, GQA 64/8 x 128, KV 8192, vocab
128256" with temperature-1.0 sampling; the greedy step is reported beside it,
and the other four workloads are measured in the same run under "configs".
Inputs are resident in HBM before timing starts and rotate over enough copies
to exceed the 256 MB Infinity Cache.

Prints ONE JSON line (rank 0) with the throughput (verified tree-nodes/s),
the roofline of the dominant call measured live with HIP events on its
stream, and the CPU oracle timed on a bounded sample on the host cores.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import hashlib
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified tree-nodes/sec + achieved HBM GB/s & MFMA util vs MI355X peak"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
COPY_CAL_BYTES = 512 << 20
PROBE_LIB = os.path.join(ROOT, "token_tree_verification_amd", "libtv_probe.so")
ATTN_SOURCES = ("token_tree_verification_amd/csrc/tv_attention.hip", "token_tree_verification_amd/csrc/tv_device.h")
ACC_SOURCES = ("token_tree_verification_amd/csrc/tv_accept.hip", "token_tree_verification_amd/csrc/tv_device.h")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c4", choices=["c1", "c2", "c3", "c4", "c5"],
                    help="headline workload (default: the largest one, c4)")
    ap.add_argument("--also", default="c1,c2,c3,c5",
                    help="other workloads measured in the same run and reported under 'configs'")
    ap.add_argument("--only", action="store_true", help="measure the headline workload alone")
    ap.add_argument("--temperature", type=float, default=None, help="sampling temperature (default: the config's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="bounded CPU oracle sample length")
    ap.add_argument("--graph", action="store_true",
                    help="time HIP-graph replays of the step instead of back-to-back launches")
    return ap.parse_args()


class Step:
    """Pre-marshalled C-ABI calls of one verification step on one input copy."""

    def __init__(self, tv, w, Q, Kc, Vc, Kt, Vt, q, p, draft, parent, greedy, temperature, seed, dev, stream):
        import torch
        self.lib = tv.library()
        B, N, Hq, Hkv, D, L, V = w.B, w.N, w.Hq, w.Hkv, w.D, w.L, w.V
        self.keep = [Q, Kc, Vc, Kt, Vt, q, p, draft, parent]
        self.anc = torch.empty((B, N), dtype=torch.int64, device=dev)
        self.depth = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.status = torch.empty((B,), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, N, Hq, D), dtype=torch.float32, device=dev)
        self.acc_len = torch.empty((B,), dtype=torch.int32, device=dev)
        self.acc_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
        self.toks = torch.empty((B, N), dtype=torch.int32, device=dev)
        aw = tv.attention_workspace_bytes(B, N, Hq, Hkv, D, L)
        self.attn_ws = torch.zeros(max(aw, 256), dtype=torch.uint8, device=dev)
        cw = tv.accept_workspace_bytes(B, N, V, greedy)
        self.acc_ws = torch.zeros(max(cw, 256), dtype=torch.uint8, device=dev)
        P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() else None
        self.stream = ctypes.c_void_p(stream.cuda_stream)
        self.mask_args = (P(parent), B, N, P(self.anc), P(self.depth), P(self.status), self.stream)
        self.attn_args = (P(Q), P(Kc), P(Vc), P(Kt), P(Vt), P(self.anc), P(self.out), B, N, Hq, Hkv, D, L,
                          ctypes.c_float(1.0 / math.sqrt(D)), P(self.attn_ws), ctypes.c_size_t(aw), self.stream)
        self.acc_args = (P(q), None if greedy else P(p), P(draft), P(parent), B, N, V, ctypes.c_uint64(seed),
                         ctypes.c_float(temperature), int(greedy), P(self.acc_len), P(self.acc_nodes), P(self.toks),
                         P(self.acc_ws), ctypes.c_size_t(cw), self.stream)

    def mask(self):
        rc = self.lib.tv_build_tree_mask(*self.mask_args)
        if rc:
            raise RuntimeError(f"tv_build_tree_mask: {rc}")

    def attention(self):
        rc = self.lib.tv_tree_attention(*self.attn_args)
        if rc:
            raise RuntimeError(f"tv_tree_attention: {rc}")

    def accept(self):
        rc = self.lib.tv_spec_accept(*self.acc_args)
        if rc:
            raise RuntimeError(f"tv_spec_accept: {rc}")

    def run(self):
        self.mask()
        self.attention()
        self.accept()

    def capture(self, torch, stream):
        """Record the three calls of the step into a HIP graph on `stream`."""
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=stream):
            self.run()
        return self.graph


def attention_bytes(w):
    kv = 2 * w.B * w.Hkv * w.L * w.D * 2
    return kv + w.B * w.N * w.Hq * w.D * 2 + 2 * w.B * w.N * w.Hkv * w.D * 2 + w.B * w.N * 8 + w.B * w.N * w.Hq * w.D * 4


def attention_flops(w, parents):
    import numpy as np
    depth_sum = 0
    for par in parents:
        d = np.zeros(len(par), dtype=np.int64)
        for i in range(1, len(par)):
            d[i] = d[par[i]] + 1
        depth_sum += int((d + 1).sum())
    return 4 * w.D * w.Hq * (w.B * w.N * w.L + depth_sum)


def accept_bytes(w, greedy):
    rows = w.N if greedy else 2 * w.N - 1
    return w.B * rows * w.V * 4 + w.B * w.N * 4 * 2


def family_bytes(w, parents, acc_len, acc_nodes, wor=False):
    """Row bytes of the sampling call's statistics: every node the walk reaches
    (the root and each accepted node) streams its family once, its target row
    and the draft rows its children were drawn from (one row per child, or
    without replacement the node's own row when it has children)."""
    import numpy as np
    total = 0
    for b in range(w.B):
        par = parents[b]
        nkids = np.zeros(w.N, dtype=np.int64)
        for i in range(1, w.N):
            nkids[int(par[i])] += 1
        visited = [0] + [int(x) for x in acc_nodes[b, :max(0, int(acc_len[b]))]]
        rows = sum(1 + (min(1, int(nkids[u])) if wor else int(nkids[u])) for u in visited)
        total += rows * w.V * 4
    return total


def greedy_bytes(w, parents, draft, q_argmax):
    """Row bytes of the greedy call's statistics as a level-by-level search
    reads them: the root's target row and the target row of every node whose
    path matches (each draft token on it equals its parent's target argmax)."""
    import numpy as np
    total = 0
    for b in range(w.B):
        par = parents[b]
        match = np.zeros(w.N, dtype=bool)
        match[0] = True
        for i in range(1, w.N):  # parent[i] < i
            match[i] = match[int(par[i])] and int(draft[b, i]) == int(q_argmax[b, int(par[i])])
        total += int(match.sum()) * w.V * 4
    return total


def walk_bytes(w, parents, acc_len, acc_nodes, team_size):
    """Row bytes the sampling walk reads beside the statistics, from the
    accepted paths (independent siblings): at every node on the path and at
    the stop node, each rejected child costs one pass over its p row, and the
    first rejection at a node also reads the node's q row (later passes keep
    the residual on chip); a walk that ends at a leaf draws from the leaf's q
    row in one member's slice (V / team_size logits)."""
    total = 0
    for b in range(w.B):
        par = parents[b]
        kids = [[] for _ in range(w.N)]
        for i in range(1, w.N):
            kids[int(par[i])].append(i)
        path = [int(x) for x in acc_nodes[b, :max(0, int(acc_len[b]))]]
        visited = [0] + path
        rows = 0
        for k, u in enumerate(visited):
            rej = kids[u].index(path[k]) if k < len(path) else len(kids[u])
            rows += rej + (1 if rej > 0 else 0)
        total += rows * w.V * 4
        if not kids[visited[-1]]:
            total += (w.V + team_size - 1) // team_size * 4
    return total


def sleep_cycles_per_ms(torch, stream):
    """Shader-clock cycles of torch's spin kernel per millisecond on this device."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    cyc = 2_000_000
    torch.cuda._sleep(cyc)  # first launch pays the module load
    torch.cuda.synchronize()
    a.record(stream)
    torch.cuda._sleep(cyc)
    b.record(stream)
    torch.cuda.synchronize()
    return cyc / max(a.elapsed_time(b), 1e-3)


def time_batch(fn, steps, stream, torch, lead_cycles):
    """Mean device time per call of ``steps`` back-to-back launches of one call
    (queued behind a spin kernel, so host launch latency is hidden)."""
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(lead_cycles))
    start.record(stream)
    for s in range(steps):
        fn(s)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def copy_calibration(torch, dev, nbytes=COPY_CAL_BYTES):
    """One plain elementwise copy (read nbytes, write nbytes) outside the timed
    region: under rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE give the factor
    that turns those counters into bytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def achievable_peaks(torch, dev, stream):
    """The device's reachable rates in this run, beside the spec peaks: the
    probe library's streaming read (2 GiB of 16-byte loads, a contiguous range
    per workgroup; ordinary and non-temporal loads) and pure MFMA loop
    (four independent v_mfma_f32_32x32x16_bf16 chains per wave, four waves per
    SIMD) on constant operands and on random ones (real data draws more power,
    so the chip holds a lower clock), a plain copy (512 MiB read plus 512 MiB written) and a library bf16
    GEMM (torch.matmul, 16384^3)."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps / 1e3  # seconds per call
    probe = ctypes.CDLL(PROBE_LIB)
    probe.tv_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_void_p]
    probe.tv_probe_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe.tv_probe_mfma_loop_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    probe.tv_probe_mfma_loop_flops.restype = ctypes.c_double
    st = ctypes.c_void_p(stream.cuda_stream)

    def call(rc):
        if rc != 0:
            raise RuntimeError(f"probe call failed ({rc})")

    out = {}
    nblk = 2048  # the fastest of 512 .. 16384 workgroups on this device
    sink = torch.empty(4096 * 256, dtype=torch.float32, device=dev)
    big = torch.ones((2 << 30) // 4, dtype=torch.float32, device=dev)
    for nt, key in ((0, "hbm_read_GB/s"), (1, "hbm_read_nontemporal_GB/s")):
        t = timed(lambda: call(probe.tv_probe_stream_read(ctypes.c_void_p(big.data_ptr()), big.numel() * 4, nt,
                                                          ctypes.c_void_p(sink.data_ptr()), nblk, st)), 5)
        out[key] = round(big.numel() * 4 / t / 1e9, 1)
    del big
    mblk, iters = 1024, 4096  # four workgroups of four waves per CU
    for rnd, key in ((0, "mfma_loop_bf16_TFLOP/s"), (1, "mfma_loop_bf16_random_TFLOP/s")):
        t = timed(lambda: call(probe.tv_probe_mfma_loop(mblk, iters, rnd, ctypes.c_void_p(sink.data_ptr()), st)), 3)
        out[key] = round(probe.tv_probe_mfma_loop_flops(mblk, iters) / t / 1e12, 1)
    del sink
    src = torch.ones(COPY_CAL_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    out["copy_GB/s"] = round(2 * COPY_CAL_BYTES / timed(lambda: dst.copy_(src), 10) / 1e9, 1)
    del src, dst
    n = 16384
    x = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    y = torch.randn((n, n), dtype=torch.bfloat16, device=dev)
    out["bf16_gemm_TFLOP/s"] = round(2 * n ** 3 / timed(lambda: torch.matmul(x, y), 3) / 1e12, 1)
    del x, y
    torch.cuda.synchronize()
    return out


def kernel_sources_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _profile_record(path, kernel_key, files):
    """The JSON record of ``kernel_key`` in a committed rocprofv3 summary under
    profiles/, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", path)
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get("kernels", {}).get(kernel_key)
    if not rec or rec.get("sources_sha256") != kernel_sources_digest(files):
        return None
    return rec


def counted_traffic(workload, kernel_key, files):
    """HBM bytes per launch of ``kernel_key`` on ``workload`` (FETCH_SIZE plus
    WRITE_SIZE, calibrated on a plain copy) from the committed summary."""
    rec = _profile_record(f"traffic_{workload}.md", kernel_key, files)
    return None if rec is None else int(rec["fetch_bytes"]) + int(rec["write_bytes"])


def counted_mfma(workload, files, avg_us):
    """MFMA FLOPs the attention kernel issues per launch on ``workload``, from
    the committed counter summary (calibrated against the probe's MFMA loop),
    and their rate over the live duration as a fraction of the bf16 peak."""
    rec = _profile_record(f"mfma_{workload}.md", "tree_attention_kernel", files)
    if rec is None:
        return None
    issued = float(rec["mfma_flops_issued"])
    return {"flops_issued": issued, "per_alg_flop": rec["mfma_flops_per_alg_flop"],
            "util": round(issued / (avg_us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4)}


def cpu_baseline(w, inputs, temperature, seconds):
    """The oracle as it stands (numpy fp64 attention, C walk) on the host
    cores, on a bounded sample of the workload: whole sequences (every head of
    the attention, then the sampling walk), one after another, until about
    ``seconds`` have been spent (at least one).  Attention and walk are timed
    separately.  numpy's BLAS pool is set explicitly to the host's CPU share
    (OMP_NUM_THREADS when the environment fixes it, else os.cpu_count())."""
    import numpy as np
    import oracle
    from workloads import bf16_to_f64
    Q, Kc, Vc, Kt, Vt, q, p, draft, parent = inputs
    host_cpus = os.cpu_count() or 1
    threads = int(os.environ.get("OMP_NUM_THREADS", host_cpus) or host_cpus)
    limiter = None
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=threads, user_api="blas")
    except Exception:
        pass
    try:
        parn = parent.cpu().numpy()
        t_attn = t_acc = 0.0
        seqs = 0
        while seqs < w.B:
            b = seqs
            host = [bf16_to_f64(t[b:b + 1]) for t in (Q, Kc, Vc, Kt, Vt)]
            t0 = time.perf_counter()
            oracle.tree_mask(parn[b:b + 1])
            oracle.tree_attention(*host, parn[b:b + 1])
            t1 = time.perf_counter()
            qn, pn, dn = (t[b:b + 1].cpu().numpy() for t in (q, p, draft))
            t2 = time.perf_counter()
            oracle.spec_accept(qn, pn, dn, parn[b:b + 1], seed=0, temperature=temperature)
            t3 = time.perf_counter()
            t_attn += t1 - t0
            t_acc += t3 - t2
            seqs += 1
            if t_attn + t_acc >= seconds:
                break
    finally:
        if limiter is not None:
            limiter.unregister()
    nodes = seqs * (w.N - 1)
    return {"value": round(nodes / (t_attn + t_acc), 3), "unit": "tree-nodes/s", "cores": threads,
            "kind": "oracle", "host_cpus": host_cpus, "blas_threads": threads,
            "attention_s": round(t_attn, 3), "accept_s": round(t_acc, 3),
            "sample": f"{seqs} of the workload's {w.B} sequence(s): mask + fp64 attention over every head + "
                      f"sampling walk at T={temperature}, {t_attn:.1f} s attention and {t_acc:.1f} s walk"}


def measure(name, args, tv, torch, dev, stream, lead_of, headline):
    """Time one workload: whole sampling and greedy steps, then each call on
    its own.  Returns the result record and (headline only) the first input
    copy for the CPU baseline."""
    from workloads import CONFIGS, CONFIG_TEXT, accept_inputs, attention_inputs

    w = CONFIGS[name]
    temps = [t for t in w.temperatures if t > 0]
    T = args.temperature if (args.temperature is not None and headline) else (temps[0] if temps else 1.0)
    parents = w.parents()
    per_copy = attention_bytes(w) + accept_bytes(w, False)
    ncopies = max(1, min(16, math.ceil(1.5 * MALL_BYTES / per_copy)))
    copies, first_inputs = [], None
    for c in range(ncopies):
        Q, Kc, Vc, Kt, Vt = attention_inputs(w, device=dev, seed=w.data_seed + 100 * c)
        q, p, draft, parent = accept_inputs(w, device=dev, seed=w.data_seed + 100 * c, parent=parents)
        if c == 0 and headline:
            first_inputs = (Q, Kc, Vc, Kt, Vt, q, p, draft, parent)
        copies.append(dict(
            sample=Step(tv, w, Q, Kc, Vc, Kt, Vt, q, p, draft, parent, False, T, w.philox_seed, dev, stream),
            greedy=Step(tv, w, Q, Kc, Vc, Kt, Vt, q, p, draft, parent, True, 1.0, w.philox_seed, dev, stream)))
    torch.cuda.synchronize()

    for s in range(args.warmup):
        copies[s % ncopies]["sample"].run()
        copies[s % ncopies]["greedy"].run()
    torch.cuda.synchronize()
    use_graph = args.graph
    if use_graph:
        for c in copies:
            c["sample"].capture(torch, stream)
            c["greedy"].capture(torch, stream)
        torch.cuda.synchronize()
        for s in range(args.warmup):
            copies[s % ncopies]["sample"].graph.replay()
            copies[s % ncopies]["greedy"].graph.replay()
        torch.cuda.synchronize()

    def full(mode):
        if use_graph:
            return lambda s: copies[s % ncopies][mode].graph.replay()
        return lambda s: copies[s % ncopies][mode].run()

    # timed: whole steps, sampling mode (headline) and greedy mode
    ms_step = time_batch(full("sample"), args.steps, stream, torch, lead_of(3 * args.steps))
    ms_greedy = time_batch(full("greedy"), args.steps, stream, torch, lead_of(3 * args.steps))
    # per-call durations: `steps` launches of one call back to back (rotating
    # over the input copies) between two events on the launch stream
    calls = {"mask": lambda s: copies[s % ncopies]["sample"].mask(),
             "attention": lambda s: copies[s % ncopies]["sample"].attention(),
             "accept": lambda s: copies[s % ncopies]["sample"].accept(),
             "accept_greedy": lambda s: copies[s % ncopies]["greedy"].accept()}
    per = {n: time_batch(fn, args.steps, stream, torch, lead_of(args.steps)) for n, fn in calls.items()}
    # the rows the sampling call reads on each copy (its outputs after the timed
    # calls): the families of the nodes its walk reaches and the walk's row
    # passes, averaged over the copies
    team_size = tv.accept_plan(w.B, w.N, w.V, False)[0]
    outs = [(c["sample"].acc_len.cpu().numpy(), c["sample"].acc_nodes.cpu().numpy()) for c in copies]
    f_bytes = sum(family_bytes(w, parents, al, an) for al, an in outs) / len(outs)
    w_bytes = sum(walk_bytes(w, parents, al, an, team_size) for al, an in outs) / len(outs)
    # the greedy call's rows: the matching levels of each copy's trees
    g_rows = sum(greedy_bytes(w, parents, c["greedy"].keep[7].cpu().numpy(),
                              c["greedy"].keep[5].argmax(dim=-1).cpu().numpy()) for c in copies) / len(copies)
    del copies
    torch.cuda.synchronize()

    nodes = w.B * (w.N - 1)
    a_bytes = attention_bytes(w)
    a_flops = attention_flops(w, parents)
    c_full = accept_bytes(w, False)  # what a pass over every row would read
    c_stream = int(round(f_bytes)) + w.B * w.N * 4 * 2
    c_bytes = c_stream + int(round(w_bytes))
    g_bytes = int(round(g_rows)) + w.B * w.N * 4 * 2
    attn_gbs = a_bytes / (per["attention"] / 1e3) / 1e9
    attn_tflops = a_flops / (per["attention"] / 1e3) / 1e12
    acc_gbs = c_bytes / (per["accept"] / 1e3) / 1e9
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    mfma_bound = a_flops / a_bytes > ridge
    dominant = "attention" if per["attention"] >= per["accept"] else "accept"
    if dominant == "attention":
        if mfma_bound:
            roof = {"bound": "mfma", "achieved": round(attn_tflops, 3), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
        else:
            roof = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(attn_gbs / HBM_PEAK_GBS, 4)}
        roof["kernel"] = "tv_tree_attention (one launch of tv::tree_attention_kernel / tree_attention_wide_kernel)"
        roof["algorithmic_bytes"] = a_bytes
        roof["algorithmic_flops"] = a_flops
        roof["avg_us"] = round(per["attention"] * 1e3, 3)
        roof["traffic"] = counted_traffic(w.name, "tree_attention_kernel", ATTN_SOURCES)
        mf = counted_mfma(w.name, ATTN_SOURCES, per["attention"] * 1e3)
        if mf is not None:
            roof["mfma_counters"] = mf
    else:
        roof = {"bound": "hbm", "achieved": round(acc_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(acc_gbs / HBM_PEAK_GBS, 4),
                "kernel": "tv::spec_accept_kernel<false, ...> (tv_spec_accept sampling, one launch)",
                "algorithmic_bytes": c_bytes, "stream_bytes": c_stream, "walk_bytes": c_bytes - c_stream,
                "all_rows_bytes": c_full, "avg_us": round(per["accept"] * 1e3, 3)}
        roof["traffic"] = counted_traffic(w.name, "spec_accept_kernel<false, true>", ACC_SOURCES)
    rec = {
        "workload": f"{w.name}: {CONFIG_TEXT[w.name]}",
        "value": round(nodes / (ms_step / 1e3), 1),
        "ms_per_step": round(ms_step, 5),
        "config": {"workload": f"{w.name}: {CONFIG_TEXT[w.name]}", "batch": w.B, "tree_nodes": w.N,
                   "draft_nodes": w.N - 1, "heads_q_kv": [w.Hq, w.Hkv], "head_dim": w.D, "kv_len": w.L,
                   "vocab": w.V, "mode": f"sampling T={T}", "input_copies": ncopies,
                   "launch": "hip-graph replay" if use_graph else "back-to-back launches on one stream"},
        "roofline": roof,
        "calls_us": {k: round(v * 1e3, 3) for k, v in per.items()},
        "attention": {"GB/s": round(attn_gbs, 1), "TFLOP/s": round(attn_tflops, 3),
                      "hbm_frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                      "mfma_frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                      "bound": "mfma" if mfma_bound else "hbm"},
        "accept": {"GB/s": round(acc_gbs, 1), "hbm_frac": round(acc_gbs / HBM_PEAK_GBS, 4),
                   "bytes": c_bytes, "walk_bytes": c_bytes - c_stream, "all_rows_bytes": c_full,
                   # time of a pass over every row at the HBM peak, over this call's time
                   "vs_all_rows_at_peak": round(c_full / (HBM_PEAK_GBS * 1e9) / (per["accept"] / 1e3), 3),
                   "greedy_bytes": g_bytes, "greedy_all_rows_bytes": accept_bytes(w, True),
                   "greedy_GB/s": round(g_bytes / (per["accept_greedy"] / 1e3) / 1e9, 1),
                   "greedy_hbm_frac": round(g_bytes / (per["accept_greedy"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                   "greedy_vs_all_rows_at_peak": round(accept_bytes(w, True) / (HBM_PEAK_GBS * 1e9)
                                                       / (per["accept_greedy"] / 1e3), 3)},
        "greedy": {"value": round(nodes / (ms_greedy / 1e3), 1), "ms_per_step": round(ms_greedy, 5)},
        "temperature": T,
    }
    return rec, first_inputs


def measure_extras(args, tv, torch, dev, stream, lead_of):
    """The steps around verification, on the headline workload's shapes: the
    KV commit of the accepted paths, and one step of dynamic tree construction
    (expanding ten frontier nodes per sequence with their top-10 tokens, then
    the re-ranking of the 511-slot pool down to 64 nodes)."""
    from workloads import CONFIGS, accept_inputs, attention_inputs
    w = CONFIGS[args.config]
    out = {}
    # KV commit: the sampling walk's paths of this workload, appended after L
    q, p, draft, parent = accept_inputs(w, device=dev)
    a, nodes, _ = tv.spec_accept(q, p, draft, parent, seed=w.philox_seed, temperature=1.0)
    del q, p
    _, _, _, Kt, Vt = attention_inputs(w, device=dev, L=0)
    Kc = torch.zeros((w.B, w.Hkv, w.L + w.N, w.D), dtype=torch.bfloat16, device=dev)
    Vc = torch.zeros_like(Kc)
    cl = torch.full((w.B,), w.L, dtype=torch.int32, device=dev)
    nl = torch.empty_like(cl)
    st = torch.empty_like(cl)
    lib = tv.library()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(stream.cuda_stream)
    args_c = (P(Kt), P(Vt), P(a), P(nodes), P(cl), P(Kc), P(Vc), P(nl), P(st), w.B, w.N, w.Hkv, w.D, w.L + w.N, sp)

    def commit(s):
        rc = lib.tv_commit_kv(*args_c)
        if rc:
            raise RuntimeError(f"tv_commit_kv: {rc}")
    ms = time_batch(commit, args.steps, stream, torch, lead_of(args.steps))
    rows = int((a.clamp(min=-1) + 1).sum().item())
    cbytes = rows * w.Hkv * w.D * 2 * 2 * 2  # K and V rows, read and written
    out["commit_kv"] = {"us": round(ms * 1e3, 3), "rows": rows, "bytes": cbytes,
                        "GB/s": round(cbytes / (ms / 1e3) / 1e9, 1)}
    del Kc, Vc, Kt, Vt
    # dynamic tree construction: one middle expansion step and the re-ranking
    B, F, K, V = w.B, 10, 10, w.V
    Pn = 1 + K + 5 * K * K
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    root_logits = torch.randn((B, 1, V), generator=g, device=dev) * 2.0
    logits = torch.randn((B, F, V), generator=g, device=dev) * 2.0
    pool = tv.tree_pool(B, Pn, dev)
    frontier = tv.tree_expand(root_logits, None, pool, 1, K, F, 1.0)
    nxt = torch.empty((B, F), dtype=torch.int32, device=dev)
    args_e = (P(logits), P(frontier), None, B, F, V, K, ctypes.c_float(1.0), P(pool[0]), P(pool[1]), P(pool[2]), Pn,
              1 + K, P(nxt), F, sp)

    def expand(s):
        rc = lib.tv_tree_expand(*args_e)
        if rc:
            raise RuntimeError(f"tv_tree_expand: {rc}")
    ms = time_batch(expand, args.steps, stream, torch, lead_of(args.steps))
    ebytes = B * F * V * 4
    out["tree_expand"] = {"us": round(ms * 1e3, 3), "bytes": ebytes, "GB/s": round(ebytes / (ms / 1e3) / 1e9, 1),
                          "hbm_frac": round(ebytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                          "shape": f"{B} sequences x {F} frontier rows x vocab {V}, top-{K}"}
    outs = [torch.empty((B, w.N), dtype=torch.int32, device=dev) for _ in range(3)]
    nn = torch.empty((B,), dtype=torch.int32, device=dev)
    args_s = (P(pool[0]), P(pool[1]), P(pool[2]), B, Pn, 1 + K + F * K, w.N, *(P(o) for o in outs), P(nn), sp)

    def select(s):
        rc = lib.tv_tree_select(*args_s)
        if rc:
            raise RuntimeError(f"tv_tree_select: {rc}")
    ms = time_batch(select, args.steps, stream, torch, lead_of(args.steps))
    out["tree_select"] = {"us": round(ms * 1e3, 3), "shape": f"{B} pools of {1 + K + F * K} slots -> {w.N} nodes"}
    del logits, root_logits, pool
    torch.cuda.synchronize()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (verification of independent "
              f"sequences shards by batch with no communication).", file=sys.stderr)
        return 2
    import torch

    import token_tree_verification_amd as tv
    from workloads import CONFIGS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)  # every call of the step is issued (and captured) here
    torch.cuda.set_stream(stream)

    copy_calibration(torch, dev)
    cyc_ms = sleep_cycles_per_ms(torch, stream)
    # enough lead for the host to queue every call of the timed loop
    lead = lambda calls: cyc_ms * max(2.0, 0.05 * calls)

    head, first_inputs = measure(args.config, args, tv, torch, dev, stream, lead, True)
    print(f"[bench] {args.config}: {head['ms_per_step'] * 1e3:.1f} us/step, calls_us {head['calls_us']}",
          file=sys.stderr, flush=True)
    extras = measure_extras(args, tv, torch, dev, stream, lead)
    print(f"[bench] around verification: {extras}", file=sys.stderr, flush=True)
    others = {}
    if not args.only:
        for name in [c.strip() for c in args.also.split(",") if c.strip()]:
            if name == args.config or name not in CONFIGS:
                continue
            rec, _ = measure(name, args, tv, torch, dev, stream, lead, False)
            rec.pop("config", None)
            others[name] = rec
            print(f"[bench] {name}: {rec['ms_per_step'] * 1e3:.1f} us/step, calls_us {rec['calls_us']}",
                  file=sys.stderr, flush=True)

    roof = head["roofline"]
    peaks = achievable_peaks(torch, dev, stream)
    # MFMA work on real data is held to the clock of the random-operand loop
    reach = (peaks["mfma_loop_bf16_random_TFLOP/s"] if roof["unit"] == "TFLOP/s" else
             max(peaks["hbm_read_GB/s"], peaks["hbm_read_nontemporal_GB/s"]))
    roof["frac_of_achievable"] = round(roof["achieved"] / reach, 4)

    res = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tree-nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": roof,
        "calls_us": head["calls_us"],
        "attention": head["attention"],
        "accept": head["accept"],
        "greedy": head["greedy"],
        "achievable": peaks,
        "around_verification": extras,
        "configs": others,
    }
    if not args.no_cpu_baseline:
        w = CONFIGS[args.config]
        res["cpu_baseline"] = cpu_baseline(w, first_inputs, head["temperature"], args.cpu_seconds)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
