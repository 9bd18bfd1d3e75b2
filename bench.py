#!/usr/bin/env python3
"""Benchmark of the tree-packed chunkwise KDA hot path on one MI355X.

One step = forward + backward of one KDA layer (16 heads, d = 128, chunk 64,
bf16 q/k/v, fp32 gates and state) over the whole synthetic rollout tree of
the workload (default: complete 4-ary tree of depth 3, segment lengths
U{256..2048}), with the plan built and uploaded before the timed region (the
plan belongs to the tree and is shared by every KDA layer of a model; its
host time is reported separately as plan_ms).

Prints one JSON line: unique tokens/s, roofline of the dominant kernel (its
launch durations measured live inside the timed region with hipEvents on the
launch stream through the library's timing hook, which times that kernel
alone there; every kernel's durations come from a few more steps after it),
the float64 CPU oracle timed on a bounded sample of the same workload, and
the speedup over trajectory-expanded execution of the same tree with the
same kernels.

    python bench.py [--steps K] [--warmup W] [--workload 2] [--expanded-steps 3]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "unique tokens/s, tree-packed KDA fwd+bwd @16 heads d=128; % of MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA


def _progress(msg):
    """A progress line on stderr (the result is the one JSON line on stdout)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--expanded-steps", type=int, default=3)
    ap.add_argument("--attn-steps", type=int, default=3,
                    help="timed steps of the tree attention measurement (0: skip)")
    ap.add_argument("--hybrid-steps", type=int, default=1,
                    help="timed steps of the hybrid layer group (0: skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-configs", dest="extra_configs", action="store_false",
                    help="skip the forward-only and step-wise workloads and the gather")
    ap.add_argument("--no-timing", action="store_true",
                    help="do not record per-kernel launch events in the timed region")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (1 GiB read + 1 GiB "
                         "written per launch, 3 launches), to scale HBM byte counters")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 28  # floats: 1 GiB
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n * 4,
                                           "bytes_written_per_launch": n * 4, "launches": 3}}))


# ---------------------------------------------------------------------------
# algorithmic bytes (per unique token at H heads, head dim D; bf16 inputs)
# ---------------------------------------------------------------------------

def path_bytes_per_token(H, D, in_bytes=2):
    """Minimum HBM traffic of the whole layer per unique token: forward reads
    q,k,v (bf16), g (fp32 per channel), beta, writes o (fp32); backward
    re-reads the inputs, reads dO (bf16), writes dq, dk, dv, dg (fp32), dbeta."""
    fwd = H * (3 * D * in_bytes + D * 4 + 4 + D * 4)
    bwd = H * (3 * D * in_bytes + D * 4 + 4 + D * in_bytes + 4 * D * 4 + 4)
    return fwd, bwd


# HBM bytes per launch of a kernel (mean over the launches of a call), from
# rocprofv3 FETCH_SIZE / WRITE_SIZE runs scaled by a plain device copy's counts
# (profiles/*_hbm_traffic.md).  A figure
# holds only for the kernel sources and workload it was measured on: the
# sources are hashed at run time and the figure is dropped when they differ.
# the kernel whose launches the headline's timed region carries events for
DOMINANT = "kda_bwd_chunk_grad"

MEASURED_TRAFFIC = {
    "kda_bwd_chunk_grad": {"sources": ("kda_grad.hip", "chunk.h", "common.h"),
                           "sha256_16": "d71ffa3564731483", "workload": 2,
                           "bytes_per_launch": 2196944092},
}


def measured_traffic(kernel, workload):
    import hashlib
    m = MEASURED_TRAFFIC.get(kernel)
    if m is None or m["workload"] != workload:
        return None
    csrc = os.path.join(ROOT, "tree_packed_chunkwise_amd", "csrc")
    h = hashlib.sha256()
    for f in m["sources"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return m["bytes_per_launch"] if h.hexdigest()[:16] == m["sha256_16"] else None


def image_bytes(B, D, in_bytes):
    """(image head, image as used) bytes of one chunk-head: the fp16 LDS
    image of a chunk step (layout in csrc/chunk.h); the head is everything
    but V."""
    head = 2 * (2 * B * D + D * B + 2 * B * B + B * 24) + 4 * D + 8 * B
    return head, head + in_bytes * B * D


def replay_ablation(dev, H=16, D=128):
    """Replay versus exact-fork-state starts, per handoff depth (the synthetic
    analogue of thelatestinai.com Figure 5): on a complete binary tree of
    depth 5 (segments of 64-256 tokens, bf16 inputs), the forward output of
    each plan mode against the trajectory-expanded run of the same kernels
    (every trajectory on its own B-aligned grid), as relative L2 over the rows
    at each handoff depth (side starts on the row's root path in the min-call
    plan)."""
    import torch
    from tree_packed_chunkwise_amd import binding as B
    from tree_packed_chunkwise_amd import synth
    rng = np.random.Generator(np.random.PCG64(55))
    spec = synth.tree_kary(2, 5, 64, 256, rng, name="binary_d5")
    n_rows = int(np.sum(spec.seg_len))
    inp = synth.make_kda_inputs_device(5500, n_rows, H, D, D, dev, True)
    outs, plans = {}, {}
    for name, mode in (("mincall", B.MINCALL), ("expanded", B.EXPANDED), ("noreplay", B.NOREPLAY),
                       ("nodewise", B.NODEWISE)):
        pl = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 64, mode)
        f = B.kda_tree_fwd(pl, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], None, inp["scale"])
        o = f["o"]
        if mode == B.EXPANDED:   # packed rows -> compact rows (identical copies)
            ri = torch.from_numpy(np.asarray(pl.export("ROW_INDEX"), np.int64)).to(dev)
            oc = torch.empty(n_rows, H, D, device=dev)
            oc[ri] = o
            o = oc
        outs[name], plans[name] = o.double(), pl
    torch.cuda.synchronize()
    p0 = plans["mincall"]
    cont, parent = p0.export("SEG_IS_CONT"), spec.parent
    hd = np.zeros(len(parent), np.int64)
    for v in range(len(parent)):   # parents precede children in id order here
        hd[v] = 0 if parent[v] < 0 else hd[parent[v]] + (0 if cont[v] else 1)
    row_hd = np.repeat(hd, spec.seg_len)
    res = {"tree": f"complete binary, depth 5, {len(parent)} segments, {n_rows} rows, "
                   f"{H} heads, d={D}, bf16, chunk 64",
           "reference": "trajectory-expanded run of the same kernels",
           "handoff_depth": list(range(int(row_hd.max()) + 1)),
           "rows": [int(np.sum(row_hd == d_)) for d_ in range(int(row_hd.max()) + 1)]}
    ref = outs["expanded"]
    for name in ("mincall", "noreplay", "nodewise"):
        errs = []
        for d_ in res["handoff_depth"]:
            sel = torch.from_numpy(np.nonzero(row_hd == d_)[0]).to(dev)
            a_, b_ = outs[name][sel], ref[sel]
            errs.append(float(torch.linalg.norm(a_ - b_) / torch.linalg.norm(b_)))
        res[f"{name}_rel_l2"] = [float(f"{e:.3e}") for e in errs]
    return res


def measure_window(w, dev, steps, ms_single):
    """A sharing window on the benchmark tree: the producer call holds the
    root and its children (depth <= 1), the 16 depth-2 subtrees run as 4
    consumer microbatches started from the producer's end states, and their
    start-state gradients accumulate before the producer backward.  Forward
    and backward of the whole window per step; ms_single is the single packed
    call on the same tree."""
    import torch
    from tree_packed_chunkwise_amd import synth
    from tree_packed_chunkwise_amd.window import SharingWindow
    try:
        win = SharingWindow(w.tree.parent, w.tree.seg_len, 1, 4, chunk=w.chunk)
    except ValueError as exc:   # e.g. a trunk tree with fewer than 4 subtrees below depth 1
        return {"skipped": str(exc)}
    N, H, D = win.n_rows, w.H, w.dk
    inp = synth.make_kda_inputs_device(9100, N, H, D, D, dev, w.bf16)
    gen = torch.Generator(device=dev)
    gen.manual_seed(9101)
    dO = torch.randn(N, H, D, device=dev, generator=gen).to(inp["q"].dtype)
    dhl = torch.randn(win.n_leaf, H, D, D, device=dev, generator=gen)

    def step():
        return win.run(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["scale"],
                       dO=dO, dh_leaf=dhl)
    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"producer": "depth <= 1 (5 segments), %d rows" % win.rows_p,
            "consumers": "16 depth-2 subtrees in 4 microbatches, rows %s" % [m["rows"] for m in win.micro],
            "ms_per_step": round(ms, 3), "unique_tokens_per_s": round(N / (ms / 1e3), 1),
            "vs_single_call": round(ms_single / ms, 3)}


def method_bytes(name, info, H, D, in_bytes=2):
    """Algorithmic bytes of all launches of a kernel class in one step, from
    the method's own inputs and outputs per row (path_bytes_per_token): the
    chunk-local gradient pass carries the reverse pass's input and output
    traffic (q, k, v, g, beta re-read, dO read, dq, dk, dv, dg, dbeta
    written) for every packed row (unique rows plus replayed rows); the
    chunk pass carries the forward's input reads (q, k, v, g, beta) and the
    forward rounds its output writes (o) plus the handoff and leaf states."""
    P, Nrow = info["n_packed"], info["n_rows"]
    fwd_b, bwd_b = path_bytes_per_token(H, D, in_bytes)
    st = D * D * 4 * H
    if name == "kda_bwd_chunk_grad":
        return P * bwd_b
    if name == "kda_chunk_decay":
        return P * H * (3 * D * in_bytes + D * 4 + 4)
    if name == "kda_fwd_round":
        return Nrow * H * D * 4 + (info["n_buf"] + info["n_leaf"]) * st
    return None


def kernel_bytes(name, info, H, D, in_bytes=2):
    """Bytes of all launches of one kernel class in one step under this
    design: what its role reads and writes once, including the design's own
    intermediates (chunk images, fp16 per-chunk states, dy, dO tiles;
    documented per kernel in the design doc).  P = packed rows (unique rows +
    replayed rows), C = chunks, per head; states are D x D fp32."""
    P = info["n_packed"]
    Nrow = info["n_rows"]
    C = info["n_chunks"]
    B = info["chunk"]
    f = 4
    st = D * D * f                        # one state of one head
    st16 = D * D * 2                      # the fp16 copies kept per chunk
    head, fimg = image_bytes(B, D, in_bytes)
    if name == "kda_chunk_decay":
        # reads q, k, v, g, beta; writes the chunk images
        return P * H * (3 * D * in_bytes + D * f + f) + C * H * fimg
    if name == "kda_fwd_round":
        # reads the chunk images; writes o (unique rows), the start state of
        # every chunk, handoff and leaf states
        return (C * H * fimg + Nrow * H * D * f + C * H * st16
                + (info["n_buf"] + info["n_leaf"]) * H * st)
    if name == "kda_bwd_round":
        # reads the image heads, packed dO, leaf-state gradients; writes dy
        # (fp16), the end-state gradient of every chunk, sequence start
        # gradients
        return (C * H * head + P * H * D * (in_bytes + 2) + C * H * st16
                + (info["n_seq"] + info["n_leaf"]) * H * st)
    if name == "kda_bwd_chunk_grad":
        # reads q, k, g, beta, dy (fp16), packed dO, A / Td / V of the chunk
        # image, the start state and end-state gradient of every chunk;
        # writes dq, dk, dv, dg, dbeta
        return (P * H * (2 * D * in_bytes + D * f + f + D * 2 + D * in_bytes + 4 * D * f + f)
                + C * H * ((B * B + B * 24) * 2 + B * D * in_bytes + 2 * st16))
    if name == "kda_bwd_gather_dO":
        return Nrow * H * D * in_bytes + P * H * D * in_bytes
    return None


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def _oracle_head(args):
    sub_parent, sub_len, q, k, v, g, beta, dO, dhl, scale = args
    from oracle import kda as okda
    from oracle.tree import Tree
    t = Tree(sub_parent, sub_len)
    h0 = np.zeros((1, 1, q.shape[2], v.shape[2]))
    okda.tree_fwd(t, q, k, v, g, beta, h0, scale)
    okda.tree_bwd(t, q, k, v, g, beta, h0, scale, dO, dhl)
    return True


def cpu_baseline(spec, inp, dO, dhl_full, H, leaves):
    """Oracle forward + backward, all heads (one process per head), on the
    subtree root -> first child -> first grandchild -> its leaves."""
    import multiprocessing as mp
    from oracle.tree import Tree
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    keep = [t.roots[0]]
    c1 = t.children[keep[0]][0]
    c2 = t.children[c1][0]
    keep += [c1, c2]
    stack = list(t.children[c2])
    while stack:
        v = stack.pop()
        keep.append(v)
        stack.extend(t.children[v])
    keep = sorted(keep)
    idx = {v: i for i, v in enumerate(keep)}
    sub_parent = np.array([-1 if t.parent[v] < 0 else idx[int(t.parent[v])] for v in keep])
    sub_len = np.array([int(t.seg_len[v]) for v in keep])
    rows = np.concatenate([t.seg_rows(v) for v in keep])
    sub_leaves = [v for v in keep if not t.children[v]]
    li = [leaves.index(v) for v in sub_leaves]
    n_sub = len(rows)
    cores = min(16, os.cpu_count() or 1)
    tasks = []
    for h in range(H):
        sl = lambda a: np.ascontiguousarray(a[rows][:, h:h + 1], dtype=np.float64)
        tasks.append((sub_parent, sub_len, sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.g),
                      np.ascontiguousarray(inp.beta[rows][:, h:h + 1], dtype=np.float64),
                      sl(dO), np.ascontiguousarray(dhl_full[li][:, h:h + 1], dtype=np.float64),
                      inp.scale))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        pool.map(_oracle_head, tasks)
    wall = time.perf_counter() - t0
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": n_sub / wall, "unit": "unique tokens/s", "cores": cores, "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": model,
            "sample": (f"float64 numpy oracle forward+backward of all {H} heads (one process "
                       f"per head, {cores} workers) on a {n_sub}-row subtree of the workload "
                       f"tree (root, its first child and first grandchild, and that "
                       f"grandchild's {len(sub_leaves)} leaves); {wall:.1f} s wall")}


# ---------------------------------------------------------------------------
# the config-4 pieces: tree attention (matrix-core bound) and the hybrid group
# ---------------------------------------------------------------------------

def attention_pairs(plan, seg_len):
    """(query, key) pairs of the ancestor mask, per head."""
    seg_len = np.asarray(seg_len, dtype=np.int64)
    ptr = plan.export("ATT_ANC_PTR")
    anc = plan.export("ATT_ANC")
    pairs = 0
    for v in range(len(seg_len)):
        a_rows = int(seg_len[anc[ptr[v]:ptr[v + 1]]].sum())
        pairs += int(seg_len[v]) * a_rows + int(seg_len[v]) * (int(seg_len[v]) + 1) // 2
    return pairs


def measure_attention(steps):
    """Tree attention forward and backward on the hybrid group's tree (the
    4-ary depth-3 tree of the forward workload), 16 heads, d = 128, bf16.
    Algorithmic FLOPs: 4 d per (query, key) pair and head forward (QK^T and
    PV), 10 d backward (recomputed QK^T, dP, dV, dK, dQ)."""
    import torch
    from tree_packed_chunkwise_amd import binding as B
    from tree_packed_chunkwise_amd import synth
    try:
        w = synth.workload(4)
        plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, 64)
        N, H, D = plan.info["n_rows"], 16, 128
        pairs = attention_pairs(plan, w.tree.seg_len)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(11)
        mk = lambda: torch.randn(N, H, D, generator=gen, device="cuda").to(torch.bfloat16)
        q, k, v, dO = mk(), mk(), mk(), mk()
        o, lse = B.tree_attn_fwd(plan, q, k, v)
        dq, dk, dv = B.tree_attn_bwd(plan, q, k, v, o, lse, dO)
        torch.cuda.synchronize()
        B.timing_enable(True)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        for _ in range(steps):
            B.tree_attn_fwd(plan, q, k, v, out=(o, lse))
        e[1].record()
        for _ in range(steps):
            B.tree_attn_bwd(plan, q, k, v, o, lse, dO, out=(dq, dk, dv))
        e[2].record()
        torch.cuda.synchronize()
        kt = B.timing_read()
        B.timing_enable(False)
        fms, bms = e[0].elapsed_time(e[1]) / steps, e[1].elapsed_time(e[2]) / steps
        ff, bf = 4 * pairs * D * H, 10 * pairs * D * H
        kern = {n: round(ms / max(c, 1), 4) for n, (c, ms) in kt.items()}
        fa = ff / (kern.get("tree_attn_fwd", fms) * 1e-3) / 1e12
        return {"workload": f"{w.tree.name} tree, {N} rows, 16 heads, d=128, bf16",
                "pairs_per_head": pairs, "fwd_ms": round(fms, 3), "bwd_ms": round(bms, 3),
                "roofline": {"bound": "mfma", "kernel": "tree_attn_fwd", "achieved": round(fa, 1),
                             "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(fa / BF16_PEAK_TFLOPS, 4), "traffic": None},
                "bwd_tflops": round(bf / (bms * 1e-3) / 1e12, 1),
                "kernel_avg_ms": kern, "finite": bool(torch.isfinite(o).all())}
    except Exception as exc:  # reported, never fatal to the headline line
        return {"error": repr(exc)}


def measure_router(steps):
    """Occurrence-weighted MoE router statistics (forward: loads, probability
    and z-loss sums, top-8 per row; reverse: logit gradients) over the compact
    rows of the fwd+bwd workload's tree, 128 experts, bf16 logits; and the
    same kernels over the trajectory-expanded rows (every position routed,
    count 1) for comparison.  Algorithmic bytes: forward reads the logits
    (2 B x 128) and the count (4 B) of every row and writes its top-8 indices
    and probabilities (64 B); reverse reads logits and count and writes fp32
    gradients (512 B)."""
    import torch
    from tree_packed_chunkwise_amd import binding as B
    from tree_packed_chunkwise_amd import synth
    try:
        w = synth.workload(2)
        plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, 64)
        N, E, K = plan.info["n_rows"], 128, 8
        gen = torch.Generator(device="cuda")
        gen.manual_seed(13)
        x = (2 * torch.randn(N, E, generator=gen, device="cuda")).to(torch.bfloat16)
        g = torch.randn(E, generator=gen, device="cuda")
        q = plan.device_table("ROW_MULT")
        # trajectory-expanded rows: every root-to-leaf path in position order
        par, ln, r0 = (np.asarray(a, np.int64) for a in (w.tree.parent, w.tree.seg_len, w.tree.seg_row))
        rows = []
        for leaf in plan.export("LEAF_SEG"):
            path, v = [], int(leaf)
            while v >= 0:
                path.append(v)
                v = int(par[v])
            rows.append(np.concatenate([np.arange(r0[s], r0[s] + ln[s]) for s in reversed(path)]))
        rows = torch.from_numpy(np.concatenate(rows)).cuda()
        xe = x.index_select(0, rows).contiguous()
        qe = torch.ones(xe.shape[0], dtype=torch.int32, device="cuda")

        def timed(xx, qq):
            out = B.moe_router_stats(xx, qq, K)
            dx = B.moe_router_stats_bwd(xx, qq, g, 0.1)
            torch.cuda.synchronize()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            for _ in range(steps):
                B.moe_router_stats(xx, qq, K)
            e[1].record()
            for _ in range(steps):
                B.moe_router_stats_bwd(xx, qq, g, 0.1, out=dx)
            e[2].record()
            torch.cuda.synchronize()
            return out, e[0].elapsed_time(e[1]) / steps, e[1].elapsed_time(e[2]) / steps
        out, fms, bms = timed(x, q)
        oute, fe, be = timed(xe, qe)
        same = bool(torch.equal(out["load"], oute["load"]) and torch.equal(out["n_tok"], oute["n_tok"]))
        fb, bb = N * (E * 2 + 4 + K * 8), N * (E * 2 + 4 + E * 4)
        return {"workload": f"{w.tree.name} tree, {N} rows, {int(xe.shape[0])} positions, "
                            f"{E} experts, top-{K}, bf16 logits",
                "fwd_ms": round(fms, 4), "bwd_ms": round(bms, 4),
                "fwd_GBps": round(fb / (fms * 1e-3) / 1e9, 1),
                "bwd_GBps": round(bb / (bms * 1e-3) / 1e9, 1),
                "expanded_fwd_ms": round(fe, 4), "expanded_bwd_ms": round(be, 4),
                "speedup": round((fe + be) / (fms + bms), 3),
                "loads_equal_expanded": same}
    except Exception as exc:  # reported, never fatal to the headline line
        return {"error": repr(exc)}


def measure_l1(seed=17):
    """Compression-oriented microbatches (kda_l1_plan, host) for a synthetic
    rollout batch: 48 trees shaped like the workload trees (4-ary, depth 2 or
    3, segments of U{256..2048} tokens), 64k-token microbatch budget.  The
    bound is the forest's own compression (no tree cut)."""
    import time as _t
    from tree_packed_chunkwise_amd import binding as B
    from tree_packed_chunkwise_amd import synth
    try:
        rng = np.random.Generator(np.random.PCG64(seed))
        parents, lens = [], []
        for i in range(48):
            spec = synth.tree_kary(4, 2 + (i % 2), 256, 2048, rng)
            off = len(parents)
            parents += [int(p) + off if p >= 0 else -1 for p in spec.parent]
            lens += [int(x) for x in spec.seg_len]
        budget = 65536
        t0 = _t.perf_counter()
        r = B.l1_plan(parents, lens, budget)
        ms = (_t.perf_counter() - t0) * 1e3
        par = np.asarray(parents)
        ln = np.asarray(lens, np.int64)
        endp = np.zeros(len(par), np.int64)
        for v in range(len(par)):   # parents precede children here
            endp[v] = (endp[par[v]] if par[v] >= 0 else 0) + ln[v]
        leaf = np.ones(len(par), bool)
        leaf[par[par >= 0]] = False
        return {"workload": f"48 trees (4-ary, depth 2-3, U{{256..2048}}), {int(ln.sum())} unique "
                            f"tokens, {int(endp[leaf].sum())} trajectory tokens, budget {budget}",
                "microbatches": int(len(r["unique"])), "compression": round(r["compression"], 4),
                "balance": round(r["balance"], 4),
                "bound": round(float(endp[leaf].sum() / ln.sum()), 4),
                "plan_ms": round(ms, 3)}
    except Exception as exc:  # reported, never fatal to the headline line
        return {"error": repr(exc)}


def measure_hybrid(steps):
    """The hybrid layer group (3 KDA layers, tree attention, log-prob gather,
    hidden 2048, vocab 32000, bf16) forward + backward on the same tree."""
    import torch
    from tree_packed_chunkwise_amd import binding as B
    from tree_packed_chunkwise_amd import synth
    from tree_packed_chunkwise_amd.hybrid import HybridGroup, gather_maps
    try:
        w = synth.workload(4)
        plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, 64)
        N = plan.info["n_rows"]
        model = HybridGroup(2048, 16, 128, 32000, n_kda=3, seed=0, dtype=torch.bfloat16,
                            device="cuda")
        gen = torch.Generator(device="cuda")
        gen.manual_seed(12)
        tokens = torch.randint(0, 32000, (N,), generator=gen, device="cuda")
        maps = gather_maps(plan, tokens, "cuda")
        dlogp = torch.randn(plan.info["n_pos"], generator=gen, device="cuda")

        def step():
            model.zero_grad(set_to_none=True)
            logp = model(plan, tokens, maps)
            (logp * dlogp).sum().backward()
        step()
        torch.cuda.synchronize()
        B.timing_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        kt = B.timing_read()
        B.timing_enable(False)
        ms = e0.elapsed_time(e1) / steps
        tree_ms = sum(t for _, t in kt.values()) / steps
        return {"workload": f"{w.tree.name} tree, {N} rows, {plan.info['n_pos']} positions, "
                            "hidden 2048, 16 heads d=128, vocab 32000, bf16",
                "ms_per_step": round(ms, 2), "unique_tokens_per_s": round(N / (ms * 1e-3), 1),
                "tree_kernels_ms": round(tree_ms, 2),
                "dense_and_torch_ms": round(ms - tree_ms, 2)}
    except Exception as exc:
        return {"error": repr(exc)}


def expanded_batched(w, dev, steps, n_exp_rows, need_bytes, scale):
    """Trajectory-expanded execution in batches of whole trajectories that
    fit in device memory, times summed: each batch is the forest of its
    trajectories' root paths run in EXPANDED mode (every trajectory its own
    full-prefix sequence), on fresh inputs of the same distributions (the
    timing does not depend on the values).  Returns (ms per step, batches)."""
    import torch
    from tree_packed_chunkwise_amd import binding as B
    from tree_packed_chunkwise_amd import synth
    H, D = w.H, w.dk
    dt = torch.bfloat16 if w.bf16 else torch.float32
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    par = np.asarray(w.tree.parent)
    lens = np.asarray(w.tree.seg_len, np.int64)
    has_child = np.zeros(len(par), bool)
    has_child[par[par >= 0]] = True
    paths = []
    for leaf in np.nonzero(~has_child)[0]:
        p, x = [], int(leaf)
        while x >= 0:
            p.append(x)
            x = int(par[x])
        paths.append(p[::-1])
    free, _ = torch.cuda.mem_get_info(dev)
    cap = max(1, int(0.7 * free / (need_bytes / n_exp_rows)))   # expanded rows per batch
    batches, cur, rows = [], [], 0
    for p in paths:
        t = int(lens[p].sum())
        if cur and rows + t > cap:
            batches.append(cur)
            cur, rows = [], 0
        cur.append(p)
        rows += t
    batches.append(cur)
    total = 0.0
    for bi, bp in enumerate(batches):
        segs = sorted({x for p in bp for x in p})
        idx = {x: j for j, x in enumerate(segs)}
        sp = np.array([idx[int(par[x])] if par[x] >= 0 else -1 for x in segs], np.int32)
        sl = lens[segs].astype(np.int32)
        bplan = B.KDAPlan(sp, sl, None, w.chunk, B.EXPANDED)
        bi_ = bplan.info
        bin_ = synth.make_kda_inputs_device(7700 + bi, int(sl.sum()), H, D, D, dev, w.bf16)
        mg = torch.Generator(device=dev)
        mg.manual_seed(7800 + bi)
        dOb = torch.randn((bi_["n_out_rows"], H, D), device=dev, generator=mg).to(dt)
        dhb = torch.randn((bi_["n_leaf"], H, D, D), device=dev, generator=mg)
        bfo = B.alloc_fwd(bplan, H, D, dev)
        bbo = B.alloc_bwd(bplan, H, D, dev)

        def bstep():
            B.kda_tree_fwd(bplan, bin_["q"], bin_["k"], bin_["v"], bin_["g"], bin_["beta"],
                           None, scale, out=bfo)
            B.kda_tree_bwd(bplan, bin_["q"], bin_["k"], bin_["v"], bin_["g"], bin_["beta"],
                           bfo["saved"], dOb, dhb, None, scale, out=bbo)
        bstep()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            bstep()
        e1.record()
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1) / steps
        del bfo, bbo, dOb, dhb, bin_
        torch.cuda.empty_cache()
    return total, len(batches)


def expanded_need_bytes(w):
    """Device bytes of one EXPANDED call of the whole tree (outputs, saved
    state, workspaces, and the expanded copies of the inputs)."""
    from tree_packed_chunkwise_amd import binding as B
    H, D = w.H, w.dk
    ep = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk, B.EXPANDED)
    ei = ep.info
    need = (ep.saved_bytes(H, D) + ep.fwd_ws_bytes(H, D) + ep.bwd_ws_bytes(H, D)
            + ei["n_out_rows"] * H * D * (5 * 4 + 2) + ei["n_packed"] * H * D * 14)
    return need, ei


def _timed(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def measure_config_forward(dev, steps, warmup):
    """The forward-only workload on its own tree (complete 4-ary tree of depth
    3 drawn with seed 1, U{256..2048} segments), one KDA layer forward, 16
    heads, d = 128, bf16 q/k/v: unique tokens/s and the forward's roofline
    (28,736 B per unique token at 16 heads plus the handoff and leaf
    states)."""
    import torch
    from tree_packed_chunkwise_amd import binding as B
    from tree_packed_chunkwise_amd import synth
    try:
        w = synth.workload(1)
        H, D = w.H, w.dk
        plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk)
        info = plan.info
        N = info["n_rows"]
        inp = synth.make_kda_inputs_device(7300, N, H, D, D, dev, w.bf16)
        fo = B.alloc_fwd(plan, H, D, dev)
        fwd = lambda: B.kda_tree_fwd(plan, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                                     None, inp["scale"], out=fo)
        ms = _timed(fwd, steps, warmup)
        fwd_b, _ = path_bytes_per_token(H, D, 2)
        byts = N * fwd_b + (info["n_buf"] + info["n_leaf"]) * H * D * D * 4
        ach = byts / (ms * 1e-3) / 1e9
        return {"workload": w.name, "unique_rows": N, "expanded_rows": int(info["n_expanded"]),
                "rounds": int(info["n_rounds"]), "replay_rows": int(info["R"]),
                "ms_per_step": round(ms, 4), "unique_tokens_per_s": round(N / (ms * 1e-3), 1),
                "path_roofline": {"bound": "hbm", "bytes_per_step": int(byts),
                                  "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(ach / HBM_PEAK_GBS, 5)},
                "finite": bool(torch.isfinite(fo["o"]).all())}
    except Exception as exc:  # reported, never fatal to the headline line
        return {"error": repr(exc)}


def measure_config_stepwise(dev, steps, warmup, expanded_steps):
    """The step-wise workload: 32,768-token trunk with 256 branches of 1-6
    segments (U{128..1024} tokens), one KDA layer forward + backward, 16
    heads, d = 128, bf16: unique tokens/s, the path roofline (86,208 B per
    unique token plus states), and the speedup over trajectory-expanded
    execution of the same tree (batched to fit device memory)."""
    import torch
    from tree_packed_chunkwise_amd import binding as B
    from tree_packed_chunkwise_amd import synth
    try:
        w = synth.workload(3)
        H, D = w.H, w.dk
        plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk)
        info = plan.info
        N = info["n_rows"]
        inp = synth.make_kda_inputs_device(7400, N, H, D, D, dev, w.bf16)
        gen = torch.Generator(device=dev)
        gen.manual_seed(7401)
        dO = torch.randn(N, H, D, generator=gen, device=dev).to(torch.bfloat16)
        dhl = torch.randn(info["n_leaf"], H, D, D, generator=gen, device=dev)
        fo = B.alloc_fwd(plan, H, D, dev)
        bo = B.alloc_bwd(plan, H, D, dev)

        def step():
            B.kda_tree_fwd(plan, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], None,
                           inp["scale"], out=fo)
            B.kda_tree_bwd(plan, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], fo["saved"],
                           dO, dhl, None, inp["scale"], out=bo)
        ms = _timed(step, steps, warmup)
        ok = bool(torch.isfinite(fo["o"]).all() and torch.isfinite(bo["dq"]).all())
        fwd_b, bwd_b = path_bytes_per_token(H, D, 2)
        st = H * D * D * 4
        byts = N * (fwd_b + bwd_b) + (info["n_buf"] + info["n_leaf"]) * 2 * st
        ach = byts / (ms * 1e-3) / 1e9
        res = {"workload": w.name, "unique_rows": N, "expanded_rows": int(info["n_expanded"]),
               "rounds": int(info["n_rounds"]), "replay_rows": int(info["R"]),
               "sequences": int(info["n_seq"]),
               "ms_per_step": round(ms, 4), "unique_tokens_per_s": round(N / (ms * 1e-3), 1),
               "path_roofline": {"bound": "hbm", "bytes_per_step": int(byts),
                                 "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(ach / HBM_PEAK_GBS, 5)},
               "finite": ok}
        del fo, bo, dO, dhl, inp
        torch.cuda.empty_cache()
        if expanded_steps > 0:
            need, ei = expanded_need_bytes(w)
            ems, nb = expanded_batched(w, dev, expanded_steps, int(ei["n_packed"]), need,
                                       1.0 / float(np.sqrt(D)))
            res["expanded"] = {"ms_per_step": round(ems, 3), "speedup": round(ems / ms, 3),
                               "expanded_rows": int(ei["n_packed"]), "batches": nb,
                               "note": "trajectory batches that fit device memory, times summed"}
        return res
    except Exception as exc:  # reported, never fatal to the headline line
        return {"error": repr(exc)}


def measure_gather(steps):
    """gather_logprobs and its backward at vocabulary 32000 over the compact
    rows of the hybrid workload's tree (bf16 logits, every trajectory
    position): HBM-bound, the forward reads every logit once (plus the
    position tables and outputs), the backward reads the logits and writes
    their gradients once."""
    import torch
    from tree_packed_chunkwise_amd import binding as B
    from tree_packed_chunkwise_amd import synth
    try:
        w = synth.workload(4)
        plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, 64)
        N, V, P = plan.info["n_rows"], 32000, plan.info["n_pos"]
        gen = torch.Generator(device="cuda")
        gen.manual_seed(14)
        z = (3 * torch.randn(N, V, generator=gen, device="cuda")).to(torch.bfloat16)
        tokens = torch.randint(0, V, (N,), generator=gen, device="cuda")
        pos_row = plan.device_table("POS_ROW")
        tgt = tokens[plan.device_table("POS_NEXT_ROW").long()].to(torch.int32).contiguous()
        rp_ptr, rp_idx = plan.device_table("ROW_POS_PTR"), plan.device_table("ROW_POS_IDX")
        dlogp = torch.randn(P, generator=gen, device="cuda")
        logp, lse = B.gather_logprobs(z, pos_row, tgt)
        dz = B.gather_logprobs_bwd(z, lse, rp_ptr, rp_idx, tgt, dlogp)
        fms = _timed(lambda: B.gather_logprobs(z, pos_row, tgt, out=(logp, lse)), steps, 1)
        bms = _timed(lambda: B.gather_logprobs_bwd(z, lse, rp_ptr, rp_idx, tgt, dlogp, out=dz),
                     steps, 1)
        fb = N * V * 2 + P * 12 + N * 4          # logits; pos_row, target, logp; lse
        bb = 2 * N * V * 2 + N * 8 + P * 12      # logits in, gradients out; lse, CSR; dlogp, ...
        fa, ba = fb / (fms * 1e-3) / 1e9, bb / (bms * 1e-3) / 1e9
        roof = lambda a_, b_: {"bound": "hbm", "achieved": round(a_, 1), "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": round(a_ / HBM_PEAK_GBS, 4),
                               "bytes_per_launch": int(b_)}
        return {"workload": f"{w.tree.name} tree, {N} rows, {P} positions, vocab {V}, bf16 logits",
                "fwd_ms": round(fms, 4), "bwd_ms": round(bms, 4),
                "fwd_roofline": roof(fa, fb), "bwd_roofline": roof(ba, bb),
                "expanded_logit_bytes_avoided": int((P - N) * V * 2)}
    except Exception as exc:  # reported, never fatal to the headline line
        return {"error": repr(exc)}


# ---------------------------------------------------------------------------

def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {a.gpus})", file=sys.stderr)
        sys.exit(2)
    if a.copy_calibration:
        copy_calibration()
        return
    import torch
    from tree_packed_chunkwise_amd import binding as B
    from tree_packed_chunkwise_amd import synth

    w = synth.workload(a.workload)
    H, D = w.H, w.dk
    rng = synth.workload_rng(w)
    t0 = time.perf_counter()
    plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk)
    plan_host_ms = (time.perf_counter() - t0) * 1e3
    info = plan.info
    N = info["n_rows"]
    inp = synth.make_kda_inputs(rng, N, H, D, D, bf16=w.bf16)
    dO_np, dhl_np = synth.make_upstream(rng, N, info["n_leaf"], H, D, D, bf16=w.bf16)
    # the CPU baseline runs first, in forked workers, before anything touches the GPU
    cpu = None
    if not a.no_cpu_baseline:
        _progress("cpu baseline (oracle)")
        cpu = cpu_baseline(w.tree, inp, dO_np, dhl_np, H, list(plan.export("LEAF_SEG")))
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.bf16 else torch.float32
    f = lambda x, d: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(dev).to(d)
    q, k, v = f(inp.q, dt), f(inp.k, dt), f(inp.v, dt)
    g, beta = f(inp.g, torch.float32), f(inp.beta, torch.float32)
    dO, dhl = f(dO_np, dt), f(dhl_np, torch.float32)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    plan.device(dev)
    torch.cuda.synchronize()
    upload_ms = (time.perf_counter() - t0) * 1e3

    fo = B.alloc_fwd(plan, H, D, dev)
    bo = B.alloc_bwd(plan, H, D, dev)

    def step():
        B.kda_tree_fwd(plan, q, k, v, g, beta, None, inp.scale, out=fo)
        B.kda_tree_bwd(plan, q, k, v, g, beta, fo["saved"], dO, dhl, None, inp.scale, out=bo)

    _progress(f"headline: {a.warmup} warmup + {a.steps} timed steps")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    if not a.no_timing:
        # inside the headline's timed region only the dominant kernel (the
        # chunk-local gradients) carries timing events
        B.timing_enable(True, only=DOMINANT)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(a.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    kt, kt_all, all_steps = {}, {}, 3
    if not a.no_timing:
        kt = B.timing_read()
        # every kernel, over a few more steps of the same schedule
        B.timing_enable(True)
        for _ in range(all_steps):
            step()
        torch.cuda.synchronize()
        kt_all = B.timing_read()
        B.timing_enable(False)

    # fwd / bwd split (one extra step each, untimed for the headline)
    ef = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ef[0].record()
    B.kda_tree_fwd(plan, q, k, v, g, beta, None, inp.scale, out=fo)
    ef[1].record()
    B.kda_tree_bwd(plan, q, k, v, g, beta, fo["saved"], dO, dhl, None, inp.scale, out=bo)
    ef[2].record()
    torch.cuda.synchronize()
    fwd_ms, bwd_ms = ef[0].elapsed_time(ef[1]), ef[1].elapsed_time(ef[2])
    ok = bool(torch.isfinite(fo["o"]).all() and torch.isfinite(bo["dq"]).all())

    # the same step with every kernel on the caller's stream (no overlap of the
    # chunk passes with the round chains): per-kernel times without sharing
    # the GPU, and the step time of that schedule
    kt_seq, seq_ms = {}, None
    if not a.no_timing:
        B.set_overlap(False)
        try:
            step()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(2):
                step()
            e1.record()
            torch.cuda.synchronize()
            seq_ms = e0.elapsed_time(e1) / 2
            B.timing_enable(True)
            for _ in range(2):
                step()
            torch.cuda.synchronize()
            kt_seq = B.timing_read()
            B.timing_enable(False)
        finally:
            B.set_overlap(True)

    value = N / (ms * 1e-3)
    fwd_b, bwd_b = path_bytes_per_token(H, D, 2 if w.bf16 else 4)
    st = H * D * D * 4
    extra = (info["n_buf"] * 2 * st + info["n_leaf"] * 2 * st)  # handoff and leaf states + grads
    step_bytes = N * (fwd_b + bwd_b) + extra
    path_frac = (step_bytes / (ms * 1e-3)) / (HBM_PEAK_GBS * 1e9)

    roof = None
    kernels = {}
    if kt_all:
        for name, (cnt, tot) in kt_all.items():
            kernels[name] = {"launches_per_step": cnt / all_steps, "ms_per_step": tot / all_steps,
                             "avg_launch_ms": tot / max(cnt, 1)}
        dom = max(kernels, key=lambda n: kernels[n]["ms_per_step"])
        # the dominant kernel's launches as timed inside the headline region
        # (the separate pass's figures if another kernel dominates)
        live = dom in kt
        cnt, tot = kt[dom] if live else kt_all[dom]
        nst = a.steps if live else all_steps
        kb = method_bytes(dom, info, H, D, 2 if w.bf16 else 4)
        kd = kernel_bytes(dom, info, H, D, 2 if w.bf16 else 4)
        if kb is not None:
            lps = cnt / nst
            avg = tot / max(cnt, 1)
            per_launch = kb / lps
            achieved = per_launch / (avg * 1e-3) / 1e9
            roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5),
                    "traffic": measured_traffic(dom, a.workload), "bytes_per_launch": int(per_launch),
                    "design_bytes_per_launch": int(kd / lps) if kd is not None else None,
                    "avg_launch_ms": round(avg, 4), "launches_per_step": lps,
                    "timed": "headline region" if live else "separate pass"}
            if dom in kt_seq:
                cnt_s, tot_s = kt_seq[dom]
                ms_s = tot_s / 2   # per step
                roof["single_stream"] = {
                    "ms_per_step": round(ms_s, 4), "achieved": round(kb / (ms_s * 1e-3) / 1e9, 2),
                    "frac": round(kb / (ms_s * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                    "step_ms": round(seq_ms, 4)}

    # the same tree and kernels under the other plan modes: trajectory-expanded
    # execution (no sharing), and the two exact-fork-state ablations of the
    # replay rule (no-replay: min-call packing with cut chunk grids;
    # node-wise: one sequence per segment)
    def time_mode(mode, steps, seed):
        mplan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk, mode)
        mi = mplan.info
        mg = torch.Generator(device=dev)
        mg.manual_seed(seed)
        dOm = torch.randn((mi["n_out_rows"], H, D), device=dev, generator=mg).to(dt)
        mfo = B.alloc_fwd(mplan, H, D, dev)
        mbo = B.alloc_bwd(mplan, H, D, dev)

        def mstep():
            B.kda_tree_fwd(mplan, q, k, v, g, beta, None, inp.scale, out=mfo)
            B.kda_tree_bwd(mplan, q, k, v, g, beta, mfo["saved"], dOm, dhl, None, inp.scale,
                           out=mbo)
        mstep()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            mstep()
        e1.record()
        torch.cuda.synchronize()
        mms = e0.elapsed_time(e1) / steps
        del mfo, mbo, dOm
        return mms, mi

    def fits(mode):
        """Whether the plan mode's outputs and workspaces fit in free device
        memory (the trajectory-expanded run of the step-wise tree does not:
        ~4.8 M rows)."""
        mp = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk, mode)
        mi = mp.info
        rows = mi["n_out_rows"] * H * D
        need = (mp.saved_bytes(H, D) + mp.fwd_ws_bytes(H, D) + mp.bwd_ws_bytes(H, D)
                + rows * (5 * 4 + 2))   # o, dq, dk, dv, dg (fp32) and dO (bf16)
        free, _ = torch.cuda.mem_get_info(dev)
        return need < 0.9 * free, mi

    expanded, modes = None, None
    if a.expanded_steps > 0:
        _progress("trajectory-expanded run and plan modes")
        ok_e, ei = fits(B.EXPANDED)
        if ok_e:
            ems, ei = time_mode(B.EXPANDED, a.expanded_steps, 7)
            expanded = {"ms_per_step": round(ems, 3), "speedup": round(ems / ms, 3),
                        "expanded_rows": int(ei["n_packed"])}
        else:
            need, ei = expanded_need_bytes(w)
            ems, nb = expanded_batched(w, dev, a.expanded_steps, int(ei["n_packed"]), need,
                                       inp.scale)
            expanded = {"ms_per_step": round(ems, 3), "speedup": round(ems / ms, 3),
                        "expanded_rows": int(ei["n_packed"]),
                        "batches": nb, "note": "trajectory batches that fit device memory, "
                                                "times summed"}
        modes = {"mincall": {"ms_per_step": round(ms, 3), "rounds": int(info["n_rounds"]),
                             "sequences": int(info["n_seq"]), "chunks": int(info["n_chunks"]),
                             "replay_rows": int(info["R"])}}
        for name, mode in (("noreplay", B.NOREPLAY), ("nodewise", B.NODEWISE),
                           ("mincall_short", B.MINCALL_SHORT)):
            if not fits(mode)[0]:
                modes[name] = {"skipped": "does not fit in device memory in one call"}
                continue
            mms, mi = time_mode(mode, a.expanded_steps, 9)
            modes[name] = {"ms_per_step": round(mms, 3), "rounds": int(mi["n_rounds"]),
                           "sequences": int(mi["n_seq"]), "chunks": int(mi["n_chunks"]),
                           "replay_rows": int(mi["R"]),
                           "unique_tokens_per_s": round(N / (mms / 1e3), 1)}

    _progress("replay ablation, sharing window, attention, router, L1, hybrid group")
    ablation = replay_ablation(dev) if a.expanded_steps > 0 else None
    window = measure_window(w, dev, a.expanded_steps, ms) if a.expanded_steps > 0 else None
    attention = measure_attention(a.attn_steps) if a.attn_steps > 0 else None
    router = measure_router(10) if a.attn_steps > 0 else None
    l1plan = measure_l1()
    hybrid = measure_hybrid(a.hybrid_steps) if a.hybrid_steps > 0 else None
    del fo, bo
    torch.cuda.empty_cache()
    cfg_fwd = cfg_step = gather = None
    if a.workload == 2 and a.extra_configs:
        _progress("forward-only workload")
        cfg_fwd = measure_config_forward(dev, a.steps, a.warmup)
        _progress("step-wise workload")
        cfg_step = measure_config_stepwise(dev, max(3, a.steps // 4), 1, a.expanded_steps)
        _progress("gather at vocabulary 32000")
        gather = measure_gather(5)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "unique tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "tree": w.tree.name, "heads": H, "d": D,
                   "chunk": w.chunk, "unique_rows": N, "expanded_rows": int(info["n_expanded"]),
                   "rounds": info["n_rounds"], "replay_rows": int(info["R"]),
                   "seq_per_round": [int(x) for x in np.diff(plan.export("ROUND_SEQ_PTR"))],
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "path_roofline": {"bound": "hbm", "bytes_per_step": int(step_bytes),
                          "achieved": round(step_bytes / (ms * 1e-3) / 1e9, 2),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(path_frac, 5)},
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4),
        "plan_host_ms": round(plan_host_ms, 3), "plan_upload_ms": round(upload_ms, 3),
        "expanded": expanded, "plan_modes": modes, "sharing_window": window,
        "replay_ablation": ablation,
        "kernels": kernels,
        "kernels_single_stream": {n: {"launches_per_step": c / 2, "ms_per_step": round(t / 2, 4)}
                                  for n, (c, t) in sorted(kt_seq.items())},
        "finite": ok,
        "tree_attention": attention, "hybrid_group": hybrid, "moe_router": router, "l1_planner": l1plan,
        "config_forward": cfg_fwd, "config_stepwise": cfg_step, "gather": gather,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
