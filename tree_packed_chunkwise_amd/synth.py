"""Seeded synthetic workloads: rollout-tree shapes and per-row input tensors.

This module is shared by the tests, the benchmark and the smoke check. It
holds no arithmetic of the method itself (no recurrence, no planning, no
log-softmax): only tree shapes, random draws and input-format rounding.

Tree shapes stand in for the agentic rollout trees of the HARTS pages
(arXiv 2608.28158, abstract: "irregular rollout trees"; Figure 1(a): boxes
are contiguous token ranges shared by several trajectories).  No benchmark
item (SWE-bench, tau^3-Bench) is reproduced: every token, length and value
is drawn from a seeded PCG64 generator.

A tree is given as three arrays, in segment-id order:
  parent[i]  parent segment id, -1 for a root
  seg_len[i] number of tokens of segment i (> 0)
  seg_row[i] first compact row of segment i (segments occupy disjoint,
             contiguous row ranges; default: packed in id order)
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class TreeSpec:
    parent: np.ndarray   # int32 [n_seg]
    seg_len: np.ndarray  # int32 [n_seg]
    seg_row: np.ndarray  # int64 [n_seg]
    name: str = ""

    @property
    def n_seg(self) -> int:
        return int(self.parent.shape[0])

    @property
    def n_rows(self) -> int:
        return int(self.seg_len.astype(np.int64).sum())


def _mk(parent, seg_len, name, seg_row=None) -> TreeSpec:
    parent = np.asarray(parent, dtype=np.int32)
    seg_len = np.asarray(seg_len, dtype=np.int32)
    if seg_row is None:
        seg_row = np.zeros(len(seg_len), dtype=np.int64)
        if len(seg_len):
            seg_row[1:] = np.cumsum(seg_len.astype(np.int64))[:-1]
    return TreeSpec(parent, seg_len, np.asarray(seg_row, dtype=np.int64), name)


def tree_fig1() -> TreeSpec:
    """The five-segment tree of Figure 1(a) with the lengths of the tiny
    workload: A(40) -> {B(30) -> {D(25), E(15)}, C(20)}; ids A=0 B=1 C=2 D=3 E=4."""
    return _mk([-1, 0, 0, 1, 1], [40, 30, 20, 25, 15], "fig1_tiny")


def tree_kary(branch: int, depth: int, lo: int, hi: int, rng: np.random.Generator,
              name: str = "kary") -> TreeSpec:
    """Complete `branch`-ary tree with `depth` levels below the root, segment
    ids in breadth-first order, lengths uniform in [lo, hi] drawn in id order."""
    parent = [-1]
    frontier = [0]
    for _ in range(depth):
        nxt = []
        for p in frontier:
            for _ in range(branch):
                parent.append(p)
                nxt.append(len(parent) - 1)
        frontier = nxt
    seg_len = rng.integers(lo, hi + 1, size=len(parent))
    return _mk(parent, seg_len, name)


def tree_stepwise(trunk: int, n_branch: int, seg_lo: int, seg_hi: int,
                  max_chain: int, rng: np.random.Generator,
                  name: str = "stepwise") -> TreeSpec:
    """A long shared trunk with `n_branch` branches forking at uniformly random
    trunk positions in [1, trunk-1] (repeats allowed). Each branch is a chain of
    U{1..max_chain} segments of U{seg_lo..seg_hi} tokens.  The trunk is cut
    into segments at the distinct fork positions; trunk segments get the
    first ids (in trunk order), then branch segments, branch by branch in
    draw order."""
    forks = rng.integers(1, trunk, size=n_branch)
    chain_n = rng.integers(1, max_chain + 1, size=n_branch)
    chain_lens = [rng.integers(seg_lo, seg_hi + 1, size=int(c)) for c in chain_n]
    cuts = np.unique(forks)
    bounds = np.concatenate([[0], cuts, [trunk]])
    parent, seg_len = [], []
    end_to_seg = {}
    for i in range(len(bounds) - 1):
        parent.append(i - 1)
        seg_len.append(int(bounds[i + 1] - bounds[i]))
        end_to_seg[int(bounds[i + 1])] = i
    for f, lens in zip(forks, chain_lens):
        p = end_to_seg[int(f)]
        for L in lens:
            parent.append(p)
            seg_len.append(int(L))
            p = len(parent) - 1
    return _mk(parent, seg_len, name)


def tree_path(lengths, name="path") -> TreeSpec:
    """A single chain of segments (one trajectory)."""
    n = len(lengths)
    return _mk([-1] + list(range(n - 1)), lengths, name)


def tree_random(rng: np.random.Generator, n_seg: int, len_lo: int, len_hi: int,
                max_children: int | None = None, n_roots: int = 1,
                name: str = "random") -> TreeSpec:
    """Random forest: segment i>=n_roots picks a uniformly random earlier
    segment as parent (optionally capped at max_children)."""
    n_roots = max(1, min(n_roots, n_seg))
    parent = [-1] * n_roots
    nchild = [0] * n_roots
    for i in range(n_roots, n_seg):
        while True:
            p = int(rng.integers(0, i))
            if max_children is None or nchild[p] < max_children:
                break
        parent.append(p)
        nchild[p] += 1
        nchild.append(0)
    seg_len = rng.integers(len_lo, len_hi + 1, size=n_seg)
    return _mk(parent, seg_len, name)


def shuffled_rows(spec: TreeSpec, rng: np.random.Generator) -> TreeSpec:
    """Same tree, but segments placed in the compact row space in a random
    order (exercises seg_row != id order)."""
    perm = rng.permutation(spec.n_seg)
    seg_row = np.zeros(spec.n_seg, dtype=np.int64)
    off = 0
    for s in perm:
        seg_row[s] = off
        off += int(spec.seg_len[s])
    return TreeSpec(spec.parent.copy(), spec.seg_len.copy(), seg_row, spec.name + "_perm")


# ---------------------------------------------------------------------------
# Input tensors
# ---------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to the nearest bfloat16 (ties to even),
    returned as float32 (exactly representable).  Finite inputs only."""
    f = np.array(x, dtype=np.float32, copy=True)
    u = f.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return f


def bf16_bits(x_f32_bf16exact: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exact bfloat16."""
    u = np.ascontiguousarray(x_f32_bf16exact, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


@dataclass
class KDAInputs:
    q: np.ndarray      # [N,H,dk] float32 (bf16-exact when bf16=True)
    k: np.ndarray      # [N,H,dk]
    v: np.ndarray      # [N,H,dv]
    g: np.ndarray      # [N,H,dk] float32, log-decay per channel (<= 0)
    beta: np.ndarray   # [N,H]    float32 in (0,1)
    h0: np.ndarray     # [n_root,H,dk,dv] float32
    scale: float
    bf16: bool
    extra: dict = field(default_factory=dict)


def _l2n(x):
    n = np.sqrt(np.einsum("...i,...i->...", x, x))[..., None]
    x /= n
    return x


def softplus(x):
    """log(1 + e^x), computed stably."""
    return np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x)))


def make_kda_inputs(rng: np.random.Generator, n_rows: int, H: int, dk: int, dv: int,
                    n_root: int = 1, bf16: bool = True, gate_mean: float = 2.0,
                    gate: str = "default", beta_mode: str = "default",
                    h0_mode: str = "zero") -> KDAInputs:
    """Per-row KDA inputs with the workload's value distributions:
    q,k ~ N(0,1) L2-normalised per head; v ~ N(0,1); beta = sigmoid(N(0,1));
    per-channel log-gate g = -softplus(N(gate_mean,1)).  Draws are float32;
    q,k,v are rounded to bf16 (RNE) when bf16=True.  Draw order: q, k, v,
    beta-pre, g-pre, h0.

    Test-only variants: gate="weak" draws g = -softplus(N(-4,1)) (slow decay,
    so boundary states stay visible), gate="zero" sets g = 0, gate="strong"
    draws g = -softplus(N(8,1)) (about 120 of decay over 15 rows), gate=
    "extreme" g = -softplus(N(40,5)) (every row decays past fp32 range of
    e^(15 g)), gate="mixed" draws each row (all heads and channels) from the
    strong law with probability 1/8 and from the workload law otherwise;
    beta_mode "zero"/"one" pin beta; h0_mode="randn" draws h0 ~
    N(0,1)/sqrt(dk)."""
    f32 = np.float32
    q = _l2n(rng.standard_normal((n_rows, H, dk), dtype=f32))
    k = _l2n(rng.standard_normal((n_rows, H, dk), dtype=f32))
    v = rng.standard_normal((n_rows, H, dv), dtype=f32)
    bpre = rng.standard_normal((n_rows, H), dtype=f32)
    gpre = rng.standard_normal((n_rows, H, dk), dtype=f32)
    if gate == "weak":
        g = -softplus(gpre - np.float32(4.0))
    elif gate == "zero":
        g = np.zeros_like(gpre)
    elif gate == "strong":
        g = -softplus(gpre + np.float32(8.0))
    elif gate == "extreme":
        g = -softplus(np.float32(5.0) * gpre + np.float32(40.0))
    elif gate == "mixed":
        strong = rng.random(n_rows) < 0.125
        g = -softplus(gpre + np.where(strong, np.float32(8.0), np.float32(gate_mean))[:, None, None]
                      .astype(np.float32))
    else:
        g = -softplus(gpre + np.float32(gate_mean))
    beta = 1.0 / (1.0 + np.exp(-bpre))
    if beta_mode == "zero":
        beta = np.zeros_like(beta)
    elif beta_mode == "one":
        beta = np.ones_like(beta)
    if h0_mode == "randn":
        h0 = rng.standard_normal((n_root, H, dk, dv), dtype=f32) / np.sqrt(dk)
    else:
        h0 = np.zeros((n_root, H, dk, dv), dtype=f32)
    cast = round_bf16 if bf16 else (lambda a: np.asarray(a, dtype=np.float32))
    return KDAInputs(q=cast(q), k=cast(k), v=cast(v),
                     g=np.asarray(g, dtype=np.float32),
                     beta=np.asarray(beta, dtype=np.float32),
                     h0=np.asarray(h0, dtype=np.float32),
                     scale=1.0 / np.sqrt(dk), bf16=bf16)


def make_upstream(rng: np.random.Generator, n_out_rows: int, n_leaf: int, H: int, dk: int,
                  dv: int, bf16: bool = True, dh_leaf: str = "randn"):
    """Upstream gradients: dO ~ N(0,1) per output row (bf16-rounded when
    bf16=True), dh_leaf ~ N(0,1) fp32 (or zeros when dh_leaf='zero')."""
    dO = rng.standard_normal((n_out_rows, H, dv), dtype=np.float32)
    dO = round_bf16(dO) if bf16 else dO
    if dh_leaf == "zero":
        dhl = np.zeros((n_leaf, H, dk, dv), dtype=np.float32)
    else:
        dhl = rng.standard_normal((n_leaf, H, dk, dv), dtype=np.float32)
    return dO, dhl


def make_kda_inputs_device(seed: int, n_rows: int, H: int, dk: int, dv: int, device,
                           bf16: bool = True, gate: str = "default"):
    """The make_kda_inputs distributions drawn on a device with a seeded torch
    generator (for full-size workloads, whose host draws would take minutes):
    q,k ~ N(0,1) L2-normalised per head, v ~ N(0,1) (bf16 when bf16=True),
    beta = sigmoid(N(0,1)), g = -softplus(N(2,1)) fp32 (gate="weak":
    -softplus(N(-4,1)); gate="strong": -softplus(N(8,1))).  Returns a dict of
    device tensors; draw order q, k, v, beta-pre, g-pre."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dt = torch.bfloat16 if bf16 else torch.float32

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    q = torch.nn.functional.normalize(randn(n_rows, H, dk), dim=-1).to(dt)
    k = torch.nn.functional.normalize(randn(n_rows, H, dk), dim=-1).to(dt)
    v = randn(n_rows, H, dv).to(dt)
    beta = torch.sigmoid(randn(n_rows, H))
    shift = {"default": 2.0, "weak": -4.0, "strong": 8.0}[gate]
    g = -torch.nn.functional.softplus(randn(n_rows, H, dk) + shift)
    return dict(q=q, k=k, v=v, beta=beta, g=g, scale=1.0 / float(np.sqrt(dk)))


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    tree: TreeSpec
    H: int
    dk: int
    dv: int
    chunk: int
    bf16: bool
    backward: bool
    seed: int


def workload(idx: int, seed: int | None = None) -> Workload:
    """idx 0: tiny Figure-1 tree, H=2, d=64, chunk 16, fp32, fwd+bwd.
    idx 1: complete 4-ary tree of depth 3 (85 segments, 64 leaves), lengths
           U{256..2048}, H=16, d=128, chunk 64, bf16 q/k/v, forward.
    idx 2: same tree and layer as 1, forward + backward.
    idx 3: step-wise tree: 32768-token trunk, 256 branches at U{1..32767},
           each 1-6 segments of U{128..1024}; H=16, d=128, chunk 64, fwd+bwd.
    idx 4: the idx-1 tree under a 3-KDA + 1 attention group (tree only here).
    The seed defaults to the workload index (idx 4 reuses idx 1's tree)."""
    s = idx if seed is None else seed
    if idx == 0:
        return Workload("tiny_fig1_h2_d64_c16_fp32", tree_fig1(), 2, 64, 64, 16, False, True, s)
    if idx in (1, 2, 4):
        ts = 1 if (idx == 4 and seed is None) else s
        t = tree_kary(4, 3, 256, 2048, np.random.Generator(np.random.PCG64(ts)), "kary4_d3")
        nm = {1: "kary4_depth3_h16_d128_c64_fwd", 2: "kary4_depth3_h16_d128_c64_fwdbwd",
              4: "kary4_depth3_hybrid_group"}[idx]
        return Workload(nm, t, 16, 128, 128, 64, True, idx != 1, s)
    if idx == 3:
        t = tree_stepwise(32768, 256, 128, 1024, 6, np.random.Generator(np.random.PCG64(s)),
                          "stepwise_trunk32k")
        return Workload("stepwise_trunk32k_b256_h16_d128_c64_fwdbwd", t, 16, 128, 128, 64,
                        True, True, s)
    raise ValueError(idx)


def workload_rng(w: Workload) -> np.random.Generator:
    """Generator for the per-row draws of a workload (after the tree)."""
    return np.random.Generator(np.random.PCG64(1000 + w.seed))
