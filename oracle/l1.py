"""Compression-oriented microbatches of whole trajectories: their definition
and a brute-force optimum for tiny forests (oracle; test infrastructure only).

Sources: HARTS abstract (a two-level planner constructs compression-oriented
microbatches); thelatestinai.com Figure 1(c) (L1 constructs
compression-oriented microbatches); Table 4 (planners compared by
compression and balance).  The pages print no algorithm or formula; the
plainest reading, taken here:
  * a microbatch is a set of whole trajectories (root-to-leaf paths); it holds
    every compact row of those paths once, so its load is its unique token
    count (the union of the paths' rows) and it must stay within the token
    budget (a trajectory longer than the budget goes alone);
  * compression = sum of the trajectories' lengths / sum of the microbatches'
    unique tokens (a tree cut over two microbatches pays its shared prefix
    twice);
  * balance = mean microbatch load / largest microbatch load.
`evaluate` computes these for any assignment; `optimum` enumerates every
partition of the leaves of a tiny forest.
"""
from __future__ import annotations

import numpy as np

from .tree import Tree


def path_segments(tree: Tree, leaf: int) -> list:
    return tree.path(leaf)


def evaluate(tree: Tree, leaf_mb, capacity: int):
    """leaf_mb[i]: microbatch of tree.leaves[i].  Returns dict(unique per
    microbatch, expanded per microbatch, compression, balance, feasible)."""
    leaf_mb = np.asarray(leaf_mb, dtype=np.int64)
    n_mb = int(leaf_mb.max()) + 1 if len(leaf_mb) else 0
    segs = [set() for _ in range(n_mb)]
    exp = np.zeros(n_mb, dtype=np.int64)
    single = np.zeros(n_mb, dtype=bool)
    for i, leaf in enumerate(tree.leaves):
        m = int(leaf_mb[i])
        p = path_segments(tree, leaf)
        segs[m].update(p)
        exp[m] += int(sum(tree.seg_len[s] for s in p))
    uniq = np.array([sum(int(tree.seg_len[s]) for s in ss) for ss in segs], dtype=np.int64)
    counts = np.bincount(leaf_mb, minlength=n_mb)
    for m in range(n_mb):
        single[m] = counts[m] == 1
    feasible = bool(np.all((uniq <= capacity) | single) and np.all(counts > 0))
    comp = float(exp.sum() / uniq.sum()) if n_mb else 1.0
    bal = float(uniq.mean() / uniq.max()) if n_mb else 1.0
    return dict(unique=uniq, expanded=exp, compression=comp, balance=bal, feasible=feasible)


def _partitions(items):
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for part in _partitions(rest):
        for i in range(len(part)):
            yield part[:i] + [[first] + part[i]] + part[i + 1:]
        yield [[first]] + part


def optimum(tree: Tree, capacity: int):
    """Best feasible assignment by exhaustive search (leaves <= 8): the most
    compression, then the best balance.  Returns (compression, balance)."""
    n = len(tree.leaves)
    best = None
    for part in _partitions(list(range(n))):
        mb = np.zeros(n, dtype=np.int64)
        for m, blk in enumerate(part):
            mb[blk] = m
        ev = evaluate(tree, mb, capacity)
        if not ev["feasible"]:
            continue
        key = (round(ev["compression"], 12), round(ev["balance"], 12))
        if best is None or key > best:
            best = key
    return best
