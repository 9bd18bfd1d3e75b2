"""Occurrence-count-weighted MoE router statistics, float64 (oracle; test
infrastructure only).

Sources: HARTS abstract (for deterministic top-k routing without token
dropping, occurrence counts restore MoE objective weights and expert-load
statistics); thelatestinai.com Figure 1 caption (the occurrence count of a
shared row restores MoE objective weights and expert-load counts without
repeating routing or expert computation; q_B = 2 for the row shared by two
trajectories); Figure C.1(d) (compact routing uses multiplicity-weighted
router losses and expert-load counts).

The pages print no formula; the plainest reading, taken here:
  * the statistics are those of the trajectory-expanded batch: every position
    of every root-to-leaf trajectory routes with the router logits x of its
    own token (one row of the compact [rows, E] logits);
  * deterministic top-k: the k largest logits of a position, equal logits
    ordered by the lower expert index (no token is dropped);
  * per position p = softmax(x), lse = logsumexp(x);
  * load[e] = number of positions whose top-k holds e; psum[e] = sum of p[e];
    zsum = sum of lse^2; T = number of positions.  A load-balancing loss
    E * sum_e (load[e] / (k T)) * (psum[e] / T) and a z-loss zsum / T are
    assembled from these by the caller;
  * reverse mode: given gP = dL/dpsum and gz = dL/dzsum, each position adds
    p * (gP - <p, gP>) + 2 * lse * gz * p to the gradient of its row's
    logits (top-k membership carries no gradient).
Everything below is computed the expanded way, trajectory by trajectory and
position by position; the occurrence count of a row is counted the same way.
"""
from __future__ import annotations

import numpy as np

from .tree import Tree


def occurrence(tree: Tree) -> np.ndarray:
    """Number of trajectory positions that read each compact row (one per
    root-to-leaf path through the row), counted over the expanded paths."""
    q = np.zeros(tree.n_rows, dtype=np.int64)
    for leaf in tree.leaves:
        np.add.at(q, tree.path_rows(leaf), 1)
    return q


def topk_rows(x: np.ndarray, k: int) -> np.ndarray:
    """[n, k] expert indices of the k largest logits per row, larger first,
    equal logits by the lower index (a stable sort of -x)."""
    return np.argsort(-np.asarray(x, dtype=np.float64), axis=1, kind="stable")[:, :k]


def _softmax_lse(x: np.ndarray):
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    s = e.sum(axis=1, keepdims=True)
    return e / s, (m + np.log(s))[:, 0]


def expanded_stats(tree: Tree, x: np.ndarray, k: int):
    """(load [E] int64, psum [E], zsum, T) over every position of every
    trajectory."""
    E = x.shape[1]
    load = np.zeros(E, dtype=np.int64)
    psum = np.zeros(E, dtype=np.float64)
    zsum = 0.0
    T = 0
    for leaf in tree.leaves:
        rows = tree.path_rows(leaf)
        xs = np.asarray(x[rows], dtype=np.float64)
        p, lse = _softmax_lse(xs)
        top = topk_rows(xs, k)
        np.add.at(load, top.ravel(), 1)
        psum += p.sum(axis=0)
        zsum += float((lse * lse).sum())
        T += len(rows)
    return load, psum, zsum, T


def expanded_grad(tree: Tree, x: np.ndarray, g_psum: np.ndarray, g_z: float) -> np.ndarray:
    """Gradient of L = <g_psum, psum> + g_z * zsum with respect to the compact
    logits: each position's contribution added into its row."""
    gP = np.asarray(g_psum, dtype=np.float64)
    dx = np.zeros(x.shape, dtype=np.float64)
    for leaf in tree.leaves:
        rows = tree.path_rows(leaf)
        p, lse = _softmax_lse(x[rows])
        dot = p @ gP
        g = p * (gP[None, :] - dot[:, None]) + 2.0 * g_z * lse[:, None] * p
        np.add.at(dx, rows, g)
    return dx


def row_topk(x: np.ndarray, k: int):
    """Per compact row: (top-k indices [n, k], their softmax probabilities)."""
    p, _ = _softmax_lse(x)
    top = topk_rows(x, k)
    return top, np.take_along_axis(p, top, axis=1)
