"""Pins of the occurrence-weighted router-statistics oracle (oracle.moe)."""
import numpy as np
import scipy.special

from oracle import moe
from oracle.tree import Tree
from tree_packed_chunkwise_amd import synth


def _leaves_below(parent):
    """Leaves in each segment's subtree, from the parent array alone."""
    n = len(parent)
    kids = [[] for _ in range(n)]
    for v, p in enumerate(parent):
        if p >= 0:
            kids[p].append(v)
    cnt = [0] * n

    def walk(v):
        cnt[v] = 1 if not kids[v] else sum(walk(c) for c in kids[v])
        return cnt[v]
    for v in range(n):
        if parent[v] < 0:
            walk(v)
    return cnt


def test_occurrence_figure1():
    # Figure 1(a): B is shared by T1 and T2 (the caption's q_B = 2), A by all
    # three trajectories, C, D, E by one each
    spec = synth.tree_fig1()   # A -> {B -> {D, E}, C}
    t = Tree(spec.parent, spec.seg_len)
    q = moe.occurrence(t)
    want = {0: 3, 1: 2, 2: 1, 3: 1, 4: 1}
    for v, c in want.items():
        assert np.all(q[t.seg_rows(v)] == c), v


def test_occurrence_is_leaf_count_of_segment():
    rng = np.random.Generator(np.random.PCG64(3))
    for _ in range(10):
        spec = synth.tree_random(rng, 12, 1, 9, n_roots=2)
        t = Tree(spec.parent, spec.seg_len, spec.seg_row)
        q = moe.occurrence(t)
        cnt = _leaves_below(list(spec.parent))
        for v in range(len(spec.parent)):
            assert np.all(q[t.seg_rows(v)] == cnt[v])


def test_hand_counted_loads():
    # A -> {B -> {D, E}, C}, one row per segment (rows A0 B1 C2 D3 E4);
    # trajectories A-B-D, A-B-E, A-C: 8 positions.  Top-2 per row: A {0,1},
    # B {1,2}, C {2,3}, D {3,0}, E {0,2}; A is read 3 times, B twice:
    #   e0: 3 (A) + 1 (D) + 1 (E) = 5;  e1: 3 (A) + 2 (B) = 5;
    #   e2: 2 (B) + 1 (C) + 1 (E) = 4;  e3: 1 (C) + 1 (D) = 2
    t = Tree([-1, 0, 0, 1, 1], [1, 1, 1, 1, 1])
    x = np.array([[4, 3, 1, 0],
                  [0, 4, 3, 1],
                  [0, 1, 4, 3],
                  [3, 0, 1, 4],
                  [4, 0, 3, 1]], dtype=np.float64)
    load, psum, zsum, T = moe.expanded_stats(t, x, 2)
    assert T == 8
    assert load.tolist() == [5, 5, 4, 2]


def test_invariants():
    rng = np.random.Generator(np.random.PCG64(5))
    spec = synth.tree_random(rng, 9, 3, 40, n_roots=2)
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    E, k = 16, 4
    x = rng.standard_normal((t.n_rows, E)) * 2
    load, psum, zsum, T = moe.expanded_stats(t, x, k)
    assert T == t.n_expanded()
    assert load.sum() == k * T                       # every position routes to k experts
    np.testing.assert_allclose(psum.sum(), T, rtol=1e-12)   # probabilities sum to one
    assert zsum > 0


def test_single_path_is_plain_per_token():
    # no sharing: every row is read once, the statistics are per-token ones
    spec = synth.tree_path([7, 5, 9])
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    rng = np.random.Generator(np.random.PCG64(7))
    E, k = 12, 3
    x = rng.standard_normal((t.n_rows, E))
    load, psum, zsum, T = moe.expanded_stats(t, x, k)
    p = scipy.special.softmax(x, axis=1)
    lse = scipy.special.logsumexp(x, axis=1)
    np.testing.assert_allclose(psum, p.sum(axis=0), rtol=1e-13)
    np.testing.assert_allclose(zsum, (lse ** 2).sum(), rtol=1e-13)
    ref = np.zeros(E, dtype=np.int64)
    for r in range(t.n_rows):
        for e in sorted(range(E), key=lambda e: (-x[r, e], e))[:k]:
            ref[e] += 1
    assert load.tolist() == ref.tolist()


def test_topk_ties_prefer_lower_index():
    x = np.array([[1.0] * 8, [2, 5, 5, 1, 5, 0, 0, 0]], dtype=np.float64)
    top = moe.topk_rows(x, 3)
    assert top[0].tolist() == [0, 1, 2]
    assert top[1].tolist() == [1, 2, 4]


def test_grad_matches_finite_differences():
    t = Tree([-1, 0, 0, 1, 1], [2, 3, 1, 2, 2])
    rng = np.random.Generator(np.random.PCG64(9))
    E = 6
    x = rng.standard_normal((t.n_rows, E))
    gP = rng.standard_normal(E)
    gz = 0.37

    def L(xx):
        _, ps, zs, _ = moe.expanded_stats(t, xx, 2)
        return float(gP @ ps + gz * zs)
    g = moe.expanded_grad(t, x, gP, gz)
    h = 1e-6
    fd = np.zeros_like(x)
    for r in range(t.n_rows):
        for e in range(E):
            xp, xm = x.copy(), x.copy()
            xp[r, e] += h
            xm[r, e] -= h
            fd[r, e] = (L(xp) - L(xm)) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8)
