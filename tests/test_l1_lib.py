"""Host tests of the compression-oriented microbatch planner (kda_l1_plan)
against the microbatch definition and the exhaustive optimum (oracle.l1)."""
import numpy as np
import pytest

from oracle import l1
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth


def _tree(spec):
    return Tree(spec.parent, spec.seg_len, spec.seg_row)


def _check_consistent(spec, budget, r):
    t = _tree(spec)
    ev = l1.evaluate(t, r["leaf_mb"], budget)
    assert ev["feasible"]
    assert ev["unique"].tolist() == r["unique"].tolist()
    assert ev["expanded"].tolist() == r["expanded"].tolist()
    assert abs(ev["compression"] - r["compression"]) < 1e-12
    return t, ev


@pytest.mark.parametrize("budget,comp", [(1000, 240 / 130), (110, 240 / 170), (100, 1.0)])
def test_figure1_budgets(budget, comp):
    spec = synth.tree_fig1()
    r = B.l1_plan(spec.parent, spec.seg_len, budget)
    _check_consistent(spec, budget, r)
    assert abs(r["compression"] - comp) < 1e-12


def test_trees_that_fit_stay_whole():
    rng = np.random.Generator(np.random.PCG64(2))
    parents, lens = [], []
    for _ in range(12):   # a forest of small trees
        spec = synth.tree_random(rng, int(rng.integers(1, 7)), 5, 60)
        off = len(parents)
        parents += [p + off if p >= 0 else -1 for p in spec.parent]
        lens += list(spec.seg_len)
    t = Tree(parents, lens)
    sizes = {}
    for v in range(len(parents)):
        sizes[t.root_of(v)] = sizes.get(t.root_of(v), 0) + lens[v]
    budget = max(sizes.values())
    r = B.l1_plan(parents, lens, budget)
    ev = l1.evaluate(t, r["leaf_mb"], budget)
    assert ev["feasible"]
    # no tree is cut: all its trajectories share one microbatch, so the
    # compression is the whole forest's
    mb_of_root = {}
    for i, leaf in enumerate(t.leaves):
        assert mb_of_root.setdefault(t.root_of(leaf), r["leaf_mb"][i]) == r["leaf_mb"][i]
    assert abs(r["compression"] - t.n_expanded() / t.n_rows) < 1e-12


def test_near_the_optimum_on_tiny_forests():
    rng = np.random.Generator(np.random.PCG64(1))
    ratios = []
    for _ in range(120):
        spec = synth.tree_random(rng, int(rng.integers(2, 9)), 1, 30,
                                 n_roots=int(rng.integers(1, 3)))
        t = _tree(spec)
        if len(t.leaves) > 7:
            continue
        maxpath = max(t.end[l] for l in t.leaves)
        budget = int(rng.integers(maxpath, t.n_rows + 2))
        r = B.l1_plan(spec.parent, spec.seg_len, budget)
        _check_consistent(spec, budget, r)
        ratios.append(r["compression"] / l1.optimum(t, budget)[0])
    ratios = np.array(ratios)
    assert ratios.min() >= 0.8 and ratios.mean() >= 0.98, (ratios.min(), ratios.mean())


def test_large_tree_is_cut_within_budget():
    rng = np.random.Generator(np.random.PCG64(5))
    spec = synth.tree_kary(4, 3, 256, 2048, rng)
    budget = 32768
    r = B.l1_plan(spec.parent, spec.seg_len, budget)
    t, ev = _check_consistent(spec, budget, r)
    assert r["unique"].max() <= budget and len(r["unique"]) > 1
    assert r["compression"] > 1.0


def test_bad_arguments():
    with pytest.raises(B.KDAError):
        B.l1_plan([-1, 0], [3, 4], 0)
    with pytest.raises(B.KDAError):
        B.l1_plan([1, 0], [3, 4], 10)
    with pytest.raises(B.KDAError):
        B.l1_plan([-1, 0], [3, 0], 10)
