"""Pins of the microbatch definition and exhaustive optimum (oracle.l1)."""
import numpy as np

from oracle import l1
from oracle.tree import Tree
from tree_packed_chunkwise_amd import synth


def _fig1():
    spec = synth.tree_fig1()   # A40 -> {B30 -> {D25, E15}, C20}; leaves C, D, E
    return Tree(spec.parent, spec.seg_len)


def test_whole_tree_fits():
    # trajectories A-C (60), A-B-D (95), A-B-E (85): 240 positions, 130 unique
    t = _fig1()
    ev = l1.evaluate(t, [0, 0, 0], 130)
    assert ev["feasible"] and ev["unique"].tolist() == [130] and ev["expanded"].tolist() == [240]
    assert abs(ev["compression"] - 240 / 130) < 1e-15 and ev["balance"] == 1.0
    assert abs(l1.optimum(t, 1000)[0] - 240 / 130) < 1e-12


def test_budget_110_hand_optimum():
    # budget 110: {A-B-D, A-B-E} = A+B+D+E = 110 fits, A-C alone (60):
    # 240 / 170; every other feasible split pays more prefix
    # ({A-B-D}, {A-B-E, A-C} = 95 + 105 = 200), and A-C cannot join the pair
    t = _fig1()
    leaves = t.leaves            # C, D, E (ascending ids 2, 3, 4)
    assert leaves == [2, 3, 4]
    ev = l1.evaluate(t, [1, 0, 0], 110)
    assert ev["feasible"] and sorted(ev["unique"].tolist()) == [60, 110]
    comp, bal = l1.optimum(t, 110)
    assert abs(comp - 240 / 170) < 1e-12
    assert abs(bal - (85 / 110)) < 1e-12


def test_budget_100_all_apart():
    # budget 100: no two trajectories fit together (105, 110, 115 > 100)
    t = _fig1()
    comp, bal = l1.optimum(t, 100)
    assert abs(comp - 1.0) < 1e-12
    assert abs(bal - (80 / 95)) < 1e-12
    assert not l1.evaluate(t, [0, 0, 1], 100)["feasible"]


def test_unique_is_union_of_path_rows():
    rng = np.random.Generator(np.random.PCG64(4))
    for _ in range(10):
        spec = synth.tree_random(rng, 9, 1, 20, n_roots=2)
        t = Tree(spec.parent, spec.seg_len, spec.seg_row)
        mb = rng.integers(0, 3, size=len(t.leaves))
        mb[: min(3, len(mb))] = np.arange(min(3, len(mb)))
        ev = l1.evaluate(t, mb, 10 ** 9)
        for m in range(int(mb.max()) + 1):
            rows = [t.path_rows(l) for i, l in enumerate(t.leaves) if mb[i] == m]
            assert ev["unique"][m] == len(np.unique(np.concatenate(rows)))
            assert ev["expanded"][m] == sum(len(r) for r in rows)


def test_single_path_has_no_compression():
    spec = synth.tree_path([5, 7, 3])
    t = Tree(spec.parent, spec.seg_len)
    assert l1.optimum(t, 100) == (1.0, 1.0)
