"""Host-side construction of a sharing window (tree_packed_chunkwise_amd.window):
the row layout tiles the tree with every part contiguous, the producer holds
every segment down to the split depth, each consumer root is handed its
parent's producer leaf state, and every tree leaf is covered exactly once."""
import numpy as np
import pytest

from oracle.tree import Tree
from tree_packed_chunkwise_amd import synth
from tree_packed_chunkwise_amd.window import SharingWindow


@pytest.mark.parametrize("split,n_micro", [(0, 1), (0, 3), (1, 2), (1, 4)])
def test_window_construction(split, n_micro):
    rng = np.random.Generator(np.random.PCG64(5))
    spec = synth.tree_kary(3, 3, 20, 90, rng)
    t = Tree(spec.parent, spec.seg_len)
    w = SharingWindow(spec.parent, spec.seg_len, split, n_micro, chunk=16)
    t2 = Tree(spec.parent, spec.seg_len, w.seg_row)          # the layout tiles [0, N)
    assert t2.n_rows == t.n_rows == w.n_rows
    prod = [v for v in range(t.n) if t.depth(v) <= split]
    assert w.rows_p == sum(int(t.seg_len[v]) for v in prod)
    assert all(w.seg_row[v] < w.rows_p for v in prod)
    # microbatches: contiguous row ranges after the producer, in order
    r = w.rows_p
    for m in w.micro:
        assert m["base"] == r
        r += m["rows"]
    assert r == w.n_rows
    # every consumer root starts from its parent's producer leaf state
    p_leaves = [prod[int(i)] for i in w.plan_p.export("LEAF_SEG")]
    heads = [v for v in range(t.n) if t.depth(v) == split + 1]
    seen = []
    for m in w.micro:
        for h_src in m["h0_src"]:
            assert 0 <= h_src < len(p_leaves)
        seen += m["h0_src"]
        # the CSR of each microbatch lists each of its roots exactly once
        assert sorted(m["idx"]) == list(range(m["n_root"]))
    assert len(seen) == len(heads)
    # every tree leaf is produced exactly once (producer or one microbatch)
    leaves = sorted(w.p_full_dst + [i for m in w.micro for i in m["leaf_full"]])
    assert leaves == list(range(len(t.leaves)))
