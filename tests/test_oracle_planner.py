"""Pins of the min-call planner oracle (oracle.planner): exhaustive search,
the worked examples of Figures 1 and 2(c), the closed form of the replay
total, and special cases with known round counts."""
from pathlib import Path

import numpy as np
import pytest

from oracle import planner
from oracle.tree import Tree, TreeError
from tree_packed_chunkwise_amd import synth

GOLDEN = Path(__file__).parent / "golden"


def _load_golden(name):
    names, parent, lens, calls, cont = [], [], [], [], []
    chunk = None
    for line in (GOLDEN / name).read_text().splitlines():
        if not line or line.startswith("#"):
            continue
        f = line.split()
        if f[0] == "tree":
            names.append(f[1])
            parent.append(f[2])
            lens.append(int(f[3]))
        elif f[0] == "chunk":
            chunk = int(f[1])
        elif f[0] == "call":
            calls.append(sorted(f[1:]))
        elif f[0] == "continuations":
            cont = f[1:]
    idx = {n: i for i, n in enumerate(names)}
    par = [-1 if p == "-" else idx[p] for p in parent]
    return names, par, lens, chunk, calls, cont


def _calls_of(plan, names):
    out = []
    for r in range(plan.n_rounds):
        seqs = []
        for s in range(plan.round_seq_ptr[r], plan.round_seq_ptr[r + 1]):
            segs = [v for v in range(len(names)) if plan.seg_seq[v] == s]
            seqs.append(">".join(names[v] for v in sorted(segs)))
        out.append(sorted(seqs))
    return out


@pytest.mark.parametrize("fixture", ["fig1_plan.txt", "fig2c_plan.txt"])
def test_worked_examples(fixture):
    names, par, lens, chunk, calls, cont = _load_golden(fixture)
    t = Tree(par, lens)
    p = planner.build_plan(t, chunk)
    assert p.n_rounds == len(calls)
    assert _calls_of(p, names) == calls
    for n in cont:
        assert p.seg_is_cont[names.index(n)] == 1
    # replay-started sequences carry replay rows and write no outputs there
    for s in range(p.n_seq):
        r = p.seq_replay[s]
        rows = slice(p.seq_row_ptr[s], p.seq_row_ptr[s] + r)
        assert np.all(p.out_row[rows] == -1)


def test_fig1_replay_lengths():
    # chunk 16: C forks at 40 -> b = 32, r = 8; E forks at 70 -> b = 64, r = 6
    t = Tree([-1, 0, 0, 1, 1], [40, 30, 20, 25, 15])
    p = planner.build_plan(t, 16)
    assert p.R == 14
    assert list(p.seg_b[[2, 4]]) == [32, 64]
    assert list(p.seg_replay[[2, 4]]) == [8, 6]


def _rand_tree(rng, max_seg=9):
    n = int(rng.integers(1, max_seg + 1))
    spec = synth.tree_random(rng, n, 1, 40, n_roots=int(rng.integers(1, 3)))
    return Tree(spec.parent, spec.seg_len)


@pytest.mark.parametrize("B", [4, 8, 16])
def test_dp_matches_exhaustive_search(B):
    rng = np.random.Generator(np.random.PCG64(B))
    for _ in range(300):
        t = _rand_tree(rng)
        cont, _, rounds = planner.dp_mincall(t, B)
        assert rounds == planner.exhaustive_min_rounds(t, B)
        sim = planner.simulate(t, B, cont)
        assert sim[0] == rounds
        assert sim[1] == planner.replay_closed_form(t, B)


def test_path_is_one_round():
    for lens in ([5], [100, 3, 64, 7], [64, 64, 64]):
        t = Tree([-1] + list(range(len(lens) - 1)), lens)
        for B in (1, 16, 64):
            assert planner.dp_mincall(t, B)[2] == 1


def test_forks_in_first_chunk_one_round():
    # every fork position < B: every side branch restarts from h0 in round 1
    t = Tree([-1, 0, 0, 1, 1, 2], [3, 4, 5, 2, 3, 50])
    p = planner.build_plan(t, 16)
    assert p.n_rounds == 1
    assert np.all(p.seq_init_kind == 0)


@pytest.mark.parametrize("k,depth", [(2, 2), (3, 3), (4, 3)])
def test_complete_kary_rounds(k, depth):
    # all segments >= B: every side branch waits one round per level
    rng = np.random.Generator(np.random.PCG64(k * 10 + depth))
    spec = synth.tree_kary(k, depth, 64, 300, rng)
    t = Tree(spec.parent, spec.seg_len)
    assert planner.dp_mincall(t, 64)[2] == depth + 1


def test_handoff_buffers_are_written_before_read():
    rng = np.random.Generator(np.random.PCG64(11))
    for _ in range(100):
        t = _rand_tree(rng, 12)
        p = planner.build_plan(t, 8)
        for s in range(p.n_seq):
            if p.seq_init_kind[s] == 1:
                b = p.seq_init_idx[s]
                assert p.seq_round[p.buf_seq[b]] < p.seq_round[s]
                c = p.buf_chunk[b]
                assert p.chunk_save[c] == b and p.chunk_len[c] == 8


def test_malformed_trees_rejected():
    with pytest.raises(TreeError):
        Tree([-1, 2, 1], [1, 1, 1])       # cycle
    with pytest.raises(TreeError):
        Tree([-1, 0], [1, 0])             # zero length
    with pytest.raises(TreeError):
        Tree([-1, 5], [1, 1])             # parent out of range
    with pytest.raises(TreeError):
        Tree([-1, 0], [2, 2], [0, 1])     # overlapping rows


# ---- exact-state starts (the no-replay ablation and node-wise execution) ----

def _exhaustive_exact_rounds(t, limit=200000):
    """Minimum rounds over every continuation assignment when side branches
    start from their exact fork states."""
    import itertools
    internal = [v for v in range(t.n) if t.children[v]]
    choices = [[-1] + t.children[v] for v in internal]
    total = 1
    for c in choices:
        total *= len(c)
    assert total <= limit
    best = None
    for combo in itertools.product(*choices):
        cont = [-1] * t.n
        for v, c in zip(internal, combo):
            cont[v] = c
        r = planner.simulate_exact(t, cont)[0]
        best = r if best is None else min(best, r)
    return best


def test_noreplay_dp_matches_exhaustive_search():
    rng = np.random.Generator(np.random.PCG64(23))
    for _ in range(300):
        t = _rand_tree(rng)
        cont, _, rounds = planner.dp_noreplay(t)
        assert rounds == _exhaustive_exact_rounds(t)
        assert planner.simulate_exact(t, cont)[0] == rounds


def test_nodewise_rounds_are_depths():
    rng = np.random.Generator(np.random.PCG64(29))
    for _ in range(100):
        t = _rand_tree(rng, 12)
        p = planner.build_plan(t, 8, planner.NODEWISE)
        assert p.n_rounds == 1 + max(t.depth(v) for v in range(t.n))
        assert p.n_seq == t.n
        assert list(p.seg_round) == [t.depth(v) for v in range(t.n)]
        assert not np.any(p.seg_is_cont)


def test_fig1_exact_modes():
    # A40 -> {B30 -> {D25, E15}, C20}: no-replay continues A > B > D and starts
    # C at 40 and E at 70 from their exact states one round later; node-wise
    # runs one segment per sequence, a round per depth
    t = Tree([-1, 0, 0, 1, 1], [40, 30, 20, 25, 15])
    p = planner.build_plan(t, 16, planner.NOREPLAY)
    assert p.n_rounds == 2 and p.R == 0
    assert list(p.seg_is_cont) == [0, 1, 0, 1, 0]
    assert list(p.seg_b[[2, 4]]) == [40, 70]
    assert list(p.buf_pos) == [40, 70]
    # the A > B > D sequence is cut at 40 and 70: chunk ends at 16, 32, 40, 48, 64, 70, 80, 95
    s0 = p.seg_seq[0]
    lens = p.chunk_len[p.seq_chunk_ptr[s0]:p.seq_chunk_ptr[s0 + 1]]
    assert list(np.cumsum(lens)) == [16, 32, 40, 48, 64, 70, 80, 95]
    q = planner.build_plan(t, 16, planner.NODEWISE)
    assert q.n_rounds == 3 and q.n_seq == 5 and q.R == 0
    assert list(q.seg_round) == [0, 1, 1, 2, 2]
    assert list(q.seq_leaf[q.seg_seq[[0, 1]]]) == [-1, -1]   # A and B end at inner segments


@pytest.mark.parametrize("mode", [planner.NOREPLAY, planner.NODEWISE])
def test_exact_mode_structure(mode):
    rng = np.random.Generator(np.random.PCG64(31 + mode))
    for _ in range(100):
        t = _rand_tree(rng, 12)
        for B in (1, 4, 16):
            p = planner.build_plan(t, B, mode)
            assert p.R == 0 and p.n_packed == t.n_rows
            assert sorted(p.row_index.tolist()) == list(range(t.n_rows))
            assert np.all(p.out_row == p.row_index) and np.all(p.chunk_len <= B)
            for s in range(p.n_seq):
                if p.seq_init_kind[s] == 1:
                    b = p.seq_init_idx[s]
                    assert p.seq_round[p.buf_seq[b]] < p.seq_round[s]
                    assert p.seq_b_head[s] == p.buf_pos[b] == t.start[p.seq_head[s]]
                    c = p.buf_chunk[b]
                    ps = p.buf_seq[b]
                    end = p.seq_b_head[ps] + (p.chunk_row0[c] + p.chunk_len[c] - p.seq_row_ptr[ps])
                    assert p.chunk_save[c] == b and end == p.buf_pos[b]


@pytest.mark.parametrize("B", [4, 8, 16])
def test_short_chain_variant_keeps_minimum_rounds(B):
    """The short-chain variant drops only continuations that cost no round:
    the round count stays the exhaustive minimum, and its sequences are never
    longer than the min-call plan's."""
    rng = np.random.Generator(np.random.PCG64(40 + B))
    for _ in range(200):
        t = _rand_tree(rng)
        cont, _, rounds = planner.dp_mincall(t, B, short=True)
        assert rounds == planner.exhaustive_min_rounds(t, B)
        assert planner.simulate(t, B, cont)[0] == rounds
        p0 = planner.build_plan(t, B, planner.MINCALL)
        p4 = planner.build_plan(t, B, planner.MINCALL_SHORT)
        assert p4.n_rounds == p0.n_rounds
        assert np.diff(p4.seq_row_ptr).max() <= np.diff(p0.seq_row_ptr).max() + B
