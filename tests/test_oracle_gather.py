"""Pins of the log-prob gather oracle (oracle.gather)."""
import numpy as np
import scipy.special

from oracle import gather
from oracle.tree import Tree
from tree_packed_chunkwise_amd import synth


def test_uniform_logits():
    V = 1000
    z = np.full((5, V), 3.25)
    logp, lse = gather.gather_fwd(z, [0, 1, 4, 4], [3, 999, 0, 0])
    np.testing.assert_allclose(logp, -np.log(V), rtol=1e-15)


def test_matches_log_softmax_on_expanded_rows():
    # compact rows serve several trajectories: the gathered values equal the
    # log-softmax of the expanded (per-trajectory) rows at each target
    spec = synth.tree_fig1()
    t = Tree(spec.parent, spec.seg_len)
    rng = np.random.Generator(np.random.PCG64(0))
    V = 97
    z = rng.standard_normal((t.n_rows, V)) * 3
    tokens = rng.integers(0, V, size=t.n_rows)
    pos_row, pos_next = t.gather_map()
    logp, _ = gather.gather_fwd(z, pos_row, tokens[pos_next])
    k = 0
    for leaf in t.leaves:
        rows = t.path_rows(leaf)
        ref = scipy.special.log_softmax(z[rows], axis=1)
        for tt in range(len(rows) - 1):
            assert abs(logp[k] - ref[tt, tokens[rows[tt + 1]]]) < 1e-12
            k += 1
    assert k == len(logp)
    # the shared root rows serve all three trajectories
    assert np.sum(pos_row == 0) == 3


def test_backward_finite_differences():
    rng = np.random.Generator(np.random.PCG64(1))
    n, V = 4, 11
    z = rng.standard_normal((n, V))
    pos_row = np.array([0, 0, 1, 3, 3, 3])
    pos_tgt = np.array([2, 2, 5, 0, 7, 10])
    dl = rng.standard_normal(len(pos_row))
    dz = gather.gather_bwd(z, pos_row, pos_tgt, dl)
    eps = 1e-6
    for i in range(n):
        for j in range(V):
            z1 = z.copy(); z1[i, j] += eps
            z2 = z.copy(); z2[i, j] -= eps
            f = (gather.gather_fwd(z1, pos_row, pos_tgt)[0] @ dl
                 - gather.gather_fwd(z2, pos_row, pos_tgt)[0] @ dl) / (2 * eps)
            assert abs(f - dz[i, j]) < 1e-8


def test_masked_entries_equal_log_softmax_of_unmasked():
    """A -inf logit has probability zero: a row with masked entries gives the
    log-softmax over its unmasked entries alone (scipy on the sub-vector), a
    masked target gets -inf, and the gradient of a masked entry's softmax part
    is zero; an all-masked row gives lse = -inf and logp = -inf everywhere."""
    rng = np.random.Generator(np.random.PCG64(3))
    V = 300
    z = rng.standard_normal((4, V)) * 2
    z[0, :256] = -np.inf            # a row whose first 256 entries are masked
    z[1, rng.choice(V, 100, replace=False)] = -np.inf
    z[3, :] = -np.inf               # every entry masked
    keep0 = np.isfinite(z[0])
    keep1 = np.isfinite(z[1])
    pos_row = np.array([0, 0, 1, 1, 2, 3])
    tgt1_masked = int(np.flatnonzero(~keep1)[0])
    pos_tgt = np.array([260, 10, int(np.flatnonzero(keep1)[3]), tgt1_masked, 5, 7])
    logp, lse = gather.gather_fwd(z, pos_row, pos_tgt)
    ref0 = scipy.special.log_softmax(z[0, keep0])
    assert abs(logp[0] - ref0[260 - 256]) < 1e-12
    assert logp[1] == -np.inf                      # masked target
    ref1 = scipy.special.log_softmax(z[1, keep1])
    assert abs(logp[2] - ref1[3]) < 1e-12
    assert logp[3] == -np.inf
    assert abs(lse[0] - scipy.special.logsumexp(z[0, keep0])) < 1e-12
    assert lse[3] == -np.inf and logp[5] == -np.inf
    dl = rng.standard_normal(len(pos_row))
    dz = gather.gather_bwd(z, pos_row, pos_tgt, dl)
    assert np.isfinite(dz).all()
    # masked non-target entries carry no gradient; the all-masked row only its target
    assert np.all(dz[0, :256][np.arange(256) != 10] == 0)
    assert dz[3, 7] == dl[5] and np.count_nonzero(dz[3]) == 1
    # unmasked part of row 0: softmax over the unmasked entries (scipy)
    p0 = scipy.special.softmax(z[0, keep0])
    exp0 = -p0 * (dl[0] + dl[1])
    exp0[260 - 256] += dl[0]
    np.testing.assert_allclose(dz[0, keep0], exp0, atol=1e-14)
