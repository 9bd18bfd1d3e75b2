"""Pins of the token-level KDA oracle (oracle.kda) against things other than
itself: closed forms, the write/read identity of the delta rule, finite
differences, and brute-force trajectory expansion."""
import numpy as np
import pytest

from oracle import kda
from oracle.tree import Tree
from tree_packed_chunkwise_amd import synth


def _inputs(T, H, dk, dv, seed, **kw):
    rng = np.random.Generator(np.random.PCG64(seed))
    return synth.make_kda_inputs(rng, T, H, dk, dv, bf16=False, **kw)


def test_beta_zero_closed_form():
    # beta = 0: the state only decays, S_t = diag(exp(G_t)) h0 with G_t the
    # cumulative log-decay, so o_t = scale * h0^T (exp(G_t) * q_t)
    inp = _inputs(23, 2, 5, 4, 1, beta_mode="zero", h0_mode="randn", gate="weak")
    o, S = kda.path_fwd(inp.h0[0], inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale)
    G = np.cumsum(inp.g.astype(np.float64), axis=0)
    for t in range(23):
        for h in range(2):
            ref = inp.scale * inp.h0[0, h].astype(np.float64).T @ (np.exp(G[t, h]) * inp.q[t, h])
            np.testing.assert_allclose(o[t, h], ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, np.exp(G[-1])[:, :, None] * inp.h0[0], rtol=1e-12)


def test_single_token_closed_form():
    # one token from a zero state: o = scale * beta * (q . k) * v
    inp = _inputs(1, 3, 7, 5, 2)
    o, S = kda.path_fwd(np.zeros((3, 7, 5)), inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale)
    for h in range(3):
        q, k, v, b = (x.astype(np.float64) for x in (inp.q[0, h], inp.k[0, h], inp.v[0, h],
                                                      inp.beta[0, h]))
        np.testing.assert_allclose(o[0, h], inp.scale * b * (q @ k) * v, rtol=1e-13)
        np.testing.assert_allclose(S[h], b * np.outer(k, v), rtol=1e-13)


def test_orthonormal_overwrite():
    # g = 0, beta = 1, orthonormal keys: each write replaces the state's
    # component along its key, so S_T = (I - K^T K) h0 + K^T V exactly.
    rng = np.random.Generator(np.random.PCG64(3))
    dk, dv, T = 8, 3, 5
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:T]
    vals = rng.standard_normal((T, dv))
    h0 = rng.standard_normal((1, dk, dv))
    z = np.zeros((T, 1, dk))
    o, S = kda.path_fwd(h0, keys[:, None], keys[:, None], vals[:, None], z, np.ones((T, 1)), 1.0)
    ref = (np.eye(dk) - keys.T @ keys) @ h0[0] + keys.T @ vals
    np.testing.assert_allclose(S[0], ref, atol=1e-12)
    # reading with the last written key returns its value
    np.testing.assert_allclose(o[-1, 0], vals[-1], atol=1e-12)


def _loss(fn_args, dO, dSf, S0):
    o, S = kda.path_fwd(S0, *fn_args)
    return float((o * dO).sum() + (S * dSf).sum())


@pytest.mark.parametrize("gate", ["default", "weak"])
def test_path_bwd_finite_differences(gate):
    T, H, dk, dv = 6, 1, 4, 3
    inp = _inputs(T, H, dk, dv, 4, gate=gate, h0_mode="randn")
    rng = np.random.Generator(np.random.PCG64(5))
    dO = rng.standard_normal((T, H, dv))
    dSf = rng.standard_normal((H, dk, dv))
    args = [np.asarray(x, np.float64) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
    S0 = np.asarray(inp.h0[0], np.float64)
    dq, dk_, dv_, dg, db, dS0, _ = kda.path_bwd(S0, *args, inp.scale, dO, dSf)
    grads = [dq, dk_, dv_, dg, db]
    eps = 1e-6
    for ai in range(5):
        for idx in np.ndindex(args[ai].shape):
            a1 = [a.copy() for a in args]
            a2 = [a.copy() for a in args]
            a1[ai][idx] += eps
            a2[ai][idx] -= eps
            fd = (_loss(a1 + [inp.scale], dO, dSf, S0) - _loss(a2 + [inp.scale], dO, dSf, S0)) / (2 * eps)
            assert abs(fd - grads[ai][idx]) <= 1e-6 * max(1.0, abs(fd)), (ai, idx, fd, grads[ai][idx])
    for idx in np.ndindex(S0.shape):
        s1 = S0.copy(); s1[idx] += eps
        s2 = S0.copy(); s2[idx] -= eps
        fd = (_loss(args + [inp.scale], dO, dSf, s1) - _loss(args + [inp.scale], dO, dSf, s2)) / (2 * eps)
        assert abs(fd - dS0[idx]) <= 1e-6 * max(1.0, abs(fd))


def _tree_case(seed, n_seg=7, lo=1, hi=30, n_roots=1, H=2, dk=6, dv=5):
    rng = np.random.Generator(np.random.PCG64(seed))
    spec = synth.tree_random(rng, n_seg, lo, hi, n_roots=n_roots)
    if seed % 2:
        spec = synth.shuffled_rows(spec, rng)
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    inp = synth.make_kda_inputs(rng, t.n_rows, H, dk, dv, n_root=len(t.roots), bf16=False,
                                gate="weak", h0_mode="randn")
    return t, inp, rng


@pytest.mark.parametrize("seed", range(6))
def test_tree_equals_expansion_bitwise(seed):
    # every root-to-leaf path run on its own gives, bit for bit, the tree
    # result at its rows and its leaf state
    t, inp, _ = _tree_case(seed, n_roots=1 + seed % 2)
    o, hl = kda.tree_fwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale)
    outs, finals = kda.expanded_fwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale)
    for i, l in enumerate(t.leaves):
        rows = t.path_rows(l)
        assert np.array_equal(o[rows], outs[i])
    assert np.array_equal(hl, finals)


@pytest.mark.parametrize("seed", range(4))
def test_tree_grads_equal_sum_over_trajectories(seed):
    # each trajectory position has its own loss: with compact dO equal to the
    # sum of per-trajectory dO', tree gradients equal the summed expanded ones
    t, inp, rng = _tree_case(seed, n_roots=1 + seed % 2)
    H, dv = inp.v.shape[1], inp.v.shape[2]
    dO_traj = [rng.standard_normal((len(t.path_rows(l)), H, dv)) for l in t.leaves]
    dhl = rng.standard_normal((len(t.leaves),) + inp.h0.shape[1:])
    dO = np.zeros((t.n_rows, H, dv))
    for i, l in enumerate(t.leaves):
        np.add.at(dO, t.path_rows(l), dO_traj[i])
    tree = kda.tree_bwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale, dO, dhl)
    exp = kda.expanded_bwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale, dO_traj, dhl)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        acc = np.zeros_like(tree[name])
        for e in exp:
            np.add.at(acc, e["rows"], e[name])
        np.testing.assert_allclose(tree[name], acc, rtol=1e-10, atol=1e-12)
    dh0 = np.zeros_like(tree["dh0"])
    for i, l in enumerate(t.leaves):
        dh0[t.root_index[t.root_of(l)]] += exp[i]["dh0"]
    np.testing.assert_allclose(tree["dh0"], dh0, rtol=1e-10, atol=1e-12)
