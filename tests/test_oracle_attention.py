"""Pins of the tree-ancestor attention oracle (oracle/attention.py) against
what the mathematics fixes: causal attention on a path (torch's
scaled_dot_product_attention, float64), trajectory expansion, central finite
differences, and autograd of the expanded runs."""
import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle.tree import Tree
from tree_packed_chunkwise_amd import synth


def _inputs(rng, N, H, d):
    q = rng.standard_normal((N, H, d))
    k = rng.standard_normal((N, H, d))
    v = rng.standard_normal((N, H, d))
    return q, k, v


def _sdpa(q, k, v, scale):
    """causal attention of one sequence [T,H,d] via torch (float64)."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True,
                                                         scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


def test_path_is_causal_attention():
    rng = np.random.Generator(np.random.PCG64(1))
    spec = synth.tree_path([7, 5, 9])
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    q, k, v = _inputs(rng, t.n_rows, 2, 8)
    o, lse = oa.tree_attention_fwd(t, q, k, v, 0.3)
    ref = _sdpa(q, k, v, 0.3)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    # lse of the first row is its single score
    np.testing.assert_allclose(lse[0], 0.3 * (q[0] * k[0]).sum(-1), rtol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rows_equal_trajectory_expansion(seed):
    rng = np.random.Generator(np.random.PCG64(10 + seed))
    spec = synth.tree_random(rng, 9, 1, 12, 3, n_roots=2)
    spec = synth.shuffled_rows(spec, rng)
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    q, k, v = _inputs(rng, t.n_rows, 2, 8)
    o, _ = oa.tree_attention_fwd(t, q, k, v, 0.25)
    seen = np.zeros(t.n_rows, dtype=bool)
    for leaf in t.leaves:
        rows = t.path_rows(leaf)
        ref = _sdpa(q[rows], k[rows], v[rows], 0.25)
        np.testing.assert_allclose(o[rows], ref, rtol=1e-11, atol=1e-12)
        seen[rows] = True
    assert seen.all()


def test_backward_finite_differences():
    rng = np.random.Generator(np.random.PCG64(3))
    spec = synth.tree_fig1()
    spec = synth._mk(spec.parent, [3, 2, 2, 3, 1], "fig1_small")
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    q, k, v = _inputs(rng, t.n_rows, 2, 4)
    dO = rng.standard_normal(q.shape)
    dq, dk, dv = oa.tree_attention_bwd(t, q, k, v, 0.5, dO)
    loss = lambda q_, k_, v_: (oa.tree_attention_fwd(t, q_, k_, v_, 0.5)[0] * dO).sum()
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            pos = "qkv".index(name)
            args_p[pos], args_m[pos] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_backward_equals_sum_over_trajectories():
    """Per-trajectory losses with their own upstream gradients; the compact
    upstream gradient of a row is the sum over the trajectories through it,
    and the tree gradients are the sums of the expanded runs' autograd
    gradients mapped to rows."""
    rng = np.random.Generator(np.random.PCG64(4))
    spec = synth.tree_random(rng, 7, 2, 9, 2)
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    q, k, v = _inputs(rng, t.n_rows, 2, 6)
    dO = np.zeros_like(q)
    gq, gk, gv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for leaf in t.leaves:
        rows = t.path_rows(leaf)
        dtraj = rng.standard_normal((len(rows), 2, 6))
        dO[rows] += dtraj
        tt = lambda x: torch.from_numpy(np.ascontiguousarray(x[rows].transpose(1, 0, 2)))[None].requires_grad_()
        Q, K, V = tt(q), tt(k), tt(v)
        o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=0.4)
        (o * torch.from_numpy(dtraj.transpose(1, 0, 2))[None]).sum().backward()
        back = lambda G: G.grad[0].numpy().transpose(1, 0, 2)
        gq[rows] += back(Q)
        gk[rows] += back(K)
        gv[rows] += back(V)
    dq, dk, dv = oa.tree_attention_bwd(t, q, k, v, 0.4, dO)
    np.testing.assert_allclose(dq, gq, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dk, gk, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dv, gv, rtol=1e-10, atol=1e-11)
