"""Tree-ancestor softmax attention over compact rows, float64 (oracle; test
infrastructure only).

Sources: HARTS Figure 1(b) caption (thelatestinai.com): full attention reads
ancestor keys and values; Figure C.1(c): attention over the compact layout
with a tree mask; Table 1: the hybrid models mix KDA layers with full
attention layers.  Reading taken (the pages print no formula): plain
multi-head softmax attention in which the query at trajectory position t of
segment v sees exactly the keys of the rows on its own root path at
positions <= t, i.e. every row of every ancestor segment of v and the rows of
v up to and including itself.  Because every trajectory through a row shares
that row's whole root path, the result is the same for all of them, which is
what lets one compact row serve them all.

    s_rj  = scale * q_r . k_j                   for j in keys(r)
    o_r   = sum_j softmax_j(s_r) v_j,  lse_r = logsumexp_j s_rj

Reverse mode (written from the chain rule of the softmax):
    p_rj = exp(s_rj - lse_r);  dv_j += p_rj do_r;  dp_rj = do_r . v_j
    ds_rj = p_rj (dp_rj - sum_j' p_rj' dp_rj');   dq_r = scale sum_j ds_rj k_j
    dk_j += scale ds_rj q_r

Pins (tests/test_oracle_attention.py): a path reduces to causal attention
(torch's scaled_dot_product_attention in float64); every row equals the
trajectory-expanded causal attention of each trajectory through it; the
backward agrees with central finite differences and with autograd of the
expanded runs summed over trajectories.
"""
from __future__ import annotations

import numpy as np

from oracle.tree import Tree


def _keys_of_segment(tree: Tree, v: int) -> np.ndarray:
    """Compact rows of v's root path (ancestors first, then v itself)."""
    return tree.path_rows(v)


def tree_attention_fwd(tree: Tree, q, k, v, scale):
    """q, k [N,H,d]; v [N,H,dv].  Returns o [N,H,dv], lse [N,H] (float64)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    N, H, _ = q.shape
    o = np.zeros((N, H, v.shape[2]))
    lse = np.zeros((N, H))
    for s in range(tree.n):
        keys = _keys_of_segment(tree, s)
        rows = tree.seg_rows(s)
        n_anc = len(keys) - len(rows)
        # query m of the segment sees keys[: n_anc + m + 1]
        mask = np.arange(len(keys))[None, :] <= (n_anc + np.arange(len(rows)))[:, None]
        for h in range(H):
            sc = scale * q[rows, h] @ k[keys, h].T
            sc = np.where(mask, sc, -np.inf)
            m = sc.max(axis=1, keepdims=True)
            e = np.exp(sc - m)
            z = e.sum(axis=1, keepdims=True)
            o[rows, h] = (e / z) @ v[keys, h]
            lse[rows, h] = (m + np.log(z))[:, 0]
    return o, lse


def tree_attention_bwd(tree: Tree, q, k, v, scale, dO):
    """Gradients (dq, dk, dv) of sum(dO * o) for tree_attention_fwd."""
    q, k, v, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dO))
    N, H, _ = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for s in range(tree.n):
        keys = _keys_of_segment(tree, s)
        rows = tree.seg_rows(s)
        n_anc = len(keys) - len(rows)
        mask = np.arange(len(keys))[None, :] <= (n_anc + np.arange(len(rows)))[:, None]
        for h in range(H):
            sc = scale * q[rows, h] @ k[keys, h].T
            sc = np.where(mask, sc, -np.inf)
            m = sc.max(axis=1, keepdims=True)
            p = np.exp(sc - m)
            p /= p.sum(axis=1, keepdims=True)
            do = dO[rows, h]
            dv[keys, h] += p.T @ do
            dp = do @ v[keys, h].T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq[rows, h] += scale * ds @ k[keys, h]
            dk[keys, h] += scale * ds.T @ q[rows, h]
    return dq, dk, dv
