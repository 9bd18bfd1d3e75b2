"""Token-by-token KDA recurrence over paths and trees, forward and reverse
mode, in float64 (oracle; test infrastructure only).

The HARTS pages name KDA layers ("KDA:MLA per group", Table 1) and say that
linear attention consumes a recurrent state and produces a branch-specific
next state (Figure 1(b)), but print no update rule.  The reading fixed for
this build is the gated delta rule with a per-channel decay.  Per head, per
token t, with state S (dk x dv):

    a    = exp(g_t)                      (per key channel, g_t <= 0)
    Sbar = diag(a) S                     decay first
    u    = beta_t * (v_t - Sbar^T k_t)   delta-rule write strength
    S    = Sbar + k_t u^T                write second
    o_t  = scale * S^T q_t               read after the write

Tree semantics (Figure 1(b), Figure 2(b), abstract "differentiable
boundary-state handoff"): a segment starts from the state its parent ended
with; a root starts from its own h0.  Each trajectory position has its own
output and loss, so a compact row's output is shared by every trajectory
through it, and the gradient reaching a shared state is the sum over its
children (the RL reading of Figure 1: one row serves several trajectories).

Pins (tests/test_oracle_kda.py): closed forms for beta = 0 and for a single
token; the orthonormal-key write/read identity of the delta rule; central
finite differences of the forward for every gradient; tree result equal,
bit for bit, to every root-to-leaf path run on its own; tree gradients equal
to the sum over trajectories of the expanded gradients.
"""
from __future__ import annotations

import numpy as np

from .tree import Tree

CKPT = 64  # tokens between stored states in the reverse sweep


def _f64(*xs):
    return [np.asarray(x, dtype=np.float64) for x in xs]


def path_fwd(S0, q, k, v, g, beta, scale, want_states=False):
    """Run the recurrence over one path.

    S0 [H,dk,dv]; q,k,g [T,H,dk]; v [T,H,dv]; beta [T,H].
    Returns o [T,H,dv], S_final [H,dk,dv] (and the T+1 states if asked)."""
    S = np.array(S0, dtype=np.float64, copy=True)
    q, k, v, g, beta = _f64(q, k, v, g, beta)
    T = q.shape[0]
    o = np.empty(v.shape, dtype=np.float64)
    states = [S.copy()] if want_states else None
    for t in range(T):
        a = np.exp(g[t])
        Sb = a[:, :, None] * S
        u = beta[t][:, None] * (v[t] - np.einsum("hkv,hk->hv", Sb, k[t]))
        S = Sb + k[t][:, :, None] * u[:, None, :]
        o[t] = scale * np.einsum("hkv,hk->hv", S, q[t])
        if want_states:
            states.append(S.copy())
    if want_states:
        return o, S, states
    return o, S


def path_bwd(S0, q, k, v, g, beta, scale, dO, dS_final, record=None):
    """Reverse mode of path_fwd.

    dO [T,H,dv] (output gradients), dS_final [H,dk,dv] (gradient of the final
    state).  `record` is an optional set of token boundaries j in [0,T]; the
    gradient with respect to the state after j tokens is returned for each.
    Returns (dq, dk, dv, dg, dbeta, dS0, recorded)."""
    q, k, v, g, beta, dO = _f64(q, k, v, g, beta, dO)
    T = q.shape[0]
    H, dk_, dv_ = np.shape(S0)
    # forward sweep keeping a state every CKPT tokens
    ck = {}
    S = np.array(S0, dtype=np.float64, copy=True)
    for t in range(T):
        if t % CKPT == 0:
            ck[t] = S.copy()
        a = np.exp(g[t])
        Sb = a[:, :, None] * S
        u = beta[t][:, None] * (v[t] - np.einsum("hkv,hk->hv", Sb, k[t]))
        S = Sb + k[t][:, :, None] * u[:, None, :]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    dg = np.zeros_like(g)
    db = np.zeros_like(beta)
    dS = np.array(dS_final, dtype=np.float64, copy=True)
    rec = {}
    if record is not None and T in record:
        rec[T] = dS.copy()
    for w0 in reversed(range(0, T, CKPT)):
        w1 = min(T, w0 + CKPT)
        # recompute the window's states
        Ss = [ck[w0]]
        for t in range(w0, w1):
            a = np.exp(g[t])
            Sb = a[:, :, None] * Ss[-1]
            u = beta[t][:, None] * (v[t] - np.einsum("hkv,hk->hv", Sb, k[t]))
            Ss.append(Sb + k[t][:, :, None] * u[:, None, :])
        for t in reversed(range(w0, w1)):
            Sp = Ss[t - w0]
            Sn = Ss[t - w0 + 1]
            a = np.exp(g[t])
            Sb = a[:, :, None] * Sp
            e = v[t] - np.einsum("hkv,hk->hv", Sb, k[t])
            u = beta[t][:, None] * e
            # o_t = scale * S^T q_t
            dS = dS + scale * q[t][:, :, None] * dO[t][:, None, :]
            dq[t] = scale * np.einsum("hkv,hv->hk", Sn, dO[t])
            # S = Sb + k u^T
            du = np.einsum("hkv,hk->hv", dS, k[t])
            dk[t] = np.einsum("hkv,hv->hk", dS, u)
            # u = beta * e
            db[t] = (du * e).sum(-1)
            de = beta[t][:, None] * du
            # e = v - Sb^T k
            dvv[t] = de
            dSb = dS - k[t][:, :, None] * de[:, None, :]
            dk[t] -= np.einsum("hkv,hv->hk", Sb, de)
            # Sb = diag(a) S_prev
            dg[t] = a * (dSb * Sp).sum(-1)
            dS = a[:, :, None] * dSb
            if record is not None and t in record:
                rec[t] = dS.copy()
    if record is not None and 0 in record and T == 0:
        rec[0] = dS.copy()
    return dq, dk, dvv, dg, db, dS, rec


def _h0_for(tree: Tree, h0, v):
    return np.asarray(h0[tree.root_index[tree.root_of(v)]], dtype=np.float64)


def tree_fwd(tree: Tree, q, k, v, g, beta, h0, scale, keep_start_states=False):
    """Forward over the compact rows of a tree.

    q,k,g [N,H,dk]; v [N,H,dv]; beta [N,H]; h0 [n_root,H,dk,dv].
    Returns o [N,H,dv], h_leaf [n_leaf,H,dk,dv] (leaves ascending), and the
    start state of every segment when keep_start_states is set."""
    H = q.shape[1]
    dv_ = v.shape[2]
    o = np.zeros((tree.n_rows, H, dv_), dtype=np.float64)
    h_leaf = np.zeros((len(tree.leaves),) + np.shape(h0)[1:], dtype=np.float64)
    end_state = {}
    left = {u: len(tree.children[u]) for u in range(tree.n)}
    starts = {}
    for s in tree.preorder:
        p = int(tree.parent[s])
        S0 = _h0_for(tree, h0, s) if p < 0 else end_state[p]
        if p >= 0:
            left[p] -= 1
            if left[p] == 0:
                end_state.pop(p)
        if keep_start_states:
            starts[s] = S0.copy()
        r = tree.seg_rows(s)
        oo, S = path_fwd(S0, q[r], k[r], v[r], g[r], beta[r], scale)
        o[r] = oo
        if tree.children[s]:
            end_state[s] = S
        else:
            h_leaf[tree.leaf_index[s]] = S
    if keep_start_states:
        return o, h_leaf, starts
    return o, h_leaf


def tree_bwd(tree: Tree, q, k, v, g, beta, h0, scale, dO, dh_leaf, boundaries=()):
    """Reverse mode of tree_fwd.

    dO [N,H,dv] per compact row; dh_leaf [n_leaf,H,dk,dv].
    `boundaries` is a list of (segment v, trajectory position b): for each,
    the total gradient with respect to the state after position b-1 on the
    root path of v (the state shared by everything below that position).
    Returns dict with dq, dk, dv, dg, dbeta [per compact row], dh0
    [n_root,...], and 'boundary' (list aligned with `boundaries`)."""
    _, _, starts = tree_fwd(tree, q, k, v, g, beta, h0, scale, keep_start_states=True)
    H = q.shape[1]
    out = {n: np.zeros(np.shape(x), dtype=np.float64) for n, x in
           (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    dh0 = np.zeros(np.shape(h0), dtype=np.float64)
    # where each requested boundary falls: segment a on the path, local index
    req = {}
    for i, (vv, b) in enumerate(boundaries):
        for a in tree.path(vv):
            if tree.start[a] < b <= tree.end[a]:
                req.setdefault(a, []).append((int(b - tree.start[a]), i))
                break
        else:
            raise ValueError("boundary outside the path")
    bres = [None] * len(boundaries)
    dstart = {}
    for s in reversed(tree.preorder):
        if tree.children[s]:
            dS_end = sum(dstart.pop(c) for c in tree.children[s])
        else:
            dS_end = np.asarray(dh_leaf[tree.leaf_index[s]], dtype=np.float64)
        r = tree.seg_rows(s)
        wanted = {j for j, _ in req.get(s, [])}
        dq, dk, dvv, dg, db, dS0, rec = path_bwd(starts[s], q[r], k[r], v[r], g[r], beta[r],
                                                scale, dO[r], dS_end, record=wanted)
        for j, i in req.get(s, []):
            bres[i] = rec[j]
        out["dq"][r] = dq
        out["dk"][r] = dk
        out["dv"][r] = dvv
        out["dg"][r] = dg
        out["dbeta"][r] = db
        if int(tree.parent[s]) < 0:
            dh0[tree.root_index[s]] += dS0
        else:
            dstart[s] = dS0
    out["dh0"] = dh0
    out["boundary"] = bres
    return out


def expanded_fwd(tree: Tree, q, k, v, g, beta, h0, scale):
    """Every trajectory (leaf ascending) run as an independent path from its
    root's h0.  Returns list of o_tau [L,H,dv] and h_final [n_leaf,...]."""
    outs, finals = [], []
    for l in tree.leaves:
        rows = tree.path_rows(l)
        o, S = path_fwd(_h0_for(tree, h0, l), q[rows], k[rows], v[rows], g[rows], beta[rows],
                        scale)
        outs.append(o)
        finals.append(S)
    return outs, np.stack(finals)


def expanded_bwd(tree: Tree, q, k, v, g, beta, h0, scale, dO_traj, dh_leaf):
    """Per-trajectory reverse mode; dO_traj is a list of [L,H,dv] arrays.
    Returns per-trajectory gradient dicts (position order) and dh0 per leaf."""
    res = []
    for i, l in enumerate(tree.leaves):
        rows = tree.path_rows(l)
        dq, dk, dvv, dg, db, dS0, _ = path_bwd(_h0_for(tree, h0, l), q[rows], k[rows], v[rows],
                                               g[rows], beta[rows], scale, dO_traj[i],
                                               dh_leaf[i])
        res.append(dict(rows=rows, dq=dq, dk=dk, dv=dvv, dg=dg, dbeta=db, dh0=dS0))
    return res
