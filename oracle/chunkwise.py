"""Chunk form of the KDA recurrence, executed over a packed plan, forward and
reverse mode, float64 (oracle; test infrastructure only).

Sources: HARTS abstract (chunkwise linear attention with differentiable
boundary-state handoff and bounded replay); Figure 2(c) (all sequences of a
round form one packed call; a later round may start only from states made
by earlier rounds); Figure C.1(b) (side sequences start from a boundary
state and replay the parent's tail inside the core without writing
outputs).  The chunk algebra below is the standard WY/UT form of the gated
delta rule of oracle.kda, written with exact per-pair decays (no reference
points, no factorisation), so it cannot overflow: every exponent used is
<= 0.

Per chunk of C rows (one head), with start state h (dk x dv):
    Gam_i  = sum_{s<=i} g_s                      (inclusive, per channel)
    A_ij   = sum_c k_ic k_jc exp(Gam_ic - Gam_jc)   j <  i
    P_ij   = sum_c q_ic k_jc exp(Gam_ic - Gam_jc)   j <= i
    T      = (I + diag(beta) A)^-1
    delta  = T diag(beta) (V - (K * e^Gam) h)        the delta-rule writes u_t
    O      = scale * ((Q * e^Gam) h + P delta)
    h'     = diag(e^Gam_C) h + (K * e^(Gam_C - Gam))^T delta

Reverse mode (derived from the forward above; pinned against the token-level
reverse mode of oracle.kda, which is itself pinned by finite differences):
    ddelta = scale P^T dO + (K e^(Gam_C-Gam)) dh'
    dy     = T^T ddelta
    dh     = diag(e^Gam_C) dh' + scale (Q e^Gam)^T dO - (diag(beta) K e^Gam)^T dy
    dV     = diag(beta) dy
    dbeta  = rowsum(dy * (V - (K e^Gam) h - A delta))
    dA     = -diag(beta) (dy delta^T)   (strict lower);  dP = scale dO delta^T (lower)
    and the q, k, Gam chains through e^Gam, e^(Gam_C-Gam), A and P; dg is the
    reverse cumulative sum of dGam within the chunk.

Pins (tests/test_oracle_chunkwise.py): chunk sizes 1, 16, 64 all equal the
token recurrence; plan execution equals oracle.kda.tree_fwd / tree_bwd; every
handoff buffer is read only in a round after the one that wrote it.
"""
from __future__ import annotations

import numpy as np

from .planner import EXPANDED, Plan
from .tree import Tree


def _decay(Gam):
    """exp(Gam_i - Gam_j) for j <= i, zero above the diagonal. [C,C,dk]"""
    C = Gam.shape[0]
    diff = Gam[:, None, :] - Gam[None, :, :]
    low = np.tril(np.ones((C, C), dtype=bool))
    return np.where(low[:, :, None], np.exp(np.where(low[:, :, None], diff, 0.0)), 0.0)


def chunk_fwd(h, q, k, v, g, beta, scale):
    """One chunk, one head.  Returns (O, h_new, cache)."""
    C = q.shape[0]
    Gam = np.cumsum(g, axis=0)
    D = _decay(Gam)
    strict = np.tril(np.ones((C, C)), -1)
    A = np.einsum("ic,jc,ijc->ij", k, k, D) * strict
    P = np.einsum("ic,jc,ijc->ij", q, k, D)
    T = np.linalg.inv(np.eye(C) + beta[:, None] * A)
    eG = np.exp(Gam)
    Kt = k * eG
    Qt = q * eG
    GC = Gam[-1]
    Kh = k * np.exp(GC[None, :] - Gam)
    delta = T @ (beta[:, None] * (v - Kt @ h))
    O = scale * (Qt @ h + P @ delta)
    h_new = np.exp(GC)[:, None] * h + Kh.T @ delta
    cache = dict(Gam=Gam, D=D, A=A, P=P, T=T, Kt=Kt, Qt=Qt, Kh=Kh, delta=delta, GC=GC)
    return O, h_new, cache


def chunk_bwd(h, q, k, v, g, beta, scale, dO, dh_new, cache=None):
    """Reverse mode of chunk_fwd.  Returns (dq, dk, dv, dg, dbeta, dh)."""
    if cache is None:
        _, _, cache = chunk_fwd(h, q, k, v, g, beta, scale)
    C = q.shape[0]
    Gam, D, A, P, T = cache["Gam"], cache["D"], cache["A"], cache["P"], cache["T"]
    Kt, Qt, Kh, delta, GC = cache["Kt"], cache["Qt"], cache["Kh"], cache["delta"], cache["GC"]
    strict = np.tril(np.ones((C, C)), -1)
    incl = np.tril(np.ones((C, C)))
    eGC = np.exp(GC)
    ddelta = scale * P.T @ dO + Kh @ dh_new
    dy = T.T @ ddelta
    dh = eGC[:, None] * dh_new + scale * Qt.T @ dO - (beta[:, None] * Kt).T @ dy
    dQt = scale * dO @ h.T
    dP = scale * (dO @ delta.T) * incl
    dA = -(beta[:, None] * (dy @ delta.T)) * strict
    dbeta = np.sum(dy * (v - Kt @ h - A @ delta), axis=1)
    dvv = beta[:, None] * dy
    dKt = -(beta[:, None] * dy) @ h.T
    dKh = delta @ dh_new.T
    deGC = np.sum(h * dh_new, axis=1)
    # products weighted by the per-pair decay
    dqP = np.einsum("ij,jc,ijc->ic", dP, k, D)     # row side of P
    dkP = np.einsum("ij,ic,ijc->jc", dP, q, D)     # column side of P
    dkAr = np.einsum("ij,jc,ijc->ic", dA, k, D)    # row side of A
    dkAc = np.einsum("ij,ic,ijc->jc", dA, k, D)    # column side of A
    eG = np.exp(Gam)
    dq = dQt * eG + dqP
    dk = dKt * eG + dKh * np.exp(GC[None, :] - Gam) + dkP + dkAr + dkAc
    dGam = dQt * Qt + dKt * Kt - dKh * Kh + q * dqP - k * dkP + k * dkAr - k * dkAc
    dGam[-1] += np.sum(dKh * Kh, axis=0) + deGC * eGC
    dg = np.cumsum(dGam[::-1], axis=0)[::-1]
    return dq, dk, dvv, dg, dbeta, dh


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def run_plan_fwd(plan: Plan, q, k, v, g, beta, h0, scale, n_leaf=None):
    """Execute a plan round by round.  Returns dict with o [n_out_rows,H,dv],
    h_leaf, buffers [n_buf,H,dk,dv] and chunk_h (start state of every chunk)."""
    q, k, v, g, beta, h0 = map(_f64, (q, k, v, g, beta, h0))
    H, dk, dv = q.shape[1], q.shape[2], v.shape[2]
    n_leaf = int(plan.seq_leaf.max()) + 1 if n_leaf is None else n_leaf
    o = np.zeros((plan.n_out_rows, H, dv))
    h_leaf = np.zeros((n_leaf, H, dk, dv))
    bufs = np.zeros((plan.n_buf, H, dk, dv))
    buf_round = -np.ones(plan.n_buf, dtype=np.int64)
    chunk_h = np.zeros((plan.n_chunks, H, dk, dv))
    for r in range(plan.n_rounds):
        for s in range(plan.round_seq_ptr[r], plan.round_seq_ptr[r + 1]):
            if plan.seq_init_kind[s] == 0:
                hs = h0[plan.seq_init_idx[s]].copy()
            else:
                bi = plan.seq_init_idx[s]
                assert 0 <= buf_round[bi] < r, "handoff buffer read before it was written"
                hs = bufs[bi].copy()
            for c in range(plan.seq_chunk_ptr[s], plan.seq_chunk_ptr[s + 1]):
                p0, L = plan.chunk_row0[c], plan.chunk_len[c]
                rows = plan.row_index[p0:p0 + L]
                outs = plan.out_row[p0:p0 + L]
                chunk_h[c] = hs
                for hh in range(H):
                    O, hn, _ = chunk_fwd(hs[hh], q[rows, hh], k[rows, hh], v[rows, hh],
                                         g[rows, hh], beta[rows, hh], scale)
                    m = outs >= 0
                    o[outs[m], hh] = O[m]
                    hs[hh] = hn
                if plan.chunk_save[c] >= 0:
                    bufs[plan.chunk_save[c]] = hs
                    buf_round[plan.chunk_save[c]] = r
            if plan.seq_leaf[s] >= 0:   # a node-wise sequence may end at an inner segment
                h_leaf[plan.seq_leaf[s]] = hs
    return dict(o=o, h_leaf=h_leaf, buffers=bufs, chunk_h=chunk_h)


def run_plan_bwd(plan: Plan, q, k, v, g, beta, h0, scale, dO, dh_leaf, fwd=None):
    """Reverse mode of run_plan_fwd, rounds in reverse order.

    dO [n_out_rows,H,dv]; dh_leaf [n_leaf,H,dk,dv].  Gradients of q,k,v,g,
    beta land in the rows they were read from (compact rows in MINCALL mode,
    packed rows in EXPANDED mode); replay rows add into their ancestor rows.
    Returns dict with dq, dk, dv, dg, dbeta, dh0, dh_boundary [n_buf,...]
    (total gradient of each handoff state) and seq_dh (start gradient of
    every sequence)."""
    q, k, v, g, beta, h0, dO, dh_leaf = map(_f64, (q, k, v, g, beta, h0, dO, dh_leaf))
    if fwd is None:
        fwd = run_plan_fwd(plan, q, k, v, g, beta, h0, scale, n_leaf=dh_leaf.shape[0])
    H = q.shape[1]
    expanded = plan.mode == EXPANDED
    n_gr = plan.n_packed if expanded else plan.n_rows
    grads = {n: np.zeros((n_gr,) + x.shape[1:]) for n, x in
             (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    seq_dh = np.zeros((plan.n_seq,) + h0.shape[1:])
    dh_boundary = np.zeros((plan.n_buf,) + h0.shape[1:])
    for r in reversed(range(plan.n_rounds)):
        for s in range(plan.round_seq_ptr[r], plan.round_seq_ptr[r + 1]):
            dh = dh_leaf[plan.seq_leaf[s]].copy() if plan.seq_leaf[s] >= 0 else np.zeros(h0.shape[1:])
            for c in reversed(range(plan.seq_chunk_ptr[s], plan.seq_chunk_ptr[s + 1])):
                b = plan.chunk_save[c]
                if b >= 0:
                    for ci in range(plan.buf_cons_ptr[b], plan.buf_cons_ptr[b + 1]):
                        cs = plan.buf_cons[ci]
                        assert plan.seq_round[cs] > r
                        dh = dh + seq_dh[cs]
                    dh_boundary[b] = dh
                p0, L = plan.chunk_row0[c], plan.chunk_len[c]
                rows = plan.row_index[p0:p0 + L]
                outs = plan.out_row[p0:p0 + L]
                grow = np.arange(p0, p0 + L) if expanded else rows
                dOc = np.zeros((L, H, dO.shape[2]))
                m = outs >= 0
                dOc[m] = dO[outs[m]]
                hs = fwd["chunk_h"][c]
                for hh in range(H):
                    dq, dk, dvv, dg, db, dh_prev = chunk_bwd(
                        hs[hh], q[rows, hh], k[rows, hh], v[rows, hh], g[rows, hh],
                        beta[rows, hh], scale, dOc[:, hh], dh[hh])
                    np.add.at(grads["dq"][:, hh], grow, dq)
                    np.add.at(grads["dk"][:, hh], grow, dk)
                    np.add.at(grads["dv"][:, hh], grow, dvv)
                    np.add.at(grads["dg"][:, hh], grow, dg)
                    np.add.at(grads["dbeta"][:, hh], grow, db)
                    dh[hh] = dh_prev
            seq_dh[s] = dh
    dh0 = np.zeros(h0.shape)
    for s in range(plan.n_seq):
        if plan.seq_init_kind[s] == 0:
            dh0[plan.seq_init_idx[s]] += seq_dh[s]
    grads.update(dh0=dh0, dh_boundary=dh_boundary, seq_dh=seq_dh)
    return grads
