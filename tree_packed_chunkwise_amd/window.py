"""Sharing windows: one producer call for a tree's shared prefix, consumer
microbatches started from its end states, and one producer backward after
the consumers' gradients have accumulated (HARTS abstract: within each
sharing window, gradients from dependent microbatches accumulate before one
backward pass through the shared prefix computation; thelatestinai.com
Figure 3: producer forward PF, consumer forward/backward Fi/Bi in 1F1B order,
producer backward PB inside the window's last consumer backward).

The split: segments at depth <= split_depth form the producer forest; every
segment at depth split_depth + 1 heads a consumer subtree, and the consumer
subtrees (ascending head id) are cut into n_micro microbatches.  A consumer
root starts from its parent's end state, which is a leaf state of the
producer call.  The calls are kda_tree_fwd / kda_tree_bwd on one plan per
part; kda_state_copy / kda_state_sum move and sum the states between them
(every sum in a fixed order).  This module is host-side orchestration and
argument marshalling; all arithmetic runs in libkda_tree.so.

Row layout: the window needs each part's rows contiguous, so it fixes the
compact layout of the whole tree (`seg_row`): the producer segments in id
order, then each microbatch's subtrees (head by head, preorder within a
subtree).  The caller lays out q, k, v, g, beta, dO in that order; every
output comes back in it.
"""
from __future__ import annotations

import numpy as np

from . import binding as B


def _depths(parent):
    n = len(parent)
    d = -np.ones(n, np.int64)
    for v in range(n):
        path = []
        u = v
        while u >= 0 and d[u] < 0:
            path.append(u)
            u = int(parent[u])
        base = -1 if u < 0 else int(d[u])
        for w in reversed(path):
            base += 1
            d[w] = base
    return d


class SharingWindow:
    def __init__(self, parent, seg_len, split_depth: int, n_micro: int, chunk: int = 64,
                 mode: int = B.MINCALL):
        parent = np.asarray(parent, np.int64)
        seg_len = np.asarray(seg_len, np.int64)
        n = len(parent)
        children = [[] for _ in range(n)]
        for v in range(n):
            if parent[v] >= 0:
                children[int(parent[v])].append(v)
        depth = _depths(parent)
        prod = [v for v in range(n) if depth[v] <= split_depth]
        heads = [v for v in range(n) if depth[v] == split_depth + 1]
        if not heads:
            raise ValueError("no segment below the split depth: nothing to share")
        if not 1 <= n_micro <= len(heads):
            raise ValueError("n_micro must be in [1, number of consumer subtrees]")

        def subtree(h):
            out, stack = [], [h]
            while stack:
                u = stack.pop()
                out.append(u)
                stack.extend(reversed(children[u]))
            return out

        groups = [list(x) for x in np.array_split(np.asarray(heads), n_micro)]
        order = list(prod)
        gsegs = []
        for gh in groups:
            segs = [u for h in gh for u in subtree(int(h))]
            gsegs.append(segs)
            order += segs
        seg_row = np.zeros(n, np.int64)
        r = 0
        for v in order:
            seg_row[v] = r
            r += int(seg_len[v])
        self.seg_row, self.n_rows, self.n_seg = seg_row, int(r), n
        self.split_depth, self.n_micro, self.chunk, self.mode = split_depth, n_micro, chunk, mode

        def local_plan(segs):
            idx = {v: i for i, v in enumerate(segs)}
            par = [idx.get(int(parent[v]), -1) for v in segs]
            lens = [int(seg_len[v]) for v in segs]
            base = int(seg_row[segs[0]])
            rows = [int(seg_row[v]) - base for v in segs]
            return B.KDAPlan(par, lens, rows, chunk, mode), base

        full_leaves = [v for v in range(n) if not children[v]]
        full_leaf_idx = {v: i for i, v in enumerate(full_leaves)}
        self.n_leaf = len(full_leaves)
        self.n_root = int(np.sum(parent < 0))
        # producer
        self.plan_p, _ = local_plan(prod)
        self.rows_p = int(sum(int(seg_len[v]) for v in prod))
        p_leaves = [prod[int(i)] for i in self.plan_p.export("LEAF_SEG")]
        p_leaf_idx = {v: i for i, v in enumerate(p_leaves)}
        # producer leaves that are leaves of the whole tree
        self.p_full_src = [p_leaf_idx[v] for v in p_leaves if not children[v]]
        self.p_full_dst = [full_leaf_idx[v] for v in p_leaves if not children[v]]
        # their end-state gradients come from the caller's dh_leaf (CSR over producer leaves)
        ptr, idx = [0], []
        for v in p_leaves:
            if not children[v]:
                idx.append(full_leaf_idx[v])
            ptr.append(len(idx))
        self.p_init_ptr, self.p_init_idx = ptr, idx
        # microbatches
        self.micro = []
        for gh, segs in zip(groups, gsegs):
            plan, base = local_plan(segs)
            roots = [segs[int(i)] for i in plan.export("ROOT_SEG")]
            m_leaves = [segs[int(i)] for i in plan.export("LEAF_SEG")]
            h0_src = [p_leaf_idx[int(parent[h])] for h in roots]
            # consumer start-state gradients -> producer leaves (ascending root index)
            cptr, cidx = [0], []
            for j in range(len(p_leaves)):
                cidx.extend(i for i, s in enumerate(h0_src) if s == j)
                cptr.append(len(cidx))
            rows = int(sum(int(seg_len[v]) for v in segs))
            self.micro.append(dict(plan=plan, base=base, rows=rows, n_root=len(roots),
                                   h0_src=h0_src, ptr=cptr, idx=cidx,
                                   leaf_full=[full_leaf_idx[v] for v in m_leaves]))
        self._dev = {}

    def _idx(self, key, vals, device):
        import torch
        k = (key, str(device))
        if k not in self._dev:
            self._dev[k] = torch.tensor(np.asarray(vals, np.int32), dtype=torch.int32, device=device)
        return self._dev[k]

    def run(self, q, k, v, g, beta, scale, h0=None, dO=None, dh_leaf=None):
        """Producer forward, then per microbatch its forward and (when dO is
        given) its backward with the start-state gradients accumulated into the
        producer's end-state gradients, then the producer backward.  Returns
        dict(o, h_leaf[, dq, dk, dv, dg, dbeta, dh0]) for the whole tree in the
        window's row layout."""
        import torch
        dev = q.device
        N, H, D = q.shape
        if N != self.n_rows:
            raise ValueError("inputs must hold the whole tree in the window's row layout")
        f32 = dict(dtype=torch.float32, device=dev)
        bwd = dO is not None
        o = torch.empty((N, H, D), **f32)
        h_leaf = torch.empty((self.n_leaf, H, D, D), **f32)
        grads = {}
        if bwd:
            grads = {n: torch.empty((N, H, D), **f32) for n in ("dq", "dk", "dv", "dg")}
            grads["dbeta"] = torch.empty((N, H), **f32)
        sl = lambda x, r0, n: None if x is None else x[r0:r0 + n]

        def fwd(plan, r0, n, hs):
            out = B.alloc_fwd(plan, H, D, dev)
            out["o"] = o[r0:r0 + n]
            return B.kda_tree_fwd(plan, sl(q, r0, n), sl(k, r0, n), sl(v, r0, n), sl(g, r0, n),
                                  sl(beta, r0, n), hs, scale, out=out)

        def bwd_call(plan, r0, n, saved, dhl, hs):
            out = B.alloc_bwd(plan, H, D, dev, boundary=False)
            for nm in ("dq", "dk", "dv", "dg", "dbeta"):
                out[nm] = grads[nm][r0:r0 + n]
            return B.kda_tree_bwd(plan, sl(q, r0, n), sl(k, r0, n), sl(v, r0, n), sl(g, r0, n),
                                  sl(beta, r0, n), saved, sl(dO, r0, n), dhl, hs, scale, out=out,
                                  boundary=False)

        # PF
        fp = fwd(self.plan_p, 0, self.rows_p, h0)
        if self.p_full_src:
            B.kda_state_copy(fp["h_leaf"], self._idx("pfs", self.p_full_src, dev), h_leaf,
                             self._idx("pfd", self.p_full_dst, dev), len(self.p_full_src))
        if bwd:
            dhl_p = torch.empty((self.plan_p.info["n_leaf"], H, D, D), **f32)
            if dh_leaf is not None:
                B.kda_state_sum(dh_leaf, self._idx("pip", self.p_init_ptr, dev),
                                self._idx("pii", self.p_init_idx, dev), dhl_p, accumulate=False)
            else:
                dhl_p.zero_()
        for mi, m in enumerate(self.micro):
            h0_m = torch.empty((m["n_root"], H, D, D), **f32)
            B.kda_state_copy(fp["h_leaf"], self._idx(("h0", mi), m["h0_src"], dev), h0_m, None,
                             m["n_root"])
            fm = fwd(m["plan"], m["base"], m["rows"], h0_m)
            lf = self._idx(("lf", mi), m["leaf_full"], dev)
            B.kda_state_copy(fm["h_leaf"], None, h_leaf, lf, len(m["leaf_full"]))
            if bwd:
                dhl_m = torch.empty((len(m["leaf_full"]), H, D, D), **f32)
                if dh_leaf is not None:
                    B.kda_state_copy(dh_leaf, lf, dhl_m, None, len(m["leaf_full"]))
                else:
                    dhl_m.zero_()
                gm = bwd_call(m["plan"], m["base"], m["rows"], fm["saved"], dhl_m, h0_m)
                B.kda_state_sum(gm["dh0"], self._idx(("cp", mi), m["ptr"], dev),
                                self._idx(("ci", mi), m["idx"], dev), dhl_p, accumulate=True)
        res = dict(o=o, h_leaf=h_leaf)
        if bwd:   # PB
            gp = bwd_call(self.plan_p, 0, self.rows_p, fp["saved"], dhl_p, h0)
            res.update(grads)
            res["dh0"] = gp["dh0"]
        return res
