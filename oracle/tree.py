"""Rollout-tree conventions (oracle; test infrastructure only).

Follows HARTS Figure 1(a) (thelatestinai.com): boxes are contiguous token
ranges; trajectories share prefixes and may need different next-token labels.
Figure 2(a): boxes are fork-free segments.  Figure C.1(a): one compact
physical ordering holds every unique token once.

Conventions (the plainest reading; the pages give none explicitly):
  * A segment starts at the trajectory position where its parent ends:
    s_root = 0, s_c = e_parent(c), e_v = s_v + len_v.
  * Segment v occupies compact rows seg_row[v] .. seg_row[v]+len_v-1.
  * Trajectories are root-to-leaf paths, ordered by leaf id ascending.
  * A forest is allowed; roots are indexed by ascending segment id.
  * Next-token targets: position t of trajectory tau (t = 0..L-2) reads the
    logit row of its own token and targets the token at position t+1 (the
    "one logit row z_B supplies T1/T2's distinct targets" example, Figure 1).
"""
from __future__ import annotations

import numpy as np


class TreeError(ValueError):
    pass


class Tree:
    def __init__(self, parent, seg_len, seg_row=None):
        parent = np.asarray(parent, dtype=np.int64)
        seg_len = np.asarray(seg_len, dtype=np.int64)
        n = int(parent.shape[0])
        if seg_len.shape != (n,):
            raise TreeError("seg_len shape")
        if n == 0:
            raise TreeError("empty tree")
        if np.any(seg_len <= 0):
            raise TreeError("segment length must be positive")
        if np.any(parent < -1) or np.any(parent >= n):
            raise TreeError("parent id out of range")
        children = [[] for _ in range(n)]
        roots = []
        for i in range(n):
            p = int(parent[i])
            if p == i:
                raise TreeError("self parent")
            if p < 0:
                roots.append(i)
            else:
                children[p].append(i)
        if not roots:
            raise TreeError("no root")
        # pre-order from the roots; a node not reached lies on a cycle
        order = []
        stack = list(reversed(roots))
        seen = np.zeros(n, dtype=bool)
        while stack:
            v = stack.pop()
            if seen[v]:
                raise TreeError("node reached twice")
            seen[v] = True
            order.append(v)
            stack.extend(reversed(children[v]))
        if not seen.all():
            raise TreeError("cycle")
        start = np.zeros(n, dtype=np.int64)
        end = np.zeros(n, dtype=np.int64)
        for v in order:
            p = int(parent[v])
            start[v] = 0 if p < 0 else end[p]
            end[v] = start[v] + seg_len[v]
        if seg_row is None:
            seg_row = np.concatenate([[0], np.cumsum(seg_len)[:-1]])
        seg_row = np.asarray(seg_row, dtype=np.int64)
        n_rows = int(seg_len.sum())
        # rows must be a partition of [0, n_rows)
        cover = np.zeros(n_rows, dtype=np.int64)
        for v in range(n):
            r0 = int(seg_row[v])
            if r0 < 0 or r0 + seg_len[v] > n_rows:
                raise TreeError("seg_row out of range")
            cover[r0:r0 + seg_len[v]] += 1
        if np.any(cover != 1):
            raise TreeError("segments overlap in the row space")
        self.n = n
        self.parent = parent
        self.seg_len = seg_len
        self.seg_row = seg_row
        self.children = children
        self.roots = roots
        self.root_index = {r: i for i, r in enumerate(roots)}
        self.preorder = order
        self.start = start
        self.end = end
        self.n_rows = n_rows
        self.leaves = [v for v in range(n) if not children[v]]
        self.leaf_index = {v: i for i, v in enumerate(self.leaves)}

    def root_of(self, v: int) -> int:
        while self.parent[v] >= 0:
            v = int(self.parent[v])
        return v

    def path(self, v: int) -> list:
        """Segments from the root down to v."""
        p = []
        while v >= 0:
            p.append(v)
            v = int(self.parent[v])
        return p[::-1]

    def depth(self, v: int) -> int:
        """Number of ancestors of segment v (a root has depth 0)."""
        return len(self.path(v)) - 1

    def seg_rows(self, v: int) -> np.ndarray:
        return np.arange(self.seg_row[v], self.seg_row[v] + self.seg_len[v], dtype=np.int64)

    def path_rows(self, v: int) -> np.ndarray:
        """Compact rows of the trajectory ending at segment v, in position order."""
        return np.concatenate([self.seg_rows(s) for s in self.path(v)])

    def subtree_tokens(self) -> np.ndarray:
        tot = self.seg_len.copy()
        for v in reversed(self.preorder):
            p = int(self.parent[v])
            if p >= 0:
                tot[p] += tot[v]
        return tot

    def n_expanded(self) -> int:
        return int(sum(self.end[l] for l in self.leaves))

    def gather_map(self):
        """(pos_row, pos_next_row) for every trajectory position that has a
        next token: trajectories by leaf id ascending, positions 0..L-2."""
        rows, nxt = [], []
        for l in self.leaves:
            pr = self.path_rows(l)
            rows.append(pr[:-1])
            nxt.append(pr[1:])
        return np.concatenate(rows), np.concatenate(nxt)
