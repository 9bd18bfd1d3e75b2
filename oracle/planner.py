"""Min-call planner for packed chunkwise linear attention (oracle; test
infrastructure only).

Sources: HARTS abstract (devfeed.tech): a linear-time planner attains the
global minimum number of sequential linear-attention calls under the packed
chunkwise-call model.  Figure 2 (thelatestinai.com): thick edges select
direct continuations; a side branch at position p can start from the state
S_B of the current call only after that call returns; three boundary cases
separate replay length from earliest legal start; all sequences of a round
form one packed call.  Figure C.1(b): side sequences start from the boundary
state and replay the parent's tail inside the core without writing outputs.
Figures D.1-D.3: R is the total replay length with chunk size B = 64.

Reading of the call model (the pages state it only in prose):
  * A call runs independent sequences.  A sequence starts from a state that
    exists before the call, at a trajectory position that is a multiple of B,
    and runs contiguous tokens down one root-to-leaf path; every chunk of it
    is a chunk of that trajectory's own B-aligned grid.
  * A child is a direct continuation (same sequence, same round, no replay)
    or side-started.  A side-started child c of v forks at p = e_v and starts
    at b = B*floor(p/B), replaying r = p - b < B rows.
  * Earliest legal start of a side child of v, with S the sequence holding v
    and b_head the position S starts at:
        case 1  r = 0:                 the state at b is made by S -> next round
        case 2  r > 0 and b > b_head:  the state at b is made by S -> next round
        case 3  b == b_head:           the state S started from already exists
                                       -> same round, replay from b_head
    (Case 3 includes a root whose fork lies inside its first chunk.)

The two-mode DP: for a node v, mode A means "the sequence holding v has not
left its head chunk by e_v" (side children start in the same round, d = 0),
mode B otherwise (d = 1).  G(v, m) is the number of rounds needed below the
round of v's sequence.  A side child c costs d + G(c, mode of c as a head);
continuing c costs G(c, mode of c inside v's sequence) and never more than
side-starting it, so the continuation is the child of largest side cost.
Rounds = 1 + G(root, mode of the root).  Ties: largest side cost, then
largest subtree token count, then smallest segment id.  Every internal node
gets a continuation, which also makes the total replay
R = sum_v (children(v) - 1) * (e_v mod B) the least possible.

Pins (tests/test_oracle_planner.py): exhaustive search over every
continuation assignment (including none) on small random trees; the worked
example of Figure 1 ([A,B,D] in call 1, then [C] and [E]); the structure of
Figure 2(c); the closed form of R; a path is one round; forks inside the
first chunk need one round; a complete k-ary tree of depth D with every
segment >= B needs D+1 rounds.
"""
from __future__ import annotations

import itertools
from dataclasses import dataclass

import numpy as np

from .tree import Tree

MINCALL = 0
EXPANDED = 1
NOREPLAY = 2   # side branches start from their exact fork state (no replay)
NODEWISE = 3   # one sequence per segment, started from its parent's end state
MINCALL_SHORT = 4   # minimum rounds; a continuation that costs no round is dropped
EXACT_MODES = (NOREPLAY, NODEWISE)
A_MODE, B_MODE = 0, 1


def _head_mode(s, e, B):
    return A_MODE if e // B == s // B else B_MODE


def dp_mincall(tree: Tree, B: int, short: bool = False):
    """Two-mode DP.  Returns (cont, G, rounds): cont[v] is the continuation
    child of v (-1 for a leaf), G[v] = (G(v,A), G(v,B)).

    short=True: where side-starting every child of v gives the same G(v, m)
    for both modes as continuing the best one, v continues none of them.  The
    round count is unchanged (G is unchanged everywhere); the sequences end
    sooner, which shortens the longest sequence of later rounds (the chain a
    round's call waits for) at the price of more replay rows."""
    n = tree.n
    sub = tree.subtree_tokens()
    G = [(0, 0)] * n
    cont = [-1] * n
    for v in reversed(tree.preorder):
        ch = tree.children[v]
        if not ch:
            continue
        base = {}
        for c in ch:
            base[c] = G[c][_head_mode(int(tree.start[c]), int(tree.end[c]), B)]
        cstar = max(ch, key=lambda c: (base[c], int(sub[c]), -c))
        cont[v] = cstar
        same_chunk = tree.end[cstar] // B == tree.start[cstar] // B
        gv, gnone = [], []
        for m in (A_MODE, B_MODE):
            d = 0 if m == A_MODE else 1
            cm = A_MODE if (m == A_MODE and same_chunk) else B_MODE
            worst = G[cstar][cm]
            for c in ch:
                if c != cstar:
                    worst = max(worst, d + base[c])
            gv.append(worst)
            gnone.append(max(d + base[c] for c in ch))
        if short and gnone == gv:
            cont[v] = -1
        G[v] = tuple(gv)
    rounds = 0
    for r in tree.roots:
        rounds = max(rounds, 1 + G[r][_head_mode(0, int(tree.end[r]), B)])
    return cont, G, rounds


def simulate(tree: Tree, B: int, cont):
    """As-soon-as-possible rounds for a continuation assignment (cont[v] is a
    child of v or -1).  Returns (rounds, R, seg_round, chain_of, chain_head,
    b_head, init) where init[chain] = ('h0', root) | ('buf', producer chain, b)."""
    n = tree.n
    chain_of = [-1] * n
    chain_head, b_head, chain_round, init = [], [], [], []
    R = 0
    for v in tree.preorder:
        p = int(tree.parent[v])
        if p < 0:
            cid = len(chain_head)
            chain_head.append(v)
            b_head.append(0)
            chain_round.append(0)
            init.append(("h0", tree.root_index[v]))
            chain_of[v] = cid
            continue
        if cont[p] == v:
            chain_of[v] = chain_of[p]
            continue
        S = chain_of[p]
        pos = int(tree.start[v])
        b = B * (pos // B)
        R += pos - b
        cid = len(chain_head)
        chain_head.append(v)
        b_head.append(b)
        if b == b_head[S]:
            chain_round.append(chain_round[S])
            init.append(init[S])
        else:
            chain_round.append(chain_round[S] + 1)
            init.append(("buf", S, b))
        chain_of[v] = cid
    seg_round = [chain_round[chain_of[v]] for v in range(n)]
    rounds = 1 + max(chain_round)
    return rounds, R, seg_round, chain_of, chain_head, b_head, init


def dp_noreplay(tree: Tree):
    """Continuations when a side branch starts from its exact fork state: that
    state exists only once the call that makes it has returned, so every side
    start costs one round and nothing is replayed.  G(v) = max(G(cont),
    max over the other children c of 1 + G(c)); the continuation is the child
    of largest G (ties as in dp_mincall: larger subtree, then smaller id).
    Returns (cont, G, rounds)."""
    n = tree.n
    sub = tree.subtree_tokens()
    G = [0] * n
    cont = [-1] * n
    for v in reversed(tree.preorder):
        ch = tree.children[v]
        if not ch:
            continue
        cstar = max(ch, key=lambda c: (G[c], int(sub[c]), -c))
        cont[v] = cstar
        G[v] = max([G[cstar]] + [1 + G[c] for c in ch if c != cstar])
    return cont, G, 1 + max(G[r] for r in tree.roots)


def simulate_exact(tree: Tree, cont):
    """Sequences when side branches start from exact fork states: a side child
    c of v starts at its own first position s_c, from the state that the
    sequence holding v emits there, one round after that sequence's round.
    Returns (rounds, seg_round, chain_of, chain_head, b_head, init) as
    simulate does."""
    n = tree.n
    chain_of = [-1] * n
    chain_head, b_head, chain_round, init = [], [], [], []
    for v in tree.preorder:
        p = int(tree.parent[v])
        if p >= 0 and cont[p] == v:
            chain_of[v] = chain_of[p]
            continue
        cid = len(chain_head)
        chain_head.append(v)
        if p < 0:
            b_head.append(0)
            chain_round.append(0)
            init.append(("h0", tree.root_index[v]))
        else:
            S = chain_of[p]
            b_head.append(int(tree.start[v]))
            chain_round.append(chain_round[S] + 1)
            init.append(("buf", S, int(tree.start[v])))
        chain_of[v] = cid
    seg_round = [chain_round[chain_of[v]] for v in range(n)]
    return 1 + max(chain_round), seg_round, chain_of, chain_head, b_head, init


def exhaustive_min_rounds(tree: Tree, B: int, limit: int = 200000):
    """Minimum rounds over every continuation assignment, where each internal
    node continues one of its children or none."""
    internal = [v for v in range(tree.n) if tree.children[v]]
    choices = [[-1] + tree.children[v] for v in internal]
    total = 1
    for c in choices:
        total *= len(c)
    if total > limit:
        raise ValueError("tree too large for exhaustive search")
    best = None
    for combo in itertools.product(*choices):
        cont = [-1] * tree.n
        for v, c in zip(internal, combo):
            cont[v] = c
        r = simulate(tree, B, cont)[0]
        best = r if best is None else min(best, r)
    return best


def replay_closed_form(tree: Tree, B: int) -> int:
    return int(sum((len(tree.children[v]) - 1) * (int(tree.end[v]) % B)
                   for v in range(tree.n) if tree.children[v]))


@dataclass
class Plan:
    """Canonical plan arrays (all int64 numpy arrays)."""
    mode: int
    B: int
    n_rounds: int
    R: int
    n_rows: int            # compact rows N
    n_packed: int          # packed rows (N + R in MINCALL)
    n_out_rows: int        # rows of o / dO (N in MINCALL, packed rows in EXPANDED)
    # per segment
    seg_round: np.ndarray
    seg_seq: np.ndarray
    seg_is_cont: np.ndarray
    seg_b: np.ndarray
    seg_replay: np.ndarray
    # per round
    round_seq_ptr: np.ndarray     # [n_rounds+1]
    # per sequence
    seq_round: np.ndarray
    seq_head: np.ndarray
    seq_leaf: np.ndarray          # leaf index (leaves ascending); -1 if the sequence ends at an
                                  # inner segment (node-wise plans)
    seq_b_head: np.ndarray
    seq_replay: np.ndarray
    seq_row_ptr: np.ndarray       # [n_seq+1] into packed rows
    seq_chunk_ptr: np.ndarray     # [n_seq+1] into chunks
    seq_init_kind: np.ndarray     # 0 = root h0, 1 = handoff buffer
    seq_init_idx: np.ndarray
    # per chunk
    chunk_seq: np.ndarray
    chunk_row0: np.ndarray        # first packed row
    chunk_len: np.ndarray
    chunk_save: np.ndarray        # buffer saved at this chunk's end, -1 if none
    # per packed row
    row_index: np.ndarray         # compact row read
    out_row: np.ndarray           # row written (-1 for replay rows)
    # per buffer
    buf_seq: np.ndarray
    buf_pos: np.ndarray           # trajectory position b of the state
    buf_chunk: np.ndarray
    buf_cons_ptr: np.ndarray      # CSR of consumer sequences
    buf_cons: np.ndarray

    @property
    def n_seq(self):
        return int(self.seq_round.shape[0])

    @property
    def n_chunks(self):
        return int(self.chunk_seq.shape[0])

    @property
    def n_buf(self):
        return int(self.buf_seq.shape[0])


def _i64(x):
    return np.asarray(x, dtype=np.int64)


def build_plan(tree: Tree, B: int, mode: int = MINCALL) -> Plan:
    n = tree.n
    if mode == EXPANDED:
        seqs = []
        for li, l in enumerate(tree.leaves):
            rows = tree.path_rows(l)
            seqs.append(dict(round=0, head=tree.root_of(l), leaf=li, b=0, r=0, rows=rows,
                             init=("h0", tree.root_index[tree.root_of(l)])))
        seg_round = np.zeros(n, np.int64)
        seg_seq = -np.ones(n, np.int64)
        seg_is_cont = np.zeros(n, np.int64)
        seg_b = -np.ones(n, np.int64)
        seg_rep = np.zeros(n, np.int64)
        n_rounds, R = 1, 0
        bufs = []
    else:
        if mode in (MINCALL, MINCALL_SHORT):
            cont, _, rounds = dp_mincall(tree, B, short=(mode == MINCALL_SHORT))
            rounds_s, R, seg_round, chain_of, chain_head, b_head, init = simulate(tree, B, cont)
        elif mode == NOREPLAY:
            cont, _, rounds = dp_noreplay(tree)
            rounds_s, seg_round, chain_of, chain_head, b_head, init = simulate_exact(tree, cont)
            R = 0
        elif mode == NODEWISE:
            cont = [-1] * n
            rounds = 1 + max(tree.depth(v) for v in range(n))
            rounds_s, seg_round, chain_of, chain_head, b_head, init = simulate_exact(tree, cont)
            R = 0
        else:
            raise ValueError("unknown mode")
        assert rounds_s == rounds
        n_rounds = rounds
        nch = len(chain_head)
        # order sequences by (round, head id)
        chain_round = [seg_round[h] for h in chain_head]
        order = sorted(range(nch), key=lambda c: (chain_round[c], chain_head[c]))
        seq_of_chain = {c: i for i, c in enumerate(order)}
        members = [[] for _ in range(nch)]
        for v in tree.preorder:
            members[chain_of[v]].append(v)
        seqs = []
        for c in order:
            h = chain_head[c]
            hp = tree.path_rows(h)
            s_h = int(tree.start[h])
            r = s_h - b_head[c]
            rep = hp[b_head[c]:s_h] if r > 0 else np.zeros(0, np.int64)
            own = np.concatenate([tree.seg_rows(v) for v in members[c]])
            leaf = members[c][-1]
            ini = init[c]
            if ini[0] == "buf":
                ini = ("buf", seq_of_chain[ini[1]], ini[2])
            seqs.append(dict(round=chain_round[c], head=h, leaf=tree.leaf_index.get(leaf, -1),
                             b=b_head[c], r=r, rows=np.concatenate([rep, own]), init=ini))
        seg_seq = _i64([seq_of_chain[chain_of[v]] for v in range(n)])
        seg_round = _i64(seg_round)
        seg_is_cont = _i64([0 if tree.parent[v] < 0 else int(cont[tree.parent[v]] == v)
                            for v in range(n)])
        if mode in (MINCALL, MINCALL_SHORT):
            seg_b = _i64([-1 if seg_is_cont[v] else B * (int(tree.start[v]) // B) for v in range(n)])
        else:
            seg_b = _i64([-1 if seg_is_cont[v] else int(tree.start[v]) for v in range(n)])
        seg_rep = _i64([0 if seg_is_cont[v] else int(tree.start[v]) - int(seg_b[v])
                        for v in range(n)])
        bufs = sorted({(s["init"][1], s["init"][2]) for s in seqs if s["init"][0] == "buf"})
    buf_id = {bk: i for i, bk in enumerate(bufs)}
    # packed rows and chunks
    row_index, out_row = [], []
    seq_row_ptr, seq_chunk_ptr = [0], [0]
    chunk_seq, chunk_row0, chunk_len, chunk_save = [], [], [], []
    for si, s in enumerate(seqs):
        base = seq_row_ptr[-1]
        rows = s["rows"]
        row_index.extend(int(x) for x in rows)
        for j in range(len(rows)):
            if j < s["r"]:
                out_row.append(-1)
            elif mode == EXPANDED:
                out_row.append(base + j)
            else:
                out_row.append(int(rows[j]))
        seq_row_ptr.append(base + len(rows))
        # chunks: the sequence's own B-grid from its start; with exact starts
        # the grid is also cut at every position a side branch starts from
        cuts = sorted(pos - s["b"] for (sp, pos) in bufs if sp == si) if mode in EXACT_MODES else []
        c0 = 0
        while c0 < len(rows):
            nxt = min(len(rows), (c0 // B + 1) * B)
            for x in cuts:
                if c0 < x < nxt:
                    nxt = x
                    break
            L = nxt - c0
            chunk_seq.append(si)
            chunk_row0.append(base + c0)
            chunk_len.append(L)
            endpos = s["b"] + c0 + L
            if mode in EXACT_MODES or L == B:
                chunk_save.append(buf_id.get((si, endpos), -1))
            else:
                chunk_save.append(-1)
            c0 = nxt
        seq_chunk_ptr.append(len(chunk_seq))
    buf_seq = _i64([bk[0] for bk in bufs])
    buf_pos = _i64([bk[1] for bk in bufs])
    buf_chunk = []
    for (si, b) in bufs:
        hits = [c for c in range(seq_chunk_ptr[si], seq_chunk_ptr[si + 1])
                if chunk_save[c] == buf_id[(si, b)]]
        assert len(hits) == 1, "handoff buffer not at exactly one chunk end"
        buf_chunk.append(hits[0])
    cons = [[] for _ in bufs]
    for si, s in enumerate(seqs):
        if s["init"][0] == "buf":
            cons[buf_id[(s["init"][1], s["init"][2])]].append(si)
    cons_ptr = [0]
    for c in cons:
        cons_ptr.append(cons_ptr[-1] + len(c))
    round_ptr = [0] * (n_rounds + 1)
    for s in seqs:
        round_ptr[s["round"] + 1] += 1
    round_ptr = np.cumsum(round_ptr)
    return Plan(
        mode=mode, B=B, n_rounds=n_rounds, R=int(R), n_rows=tree.n_rows,
        n_packed=len(row_index),
        n_out_rows=(len(row_index) if mode == EXPANDED else tree.n_rows),
        seg_round=seg_round, seg_seq=seg_seq, seg_is_cont=seg_is_cont, seg_b=seg_b,
        seg_replay=seg_rep,
        round_seq_ptr=_i64(round_ptr),
        seq_round=_i64([s["round"] for s in seqs]),
        seq_head=_i64([s["head"] for s in seqs]),
        seq_leaf=_i64([s["leaf"] for s in seqs]),
        seq_b_head=_i64([s["b"] for s in seqs]),
        seq_replay=_i64([s["r"] for s in seqs]),
        seq_row_ptr=_i64(seq_row_ptr), seq_chunk_ptr=_i64(seq_chunk_ptr),
        seq_init_kind=_i64([0 if s["init"][0] == "h0" else 1 for s in seqs]),
        seq_init_idx=_i64([s["init"][1] if s["init"][0] == "h0" else buf_id[(s["init"][1],
                                                                           s["init"][2])]
                           for s in seqs]),
        chunk_seq=_i64(chunk_seq), chunk_row0=_i64(chunk_row0), chunk_len=_i64(chunk_len),
        chunk_save=_i64(chunk_save),
        row_index=_i64(row_index), out_row=_i64(out_row),
        buf_seq=buf_seq, buf_pos=buf_pos, buf_chunk=_i64(buf_chunk),
        buf_cons_ptr=_i64(cons_ptr), buf_cons=_i64([x for c in cons for x in c]),
    )
