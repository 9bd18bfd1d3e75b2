"""Full-size parity on the benchmark workloads, in the launch configuration
bench.py times: the whole tree, all 16 heads, one forward and one backward
call through the C-ABI.

The float64 oracle cannot run a whole 100k-550k row tree, so each case puts
the upstream gradients on one trajectory only: dO is drawn on the rows of the
trajectory that ends at leaf L and is zero elsewhere, and dh_leaf is drawn
for L only.  The tree loss is then exactly that trajectory's loss (an output
row depends only on its own path prefix), so on the path rows the tree-packed
outputs and gradients must equal the oracle's single-path recurrence and
backward (float64), the root's dh0 must equal the path's start-state
gradient, and every gradient of a row off the path must be exactly zero."""
import numpy as np
import pytest

from gpu_cases import TOL, rel_l2
from oracle import kda as okda
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("widx,heads,mode", [(1, (0, 15), B.MINCALL), (2, (0, 15), B.MINCALL),
                                             (3, (5,), B.MINCALL), (2, (3,), B.NOREPLAY),
                                             (2, (3,), B.NODEWISE), (3, (5,), B.NODEWISE),
                                             (2, (7,), B.MINCALL_SHORT)])
def test_fullsize_trajectory_parity(widx, heads, mode):
    import torch
    w = synth.workload(widx)
    t = Tree(w.tree.parent, w.tree.seg_len, w.tree.seg_row)
    plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk, mode)
    info = plan.info
    N, H, D = info["n_rows"], w.H, w.dk
    leaves = [int(x) for x in plan.export("LEAF_SEG")]
    li = int(np.random.Generator(np.random.PCG64(100 + widx)).integers(len(leaves)))
    rows = t.path_rows(leaves[li])
    print(f"case {w.name} mode {mode}: rows={N} rounds={info['n_rounds']} R={info['R']} "
          f"trajectory leaf={leaves[li]} length={len(rows)} heads={heads}", flush=True)
    dev = torch.device("cuda:0")
    inp = synth.make_kda_inputs_device(7000 + widx, N, H, D, D, dev, w.bf16)
    rows_t = torch.from_numpy(rows.astype(np.int64)).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(8000 + widx)
    dt = inp["q"].dtype
    dO = torch.zeros(N, H, D, device=dev, dtype=dt)
    dO[rows_t] = torch.randn(len(rows), H, D, generator=gen, device=dev).to(dt)
    dhl = torch.zeros(len(leaves), H, D, D, device=dev)
    dhl[li] = torch.randn(H, D, D, generator=gen, device=dev)
    f = B.kda_tree_fwd(plan, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], None,
                       inp["scale"])
    g = B.kda_tree_bwd(plan, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], f["saved"],
                       dO, dhl, None, inp["scale"])
    torch.cuda.synchronize()
    print("  GPU fwd+bwd done", flush=True)

    root = t.root_index[t.root_of(leaves[li])]
    bad = {}
    for h in heads:
        pick = lambda x: x[rows_t, h:h + 1].float().cpu().numpy()
        q, k, v, gg, dOp = pick(inp["q"]), pick(inp["k"]), pick(inp["v"]), pick(inp["g"]), pick(dO)
        beta = inp["beta"][rows_t, h:h + 1].cpu().numpy()
        S0 = np.zeros((1, D, D))
        o_ref, S_ref = okda.path_fwd(S0, q, k, v, gg, beta, inp["scale"])
        dq, dk, dv, dg, db, dS0, _ = okda.path_bwd(S0, q, k, v, gg, beta, inp["scale"], dOp,
                                                  dhl[li, h:h + 1].cpu().numpy())
        got = lambda name: g[name][rows_t, h].cpu().numpy()
        errs = {
            "o": rel_l2(f["o"][rows_t, h].cpu().numpy(), o_ref[:, 0]),
            "h_leaf": rel_l2(f["h_leaf"][li, h].cpu().numpy(), S_ref[0]),
            "dq": rel_l2(got("dq"), dq[:, 0]), "dk": rel_l2(got("dk"), dk[:, 0]),
            "dv": rel_l2(got("dv"), dv[:, 0]), "dg": rel_l2(got("dg"), dg[:, 0]),
            "dbeta": rel_l2(g["dbeta"][rows_t, h].cpu().numpy(), db[:, 0]),
            "dh0": rel_l2(g["dh0"][root, h].cpu().numpy(), dS0[0]),
        }
        print(f"  head {h} rel L2:", {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
        bad.update({f"{n}[h{h}]": e for n, e in errs.items() if not e <= TOL})
    assert not bad, bad

    # rows off the trajectory carry no loss: their gradients are exactly zero
    on = torch.zeros(N, dtype=torch.bool, device=dev)
    on[rows_t] = True
    off = ~on
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        m = float(g[name][off].abs().max()) if bool(off.any()) else 0.0
        assert m == 0.0, (name, m)
    assert all(bool(torch.isfinite(f[n]).all()) for n in ("o", "h_leaf"))


@pytest.mark.parametrize("gate", ["default", "weak"])
def test_fullsize_tree_equals_expanded_bitwise(gate):
    """The whole forward-and-backward workload tree (103,568 rows), all 16
    heads: the tree-packed forward and the trajectory-expanded forward of the
    same kernels (313,736 rows) agree bit for bit at every row of every
    trajectory and at every leaf state -- replay keeps each trajectory's own
    chunk grid (HARTS abstract: bounded replay preserves the per-trajectory
    chunkwise numerical path)."""
    import torch
    w = synth.workload(2)
    plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk)
    eplan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk, B.EXPANDED)
    N = plan.info["n_rows"]
    print(f"case bitwise full size {w.name} gate={gate}: rows={N} "
          f"expanded={eplan.info['n_out_rows']} replay rows={plan.info['R']}", flush=True)
    dev = torch.device("cuda:0")
    inp = synth.make_kda_inputs_device(7100, N, w.H, w.dk, w.dv, dev, w.bf16, gate=gate)
    h0 = torch.randn(1, w.H, w.dk, w.dv, device=dev) / np.sqrt(w.dk)
    f = B.kda_tree_fwd(plan, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], h0,
                       inp["scale"])
    o_tree, hl_tree = f["o"], f["h_leaf"]
    del f
    e = B.kda_tree_fwd(eplan, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], h0,
                       inp["scale"])
    torch.cuda.synchronize()
    ri = torch.from_numpy(eplan.export("ROW_INDEX").astype(np.int64)).to(dev)
    assert bool(torch.isfinite(o_tree).all())
    same_rows = torch.eq(e["o"], o_tree.index_select(0, ri)).all(dim=2).all(dim=1)
    print(f"  rows equal: {int(same_rows.sum())} of {same_rows.numel()}", flush=True)
    assert bool(same_rows.all())
    assert torch.equal(e["h_leaf"], hl_tree)


def _subtree(t: Tree, leaves):
    """The union of the root paths of `leaves` as a tree of its own: parent,
    lengths (segments renumbered in ascending old id) and the compact rows of
    the new segments in order."""
    segs = sorted({a for l in leaves for a in t.path(l)})
    new = {a: i for i, a in enumerate(segs)}
    parent = np.array([new[t.parent[a]] if t.parent[a] >= 0 else -1 for a in segs], np.int32)
    lens = np.array([len(t.seg_rows(a)) for a in segs], np.int32)
    rows = np.concatenate([t.seg_rows(a) for a in segs]).astype(np.int64)
    return segs, new, Tree(parent, lens), rows


@pytest.mark.parametrize("gate,n_traj", [("default", 4), ("weak", 2)])
def test_fullsize_trajectories_all_heads(gate, n_traj):
    """Trajectories in different depth-1 subtrees of the 103,568-row tree (the
    shortest below each of the first n_traj children of the root), all 16
    heads, upstream gradients on their rows and leaf states: the outputs,
    leaf states, every input gradient on their rows, dh0 and the total
    gradient of every handoff state against the float64 oracle run on the
    union of their root paths (the rows off it carry no loss, and every
    handoff state off it must get a zero gradient).  Weak gates keep the
    start and handoff states visible far down the paths."""
    import torch
    w = synth.workload(2)
    t = Tree(w.tree.parent, w.tree.seg_len, w.tree.seg_row)
    plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk)
    N, H, D = plan.info["n_rows"], w.H, w.dk
    root = t.roots[0]
    picks = []
    for c in t.children[root][:n_traj]:   # the shortest trajectory below each child
        below, stack = [], [c]
        while stack:
            v = stack.pop()
            if t.children[v]:
                stack += t.children[v]
            else:
                below.append(v)
        picks.append(min(below, key=lambda l: (len(t.path_rows(l)), l)))
    segs, new, sub, rows = _subtree(t, picks)
    print(f"case {n_traj} trajectories {w.name} gate={gate}: leaves {picks}, "
          f"{len(rows)} of {N} rows, 16 heads", flush=True)
    dev = torch.device("cuda:0")
    inp = synth.make_kda_inputs_device(7200, N, H, D, D, dev, w.bf16, gate=gate)
    rows_t = torch.from_numpy(rows).to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(8200)
    dt = inp["q"].dtype
    dO = torch.zeros(N, H, D, device=dev, dtype=dt)
    dO[rows_t] = torch.randn(len(rows), H, D, generator=gen, device=dev).to(dt)
    leaves = [int(x) for x in plan.export("LEAF_SEG")]
    dhl = torch.zeros(len(leaves), H, D, D, device=dev)
    for v in picks:
        dhl[leaves.index(v)] = torch.randn(H, D, D, generator=gen, device=dev)
    h0 = torch.randn(1, H, D, D, generator=gen, device=dev) / np.sqrt(D)
    f = B.kda_tree_fwd(plan, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], h0,
                       inp["scale"])
    g = B.kda_tree_bwd(plan, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], f["saved"],
                       dO, dhl, h0, inp["scale"])
    torch.cuda.synchronize()
    print("  GPU fwd+bwd done", flush=True)
    # handoff states on the four paths, located as (subtree segment, trajectory position)
    bseq, bpos = plan.export("BUF_SEQ"), plan.export("BUF_POS")
    seq_leaf, seq_head = plan.export("SEQ_LEAF"), plan.export("SEQ_HEAD")
    on_paths, bounds = [], []
    for bi, (s, p) in enumerate(zip(bseq, bpos)):
        v = leaves[int(seq_leaf[s])] if seq_leaf[s] >= 0 else int(seq_head[s])
        seg = next(a for a in t.path(v) if t.start[a] < p <= t.end[a])
        if seg in new:
            on_paths.append(bi)
            bounds.append((new[seg], int(p)))
    host = lambda x: x.index_select(0, rows_t).float().cpu().numpy().astype(np.float64)
    q, k, v, gg, dOh = host(inp["q"]), host(inp["k"]), host(inp["v"]), host(inp["g"]), host(dO)
    beta = host(inp["beta"])
    sub_leaf = [leaves.index(segs[l]) for l in sub.leaves]
    h0h = h0.cpu().numpy().astype(np.float64)
    o_ref, hl_ref = okda.tree_fwd(sub, q, k, v, gg, beta, h0h, inp["scale"])
    r = okda.tree_bwd(sub, q, k, v, gg, beta, h0h, inp["scale"], dOh,
                      dhl[sub_leaf].cpu().numpy().astype(np.float64), boundaries=bounds)
    print("  oracle done", flush=True)
    errs = {"o": rel_l2(host(f["o"]), o_ref),
            "h_leaf": rel_l2(f["h_leaf"][sub_leaf].cpu().numpy(), hl_ref),
            "dh0": rel_l2(g["dh0"].cpu().numpy(), r["dh0"])}
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        errs[n] = rel_l2(host(g[n]), r[n])
    if bounds:
        errs["dh_boundary"] = rel_l2(g["dh_boundary"][on_paths].cpu().numpy(),
                                     np.stack(r["boundary"]))
    print(f"  {len(on_paths)} handoff states on the paths; rel L2:",
          {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, bad
    off = [bi for bi in range(len(bseq)) if bi not in set(on_paths)]
    if off:
        assert float(g["dh_boundary"][off].abs().max()) == 0.0
    on = torch.zeros(N, dtype=torch.bool, device=dev)
    on[rows_t] = True
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert float(g[name][~on].abs().max()) == 0.0, name
