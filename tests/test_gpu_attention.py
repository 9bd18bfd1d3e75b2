"""GPU parity of the tree-ancestor attention (tree_attn_fwd / tree_attn_bwd,
through the C-ABI) against the float64 oracle (oracle/attention.py).

Small trees compare every element of o, lse, dq, dk, dv.  The full-size case
runs the 4-ary depth-3 tree at 16 heads, d = 128, with the upstream gradient
on one trajectory only: rows on the path must match the oracle run on that
path alone (o and lse for every path row, the gradients because the loss is
exactly that trajectory's), and rows off the path must get exactly zero
gradients.  Bar: relative L2 <= 2e-3 per tensor (bf16 inputs)."""
import numpy as np
import pytest

from gpu_cases import TOL, rel_l2
from oracle import attention as oa
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

pytestmark = pytest.mark.gpu


def _bf16_inputs(rng, N, H, D):
    f = lambda: synth.round_bf16(rng.standard_normal((N, H, D), dtype=np.float32))
    return f(), f(), f(), f()


def _run(plan, q, k, v, dO, scale):
    import torch
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda().to(torch.bfloat16)
    qt, kt, vt, dt = t(q), t(k), t(v), t(dO)
    o, lse = B.tree_attn_fwd(plan, qt, kt, vt, scale)
    dq, dk, dv = B.tree_attn_bwd(plan, qt, kt, vt, o, lse, dt, scale)
    torch.cuda.synchronize()
    return {n: x.cpu().numpy() for n, x in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}


@pytest.mark.parametrize("kind,H,D", [("fig1", 2, 64), ("fig1", 2, 128), ("random", 2, 128),
                                      ("random", 3, 64), ("path", 1, 128)])
def test_attention_small(kind, H, D):
    rng = np.random.Generator(np.random.PCG64(hash((kind, H, D)) % 2**32))
    if kind == "fig1":
        spec = synth.tree_fig1()
    elif kind == "path":
        spec = synth.tree_path([100, 37, 64, 5])
    else:
        spec = synth.shuffled_rows(synth.tree_random(rng, 11, 1, 150, 3, n_roots=2), rng)
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    plan = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 16)
    q, k, v, dO = _bf16_inputs(rng, t.n_rows, H, D)
    scale = 1.0 / np.sqrt(D)
    print(f"case attention {kind} rows={t.n_rows} H={H} D={D} tiles={plan.info['n_att_tiles']} "
          f"items={plan.info['n_att_items']}", flush=True)
    got = _run(plan, q, k, v, dO, scale)
    o, lse = oa.tree_attention_fwd(t, q, k, v, scale)
    dq, dk, dv = oa.tree_attention_bwd(t, q, k, v, scale, dO)
    errs = {"o": rel_l2(got["o"], o), "lse": rel_l2(got["lse"], lse), "dq": rel_l2(got["dq"], dq),
            "dk": rel_l2(got["dk"], dk), "dv": rel_l2(got["dv"], dv)}
    print("  rel L2:", {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
    assert all(e <= TOL for e in errs.values()), errs


def test_attention_fullsize_trajectory():
    import torch
    w = synth.workload(4)
    t = Tree(w.tree.parent, w.tree.seg_len, w.tree.seg_row)
    plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, 64)
    N, H, D = t.n_rows, 16, 128
    leaves = [int(x) for x in plan.export("LEAF_SEG")]
    leaf = leaves[int(np.random.Generator(np.random.PCG64(77)).integers(len(leaves)))]
    rows = t.path_rows(leaf)
    print(f"case attention full size rows={N} H={H} D={D} tiles={plan.info['n_att_tiles']} "
          f"items={plan.info['n_att_items']} trajectory={len(rows)} rows", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    mk = lambda: torch.randn(N, H, D, generator=gen, device="cuda").to(torch.bfloat16)
    q, k, v = mk(), mk(), mk()
    rows_t = torch.from_numpy(rows.astype(np.int64)).cuda()
    dO = torch.zeros(N, H, D, device="cuda", dtype=torch.bfloat16)
    dO[rows_t] = torch.randn(len(rows), H, D, generator=gen, device="cuda").to(torch.bfloat16)
    scale = 1.0 / np.sqrt(D)
    o, lse = B.tree_attn_fwd(plan, q, k, v, scale)
    dq, dk, dv = B.tree_attn_bwd(plan, q, k, v, o, lse, dO, scale)
    torch.cuda.synchronize()
    print("  GPU done", flush=True)
    # the path as a tree of its own (a chain of the path's segments)
    segs = t.path(leaf)
    pt = Tree([-1] + list(range(len(segs) - 1)), [int(t.seg_len[s]) for s in segs])
    bad = {}
    for h in (0, 9):
        pick = lambda x: x[rows_t, h:h + 1].float().cpu().numpy()
        o_ref, lse_ref = oa.tree_attention_fwd(pt, pick(q), pick(k), pick(v), scale)
        gq, gk, gv = oa.tree_attention_bwd(pt, pick(q), pick(k), pick(v), scale, pick(dO))
        errs = {"o": rel_l2(pick(o), o_ref), "lse": rel_l2(lse[rows_t, h].cpu().numpy(), lse_ref[:, 0]),
                "dq": rel_l2(pick(dq), gq), "dk": rel_l2(pick(dk), gk), "dv": rel_l2(pick(dv), gv)}
        print(f"  head {h} rel L2:", {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
        bad.update({f"{n}[h{h}]": e for n, e in errs.items() if not e <= TOL})
    assert not bad, bad
    off = torch.ones(N, dtype=torch.bool, device="cuda")
    off[rows_t] = False
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert float(x[off].abs().max()) == 0.0, name
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
