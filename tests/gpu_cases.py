"""Shared helpers of the GPU parity tests: seeded inputs, the HIP path
through the ctypes binding, and the float64 oracle on the same inputs."""
from __future__ import annotations

import numpy as np

from oracle import kda as okda
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

TOL = 2e-3  # relative L2 per output tensor (bf16 inputs, fp32 state)


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (n if n > 0 else 1.0))


def to_dev(inp: synth.KDAInputs, device="cuda"):
    import torch
    dt = torch.bfloat16 if inp.bf16 else torch.float32
    f = lambda a, d: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device=device, dtype=d)
    return dict(q=f(inp.q, dt), k=f(inp.k, dt), v=f(inp.v, dt), g=f(inp.g, torch.float32),
                beta=f(inp.beta, torch.float32), h0=f(inp.h0, torch.float32))


def gpu_run(plan: B.KDAPlan, inp: synth.KDAInputs, dO=None, dh_leaf=None, h0=True):
    """Forward (and backward when dO is given) on cuda:0; numpy results."""
    import torch
    t = to_dev(inp)
    f = B.kda_tree_fwd(plan, t["q"], t["k"], t["v"], t["g"], t["beta"],
                       t["h0"] if h0 else None, inp.scale)
    res = dict(o=f["o"], h_leaf=f["h_leaf"])
    if dO is not None:
        dt = torch.bfloat16 if inp.bf16 else torch.float32
        dO_t = torch.from_numpy(np.ascontiguousarray(dO, np.float32)).to("cuda", dt)
        dhl_t = None if dh_leaf is None else torch.from_numpy(
            np.ascontiguousarray(dh_leaf, np.float32)).cuda()
        g = B.kda_tree_bwd(plan, t["q"], t["k"], t["v"], t["g"], t["beta"], f["saved"], dO_t,
                           dhl_t, t["h0"] if h0 else None, inp.scale)
        res.update(g)
    torch.cuda.synchronize()
    return {k: (v.cpu().numpy() if hasattr(v, "cpu") else v) for k, v in res.items()
            if k not in ("ws", "saved")}


def make_case(spec: synth.TreeSpec, H, D, bf16, seed, gate="default", h0_mode="zero",
              dh_leaf="randn", chunk=64, mode=B.MINCALL):
    rng = np.random.Generator(np.random.PCG64(seed))
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    inp = synth.make_kda_inputs(rng, t.n_rows, H, D, D, n_root=len(t.roots), bf16=bf16,
                                gate=gate, h0_mode=h0_mode)
    plan = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, chunk, mode)
    dO, dhl = synth.make_upstream(rng, plan.info["n_out_rows"], len(t.leaves), H, D, D,
                                  bf16=bf16, dh_leaf=dh_leaf)
    return t, inp, plan, dO, dhl


def oracle_tree(t: Tree, inp, dO, dhl, plan: B.KDAPlan | None = None, bwd=True):
    o, hl = okda.tree_fwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale)
    res = dict(o=o, h_leaf=hl)
    if bwd:
        bounds = []
        if plan is not None and plan.info["n_buf"]:
            bseq, bpos = plan.export("BUF_SEQ"), plan.export("BUF_POS")
            leaf_of_seq = plan.export("SEQ_LEAF")
            head_of_seq = plan.export("SEQ_HEAD")
            leaves = plan.export("LEAF_SEG")

            def leaf_on_path(s):
                # a node-wise sequence (one segment) may end at an inner
                # segment: any leaf below it has the same root path prefix
                if leaf_of_seq[s] >= 0:
                    return int(leaves[leaf_of_seq[s]])
                v = int(head_of_seq[s])
                while t.children[v]:
                    v = t.children[v][0]
                return v
            bounds = [(leaf_on_path(s), int(p)) for s, p in zip(bseq, bpos)]
        g = okda.tree_bwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale, dO, dhl,
                          boundaries=bounds)
        res.update(dq=g["dq"], dk=g["dk"], dv=g["dv"], dg=g["dg"], dbeta=g["dbeta"],
                   dh0=g["dh0"])
        if bounds:
            res["dh_boundary"] = np.stack(g["boundary"])
    return res


def compare(got, ref, names, tol=TOL):
    errs = {n: rel_l2(got[n], ref[n]) for n in names if n in ref}
    bad = {n: e for n, e in errs.items() if not (e <= tol)}
    return errs, bad
