"""Replay versus exact-fork-state starts per handoff depth (the synthetic
analogue of thelatestinai.com Figure 5) against the float64 oracle: on a
complete binary tree of depth 5 every plan mode -- min-call with replay,
trajectory-expanded, no-replay (side branches from their exact fork states,
chunk grids cut there) and node-wise -- must meet the tolerance at every
handoff depth (side starts on a row's root path in the min-call plan), and
the min-call output must equal the expanded output bit for bit (replay keeps
every trajectory's own chunk grid)."""
import numpy as np
import pytest

from gpu_cases import TOL, gpu_run, rel_l2
from oracle import kda as okda
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

pytestmark = pytest.mark.gpu


def test_replay_ablation_by_handoff_depth():
    rng = np.random.Generator(np.random.PCG64(61))
    spec = synth.tree_kary(2, 5, 24, 80, rng, name="binary_d5")
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    inp = synth.make_kda_inputs(rng, t.n_rows, 2, 64, 64, n_root=1, bf16=True, gate="weak",
                                h0_mode="randn")
    print(f"case binary depth 5: {t.n} segments, {t.n_rows} rows, H=2, d=64, chunk 16", flush=True)
    o_ref, _ = okda.tree_fwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale)
    outs = {}
    for name, mode in (("mincall", B.MINCALL), ("expanded", B.EXPANDED), ("noreplay", B.NOREPLAY),
                       ("nodewise", B.NODEWISE)):
        plan = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 16, mode)
        o = gpu_run(plan, inp)["o"]
        if mode == B.EXPANDED:   # packed rows -> compact rows
            oc = np.zeros((t.n_rows,) + o.shape[1:], o.dtype)
            oc[plan.export("ROW_INDEX")] = o
            o = oc
        outs[name] = o
        if mode == B.MINCALL:
            cont = plan.export("SEG_IS_CONT")
    hd = np.zeros(t.n, np.int64)
    for v in t.preorder:
        p = int(t.parent[v])
        hd[v] = 0 if p < 0 else hd[p] + (0 if cont[v] else 1)
    row_hd = np.zeros(t.n_rows, np.int64)
    for v in range(t.n):
        row_hd[t.seg_rows(v)] = hd[v]
    assert np.array_equal(outs["mincall"], outs["expanded"])
    bad = {}
    for d in range(int(row_hd.max()) + 1):
        sel = row_hd == d
        errs = {n: rel_l2(o[sel], o_ref[sel]) for n, o in outs.items()}
        print(f"  handoff depth {d} ({int(sel.sum())} rows) rel L2 vs oracle:",
              {n: f"{e:.2e}" for n, e in errs.items()}, flush=True)
        bad.update({f"{n}@{d}": e for n, e in errs.items() if not e <= TOL})
    assert int(row_hd.max()) == 5
    assert not bad, bad
