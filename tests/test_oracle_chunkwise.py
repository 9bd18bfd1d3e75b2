"""Pins of the chunk-form oracle (oracle.chunkwise): it must equal the token
recurrence of oracle.kda for every chunk size and plan, forward and reverse,
and must never read a handoff state before the round that writes it."""
import numpy as np
import pytest

from oracle import chunkwise, kda, planner
from oracle.tree import Tree
from tree_packed_chunkwise_amd import synth


def _case(seed, gate="weak", n_seg=8, lo=1, hi=40, n_roots=1, H=2, D=6, h0="randn"):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    spec = synth.tree_random(rng, n_seg, lo, hi, n_roots=n_roots)
    if seed % 3 == 1:
        spec = synth.shuffled_rows(spec, rng)
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    inp = synth.make_kda_inputs(rng, t.n_rows, H, D, D, n_root=len(t.roots), bf16=False,
                                gate=gate, h0_mode=h0)
    return t, inp, rng


@pytest.mark.parametrize("mode", [planner.MINCALL, planner.MINCALL_SHORT])
@pytest.mark.parametrize("B", [1, 4, 16, 64])
@pytest.mark.parametrize("seed", range(4))
def test_plan_forward_equals_recurrence(B, seed, mode):
    t, inp, _ = _case(seed, gate=("weak" if seed % 2 else "default"), n_roots=1 + seed % 2)
    o, hl = kda.tree_fwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale)
    p = planner.build_plan(t, B, mode)
    f = chunkwise.run_plan_fwd(p, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale,
                               n_leaf=len(t.leaves))
    np.testing.assert_allclose(f["o"], o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(f["h_leaf"], hl, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("B", [4, 16])
@pytest.mark.parametrize("seed", range(3))
def test_plan_backward_equals_recurrence(B, seed):
    t, inp, rng = _case(seed, n_roots=1 + seed % 2)
    H, D = inp.q.shape[1], inp.q.shape[2]
    dO = rng.standard_normal((t.n_rows, H, D))
    dhl = rng.standard_normal((len(t.leaves), H, D, D))
    p = planner.build_plan(t, B)
    bounds = [(t.leaves[int(p.seq_leaf[p.buf_seq[b]])], int(p.buf_pos[b])) for b in range(p.n_buf)]
    ref = kda.tree_bwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale, dO, dhl,
                       boundaries=bounds)
    got = chunkwise.run_plan_bwd(p, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale, dO,
                                 dhl)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        np.testing.assert_allclose(got[n], ref[n], rtol=1e-9, atol=1e-11)
    for b in range(p.n_buf):
        np.testing.assert_allclose(got["dh_boundary"][b], ref["boundary"][b], rtol=1e-9, atol=1e-11)


def test_expanded_plan_equals_expansion():
    t, inp, _ = _case(7, n_roots=2)
    p = planner.build_plan(t, 16, planner.EXPANDED)
    f = chunkwise.run_plan_fwd(p, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale,
                               n_leaf=len(t.leaves))
    outs, finals = kda.expanded_fwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale)
    np.testing.assert_allclose(f["o"], np.concatenate(outs), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(f["h_leaf"], finals, rtol=1e-11, atol=1e-12)


def test_chunk_size_independence_fig1():
    # the tiny workload's tree: chunk sizes 1, 16 and 64 all give the recurrence
    spec = synth.tree_fig1()
    t = Tree(spec.parent, spec.seg_len)
    rng = np.random.Generator(np.random.PCG64(0))
    inp = synth.make_kda_inputs(rng, t.n_rows, 2, 8, 8, bf16=False)
    o, hl = kda.tree_fwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale)
    for B in (1, 16, 64):
        f = chunkwise.run_plan_fwd(planner.build_plan(t, B), inp.q, inp.k, inp.v, inp.g,
                                   inp.beta, inp.h0, inp.scale, n_leaf=3)
        np.testing.assert_allclose(f["o"], o, rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(f["h_leaf"], hl, rtol=1e-11, atol=1e-13)


def test_strong_decay_chunk_no_overflow():
    # a 64-row chunk accumulates ~-140 of log-decay per channel: the per-pair
    # form must stay finite and exact
    rng = np.random.Generator(np.random.PCG64(9))
    inp = synth.make_kda_inputs(rng, 64, 1, 8, 8, bf16=False, gate_mean=4.0)
    assert inp.g.sum(0).min() < -150
    h = rng.standard_normal((8, 8))
    O, hn, _ = chunkwise.chunk_fwd(h, *(np.asarray(x[:, 0], np.float64) for x in
                                       (inp.q, inp.k, inp.v, inp.g, inp.beta)), inp.scale)
    o_ref, S_ref = kda.path_fwd(h[None], inp.q, inp.k, inp.v, inp.g, inp.beta, inp.scale)
    assert np.all(np.isfinite(O))
    np.testing.assert_allclose(O, o_ref[:, 0], rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(hn, S_ref[0], rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("mode", [planner.NOREPLAY, planner.NODEWISE])
@pytest.mark.parametrize("B", [4, 16, 64])
@pytest.mark.parametrize("seed", range(3))
def test_exact_mode_plans_equal_recurrence(mode, B, seed):
    """Side branches started from exact fork states (no replay): the same
    functions of the inputs, forward and reverse."""
    t, inp, rng = _case(20 + seed, gate=("weak" if seed % 2 else "default"), n_roots=1 + seed % 2)
    H, D = inp.q.shape[1], inp.q.shape[2]
    p = planner.build_plan(t, B, mode)
    o, hl = kda.tree_fwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale)
    f = chunkwise.run_plan_fwd(p, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale,
                               n_leaf=len(t.leaves))
    np.testing.assert_allclose(f["o"], o, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(f["h_leaf"], hl, rtol=1e-11, atol=1e-12)
    dO = rng.standard_normal((t.n_rows, H, D))
    dhl = rng.standard_normal((len(t.leaves), H, D, D))
    ref = kda.tree_bwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale, dO, dhl)
    got = chunkwise.run_plan_bwd(p, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale, dO,
                                 dhl, fwd=f)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0"):
        np.testing.assert_allclose(got[n], ref[n], rtol=1e-9, atol=1e-11)
