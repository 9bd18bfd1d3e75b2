"""GPU parity of the HIP path (through the C-ABI) against the float64 oracle.

Bar: relative L2 <= 2e-3 per output tensor (outputs, leaf states, every
gradient, handoff-state gradients); plans and indices bit-exact (checked on
the CPU in test_planner_lib.py)."""
import numpy as np
import pytest

from gpu_cases import TOL, compare, gpu_run, make_case, oracle_tree, rel_l2
from oracle import kda as okda
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

pytestmark = pytest.mark.gpu

FWD = ("o", "h_leaf")
ALL = ("o", "h_leaf", "dq", "dk", "dv", "dg", "dbeta", "dh0", "dh_boundary")


def _check(t, inp, plan, dO, dhl, tol=TOL, names=ALL):
    print(f"case rows={t.n_rows} H={inp.q.shape[1]} D={inp.q.shape[2]} B={plan.info['chunk']} "
          f"bf16={inp.bf16} rounds={plan.info['n_rounds']} R={plan.info['R']}", flush=True)
    got = gpu_run(plan, inp, dO, dhl)
    ref = oracle_tree(t, inp, dO, dhl, plan)
    errs, bad = compare(got, ref, names, tol)
    print("  rel L2:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert not bad, bad
    return got, ref


def test_tiny_workload_fwd_bwd():
    """Figure 1 tree, H=2, d=64, chunk 16, fp32 inputs, default gates."""
    w = synth.workload(0)
    t, inp, plan, dO, dhl = make_case(w.tree, 2, 64, False, 0, chunk=16)
    _check(t, inp, plan, dO, dhl)


@pytest.mark.parametrize("h0_mode,dhl", [("randn", "randn"), ("zero", "zero")])
def test_tiny_weak_gates_handoff(h0_mode, dhl):
    """Slow decay keeps boundary states visible at every row."""
    t, inp, plan, dO, dh = make_case(synth.tree_fig1(), 2, 64, False, 1, gate="weak",
                                     h0_mode=h0_mode, dh_leaf=dhl, chunk=16)
    _check(t, inp, plan, dO, dh)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("D,chunk,bf16", [(64, 16, False), (128, 64, True), (64, 64, True),
                                          (128, 16, False), (128, 64, False), (64, 16, True)])
def test_random_forests(seed, D, chunk, bf16):
    rng = np.random.Generator(np.random.PCG64(seed))
    spec = synth.tree_random(rng, 9, 1, 3 * chunk, n_roots=1 + seed % 2)
    if seed % 2:
        spec = synth.shuffled_rows(spec, rng)
    gate = ("weak", "default", "zero")[seed]
    t, inp, plan, dO, dhl = make_case(spec, 2, D, bf16, 10 + seed, gate=gate, h0_mode="randn",
                                      chunk=chunk)
    _check(t, inp, plan, dO, dhl)


@pytest.mark.parametrize("seed", range(2))
@pytest.mark.parametrize("D,chunk,bf16", [(64, 16, False), (128, 64, True)])
def test_short_chain_mode(seed, D, chunk, bf16):
    """The short-chain variant of the min-call plan: same functions."""
    rng = np.random.Generator(np.random.PCG64(60 + seed))
    spec = synth.tree_kary(3, 3, chunk, 4 * chunk, rng)
    t, inp, plan, dO, dhl = make_case(spec, 2, D, bf16, 70 + seed, gate="weak", h0_mode="randn",
                                      chunk=chunk, mode=B.MINCALL_SHORT)
    _check(t, inp, plan, dO, dhl)


@pytest.mark.parametrize("mode", [B.NOREPLAY, B.NODEWISE])
@pytest.mark.parametrize("seed", range(2))
@pytest.mark.parametrize("D,chunk,bf16", [(64, 16, False), (128, 64, True)])
def test_exact_start_modes(mode, seed, D, chunk, bf16):
    """The no-replay and node-wise plans (side branches start from their
    exact fork states, chunk grids cut there) compute the same functions."""
    rng = np.random.Generator(np.random.PCG64(40 + seed))
    spec = synth.tree_random(rng, 10, 1, 3 * chunk, n_roots=1 + seed)
    if seed:
        spec = synth.shuffled_rows(spec, rng)
    t, inp, plan, dO, dhl = make_case(spec, 2, D, bf16, 50 + seed, gate="weak", h0_mode="randn",
                                      chunk=chunk, mode=mode)
    assert plan.info["R"] == 0
    _check(t, inp, plan, dO, dhl)


@pytest.mark.parametrize("beta_mode", ["zero", "one"])
def test_degenerate_beta(beta_mode):
    rng = np.random.Generator(np.random.PCG64(7))
    spec = synth.tree_random(rng, 6, 5, 80)
    t = Tree(spec.parent, spec.seg_len)
    inp = synth.make_kda_inputs(rng, t.n_rows, 2, 64, 64, bf16=False, gate="weak",
                                beta_mode=beta_mode, h0_mode="randn")
    plan = B.KDAPlan(spec.parent, spec.seg_len, None, 16)
    dO, dhl = synth.make_upstream(rng, t.n_rows, len(t.leaves), 2, 64, 64, bf16=False)
    _check(t, inp, plan, dO, dhl)


def test_single_token_and_path():
    for lens in ([1], [64], [65, 1, 63]):
        spec = synth.tree_path(lens)
        t, inp, plan, dO, dhl = make_case(spec, 2, 64, False, 3, gate="weak", h0_mode="randn",
                                          chunk=16)
        _check(t, inp, plan, dO, dhl)


def test_expanded_mode_matches_expansion():
    rng = np.random.Generator(np.random.PCG64(21))
    spec = synth.tree_random(rng, 8, 10, 150, n_roots=2)
    t, inp, plan, dO, dhl = make_case(spec, 2, 128, True, 22, gate="weak", h0_mode="randn",
                                      chunk=64, mode=B.EXPANDED)
    got = gpu_run(plan, inp, dO, dhl)
    outs, finals = okda.expanded_fwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale)
    assert rel_l2(got["o"], np.concatenate(outs)) <= TOL
    assert rel_l2(got["h_leaf"], finals) <= TOL
    offs = np.cumsum([0] + [len(o) for o in outs])
    dO_traj = [dO[offs[i]:offs[i + 1]] for i in range(len(outs))]
    exp = okda.expanded_bwd(t, inp.q, inp.k, inp.v, inp.g, inp.beta, inp.h0, inp.scale, dO_traj,
                            dhl)
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert rel_l2(got[n], np.concatenate([e[n] for e in exp])) <= TOL, n


@pytest.mark.parametrize("mode", [B.MINCALL, B.MINCALL_SHORT])
def test_tree_equals_expanded_bitwise_on_gpu(mode):
    """Replay keeps every trajectory's chunk grid: the packed tree run and the
    trajectory-expanded run compute the same chunks from the same states, so
    outputs and leaf states agree bit for bit (with or without the short-chain
    tie-break, which changes only which sequences carry which segments)."""
    rng = np.random.Generator(np.random.PCG64(31))
    spec = synth.tree_random(rng, 10, 20, 200, n_roots=1)
    t, inp, plan, dO, dhl = make_case(spec, 2, 128, True, 32, chunk=64, h0_mode="randn",
                                      gate="weak", mode=mode)
    tree = gpu_run(plan, inp)
    eplan = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 64, B.EXPANDED)
    exp = gpu_run(eplan, inp)
    row_index = eplan.export("ROW_INDEX")
    assert np.array_equal(exp["o"], tree["o"][row_index])
    assert np.array_equal(exp["h_leaf"], tree["h_leaf"])


def test_deterministic():
    rng = np.random.Generator(np.random.PCG64(41))
    spec = synth.tree_random(rng, 8, 30, 300)
    t, inp, plan, dO, dhl = make_case(spec, 2, 128, True, 42, chunk=64)
    a = gpu_run(plan, inp, dO, dhl)
    b = gpu_run(plan, inp, dO, dhl)
    for n in ("o", "h_leaf", "dq", "dk", "dv", "dg", "dbeta", "dh0"):
        assert np.array_equal(a[n], b[n]), n


def test_overlap_matches_single_stream():
    """The chunk-parallel passes run on a second stream beside the round
    chains by default; keeping every kernel on the caller's stream must give
    the same bits (no kernel reads what a kernel beside it writes, and every
    sum has a fixed order).  The tree has four rounds, so the forward runs
    three chunk-pass groups beside the rounds and the reverse pass forks the
    chunk-local gradients twice."""
    rng = np.random.Generator(np.random.PCG64(53))
    spec = synth.tree_kary(3, 3, 40, 260, rng)
    t, inp, plan, dO, dhl = make_case(spec, 2, 128, True, 54, chunk=64, h0_mode="randn")
    assert plan.info["n_rounds"] == 4
    try:
        B.set_overlap(False)
        one = gpu_run(plan, inp, dO, dhl)
    finally:
        B.set_overlap(True)
    two = gpu_run(plan, inp, dO, dhl)
    for n in ALL:
        if one.get(n) is None:
            continue
        assert np.array_equal(one[n], two[n]), n


@pytest.mark.parametrize("gate", ["strong", "mixed", "extreme"])
@pytest.mark.parametrize("D,chunk,bf16", [(128, 64, True), (64, 16, False), (64, 64, True)])
def test_strong_gates_fwd_bwd(gate, D, chunk, bf16):
    """Decays far past the range of the factored chunk products (about 120 of
    decay over 15 rows with gate 'strong', every row past it with 'extreme',
    and rows of both kinds mixed): the rows concerned take exact per-pair
    exponentials, the results stay within 2e-3 of the oracle."""
    rng = np.random.Generator(np.random.PCG64(90))
    spec = synth.tree_random(rng, 9, 1, 3 * chunk, n_roots=1)
    t, inp, plan, dO, dhl = make_case(spec, 2, D, bf16, 91, gate=gate, h0_mode="randn",
                                      chunk=chunk)
    if gate != "extreme":
        got, _ = _check(t, inp, plan, dO, dhl)
    else:
        # a decay of about e^-40 per row leaves the gradients of the start and
        # handoff states near 1e-18 (every path to them crosses at least one
        # row's decay); they are held to 2e-3 of the size of a state gradient
        # (dh_leaf's norm), not of their own size
        got, ref = _check(t, inp, plan, dO, dhl, names=ALL[:7])
        for n in ("dh0", "dh_boundary"):
            if n in ref:
                err = np.linalg.norm(got[n] - ref[n]) / np.linalg.norm(dhl)
                print(f"  {n}: |ref| {np.linalg.norm(ref[n]):.2e}, |err| / |dh_leaf| {err:.2e}")
                assert err <= TOL, n
    for n in ALL:
        if got.get(n) is not None:
            assert np.isfinite(got[n]).all(), n


@pytest.mark.parametrize("gate", ["strong", "mixed"])
def test_tree_equals_expanded_bitwise_strong_gates(gate):
    """The rows that take exact per-pair exponentials are chosen from the rows
    up to them, so replay stays bitwise equal to the trajectory-expanded run
    with decays past the factored range too."""
    rng = np.random.Generator(np.random.PCG64(33))
    spec = synth.tree_random(rng, 10, 20, 200, n_roots=1)
    t, inp, plan, dO, dhl = make_case(spec, 2, 128, True, 34, chunk=64, h0_mode="randn",
                                      gate=gate)
    tree = gpu_run(plan, inp)
    eplan = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 64, B.EXPANDED)
    exp = gpu_run(eplan, inp)
    row_index = eplan.export("ROW_INDEX")
    assert np.isfinite(tree["o"]).all()
    assert np.array_equal(exp["o"], tree["o"][row_index])
    assert np.array_equal(exp["h_leaf"], tree["h_leaf"])


@pytest.mark.parametrize("e", [-24, -16, 12, 16, 24])
@pytest.mark.parametrize("gate,leaf_grad", [("default", "randn"), ("weak", "zero")])
def test_upstream_gradient_scale(e, gate, leaf_grad):
    """The reverse pass runs in power-of-two units chosen from the largest
    upstream gradient, so its fp16 intermediates keep their precision whether
    the loss is averaged over many positions (tiny dO) or scaled up: with dO
    and dh_leaf times 2^e every gradient is exactly 2^e times the unit-scale
    run (bitwise), and within 2e-3 of the oracle."""
    rng = np.random.Generator(np.random.PCG64(5))
    spec = synth.tree_random(rng, 9, 50, 400, n_roots=1)
    t, inp, plan, dO, dhl = make_case(spec, 2, 128, True, 6, gate=gate, h0_mode="randn",
                                      dh_leaf=leaf_grad, chunk=64)
    s = float(2.0 ** e)
    print(f"case gradient scale 2^{e} gate={gate} dh_leaf={leaf_grad}", flush=True)
    base = gpu_run(plan, inp, dO, dhl)
    got = gpu_run(plan, inp, synth.round_bf16((dO * s).astype(np.float32)), dhl * np.float32(s))
    ref = oracle_tree(t, inp, dO, dhl, plan)
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dh0", "dh_boundary"):
        if got.get(n) is not None:
            assert np.array_equal(got[n], base[n] * np.float32(s)), n
    refs = {n: (v * s if n not in ("o", "h_leaf") else v) for n, v in ref.items()}
    errs, bad = compare(got, refs, ALL)
    print("  rel L2:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert not bad, bad


@pytest.mark.parametrize("e", [-12, 12])
def test_value_range_of_the_forward(e):
    """The forward keeps the state and the delta-rule writes in fp16 matrix-core
    operands (fp32 accumulation): values v and start states h0 of magnitude
    2^-12 .. 2^12 times unit scale stay within 2e-3 (the range the header
    states)."""
    rng = np.random.Generator(np.random.PCG64(5))
    spec = synth.tree_random(rng, 9, 50, 400, n_roots=1)
    t, inp, plan, dO, dhl = make_case(spec, 2, 128, True, 6, gate="weak", h0_mode="randn",
                                      chunk=64)
    s = np.float32(2.0 ** e)
    inp = synth.KDAInputs(q=inp.q, k=inp.k, v=synth.round_bf16(inp.v * s), g=inp.g,
                          beta=inp.beta, h0=inp.h0 * s, scale=inp.scale, bf16=True)
    _check(t, inp, plan, dO, dhl)
