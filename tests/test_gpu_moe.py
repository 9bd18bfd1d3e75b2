"""GPU parity of the occurrence-weighted router statistics (through the C-ABI)
against the float64 oracle, which computes them the trajectory-expanded way.

Bar: expert loads, token counts and top-k indices bit-exact (the top-k is
decided on the same values: bf16 or fp32 logits are exact in float64);
probability sums, z-loss sums, top-k probabilities and logit gradients
within relative L2 2e-3."""
import numpy as np
import pytest

from oracle import moe
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _run(spec, E, k, bf16, seed, logits=None, g_seed=None):
    import torch
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    plan = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 64)
    rng = np.random.Generator(np.random.PCG64(seed))
    x = logits if logits is not None else rng.standard_normal((t.n_rows, E)) * 2.0
    if bf16:
        x = synth.round_bf16(np.asarray(x, np.float32))
    x = np.asarray(x, np.float32)
    xd = torch.from_numpy(x).cuda()
    if bf16:
        xd = xd.to(torch.bfloat16)
    q = plan.device_table("ROW_MULT")
    print(f"case rows={t.n_rows} E={E} k={k} bf16={bf16} seed={seed}", flush=True)
    got = B.moe_router_stats(xd, q, k)
    gP = rng.standard_normal(E)
    gz = 0.25
    dx = B.moe_router_stats_bwd(xd, q, torch.from_numpy(gP.astype(np.float32)).cuda(), gz)
    torch.cuda.synchronize()
    got = {n: v.cpu().numpy() for n, v in got.items()}
    return t, x.astype(np.float64), got, gP.astype(np.float32).astype(np.float64), gz, \
        dx.cpu().numpy()


def _check(t, x, got, k, gP, gz, dx):
    load, psum, zsum, T = moe.expanded_stats(t, x, k)
    assert int(got["n_tok"][0]) == T
    assert np.array_equal(got["load"], load)
    top, prob = moe.row_topk(x, k)
    assert np.array_equal(got["topk_idx"], top)
    errs = {"psum": _rel(got["psum"], psum), "zsum": _rel(got["zsum"], [zsum]),
            "topk_prob": _rel(got["topk_prob"], prob),
            "dlogits": _rel(dx, moe.expanded_grad(t, x, gP, gz))}
    print("  rel L2:", {n: f"{e:.1e}" for n, e in errs.items()}, flush=True)
    assert all(e <= TOL for e in errs.values()), errs


@pytest.mark.parametrize("E,k,bf16", [(64, 1, False), (128, 8, True), (256, 4, True),
                                      (64, 32, False), (512, 8, True)])
@pytest.mark.parametrize("seed", range(2))
def test_random_forests(E, k, bf16, seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    spec = synth.tree_random(rng, 10, 5, 120, n_roots=1 + seed)
    t, x, got, gP, gz, dx = _run(spec, E, k, bf16, 200 + seed)
    _check(t, x, got, k, gP, gz, dx)


def test_ties_go_to_the_lower_expert():
    # integer logits in a small range: many exact ties in every row
    spec = synth.tree_fig1()
    t = Tree(spec.parent, spec.seg_len)
    rng = np.random.Generator(np.random.PCG64(7))
    x = rng.integers(-2, 3, size=(t.n_rows, 128)).astype(np.float32)
    x[:, ::2] = np.where(x[:, ::2] == 0, np.float32(-0.0), x[:, ::2])   # -0 ties +0
    t, x, got, gP, gz, dx = _run(spec, 128, 8, True, 7, logits=x)
    _check(t, x, got, 8, gP, gz, dx)


def test_all_negative_ties_fp32():
    # k-th value negative and tied (keys of negative values), fp32 logits
    spec = synth.tree_fig1()
    t = Tree(spec.parent, spec.seg_len)
    rng = np.random.Generator(np.random.PCG64(8))
    x = -rng.integers(1, 4, size=(t.n_rows, 64)).astype(np.float32) * 0.75
    t, x, got, gP, gz, dx = _run(spec, 64, 8, False, 8, logits=x)
    _check(t, x, got, 8, gP, gz, dx)


def test_deterministic():
    rng = np.random.Generator(np.random.PCG64(11))
    spec = synth.tree_random(rng, 12, 50, 400)
    a = _run(spec, 128, 8, True, 12)
    b = _run(spec, 128, 8, True, 12)
    for n in ("load", "psum", "zsum", "n_tok", "topk_idx", "topk_prob"):
        assert np.array_equal(a[2][n], b[2][n]), n
    assert np.array_equal(a[5], b[5])


def test_full_size_kary4_tree():
    """The 4-ary depth-3 tree of the fwd+bwd workload (103,568 rows, 313,736
    positions), 128 experts, top-8, bf16 logits."""
    w = synth.workload(2)
    t, x, got, gP, gz, dx = _run(w.tree, 128, 8, True, 21)
    _check(t, x, got, 8, gP, gz, dx)
