"""The allocation-free entry point (moe_router_stats_noalloc: the library's
own scratch instead of a workspace argument) against moe_router_stats on the
same inputs, through the C-ABI: two calls in a row, the second on a smaller
input, so that the second reads nothing the first left in the shared
scratch.  Loads, token counts and top-k indices bit-exact; the float sums and
probabilities bitwise equal as well (the same kernels over the same block
partition).  Also checked against the float64 oracle at 2e-3 on the first
call."""
import numpy as np
import pytest

from oracle import moe
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

pytestmark = pytest.mark.gpu


def _outputs(n_rows, E, k, dev):
    import torch
    return dict(load=torch.full((E,), -7, dtype=torch.int64, device=dev),
                psum=torch.full((E,), float("nan"), dtype=torch.float32, device=dev),
                zsum=torch.full((1,), float("nan"), dtype=torch.float32, device=dev),
                n_tok=torch.full((1,), -7, dtype=torch.int64, device=dev),
                topk_idx=torch.full((n_rows, k), -1, dtype=torch.int32, device=dev),
                topk_prob=torch.full((n_rows, k), float("nan"), dtype=torch.float32, device=dev))


def _case(spec, E, k, bf16, seed):
    import torch
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    plan = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 64)
    rng = np.random.Generator(np.random.PCG64(seed))
    x = (rng.standard_normal((t.n_rows, E)) * 2.0).astype(np.float32)
    if bf16:
        x = synth.round_bf16(x)
    xd = torch.from_numpy(x).cuda()
    if bf16:
        xd = xd.to(torch.bfloat16)
    return t, x.astype(np.float64), xd, plan.device_table("ROW_MULT")


@pytest.mark.parametrize("E,k,bf16", [(128, 8, True), (512, 8, False)])
def test_noalloc_matches_workspace_entry_point(E, k, bf16):
    import torch
    w = synth.workload(1)
    big = w.tree
    rng = np.random.Generator(np.random.PCG64(5))
    small = synth.tree_random(rng, 12, 10, 300, n_roots=2)
    for step, (spec, seed) in enumerate(((big, 11), (small, 12))):
        t, x, xd, q = _case(spec, E, k, bf16, seed + E)
        print(f"case no-alloc step {step} rows={t.n_rows} E={E} k={k} bf16={bf16}", flush=True)
        ref = B.moe_router_stats(xd, q, k)
        got = B.moe_router_stats_noalloc(xd, q, k, _outputs(t.n_rows, E, k, xd.device))
        torch.cuda.synchronize()
        for n in ("load", "n_tok", "topk_idx", "psum", "zsum", "topk_prob"):
            a, b = got[n].cpu().numpy(), ref[n].cpu().numpy()
            assert np.array_equal(a, b), (step, n)
        if step == 1:   # the oracle on the smaller input (the first is the full-size tree)
            load, psum, zsum, T = moe.expanded_stats(t, x, k)
            assert np.array_equal(got["load"].cpu().numpy(), load)
            assert int(got["n_tok"][0]) == T
            rel = lambda a, b: float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))
            assert rel(got["psum"].cpu().numpy(), psum) <= 2e-3
            assert rel(got["zsum"].cpu().numpy(), [zsum]) <= 2e-3
