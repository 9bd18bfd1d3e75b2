"""The hybrid layer group (3 KDA layers, one tree-attention layer, per-position
log-prob gather) on the GPU against its float64 CPU reference composed from the
oracle (tests/hybrid_ref.py), at a reduced size: per-position log-probs and
the gradient of every parameter of sum(dlogp * logp).  The GPU side runs its
stream and projections in fp32 here; tree attention takes bf16 q, k, v on
both sides.

Bar: relative L2 <= 5e-3 per tensor (GROUP_TOL).  Each tree step is held to
2e-3 against the oracle on identical inputs by its own tests; here four
layers compose, each contributing about 1e-3 (the fp16 state products of the
KDA layers), and the attention inputs are rounded to bf16 at a point that
depends on that upstream error: a relative difference of 1e-3 in x moves a
sizable share of q, k, v across bf16 rounding boundaries (one ulp is 2^-8
relative), which adds about 1e-3 to the attention gradients.  Summed in
quadrature the composed bound is about 3e-3; the bar leaves margin above it."""
import numpy as np
import pytest

from gpu_cases import rel_l2
from hybrid_ref import reference_forward
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

pytestmark = pytest.mark.gpu

GROUP_TOL = 5e-3


@pytest.mark.parametrize("kind", ["fig1", "random"])
def test_hybrid_group_parity(kind):
    import torch
    from tree_packed_chunkwise_amd.hybrid import HybridGroup, gather_maps
    rng = np.random.Generator(np.random.PCG64(5))
    spec = synth.tree_fig1() if kind == "fig1" else synth.tree_random(rng, 8, 8, 60, 3)
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    plan = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 16)
    H, D, hidden, vocab = 2, 64, 128, 300
    print(f"case hybrid {kind} rows={t.n_rows} hidden={hidden} H={H} D={D} vocab={vocab}", flush=True)
    model = HybridGroup(hidden, H, D, vocab, n_kda=3, seed=3, dtype=torch.float32, device="cuda")
    tokens = torch.from_numpy(rng.integers(0, vocab, t.n_rows)).cuda()
    maps = gather_maps(plan, tokens, "cuda")
    logp = model(plan, tokens, maps)
    dlogp = torch.from_numpy(rng.standard_normal(logp.shape[0]).astype(np.float32)).cuda()
    (logp * dlogp).sum().backward()
    torch.cuda.synchronize()
    # reference on the same weights
    params = {n: p.detach().double().cpu().requires_grad_() for n, p in model.named_parameters()}
    pos_row = maps["pos_row"].cpu().numpy().astype(np.int64)
    pos_tgt = maps["pos_tgt"].cpu().numpy().astype(np.int64)
    ref = reference_forward(params, t, tokens.cpu(), pos_row, pos_tgt, H, D)
    (ref * torch.from_numpy(dlogp.cpu().numpy().astype(np.float64))).sum().backward()
    errs = {"logp": rel_l2(logp.detach().cpu().numpy(), ref.detach().numpy())}
    for n, p in model.named_parameters():
        errs[n] = rel_l2(p.grad.cpu().numpy(), params[n].grad.numpy())
    print("  rel L2:", {n: f"{e:.1e}" for n, e in errs.items()}, flush=True)
    bad = {n: e for n, e in errs.items() if not e <= GROUP_TOL}
    assert not bad, bad
