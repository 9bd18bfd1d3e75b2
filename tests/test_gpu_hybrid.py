"""The hybrid layer group (3 KDA layers, one tree-attention layer, per-position
log-prob gather) on the GPU against its float64 CPU reference composed from the
oracle (tests/hybrid_ref.py), at a reduced size on whole small trees:
per-position log-probs and the gradient of every parameter of
sum(dlogp * logp).  The GPU side runs its stream and projections in fp32
here; tree attention takes bf16 q, k, v on both sides.  (The hybrid
workload's own shape and bf16 precision: tests/test_gpu_config4.py.)

Bar: 2e-3 per tensor, except the gradients of the three attention input
projections: q, k, v are rounded to bf16 where the GPU and reference streams
differ by the KDA layers' error d (<= 4.5e-4 per call), so a share d / 2^-8
of them round to the other bf16 neighbour: about sqrt(d 2^-8) = 1.3e-3 on
q, k, v, passed on with a gain of about 2 -> 2e-3 + 2.6e-3, bar 5e-3
(derivation and measurements at full size in test_gpu_config4.py)."""
import numpy as np
import pytest

from gpu_cases import TOL, rel_l2
from hybrid_ref import reference_forward
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

pytestmark = pytest.mark.gpu

ATTN_IN_TOL = 5e-3


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
    tol = lambda n: ATTN_IN_TOL if n in ("attn.wq", "attn.wk", "attn.wv") else TOL
    bad = {n: e for n, e in errs.items() if not e <= tol(n)}
    assert not bad, bad
