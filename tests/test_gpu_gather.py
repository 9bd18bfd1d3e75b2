"""GPU parity of gather_logprobs / gather_logprobs_bwd (through the C-ABI)
against the float64 oracle (oracle/gather.py).

Small cases compare every position and every logit gradient; the full-size
case (4-ary tree, vocabulary 32000, bf16 logits, every trajectory position)
compares sampled rows, which the oracle computes one by one.  Bar: relative
L2 <= 2e-3; the gradient is stored in the logits' dtype, so for bf16 logits
the oracle's gradient is compared after the same rounding is allowed for
(bf16 storage alone is below 2^-9 per element)."""
import numpy as np
import pytest

from gpu_cases import TOL, rel_l2
from oracle import gather as og
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

pytestmark = pytest.mark.gpu


def _maps(plan):
    ex = lambda f: np.asarray(plan.export(f), dtype=np.int64)
    return ex("POS_ROW"), ex("POS_NEXT_ROW"), ex("ROW_POS_PTR"), ex("ROW_POS_IDX")


def _dev_i32(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def _star(n_children):
    """A root segment of 20 rows with `n_children` leaf segments of 3 rows: the
    root's last row predicts the first token of every child, so that one
    logit row carries n_children positions."""
    parent = np.array([-1] + [0] * n_children, dtype=np.int32)
    seg_len = np.array([20] + [3] * n_children, dtype=np.int32)
    seg_row = np.concatenate([[0], 20 + 3 * np.arange(n_children)]).astype(np.int64)
    return synth.TreeSpec(parent, seg_len, seg_row, f"star{n_children}")


@pytest.mark.parametrize("spec_name,vocab,bf16", [
    ("fig1", 1000, False), ("fig1", 1000, True), ("fig1", 1001, True),
    ("random", 4096, True), ("random", 777, False),
    # a row with more positions than a block has threads (its target columns
    # are written in several passes, some targets shared), a vocabulary
    # shorter than one 16-byte load, fp32 logits on the 16-byte path
    ("star300", 1000, True), ("fig1", 5, True), ("fig1", 4096, False)])
def test_gather_small(spec_name, vocab, bf16):
    import torch
    rng = np.random.Generator(np.random.PCG64(11 + vocab))
    if spec_name == "fig1":
        spec = synth.tree_fig1()
    elif spec_name == "star300":
        spec = _star(300)
    else:
        spec = synth.tree_random(rng, 12, 1, 40, 2)
    plan = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 16)
    N = plan.info["n_rows"]
    pos_row, pos_next, rp_ptr, rp_idx = _maps(plan)
    tokens = rng.integers(0, vocab, N)
    tgt = tokens[pos_next]
    z = rng.standard_normal((N, vocab), dtype=np.float32) * np.float32(3.0)
    z = synth.round_bf16(z) if bf16 else z
    dlogp = rng.standard_normal(len(pos_row)).astype(np.float32)
    print(f"case gather {spec_name} rows={N} vocab={vocab} bf16={bf16} n_pos={len(pos_row)}",
          flush=True)
    zt = torch.from_numpy(z).cuda().to(torch.bfloat16 if bf16 else torch.float32)
    logp, lse = B.gather_logprobs(zt, _dev_i32(pos_row), _dev_i32(tgt))
    dz = B.gather_logprobs_bwd(zt, lse, _dev_i32(rp_ptr), _dev_i32(rp_idx), _dev_i32(tgt),
                               torch.from_numpy(dlogp).cuda())
    torch.cuda.synchronize()
    ref_logp, ref_lse = og.gather_fwd(z, pos_row, tgt)
    ref_dz = og.gather_bwd(z, pos_row, tgt, dlogp)
    errs = {"logp": rel_l2(logp.cpu().numpy(), ref_logp), "lse": rel_l2(lse.cpu().numpy(), ref_lse),
            "dlogits": rel_l2(dz.float().cpu().numpy(), ref_dz)}
    print("  rel L2:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(e <= TOL for e in errs.values()), errs
    # a target column that several positions of one row share gets the exact sum
    assert np.isfinite(dz.float().cpu().numpy()).all()



@pytest.mark.parametrize("bf16", [False, True])
def test_gather_masked_entries(bf16):
    """Rows with masked (-inf) vocabulary entries: one row whose first 256
    entries are masked, rows with scattered masks, an all-masked row, and a
    masked target.  Finite values compare at 2e-3; -inf values must match."""
    import torch
    rng = np.random.Generator(np.random.PCG64(77))
    spec = synth.tree_fig1()
    plan = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 16)
    N, vocab = plan.info["n_rows"], 1000
    pos_row, pos_next, rp_ptr, rp_idx = _maps(plan)
    z = rng.standard_normal((N, vocab), dtype=np.float32) * np.float32(3.0)
    z = synth.round_bf16(z) if bf16 else z
    z[0, :256] = -np.inf
    for r in range(1, N, 3):
        z[r, rng.choice(vocab, 300, replace=False)] = -np.inf
    z[5, :] = -np.inf
    tokens = rng.integers(256, vocab, N)
    tgt = tokens[pos_next]
    masked_tgt = np.flatnonzero(~np.isfinite(z[pos_row, tgt]))
    assert len(masked_tgt) > 0
    dlogp = rng.standard_normal(len(pos_row)).astype(np.float32)
    print(f"case gather masked rows={N} vocab={vocab} bf16={bf16}", flush=True)
    zt = torch.from_numpy(z).cuda().to(torch.bfloat16 if bf16 else torch.float32)
    logp, lse = B.gather_logprobs(zt, _dev_i32(pos_row), _dev_i32(tgt))
    dz = B.gather_logprobs_bwd(zt, lse, _dev_i32(rp_ptr), _dev_i32(rp_idx), _dev_i32(tgt),
                               torch.from_numpy(dlogp).cuda())
    torch.cuda.synchronize()
    ref_logp, ref_lse = og.gather_fwd(z, pos_row, tgt)
    ref_dz = og.gather_bwd(z, pos_row, tgt, dlogp)
    got_logp, got_lse, got_dz = logp.cpu().numpy(), lse.cpu().numpy(), dz.float().cpu().numpy()
    for got, ref in ((got_logp, ref_logp), (got_lse, ref_lse)):
        assert not np.isnan(got).any()
        assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref_logp)
    errs = {"logp": rel_l2(got_logp[fin], ref_logp[fin]),
            "lse": rel_l2(got_lse[np.isfinite(ref_lse)], ref_lse[np.isfinite(ref_lse)]),
            "dlogits": rel_l2(got_dz, ref_dz)}
    print("  rel L2:", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert np.isfinite(got_dz).all()
    assert all(e <= TOL for e in errs.values()), errs


def test_gather_fullsize_sampled_rows():
    import torch
    w = synth.workload(1)
    plan = B.KDAPlan(w.tree.parent, w.tree.seg_len, w.tree.seg_row, w.chunk)
    N, V = plan.info["n_rows"], 32000
    pos_row, pos_next, rp_ptr, rp_idx = _maps(plan)
    print(f"case gather full size rows={N} vocab={V} n_pos={len(pos_row)}", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4242)
    zt = (torch.randn(N, V, generator=gen, device="cuda") * 3.0).to(torch.bfloat16)
    tokens = torch.randint(0, V, (N,), generator=gen, device="cuda")
    tgt = tokens[torch.from_numpy(pos_next).cuda()].to(torch.int32)
    dlogp = torch.randn(len(pos_row), generator=gen, device="cuda")
    logp, lse = B.gather_logprobs(zt, _dev_i32(pos_row), tgt)
    dz = B.gather_logprobs_bwd(zt, lse, _dev_i32(rp_ptr), _dev_i32(rp_idx), tgt, dlogp)
    torch.cuda.synchronize()
    print("  GPU done", flush=True)
    rng = np.random.Generator(np.random.PCG64(5))
    # sampled rows: random rows plus the row with the most positions (a root row)
    counts = np.diff(rp_ptr)
    rows = np.unique(np.concatenate([rng.choice(N, 48, replace=False), [int(np.argmax(counts))]]))
    zr = zt[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    tgt_np = tgt.cpu().numpy().astype(np.int64)
    dlogp_np = dlogp.cpu().numpy()
    # positions of the sampled rows (CSR) and their local row index
    sel = np.concatenate([rp_idx[rp_ptr[r]:rp_ptr[r + 1]] for r in rows])
    local = np.concatenate([np.full(rp_ptr[r + 1] - rp_ptr[r], i) for i, r in enumerate(rows)])
    ref_logp, ref_lse = og.gather_fwd(zr, local, tgt_np[sel])
    ref_dz = og.gather_bwd(zr, local, tgt_np[sel], dlogp_np[sel])
    errs = {"lse": rel_l2(lse.cpu().numpy()[rows], ref_lse),
            "logp": rel_l2(logp.cpu().numpy()[sel], ref_logp),
            "dlogits": rel_l2(dz[torch.from_numpy(rows).cuda()].float().cpu().numpy(), ref_dz)}
    print(f"  {len(rows)} rows, {len(sel)} positions, rel L2:",
          {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(e <= TOL for e in errs.values()), errs
    assert bool(torch.isfinite(logp).all())
