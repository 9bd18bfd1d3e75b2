"""The binding refuses tensors whose shape, dtype or size does not match the
plan before anything reaches the library: a wrong row count, a bf16 gate read
as fp32 or a short `saved` buffer would otherwise become an out-of-bounds
device access.  CPU only: every case raises before any launch (CPU tensors of
the right shapes are refused for not being device tensors)."""
import numpy as np
import pytest
import torch

from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth


@pytest.fixture(scope="module")
def plan():
    spec = synth.tree_fig1()
    return B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, 16)


def _inputs(plan, H=2, D=64, dt=torch.float32):
    N = plan.info["n_rows"]
    z = lambda *s, d=dt: torch.zeros(*s, dtype=d)
    return dict(q=z(N, H, D), k=z(N, H, D), v=z(N, H, D), g=z(N, H, D, d=torch.float32),
                beta=z(N, H, d=torch.float32))


def _fwd(plan, **kw):
    a = _inputs(plan)
    a.update(kw)
    return B.kda_tree_fwd(plan, a["q"], a["k"], a["v"], a["g"], a["beta"], a.get("h0"), None,
                          a.get("out"))


def test_fwd_accepts_shapes_then_needs_device(plan):
    with pytest.raises(B.KDAError, match="device tensors"):
        _fwd(plan)


@pytest.mark.parametrize("field,bad,msg", [
    ("q", torch.zeros(5, 2, 64), "rows"),
    ("k", torch.zeros(130, 2, 32), "shape"),
    ("v", torch.zeros(130, 2, 64, dtype=torch.bfloat16), "dtype"),
    ("g", torch.zeros(130, 2, 64, dtype=torch.bfloat16), "dtype"),
    ("beta", torch.zeros(130, 3), "shape"),
    ("h0", torch.zeros(2, 2, 64, 64), "shape"),
])
def test_fwd_rejects_bad_inputs(plan, field, bad, msg):
    with pytest.raises(B.KDAError, match=msg):
        _fwd(plan, **{field: bad})


def test_fwd_rejects_bad_outputs(plan):
    H, D = 2, 64
    i = plan.info
    ok = dict(o=torch.zeros(i["n_out_rows"], H, D), h_leaf=torch.zeros(i["n_leaf"], H, D, D),
              saved=torch.zeros(plan.saved_bytes(H, D), dtype=torch.uint8),
              ws=torch.zeros(plan.fwd_ws_bytes(H, D), dtype=torch.uint8))
    for key, bad, msg in (("o", torch.zeros(i["n_out_rows"] - 1, H, D), "shape"),
                          ("h_leaf", torch.zeros(i["n_leaf"], H, D, D, dtype=torch.float64), "dtype"),
                          ("saved", torch.zeros(plan.saved_bytes(H, D) - 16, dtype=torch.uint8),
                           "bytes")):
        out = dict(ok)
        out[key] = bad
        q = torch.zeros(i["n_rows"], H, D)
        with pytest.raises(B.KDAError, match=msg):
            # the inputs pass their checks (on the CPU they fail only the device test,
            # which the outputs' checks precede for the caller-supplied buffers)
            B._check_inputs(plan, q, q, q, q, torch.zeros(i["n_rows"], H), None)
            B._expect("o", out["o"], (i["n_out_rows"], H, D), (torch.float32,))
            B._expect("h_leaf", out["h_leaf"], (i["n_leaf"], H, D, D), (torch.float32,))
            B._expect_bytes("saved", out["saved"], plan.saved_bytes(H, D))


def test_bwd_rejects_bad_upstream(plan):
    a = _inputs(plan)
    i = plan.info
    saved = torch.zeros(plan.saved_bytes(2, 64), dtype=torch.uint8)
    with pytest.raises(B.KDAError, match="dtype"):
        B.kda_tree_bwd(plan, a["q"], a["k"], a["v"], a["g"], a["beta"], saved,
                       torch.zeros(i["n_out_rows"], 2, 64, dtype=torch.bfloat16))
    with pytest.raises(B.KDAError, match="shape"):
        B.kda_tree_bwd(plan, a["q"], a["k"], a["v"], a["g"], a["beta"], saved,
                       torch.zeros(i["n_out_rows"], 2, 64), torch.zeros(1, 2, 64, 64))
    with pytest.raises(B.KDAError, match="bytes"):
        B.kda_tree_bwd(plan, a["q"], a["k"], a["v"], a["g"], a["beta"], saved[:100],
                       torch.zeros(i["n_out_rows"], 2, 64))
    with pytest.raises(B.KDAError, match="device tensors"):
        B.kda_tree_bwd(plan, a["q"], a["k"], a["v"], a["g"], a["beta"], saved,
                       torch.zeros(i["n_out_rows"], 2, 64))


def test_gather_attention_router_state_checks(plan):
    N = plan.info["n_rows"]
    z = torch.zeros(N, 50)
    with pytest.raises(B.KDAError, match="dtype"):
        B.gather_logprobs(z, torch.zeros(7, dtype=torch.int64), torch.zeros(7, dtype=torch.int32))
    with pytest.raises(B.KDAError, match="shape"):
        B.gather_logprobs(z, torch.zeros(7, dtype=torch.int32), torch.zeros(6, dtype=torch.int32))
    with pytest.raises(B.KDAError, match="shape"):
        B.gather_logprobs_bwd(z, torch.zeros(N), torch.zeros(N, dtype=torch.int32),
                              torch.zeros(7, dtype=torch.int32), torch.zeros(7, dtype=torch.int32),
                              torch.zeros(7))
    bf = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    with pytest.raises(B.KDAError, match="rows"):
        B.tree_attn_fwd(plan, bf(N + 1, 2, 64), bf(N + 1, 2, 64), bf(N + 1, 2, 64))
    with pytest.raises(B.KDAError, match="dtype"):
        B.tree_attn_fwd(plan, bf(N, 2, 64), torch.zeros(N, 2, 64), bf(N, 2, 64))
    with pytest.raises(B.KDAError, match="shape"):
        B.tree_attn_bwd(plan, bf(N, 2, 64), bf(N, 2, 64), bf(N, 2, 64), torch.zeros(N, 2, 64),
                        torch.zeros(N, 3), bf(N, 2, 64))
    with pytest.raises(B.KDAError, match="shape"):
        B.moe_router_stats(torch.zeros(N, 128), torch.zeros(N - 1, dtype=torch.int32), 8)
    st = torch.zeros(3, 2, 8, 8)
    with pytest.raises(B.KDAError, match="exceeds"):
        B.kda_state_copy(st, None, torch.zeros(2, 2, 8, 8), None, 3)
    with pytest.raises(B.KDAError, match="needs"):
        B.kda_state_copy(st, torch.zeros(1, dtype=torch.int32), st, None, 2)
    with pytest.raises(B.KDAError, match="sums"):
        B.kda_state_sum(st, torch.zeros(5, dtype=torch.int32), torch.zeros(3, dtype=torch.int32), st,
                        False)
    with pytest.raises(B.KDAError, match="device tensors"):
        B.kda_state_copy(st, None, st, None, 3)


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan")])
def test_attention_scale_must_be_positive(plan, scale):
    # the C-ABI refuses the scale before it looks at the device plan or tensors
    L = B.load_library()
    assert L.tree_attn_fwd(plan.handle, None, 2, 64, scale, None, None, None, None, None, None) == -4
    assert L.tree_attn_bwd(plan.handle, None, 2, 64, scale, *([None] * 10), 0, None) == -4
    assert b"scale" in L.kda_last_error()


@pytest.mark.parametrize("bad", range(10))
def test_attention_pointers_must_be_aligned(plan, bad):
    # the C-ABI refuses a misaligned tensor before anything is launched: the
    # pointers below are never dereferenced (each call fails on the one offset
    # by 8 bytes, or by 2 for lse)
    L = B.load_library()
    dev_plan = 0x10000
    ptrs = [0x100000 * (i + 1) for i in range(10)]   # q k v o lse dO dq dk dv ws
    ptrs[bad] += 2 if bad == 4 else 8
    q, k, v, o, lse, dO, dq, dk, dv, ws = ptrs
    if bad <= 4:
        assert L.tree_attn_fwd(plan.handle, dev_plan, 2, 64, 0.125, q, k, v, o, lse, None) == -4
        assert b"aligned" in L.kda_last_error()
    assert L.tree_attn_bwd(plan.handle, dev_plan, 2, 64, 0.125, q, k, v, o, lse, dO, dq, dk, dv,
                           ws, 1 << 40, None) == -4
    assert b"aligned" in L.kda_last_error()
