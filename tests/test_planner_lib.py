"""Host-side tests of libkda_tree.so (no GPU needed): every declared symbol is
exported, the C++ planner's canonical arrays equal the oracle planner's bit
for bit, and malformed trees and bad arguments return status codes."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest

from oracle import moe
from oracle import planner as OP
from oracle.tree import Tree
from tree_packed_chunkwise_amd import binding as B
from tree_packed_chunkwise_amd import synth

ROOT = Path(__file__).resolve().parents[1]

MAP = {
    "SEG_ROUND": "seg_round", "SEG_SEQ": "seg_seq", "SEG_IS_CONT": "seg_is_cont",
    "SEG_B": "seg_b", "SEG_REPLAY": "seg_replay", "ROUND_SEQ_PTR": "round_seq_ptr",
    "SEQ_ROUND": "seq_round", "SEQ_HEAD": "seq_head", "SEQ_LEAF": "seq_leaf",
    "SEQ_B_HEAD": "seq_b_head", "SEQ_REPLAY": "seq_replay", "SEQ_ROW_PTR": "seq_row_ptr",
    "SEQ_CHUNK_PTR": "seq_chunk_ptr", "SEQ_INIT_KIND": "seq_init_kind",
    "SEQ_INIT_IDX": "seq_init_idx", "CHUNK_SEQ": "chunk_seq", "CHUNK_ROW0": "chunk_row0",
    "CHUNK_LEN": "chunk_len", "CHUNK_SAVE": "chunk_save", "ROW_INDEX": "row_index",
    "OUT_ROW": "out_row", "BUF_SEQ": "buf_seq", "BUF_POS": "buf_pos", "BUF_CHUNK": "buf_chunk",
    "BUF_CONS_PTR": "buf_cons_ptr", "BUF_CONS": "buf_cons",
}


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def test_header_symbols_exported(lib):
    hdr = (ROOT / "include" / "kda_tree.h").read_text()
    decl = set(re.findall(r"^\s*(?:int|int64_t|size_t|void|const char\*)\s+(\w+)\(", hdr, re.M))
    assert decl == set(B.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


def _compare(spec, chunk, mode):
    t = Tree(spec.parent, spec.seg_len, spec.seg_row)
    po = OP.build_plan(t, chunk, mode)
    pc = B.KDAPlan(spec.parent, spec.seg_len, spec.seg_row, chunk, mode)
    for f, a in MAP.items():
        got, ref = pc.export(f), getattr(po, a)
        assert got.shape == ref.shape and np.array_equal(got, ref), f
    assert np.array_equal(pc.export("ROW_MULT"), moe.occurrence(t))
    pr, pn = t.gather_map()
    assert np.array_equal(pc.export("POS_ROW"), pr)
    assert np.array_equal(pc.export("POS_NEXT_ROW"), pn)
    assert np.array_equal(pc.export("LEAF_SEG"), t.leaves)
    assert np.array_equal(pc.export("ROOT_SEG"), t.roots)
    ptr, idx = pc.export("ROW_POS_PTR"), pc.export("ROW_POS_IDX")
    for r in range(0, t.n_rows, max(1, t.n_rows // 50)):
        assert np.array_equal(idx[ptr[r]:ptr[r + 1]], np.nonzero(pr == r)[0])
    # launch order of the round kernels: each round's sequences, most chunks first
    lpt, rp, nch = pc.export("SEQ_LPT"), pc.export("ROUND_SEQ_PTR"), np.diff(pc.export("SEQ_CHUNK_PTR"))
    for r in range(len(rp) - 1):
        want = sorted(range(rp[r], rp[r + 1]), key=lambda q: (-nch[q], q))
        assert list(lpt[rp[r]:rp[r + 1]]) == want
    i = pc.info
    assert (i["n_rounds"], i["R"], i["n_packed"], i["n_out_rows"]) == \
        (po.n_rounds, po.R, po.n_packed, po.n_out_rows)
    assert i["n_expanded"] == t.n_expanded()


@pytest.mark.parametrize("seed", range(20))
def test_random_forests_bit_exact(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    for _ in range(25):
        spec = synth.tree_random(rng, int(rng.integers(1, 14)), 1, 70,
                                 n_roots=int(rng.integers(1, 3)))
        if rng.integers(0, 2):
            spec = synth.shuffled_rows(spec, rng)
        for chunk in (1, 4, 16, 64):
            for mode in (OP.MINCALL, OP.EXPANDED, OP.NOREPLAY, OP.NODEWISE, OP.MINCALL_SHORT):
                _compare(spec, chunk, mode)


@pytest.mark.parametrize("idx", [0, 1, 3])
@pytest.mark.parametrize("mode", [0, 2, 3, 4])
def test_workload_trees_bit_exact(idx, mode):
    w = synth.workload(idx)
    _compare(w.tree, w.chunk, mode)


def test_workload_plan_shapes():
    w1 = synth.workload(1)
    p1 = B.KDAPlan(w1.tree.parent, w1.tree.seg_len, None, 64)
    assert p1.info["n_rounds"] == 4
    rp = p1.export("ROUND_SEQ_PTR")
    assert list(np.diff(rp)) == [1, 9, 27, 27]
    w3 = synth.workload(3)
    p3 = B.KDAPlan(w3.tree.parent, w3.tree.seg_len, None, 64)
    assert p3.info["n_rounds"] == 2
    assert np.all(p3.export("SEQ_REPLAY") < 64)


@pytest.mark.parametrize("parent,lens,msg", [
    ([-1, 2, 1], [1, 1, 1], "cycle"),
    ([-1, 0], [1, 0], "length"),
    ([-1, 7], [1, 1], "parent"),
    ([0], [3], "parent"),
])
def test_malformed_trees_return_status(parent, lens, msg):
    with pytest.raises(B.KDAError, match=r"status -1"):
        B.KDAPlan(parent, lens, None, 16)


def test_overlapping_rows_rejected():
    with pytest.raises(B.KDAError, match=r"status -1"):
        B.KDAPlan([-1, 0], [2, 2], [0, 1], 16)


def test_bad_arguments(lib):
    h = ctypes.c_void_p()
    par = np.array([-1], np.int32)
    ln = np.array([4], np.int32)
    assert lib.kda_tree_plan(1, B._np_ptr(par), B._np_ptr(ln), None, 0, 0, ctypes.byref(h)) == -4
    assert lib.kda_tree_plan(1, B._np_ptr(par), B._np_ptr(ln), None, 16, 7, ctypes.byref(h)) == -4
    assert lib.kda_tree_plan(0, None, None, None, 16, 0, ctypes.byref(h)) == -4
    p = B.KDAPlan(par, ln, None, 16)
    # unsupported shapes report zero sizes and are rejected before any launch
    assert p.saved_bytes(2, 96) == 0
    assert lib.kda_tree_fwd(p.handle, ctypes.c_void_p(256), 2, 96, 96, 0, 1.0, *([None] * 9), 0,
                            None, 0, None) == -2
    assert lib.kda_tree_fwd(p.handle, None, 2, 64, 64, 0, 1.0, *([None] * 9), 0, None, 0,
                            None) == -4
    dev = ctypes.c_void_p(256)
    # an undersized `saved` or workspace is refused before any launch
    assert lib.kda_tree_fwd(p.handle, dev, 2, 64, 64, 0, 1.0, *([dev] * 9), 0, dev, 1 << 40,
                            None) == -3
    assert b"saved" in lib.kda_last_error()
    assert lib.kda_tree_fwd(p.handle, dev, 2, 64, 64, 0, 1.0, *([dev] * 9), 1 << 40, dev, 0,
                            None) == -3
    assert b"workspace" in lib.kda_last_error()
    assert lib.kda_tree_bwd(p.handle, dev, 2, 64, 64, 0, 1.0, *([dev] * 7), 0, *([dev] * 10),
                            1 << 40, None) == -3
    assert b"saved" in lib.kda_last_error()
    p64 = B.KDAPlan(par, ln, None, 32)
    assert p64.fwd_ws_bytes(2, 64) == 0
