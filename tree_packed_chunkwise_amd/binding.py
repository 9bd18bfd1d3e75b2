"""Thin ctypes binding over libkda_tree.so (the C-ABI of include/kda_tree.h).

Argument marshalling only: tensors are passed as raw device pointers with the
current torch stream; every step of the computation runs in the library's
HIP kernels.  torch is used for device memory and streams.  There is no CPU
fallback: if the shared library is missing, or no GPU is present when a
compute call is made, the call raises.

Names follow the C-ABI: kda_tree_plan, kda_tree_fwd, kda_tree_bwd,
gather_logprobs, gather_logprobs_bwd.
"""
from __future__ import annotations

import ctypes
import math
from pathlib import Path

import numpy as np

LIB_PATH = Path(__file__).resolve().with_name("libkda_tree.so")

MINCALL, EXPANDED, NOREPLAY, NODEWISE, MINCALL_SHORT = 0, 1, 2, 3, 4
DT_FP32, DT_BF16 = 0, 1

FIELDS = [
    "SEG_ROUND", "SEG_SEQ", "SEG_IS_CONT", "SEG_B", "SEG_REPLAY", "ROUND_SEQ_PTR", "SEQ_ROUND",
    "SEQ_HEAD", "SEQ_LEAF", "SEQ_B_HEAD", "SEQ_REPLAY", "SEQ_ROW_PTR", "SEQ_CHUNK_PTR",
    "SEQ_INIT_KIND", "SEQ_INIT_IDX", "CHUNK_SEQ", "CHUNK_ROW0", "CHUNK_LEN", "CHUNK_SAVE",
    "ROW_INDEX", "OUT_ROW", "BUF_SEQ", "BUF_POS", "BUF_CHUNK", "BUF_CONS_PTR", "BUF_CONS",
    "POS_ROW", "POS_NEXT_ROW", "ROW_POS_PTR", "ROW_POS_IDX", "LEAF_SEG", "ROOT_SEG",
    "ATT_ANC_PTR", "ATT_ANC", "ATT_SEG_TILE0", "ATT_TILE_SEG", "ATT_TILE_OFF", "ATT_QORDER",
    "ATT_KQ_PTR", "ATT_KQ", "ATT_KW_TILE", "ATT_KW_Q0", "ATT_KW_NQ", "ATT_KW_SLOT", "ROW_MULT",
    "SEQ_LPT",
]
FIELD_ID = {n: i for i, n in enumerate(FIELDS)}

# every symbol include/kda_tree.h declares
EXPORTS = [
    "kda_tree_plan", "kda_plan_destroy", "kda_plan_info", "kda_plan_export", "kda_plan_upload",
    "kda_plan_device_offset", "kda_saved_bytes", "kda_fwd_workspace_bytes",
    "kda_bwd_workspace_bytes", "kda_tree_fwd", "kda_tree_bwd", "gather_logprobs",
    "gather_logprobs_bwd", "kda_timing_enable", "kda_timing_filter", "kda_timing_read", "kda_last_error",
    "tree_attn_workspace_bytes", "tree_attn_fwd", "tree_attn_bwd", "kda_state_copy",
    "kda_state_sum", "kda_set_overlap", "moe_router_workspace_bytes", "moe_router_stats",
    "moe_router_stats_bwd", "kda_l1_plan", "moe_router_stats_noalloc",
]


class KDAError(RuntimeError):
    pass


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_seg", "n_rounds", "n_seq", "n_chunks", "n_buf", "n_leaf", "n_root", "chunk", "mode",
        "max_seq_per_round")] + [(n, ctypes.c_int64) for n in (
            "n_rows", "n_packed", "n_out_rows", "R", "n_pos", "n_expanded")] + [
        ("device_bytes", ctypes.c_size_t)] + [(n, ctypes.c_int32) for n in (
            "n_att_tiles", "n_att_items", "n_att_slots", "n_att_split")]


_LIB = None


def load_library(path: Path | str | None = None):
    """Loads libkda_tree.so once; raises if it has not been built."""
    global _LIB
    if _LIB is not None and path is None:
        return _LIB
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise KDAError(f"{p} not found: build it with `python -m tree_packed_chunkwise_amd.build`")
    L = ctypes.CDLL(str(p))
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    f32 = ctypes.c_float
    L.kda_tree_plan.argtypes = [i32, vp, vp, vp, i32, i32, ctypes.POINTER(vp)]
    L.kda_tree_plan.restype = ctypes.c_int
    L.kda_plan_destroy.argtypes = [vp]
    L.kda_plan_destroy.restype = None
    L.kda_plan_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    L.kda_plan_info.restype = ctypes.c_int
    L.kda_plan_export.argtypes = [vp, i32, vp, i64]
    L.kda_plan_export.restype = i64
    L.kda_plan_upload.argtypes = [vp, vp, sz, vp]
    L.kda_plan_upload.restype = ctypes.c_int
    L.kda_plan_device_offset.argtypes = [vp, i32]
    L.kda_plan_device_offset.restype = i64
    for n in ("kda_saved_bytes", "kda_fwd_workspace_bytes", "kda_bwd_workspace_bytes"):
        getattr(L, n).argtypes = [vp, i32, i32, i32]
        getattr(L, n).restype = sz
    L.kda_tree_fwd.argtypes = [vp, vp, i32, i32, i32, i32, f32] + [vp] * 9 + [sz, vp, sz, vp]
    L.kda_tree_fwd.restype = ctypes.c_int
    L.kda_tree_bwd.argtypes = ([vp, vp, i32, i32, i32, i32, f32] + [vp] * 7 + [sz] + [vp] * 10
                               + [sz, vp])
    L.kda_tree_bwd.restype = ctypes.c_int
    L.kda_l1_plan.argtypes = [i32, vp, vp, i64, vp, vp, vp, vp]
    L.kda_l1_plan.restype = ctypes.c_int
    L.moe_router_workspace_bytes.argtypes = [i64, i32]
    L.moe_router_workspace_bytes.restype = sz
    L.moe_router_stats.argtypes = [vp, i32, i64, i32, i32] + [vp] * 8 + [sz, vp]
    L.moe_router_stats.restype = ctypes.c_int
    L.moe_router_stats_noalloc.argtypes = [vp, i32, i64, i32, i32] + [vp] * 8
    L.moe_router_stats_noalloc.restype = ctypes.c_int
    L.moe_router_stats_bwd.argtypes = [vp, i32, i64, i32, vp, vp, f32, vp, vp]
    L.moe_router_stats_bwd.restype = ctypes.c_int
    L.gather_logprobs.argtypes = [vp, i32, i64, i32, vp, vp, i64, vp, vp, vp]
    L.gather_logprobs.restype = ctypes.c_int
    L.gather_logprobs_bwd.argtypes = [vp, i32, i64, i32, vp, vp, vp, vp, vp, vp, vp]
    L.gather_logprobs_bwd.restype = ctypes.c_int
    L.tree_attn_workspace_bytes.argtypes = [vp, i32, i32]
    L.tree_attn_workspace_bytes.restype = sz
    L.tree_attn_fwd.argtypes = [vp, vp, i32, i32, f32] + [vp] * 5 + [vp]
    L.tree_attn_fwd.restype = ctypes.c_int
    L.tree_attn_bwd.argtypes = [vp, vp, i32, i32, f32] + [vp] * 10 + [sz, vp]
    L.tree_attn_bwd.restype = ctypes.c_int
    L.kda_state_copy.argtypes = [vp, vp, vp, vp, i32, i64, vp]
    L.kda_state_copy.restype = ctypes.c_int
    L.kda_state_sum.argtypes = [vp, vp, vp, i32, i64, i32, vp, vp]
    L.kda_state_sum.restype = ctypes.c_int
    L.kda_timing_enable.argtypes = [i32]
    L.kda_timing_enable.restype = ctypes.c_int
    L.kda_timing_filter.argtypes = [ctypes.c_char_p]
    L.kda_timing_filter.restype = ctypes.c_int
    L.kda_set_overlap.argtypes = [i32]
    L.kda_set_overlap.restype = ctypes.c_int
    L.kda_timing_read.argtypes = [i32, ctypes.c_char_p, i32, ctypes.POINTER(i64),
                                  ctypes.POINTER(ctypes.c_double)]
    L.kda_timing_read.restype = ctypes.c_int
    L.kda_last_error.argtypes = []
    L.kda_last_error.restype = ctypes.c_char_p
    if path is None:
        _LIB = L
    return L


def _check(rc):
    if rc < 0:
        msg = load_library().kda_last_error().decode()
        raise KDAError(f"status {rc}: {msg}")
    return rc


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class KDAPlan:
    """Host plan (kda_tree_plan) plus its uploaded device copy per device."""

    def __init__(self, parent, seg_len, seg_row=None, chunk: int = 64, mode: int = MINCALL):
        L = load_library()
        self._parent = np.ascontiguousarray(parent, dtype=np.int32)
        self._len = np.ascontiguousarray(seg_len, dtype=np.int32)
        self._row = None if seg_row is None else np.ascontiguousarray(seg_row, dtype=np.int64)
        h = ctypes.c_void_p()
        _check(L.kda_tree_plan(len(self._parent), _np_ptr(self._parent), _np_ptr(self._len),
                               _np_ptr(self._row) if self._row is not None else None,
                               chunk, mode, ctypes.byref(h)))
        self._h = h
        pi = PlanInfo()
        _check(L.kda_plan_info(h, ctypes.byref(pi)))
        self.info = {n: getattr(pi, n) for n, _ in PlanInfo._fields_}
        self._dev = {}

    @property
    def handle(self):
        return self._h

    def export(self, field: str) -> np.ndarray:
        L = load_library()
        n = _check(L.kda_plan_export(self._h, FIELD_ID[field], None, 0))
        out = np.zeros(max(n, 1), dtype=np.int64)
        _check(L.kda_plan_export(self._h, FIELD_ID[field], _np_ptr(out), n))
        return out[:n]

    def export_all(self) -> dict:
        return {f: self.export(f) for f in FIELDS}

    def device(self, device=None):
        """int32 device copy of the plan tables (uploaded once per device)."""
        import torch
        dev = torch.device(device if device is not None else "cuda")
        key = str(dev)
        if key not in self._dev:
            nb = int(self.info["device_bytes"])
            buf = torch.empty(nb // 4, dtype=torch.int32, device=dev)
            s = torch.cuda.current_stream(dev).cuda_stream
            _check(load_library().kda_plan_upload(self._h, ctypes.c_void_p(buf.data_ptr()), nb,
                                                  ctypes.c_void_p(s)))
            torch.cuda.current_stream(dev).synchronize()
            self._dev[key] = buf
        return self._dev[key]

    def device_table(self, field: str, device=None):
        """View of one int32 table of the uploaded copy (gather map and CSR)."""
        buf = self.device(device)
        off = _check(load_library().kda_plan_device_offset(self._h, FIELD_ID[field])) // 4
        n = len(self.export(field))
        return buf[off:off + n]

    def saved_bytes(self, H, D):
        return load_library().kda_saved_bytes(self._h, H, D, D)

    def fwd_ws_bytes(self, H, D):
        return load_library().kda_fwd_workspace_bytes(self._h, H, D, D)

    def bwd_ws_bytes(self, H, D):
        return load_library().kda_bwd_workspace_bytes(self._h, H, D, D)

    def __del__(self):
        try:
            if getattr(self, "_h", None):
                load_library().kda_plan_destroy(self._h)
                self._h = None
        except Exception:
            pass


def kda_tree_plan(parent, seg_len, seg_row=None, chunk: int = 64, mode: int = MINCALL) -> KDAPlan:
    return KDAPlan(parent, seg_len, seg_row, chunk, mode)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DT_BF16
    if t.dtype == torch.float32:
        return DT_FP32
    raise KDAError(f"unsupported dtype {t.dtype}")


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise KDAError("kda kernels need device tensors (no CPU path)")
        if t is not None and not t.is_contiguous():
            raise KDAError("tensors must be contiguous")


def _expect(name, t, shape, dtypes, optional=False):
    """Refuses a tensor whose shape or dtype is not what the kernels index:
    a wrong size or element type would become an out-of-bounds device access,
    so it is caught here, before any launch."""
    import torch
    if t is None:
        if optional:
            return
        raise KDAError(f"{name} is required")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise KDAError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        raise KDAError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _expect_bytes(name, t, nbytes):
    if t is None:
        raise KDAError(f"{name} is required")
    have = t.numel() * t.element_size()
    if have < int(nbytes):
        raise KDAError(f"{name} holds {have} bytes, needs {int(nbytes)}")


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise KDAError(f"tensors on several devices: {sorted(map(str, devs))}")


def _check_inputs(plan: "KDAPlan", q, k, v, g, beta, h0):
    """q, k, v, g, beta and h0 against the plan's row and root counts."""
    import torch
    if q is None or q.dim() != 3:
        raise KDAError("q must be [rows, H, dk]")
    N, H, D = q.shape
    i = plan.info
    if N != i["n_rows"]:
        raise KDAError(f"q has {N} rows, the plan has {i['n_rows']} compact rows")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise KDAError(f"q has dtype {q.dtype}: bf16 or fp32")
    _expect("q", q, (N, H, D), None)
    _expect("k", k, (N, H, D), (q.dtype,))
    _expect("v", v, (N, H, D), (q.dtype,))
    _expect("g", g, (N, H, D), (torch.float32,))
    _expect("beta", beta, (N, H), (torch.float32,))
    _expect("h0", h0, (i["n_root"], H, D, D), (torch.float32,), optional=True)
    _same_device(q, k, v, g, beta, h0)
    return N, H, D


def alloc_fwd(plan: KDAPlan, H: int, D: int, device):
    """Output and scratch buffers of kda_tree_fwd (torch allocations)."""
    import torch
    i = plan.info
    return dict(
        o=torch.empty((i["n_out_rows"], H, D), dtype=torch.float32, device=device),
        h_leaf=torch.empty((i["n_leaf"], H, D, D), dtype=torch.float32, device=device),
        saved=torch.empty(plan.saved_bytes(H, D), dtype=torch.uint8, device=device),
        ws=torch.empty(plan.fwd_ws_bytes(H, D), dtype=torch.uint8, device=device),
    )


def kda_tree_fwd(plan: KDAPlan, q, k, v, g, beta, h0=None, scale=None, out=None):
    """Forward pass; returns dict(o, h_leaf, saved[, ws])."""
    import torch
    N, H, D = _check_inputs(plan, q, k, v, g, beta, h0)
    _need_cuda(q, k, v, g, beta, h0)
    if out is None:
        out = alloc_fwd(plan, H, D, q.device)
    i = plan.info
    _expect("o", out["o"], (i["n_out_rows"], H, D), (torch.float32,))
    _expect("h_leaf", out["h_leaf"], (i["n_leaf"], H, D, D), (torch.float32,))
    _expect_bytes("saved", out["saved"], plan.saved_bytes(H, D))
    _expect_bytes("ws", out["ws"], plan.fwd_ws_bytes(H, D))
    _need_cuda(out["o"], out["h_leaf"], out["saved"], out["ws"])
    _same_device(q, out["o"], out["h_leaf"], out["saved"], out["ws"])
    sc = float(scale) if scale is not None else 1.0 / float(np.sqrt(D))
    sv = out["saved"]
    _check(load_library().kda_tree_fwd(
        plan.handle, _p(plan.device(q.device)), H, D, v.shape[2], _dtype_code(q), sc,
        _p(q), _p(k), _p(v), _p(g), _p(beta), _p(h0), _p(out["o"]), _p(out["h_leaf"]),
        _p(sv), sv.numel() * sv.element_size(), _p(out["ws"]),
        out["ws"].numel() * out["ws"].element_size(), _stream(q)))
    return out


def alloc_bwd(plan: KDAPlan, H: int, D: int, device, boundary=True):
    import torch
    i = plan.info
    n = i["n_out_rows"]
    f = dict(dtype=torch.float32, device=device)
    return dict(
        dq=torch.empty((n, H, D), **f), dk=torch.empty((n, H, D), **f),
        dv=torch.empty((n, H, D), **f), dg=torch.empty((n, H, D), **f),
        dbeta=torch.empty((n, H), **f), dh0=torch.empty((i["n_root"], H, D, D), **f),
        dh_boundary=(torch.empty((i["n_buf"], H, D, D), **f) if boundary else None),
        ws=torch.empty(plan.bwd_ws_bytes(H, D), dtype=torch.uint8, device=device),
    )


def kda_tree_bwd(plan: KDAPlan, q, k, v, g, beta, saved, dO, dh_leaf=None, h0=None, scale=None,
                 out=None, boundary=True):
    """Reverse mode; returns dict(dq, dk, dv, dg, dbeta, dh0, dh_boundary[, ws])."""
    import torch
    N, H, D = _check_inputs(plan, q, k, v, g, beta, h0)
    i = plan.info
    n = i["n_out_rows"]
    _expect("dO", dO, (n, H, D), (q.dtype,))
    _expect("dh_leaf", dh_leaf, (i["n_leaf"], H, D, D), (torch.float32,), optional=True)
    _expect_bytes("saved", saved, plan.saved_bytes(H, D))
    _need_cuda(q, k, v, g, beta, saved, dO, dh_leaf, h0)
    if out is None:
        out = alloc_bwd(plan, H, D, q.device, boundary)
    f32 = (torch.float32,)
    for name in ("dq", "dk", "dv", "dg"):
        _expect(name, out[name], (n, H, D), f32)
    _expect("dbeta", out["dbeta"], (n, H), f32)
    _expect("dh0", out["dh0"], (i["n_root"], H, D, D), f32)
    _expect("dh_boundary", out.get("dh_boundary"), (i["n_buf"], H, D, D), f32, optional=True)
    _expect_bytes("ws", out["ws"], plan.bwd_ws_bytes(H, D))
    _need_cuda(*[out.get(x) for x in ("dq", "dk", "dv", "dg", "dbeta", "dh0", "dh_boundary", "ws")])
    _same_device(q, dO, dh_leaf, saved, *[out.get(x) for x in
                                          ("dq", "dk", "dv", "dg", "dbeta", "dh0", "dh_boundary",
                                           "ws")])
    sc = float(scale) if scale is not None else 1.0 / float(np.sqrt(D))
    _check(load_library().kda_tree_bwd(
        plan.handle, _p(plan.device(q.device)), H, D, v.shape[2], _dtype_code(q), sc,
        _p(q), _p(k), _p(v), _p(g), _p(beta), _p(h0), _p(saved),
        saved.numel() * saved.element_size(), _p(dO), _p(dh_leaf),
        _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["dg"]), _p(out["dbeta"]),
        _p(out["dh0"]), _p(out.get("dh_boundary")), _p(out["ws"]),
        out["ws"].numel() * out["ws"].element_size(), _stream(q)))
    return out


def kda_state_copy(src, src_idx, dst, dst_idx, n: int):
    """dst[dst_idx[i]] = src[src_idx[i]] for i < n over [*, H, dk, dv] fp32 state
    arrays (None index = identity; index arrays are device int32)."""
    import torch
    f32, i32 = (torch.float32,), (torch.int32,)
    if src is None or dst is None or src.dim() < 2 or tuple(src.shape[1:]) != tuple(dst.shape[1:]):
        raise KDAError("src and dst must be [*, H, dk, dv] state arrays of one state shape")
    _expect("src", src, tuple(src.shape), f32)
    _expect("dst", dst, tuple(dst.shape), f32)
    n = int(n)
    for name, t, full in (("src_idx", src_idx, src), ("dst_idx", dst_idx, dst)):
        if t is None:
            if n > full.shape[0]:
                raise KDAError(f"n = {n} exceeds the {full.shape[0]} states of the identity map")
        else:
            _expect(name, t, (t.shape[0],) if t.dim() == 1 else (-1,), i32)
            if t.shape[0] < n:
                raise KDAError(f"{name} holds {t.shape[0]} entries, needs {n}")
    _need_cuda(src, src_idx, dst, dst_idx)
    _same_device(src, src_idx, dst, dst_idx)
    elems = int(np.prod(src.shape[1:]))
    _check(load_library().kda_state_copy(_p(src), _p(src_idx), _p(dst), _p(dst_idx), int(n), elems,
                                         _stream(src)))
    return dst


def kda_state_sum(src, ptr, idx, dst, accumulate: bool):
    """dst[d] = (dst[d] if accumulate else 0) + sum of src[idx[j]], j in [ptr[d], ptr[d+1]),
    in ascending j (ptr, idx device int32)."""
    import torch
    f32, i32 = (torch.float32,), (torch.int32,)
    if dst is None or dst.dim() < 2 or ptr is None or ptr.dim() != 1:
        raise KDAError("dst must be [n_dst, H, dk, dv] and ptr [n_dst + 1]")
    n_dst = ptr.shape[0] - 1
    if n_dst > dst.shape[0]:
        raise KDAError(f"ptr describes {n_dst} sums, dst holds {dst.shape[0]} states")
    _expect("ptr", ptr, (n_dst + 1,), i32)
    _expect("dst", dst, tuple(dst.shape), f32)
    if src is not None:
        if tuple(src.shape[1:]) != tuple(dst.shape[1:]):
            raise KDAError("src and dst must hold states of one shape")
        _expect("src", src, tuple(src.shape), f32)
    if idx is not None:
        _expect("idx", idx, (idx.shape[0],) if idx.dim() == 1 else (-1,), i32)
    _need_cuda(src, ptr, idx, dst)
    _same_device(src, ptr, idx, dst)
    elems = int(np.prod(dst.shape[1:]))
    _check(load_library().kda_state_sum(_p(src), _p(ptr), _p(idx), int(ptr.shape[0] - 1), elems,
                                        1 if accumulate else 0, _p(dst), _stream(dst)))
    return dst


def gather_logprobs(logits, pos_row, pos_target, out=None):
    """logp[p] = logits[pos_row[p], pos_target[p]] - logsumexp(logits[pos_row[p]]).
    Returns (logp, lse)."""
    import torch
    if logits is None or logits.dim() != 2:
        raise KDAError("logits must be [rows, vocab]")
    n_rows, vocab = logits.shape
    _expect("logits", logits, (n_rows, vocab), (torch.bfloat16, torch.float32))
    if pos_row is None or pos_row.dim() != 1:
        raise KDAError("pos_row must be [n_pos]")
    n_pos = pos_row.shape[0]
    _expect("pos_row", pos_row, (n_pos,), (torch.int32,))
    _expect("pos_target", pos_target, (n_pos,), (torch.int32,))
    _need_cuda(logits, pos_row, pos_target)
    if out is None:
        out = (torch.empty(n_pos, dtype=torch.float32, device=logits.device),
               torch.empty(n_rows, dtype=torch.float32, device=logits.device))
    logp, lse = out
    _expect("logp", logp, (n_pos,), (torch.float32,))
    _expect("lse", lse, (n_rows,), (torch.float32,))
    _need_cuda(logp, lse)
    _same_device(logits, pos_row, pos_target, logp, lse)
    _check(load_library().gather_logprobs(_p(logits), _dtype_code(logits), n_rows, vocab,
                                          _p(pos_row), _p(pos_target), n_pos, _p(logp), _p(lse),
                                          _stream(logits)))
    return logp, lse


def gather_logprobs_bwd(logits, lse, row_pos_ptr, row_pos_idx, pos_target, dlogp, out=None):
    import torch
    if logits is None or logits.dim() != 2:
        raise KDAError("logits must be [rows, vocab]")
    n_rows, vocab = logits.shape
    _expect("logits", logits, (n_rows, vocab), (torch.bfloat16, torch.float32))
    _expect("lse", lse, (n_rows,), (torch.float32,))
    _expect("row_pos_ptr", row_pos_ptr, (n_rows + 1,), (torch.int32,))
    if pos_target is None or pos_target.dim() != 1:
        raise KDAError("pos_target must be [n_pos]")
    n_pos = pos_target.shape[0]
    _expect("row_pos_idx", row_pos_idx, (n_pos,), (torch.int32,))
    _expect("pos_target", pos_target, (n_pos,), (torch.int32,))
    _expect("dlogp", dlogp, (n_pos,), (torch.float32,))
    _need_cuda(logits, lse, row_pos_ptr, row_pos_idx, pos_target, dlogp)
    if out is None:
        out = torch.empty_like(logits)
    _expect("dlogits", out, (n_rows, vocab), (logits.dtype,))
    _need_cuda(out)
    _same_device(logits, lse, row_pos_ptr, row_pos_idx, pos_target, dlogp, out)
    _check(load_library().gather_logprobs_bwd(_p(logits), _dtype_code(logits), n_rows, vocab,
                                              _p(lse), _p(row_pos_ptr), _p(row_pos_idx),
                                              _p(pos_target), _p(dlogp), _p(out),
                                              _stream(logits)))
    return out


def l1_plan(parent, seg_len, budget: int) -> dict:
    """Compression-oriented microbatches of whole trajectories (host; see
    include/kda_tree.h).  Returns dict(leaf_mb [n_leaf], unique [n_mb],
    expanded [n_mb], compression, balance)."""
    parent = np.ascontiguousarray(parent, dtype=np.int32)
    seg_len = np.ascontiguousarray(seg_len, dtype=np.int32)
    n = len(parent)
    has_child = np.zeros(n, dtype=bool)
    has_child[parent[parent >= 0]] = True
    n_leaf = int((~has_child).sum())
    leaf_mb = np.empty(n_leaf, dtype=np.int32)
    n_mb = ctypes.c_int32(0)
    uniq = np.empty(max(n_leaf, 1), dtype=np.int64)
    expd = np.empty(max(n_leaf, 1), dtype=np.int64)
    _check(load_library().kda_l1_plan(n, _np_ptr(parent), _np_ptr(seg_len), int(budget),
                                      _np_ptr(leaf_mb), ctypes.byref(n_mb), _np_ptr(uniq),
                                      _np_ptr(expd)))
    m = n_mb.value
    uniq, expd = uniq[:m].copy(), expd[:m].copy()
    return dict(leaf_mb=leaf_mb, unique=uniq, expanded=expd,
                compression=float(expd.sum() / uniq.sum()), balance=float(uniq.mean() / uniq.max()))


def moe_router_stats(logits, row_mult, top_k: int, with_topk: bool = True):
    """Occurrence-weighted router statistics of compact rows (see
    include/kda_tree.h).  row_mult: int32 device counts, e.g.
    plan.device_table("ROW_MULT").  Returns dict(load, psum, zsum, n_tok[,
    topk_idx, topk_prob])."""
    import torch
    if logits is None or logits.dim() != 2:
        raise KDAError("logits must be [rows, n_experts]")
    n_rows, E = logits.shape
    _expect("logits", logits, (n_rows, E), (torch.bfloat16, torch.float32))
    _expect("row_mult", row_mult, (n_rows,), (torch.int32,))
    _need_cuda(logits, row_mult)
    _same_device(logits, row_mult)
    dev = logits.device
    L = load_library()
    ws = torch.empty(max(1, L.moe_router_workspace_bytes(n_rows, E)), dtype=torch.uint8, device=dev)
    out = dict(load=torch.empty(E, dtype=torch.int64, device=dev),
               psum=torch.empty(E, dtype=torch.float32, device=dev),
               zsum=torch.empty(1, dtype=torch.float32, device=dev),
               n_tok=torch.empty(1, dtype=torch.int64, device=dev))
    ti = tp = None
    if with_topk:
        ti = torch.empty((n_rows, top_k), dtype=torch.int32, device=dev)
        tp = torch.empty((n_rows, top_k), dtype=torch.float32, device=dev)
        out.update(topk_idx=ti, topk_prob=tp)
    _check(L.moe_router_stats(_p(logits), _dtype_code(logits), n_rows, E, top_k, _p(row_mult),
                              _p(ti) if ti is not None else None,
                              _p(tp) if tp is not None else None, _p(out["load"]),
                              _p(out["psum"]), _p(out["zsum"]), _p(out["n_tok"]), _p(ws),
                              ws.numel(), _stream(logits)))
    return out


def moe_router_stats_noalloc(logits, row_mult, top_k: int, out: dict, with_topk: bool = True):
    """moe_router_stats through the library's allocation-free entry point:
    every output buffer is the caller's (out: load, psum, zsum, n_tok[,
    topk_idx, topk_prob]); the scratch is the library's own."""
    import torch
    if logits is None or logits.dim() != 2:
        raise KDAError("logits must be [rows, n_experts]")
    n_rows, E = logits.shape
    _expect("logits", logits, (n_rows, E), (torch.bfloat16, torch.float32))
    _expect("row_mult", row_mult, (n_rows,), (torch.int32,))
    _expect("load", out["load"], (E,), (torch.int64,))
    _expect("psum", out["psum"], (E,), (torch.float32,))
    _expect("zsum", out["zsum"], (1,), (torch.float32,))
    _expect("n_tok", out["n_tok"], (1,), (torch.int64,))
    ti = out.get("topk_idx") if with_topk else None
    tp = out.get("topk_prob") if with_topk else None
    _expect("topk_idx", ti, (n_rows, top_k), (torch.int32,), optional=True)
    _expect("topk_prob", tp, (n_rows, top_k), (torch.float32,), optional=True)
    _need_cuda(logits, row_mult, ti, tp, *[out[x] for x in ("load", "psum", "zsum", "n_tok")])
    _check(load_library().moe_router_stats_noalloc(
        _p(logits), _dtype_code(logits), n_rows, E, top_k, _p(row_mult), _p(ti), _p(tp),
        _p(out["load"]), _p(out["psum"]), _p(out["zsum"]), _p(out["n_tok"]), _stream(logits)))
    return out


def moe_router_stats_bwd(logits, row_mult, g_psum, g_z: float, out=None):
    """dlogits of <g_psum, psum> + g_z * zsum (fp32 [n_rows, E])."""
    import torch
    if logits is None or logits.dim() != 2:
        raise KDAError("logits must be [rows, n_experts]")
    n_rows, E = logits.shape
    _expect("logits", logits, (n_rows, E), (torch.bfloat16, torch.float32))
    _expect("row_mult", row_mult, (n_rows,), (torch.int32,))
    _expect("g_psum", g_psum, (E,), (torch.float32,))
    _need_cuda(logits, row_mult, g_psum)
    if out is None:
        out = torch.empty((n_rows, E), dtype=torch.float32, device=logits.device)
    _expect("dlogits", out, (n_rows, E), (torch.float32,))
    _need_cuda(out)
    _same_device(logits, row_mult, g_psum, out)
    _check(load_library().moe_router_stats_bwd(_p(logits), _dtype_code(logits), n_rows, E,
                                               _p(row_mult), _p(g_psum), float(g_z), _p(out),
                                               _stream(logits)))
    return out


def _attn_shape(plan: KDAPlan, q):
    if q is None or q.dim() != 3:
        raise KDAError("q must be [rows, H, d]")
    N, H, D = q.shape
    if N != plan.info["n_rows"]:
        raise KDAError(f"q has {N} rows, the plan has {plan.info['n_rows']} compact rows")
    return N, H, D


def tree_attn_fwd(plan: KDAPlan, q, k, v, scale=None, out=None):
    """Tree-ancestor attention forward: q, k, v bf16 [rows, H, d] on the
    plan's compact rows.  Returns (o fp32 [rows, H, d], lse fp32 [rows, H])."""
    import torch
    N, H, D = _attn_shape(plan, q)
    bf = (torch.bfloat16,)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _expect(name, t, (N, H, D), bf)
    _need_cuda(q, k, v)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = (torch.empty(N, H, D, dtype=torch.float32, device=q.device),
               torch.empty(N, H, dtype=torch.float32, device=q.device))
    o, lse = out
    _expect("o", o, (N, H, D), (torch.float32,))
    _expect("lse", lse, (N, H), (torch.float32,))
    _need_cuda(o, lse)
    _same_device(q, k, v, o, lse)
    _check(load_library().tree_attn_fwd(plan.handle, _p(plan.device(q.device)), H, D, scale,
                                        _p(q), _p(k), _p(v), _p(o), _p(lse), _stream(q)))
    return o, lse


def tree_attn_bwd(plan: KDAPlan, q, k, v, o, lse, dO, scale=None, out=None, ws=None):
    """Gradients (dq, dk, dv) fp32 of sum(dO * o) for tree_attn_fwd; dO bf16."""
    import torch
    N, H, D = _attn_shape(plan, q)
    bf, f32 = (torch.bfloat16,), (torch.float32,)
    for name, t in (("q", q), ("k", k), ("v", v), ("dO", dO)):
        _expect(name, t, (N, H, D), bf)
    _expect("o", o, (N, H, D), f32)
    _expect("lse", lse, (N, H), f32)
    _need_cuda(q, k, v, o, lse, dO)
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if out is None:
        out = tuple(torch.empty(N, H, D, dtype=torch.float32, device=q.device) for _ in range(3))
    nb = load_library().tree_attn_workspace_bytes(plan.handle, H, D)
    if ws is None or ws.numel() * ws.element_size() < nb:
        ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = out
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _expect(name, t, (N, H, D), f32)
    _need_cuda(dq, dk, dv, ws)
    _same_device(q, k, v, o, lse, dO, dq, dk, dv, ws)
    _check(load_library().tree_attn_bwd(plan.handle, _p(plan.device(q.device)), H, D, scale,
                                        _p(q), _p(k), _p(v), _p(o), _p(lse), _p(dO), _p(dq),
                                        _p(dk), _p(dv), _p(ws), ws.numel() * ws.element_size(),
                                        _stream(q)))
    return dq, dk, dv


def set_overlap(on: bool = True):
    """Whether kda_tree_fwd / kda_tree_bwd run their chunk-parallel passes on a
    second stream beside the round chains (default) or everything on the
    caller's stream; results are bitwise the same."""
    _check(load_library().kda_set_overlap(1 if on else 0))


def timing_enable(on: bool = True, only: str | None = None):
    """Start (clearing the counters) or stop per-kernel launch timing; `only`
    limits it to one kernel class (None: every class)."""
    L = load_library()
    _check(L.kda_timing_filter(only.encode() if only else None))
    _check(L.kda_timing_enable(1 if on else 0))


def timing_read() -> dict:
    """{kernel name: (launches, total ms)} since the last timing_enable."""
    L = load_library()
    n = _check(L.kda_timing_read(-1, None, 0, None, None))
    out = {}
    for i in range(n):
        buf = ctypes.create_string_buffer(128)
        cnt = ctypes.c_int64()
        ms = ctypes.c_double()
        _check(L.kda_timing_read(i, buf, 128, ctypes.byref(cnt), ctypes.byref(ms)))
        out[buf.value.decode()] = (int(cnt.value), float(ms.value))
    return out
