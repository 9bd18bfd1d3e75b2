"""The hybrid layer group over a packed rollout tree (the Tiny-style model of
the HARTS pages: KDA layers and full-attention layers in a 3:1 mix,
thelatestinai.com Table 1; per-position log-probs from compact logit rows,
Figure C.1(d)), as torch modules whose tree-specific steps run in
libkda_tree.so:

  x = embed(tokens)                                         [rows, hidden]
  3 x KDA layer:   q, k = l2norm(x Wq), l2norm(x Wk) per head;  v = x Wv
                   beta = sigmoid(x Wb);  g = -softplus(x Wg + 2)
                   x = x + kda_tree(q, k, v, g, beta) Wo
  attention layer: x = x + tree_attn(x Wq, x Wk, x Wv) Wo    (ancestor mask)
  logits = x Wlm  [rows, vocab];  logp = gather_logprobs(logits)  per position

Residual stream without norms or feed-forward blocks; random-init weights
N(0, 1/fan_in).  Dense projections are torch matmuls (rocBLAS / hipBLASLt);
the tree steps are autograd functions over the C-ABI calls.  `dtype` is the
compute dtype of the stream and projections (bf16 for the benchmark, fp32 for
parity runs); tree attention always takes bf16 q, k, v.

`trace` (optional, a callable) receives every tree step's library inputs and
outputs as they pass: trace(kind, layer, phase, tensors) with kind in
{"kda", "attn", "gather"} and phase in {"fwd", "bwd"}.
"""
from __future__ import annotations

import math

import torch

from . import binding as B


class _KDA(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, plan, scale, trace, layer):
        f = B.kda_tree_fwd(plan, q, k, v, g, beta, None, scale)
        ctx.plan, ctx.scale, ctx.trace, ctx.layer = plan, scale, trace, layer
        ctx.save_for_backward(q, k, v, g, beta, f["saved"])
        if trace:
            trace("kda", layer, "fwd", dict(q=q, k=k, v=v, g=g, beta=beta, o=f["o"]))
        return f["o"]

    @staticmethod
    def backward(ctx, do):
        q, k, v, g, beta, saved = ctx.saved_tensors
        dO = do.to(q.dtype).contiguous()
        r = B.kda_tree_bwd(ctx.plan, q, k, v, g, beta, saved, dO, None, None, ctx.scale)
        if ctx.trace:
            ctx.trace("kda", ctx.layer, "bwd", dict(dO=dO, **{n: r[n] for n in (
                "dq", "dk", "dv", "dg", "dbeta")}))
        return (r["dq"].to(q.dtype), r["dk"].to(k.dtype), r["dv"].to(v.dtype), r["dg"],
                r["dbeta"], None, None, None, None)


class _Attn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, plan, scale, trace):
        o, lse = B.tree_attn_fwd(plan, q, k, v, scale)
        ctx.plan, ctx.scale, ctx.trace = plan, scale, trace
        ctx.save_for_backward(q, k, v, o, lse)
        if trace:
            trace("attn", 0, "fwd", dict(q=q, k=k, v=v, o=o, lse=lse))
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dO = do.to(torch.bfloat16).contiguous()
        dq, dk, dv = B.tree_attn_bwd(ctx.plan, q, k, v, o, lse, dO, ctx.scale)
        if ctx.trace:
            ctx.trace("attn", 0, "bwd", dict(dO=dO, dq=dq, dk=dk, dv=dv))
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None


class _Gather(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, pos_row, pos_tgt, row_pos_ptr, row_pos_idx, trace):
        logp, lse = B.gather_logprobs(logits, pos_row, pos_tgt)
        ctx.trace = trace
        ctx.save_for_backward(logits, lse, row_pos_ptr, row_pos_idx, pos_tgt)
        if trace:
            trace("gather", 0, "fwd", dict(logits=logits, logp=logp, lse=lse))
        return logp

    @staticmethod
    def backward(ctx, dlogp):
        logits, lse, rp_ptr, rp_idx, tgt = ctx.saved_tensors
        dl = dlogp.float().contiguous()
        dz = B.gather_logprobs_bwd(logits, lse, rp_ptr, rp_idx, tgt, dl)
        if ctx.trace:
            ctx.trace("gather", 0, "bwd", dict(dlogp=dl, dlogits=dz))
        return dz, None, None, None, None, None


def _init(rng: torch.Generator, fan_in, shape, dtype, device):
    w = torch.randn(*shape, generator=rng, dtype=torch.float32) / math.sqrt(fan_in)
    return torch.nn.Parameter(w.to(device=device, dtype=dtype))


class HybridGroup(torch.nn.Module):
    def __init__(self, hidden=2048, heads=16, head_dim=128, vocab=32000, n_kda=3, seed=0,
                 dtype=torch.bfloat16, device="cuda"):
        super().__init__()
        g = torch.Generator().manual_seed(seed)
        hd = heads * head_dim
        self.H, self.D, self.hidden, self.vocab, self.dtype = heads, head_dim, hidden, vocab, dtype
        self.embed = _init(g, 1, (vocab, hidden), dtype, device)
        self.kda = torch.nn.ModuleList()
        for _ in range(n_kda):
            layer = torch.nn.ParameterDict({
                "wq": _init(g, hidden, (hidden, hd), dtype, device),
                "wk": _init(g, hidden, (hidden, hd), dtype, device),
                "wv": _init(g, hidden, (hidden, hd), dtype, device),
                "wb": _init(g, hidden, (hidden, heads), dtype, device),
                "wg": _init(g, hidden, (hidden, hd), dtype, device),
                "wo": _init(g, hd, (hd, hidden), dtype, device)})
            self.kda.append(layer)
        self.attn = torch.nn.ParameterDict({
            "wq": _init(g, hidden, (hidden, hd), dtype, device),
            "wk": _init(g, hidden, (hidden, hd), dtype, device),
            "wv": _init(g, hidden, (hidden, hd), dtype, device),
            "wo": _init(g, hd, (hd, hidden), dtype, device)})
        self.lm = _init(g, hidden, (hidden, vocab), dtype, device)

    def forward(self, plan, tokens, maps, trace=None):
        """tokens [rows] int64 (compact rows); maps: device int32 tensors
        pos_row, pos_tgt, row_pos_ptr, row_pos_idx.  Returns logp [n_pos]."""
        N, H, D = tokens.shape[0], self.H, self.D
        x = self.embed[tokens]
        scale = 1.0 / math.sqrt(D)
        for li, L in enumerate(self.kda):
            q = torch.nn.functional.normalize((x @ L["wq"]).float().view(N, H, D), dim=-1)
            k = torch.nn.functional.normalize((x @ L["wk"]).float().view(N, H, D), dim=-1)
            v = (x @ L["wv"]).view(N, H, D)
            beta = torch.sigmoid((x @ L["wb"]).float()).contiguous()
            gate = -torch.nn.functional.softplus((x @ L["wg"]).float().view(N, H, D) + 2.0)
            o = _KDA.apply(q.to(self.dtype).contiguous(), k.to(self.dtype).contiguous(),
                           v.contiguous(), gate.contiguous(), beta, plan, scale, trace, li)
            x = x + o.to(self.dtype).reshape(N, H * D) @ L["wo"]
        A = self.attn
        bf = torch.bfloat16
        q = (x @ A["wq"]).view(N, H, D).to(bf).contiguous()
        k = (x @ A["wk"]).view(N, H, D).to(bf).contiguous()
        v = (x @ A["wv"]).view(N, H, D).to(bf).contiguous()
        o = _Attn.apply(q, k, v, plan, scale, trace)
        x = x + o.to(self.dtype).reshape(N, H * D) @ A["wo"]
        logits = (x @ self.lm).contiguous()
        return _Gather.apply(logits, maps["pos_row"], maps["pos_tgt"], maps["row_pos_ptr"],
                             maps["row_pos_idx"], trace)


def gather_maps(plan: B.KDAPlan, tokens, device):
    """Device int32 maps of the plan's trajectory positions; targets are the
    tokens of the next position."""
    import numpy as np
    ex = lambda f: torch.from_numpy(np.asarray(plan.export(f), dtype=np.int32)).to(device)
    pos_row, pos_next = ex("POS_ROW"), ex("POS_NEXT_ROW")
    return {"pos_row": pos_row, "pos_tgt": tokens[pos_next.long()].to(torch.int32).contiguous(),
            "row_pos_ptr": ex("ROW_POS_PTR"), "row_pos_idx": ex("ROW_POS_IDX")}
