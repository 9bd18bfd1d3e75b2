"""Float64 CPU reference of the hybrid layer group (test infrastructure):
the same module structure as tree_packed_chunkwise_amd.hybrid, with the
dense steps as float64 torch ops and the tree steps as autograd functions over
the oracle (oracle.kda, oracle.attention, oracle.gather).  Tree attention
inputs are rounded to bf16 as on the GPU side."""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import attention as oa
from oracle import gather as og
from oracle import kda as okda
from oracle.tree import Tree
from tree_packed_chunkwise_amd import synth


def _np(t):
    return t.detach().cpu().numpy().astype(np.float64)


class _KDARef(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, g, beta, tree, scale):
        H, D = q.shape[1], q.shape[2]
        h0 = np.zeros((len(tree.roots), H, D, v.shape[2]))
        args = tuple(_np(x) for x in (q, k, v, g, beta))
        o, _ = okda.tree_fwd(tree, *args, h0, scale)
        ctx.tree, ctx.scale, ctx.args, ctx.h0 = tree, scale, args, h0
        return torch.from_numpy(o)

    @staticmethod
    def backward(ctx, do):
        tree = ctx.tree
        H, D, Dv = ctx.args[0].shape[1], ctx.args[0].shape[2], ctx.args[2].shape[2]
        dhl = np.zeros((len(tree.leaves), H, D, Dv))
        r = okda.tree_bwd(tree, *ctx.args, ctx.h0, ctx.scale, _np(do), dhl)
        t = torch.from_numpy
        return t(r["dq"]), t(r["dk"]), t(r["dv"]), t(r["dg"]), t(r["dbeta"]), None, None


class _AttnRef(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, tree, scale):
        args = tuple(_np(x) for x in (q, k, v))
        o, _ = oa.tree_attention_fwd(tree, *args, scale)
        ctx.tree, ctx.scale, ctx.args = tree, scale, args
        return torch.from_numpy(o)

    @staticmethod
    def backward(ctx, do):
        dq, dk, dv = oa.tree_attention_bwd(ctx.tree, *ctx.args, ctx.scale, _np(do))
        t = torch.from_numpy
        return t(dq), t(dk), t(dv), None, None


class _GatherRef(torch.autograd.Function):
    @staticmethod
    def forward(ctx, logits, pos_row, pos_tgt):
        z = _np(logits)
        logp, _ = og.gather_fwd(z, pos_row, pos_tgt)
        ctx.z, ctx.pos_row, ctx.pos_tgt = z, pos_row, pos_tgt
        return torch.from_numpy(logp)

    @staticmethod
    def backward(ctx, dlogp):
        return torch.from_numpy(og.gather_bwd(ctx.z, ctx.pos_row, ctx.pos_tgt, _np(dlogp))), None, None


def _round(x):
    return torch.from_numpy(synth.round_bf16(x.detach().numpy().astype(np.float32))
                            .astype(np.float64))


def _bf16(x):
    """round to bf16 (RNE from the float32 value) without leaving autograd:
    the rounding is treated as identity in the backward, as on the GPU side."""
    return x + (_round(x) - x).detach()



def reference_forward(params: dict, tree: Tree, tokens, pos_row, pos_tgt, H, D,
                      bf16_stream=False):
    """params: float64 CPU leaf tensors named as HybridGroup's parameters.

    bf16_stream=True rounds to bf16 wherever HybridGroup with dtype bf16
    stores a bf16 tensor (every projection output, q and k after the L2
    norm, the tree steps' outputs before their projection, the residual
    stream after each add, the logits), the rounding being the identity in
    the backward.  Otherwise only the tree attention inputs are rounded, as
    in the fp32 group."""
    N = tokens.shape[0]
    R = _bf16 if bf16_stream else (lambda t: t)
    x = params["embed"][tokens]
    scale = 1.0 / math.sqrt(D)
    i = 0
    while f"kda.{i}.wq" in params:
        P = lambda n: params[f"kda.{i}.{n}"]
        q = R(torch.nn.functional.normalize(R(x @ P("wq")).view(N, H, D), dim=-1))
        k = R(torch.nn.functional.normalize(R(x @ P("wk")).view(N, H, D), dim=-1))
        v = R(x @ P("wv")).view(N, H, D)
        beta = torch.sigmoid(R(x @ P("wb")))
        g = -torch.nn.functional.softplus(R(x @ P("wg")).view(N, H, D) + 2.0)
        o = _KDARef.apply(q, k, v, g, beta, tree, scale)
        x = R(x + R(R(o).reshape(N, H * D) @ P("wo")))
        i += 1
    q = _bf16(R(x @ params["attn.wq"]).view(N, H, D))
    k = _bf16(R(x @ params["attn.wk"]).view(N, H, D))
    v = _bf16(R(x @ params["attn.wv"]).view(N, H, D))
    o = _AttnRef.apply(q, k, v, tree, scale)
    x = R(x + R(R(o).reshape(N, H * D) @ params["attn.wo"]))
    logits = R(x @ params["lm"])
    return _GatherRef.apply(logits, pos_row, pos_tgt)
