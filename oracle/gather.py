"""Per-original-position log-prob recovery from compact logit rows, float64
(oracle; test infrastructure only).

Sources: HARTS abstract (recovering log-probabilities for each original
trajectory position preserves RL objectives); Figure 1 caption (one logit
row z_B supplies the distinct target log-probs of T1 and T2); Figure C.1(d)
(mapped log-probabilities restore original token order without expanded
vocabulary-sized logits).

    logp[pos] = z[row(pos), tgt(pos)] - logsumexp(z[row(pos), :])
    dz[row, :] = sum_{pos -> row} dlogp[pos] * (onehot(tgt(pos)) - softmax(z[row]))

Masked entries (the pages leave them open; reading taken): a logit of -inf
has probability zero.  A row whose every entry is -inf has lse = -inf, its
positions get logp = -inf, and its softmax is taken as all zeros, so only the
target columns of its gradient are nonzero.

Pins (tests/test_oracle_gather.py): uniform logits give -ln V exactly;
agreement with scipy.special.log_softmax applied to expanded rows; the
backward agrees with central finite differences; a row with masked entries
equals log_softmax over its unmasked entries alone.
"""
from __future__ import annotations

import numpy as np

BLOCK = 4096  # rows per streamed block


def row_lse(z):
    """logsumexp over the last axis, streamed in row blocks, float64."""
    n = z.shape[0]
    out = np.empty(n, dtype=np.float64)
    for r0 in range(0, n, BLOCK):
        blk = np.asarray(z[r0:r0 + BLOCK], dtype=np.float64)
        m = blk.max(axis=1)
        m = np.where(np.isfinite(m), m, 0.0)   # an all -inf row sums to 0: lse = -inf
        with np.errstate(divide="ignore"):
            out[r0:r0 + BLOCK] = m + np.log(np.exp(blk - m[:, None]).sum(axis=1))
    return out


def gather_fwd(z, pos_row, pos_tgt):
    """Returns (logp [n_pos], lse [n_rows])."""
    lse = row_lse(z)
    pos_row = np.asarray(pos_row, dtype=np.int64)
    pos_tgt = np.asarray(pos_tgt, dtype=np.int64)
    zt = np.asarray(z[pos_row, pos_tgt], dtype=np.float64)
    lr = lse[pos_row]
    with np.errstate(invalid="ignore"):
        logp = np.where(lr == -np.inf, -np.inf, zt - lr)
    return logp, lse


def gather_bwd(z, pos_row, pos_tgt, dlogp, rows=None):
    """dz for the listed rows (all rows when rows is None)."""
    pos_row = np.asarray(pos_row, dtype=np.int64)
    pos_tgt = np.asarray(pos_tgt, dtype=np.int64)
    dlogp = np.asarray(dlogp, dtype=np.float64)
    n = z.shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    wsum = np.zeros(n)
    np.add.at(wsum, pos_row, dlogp)
    zr = np.asarray(z[rows], dtype=np.float64)
    m = zr.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    p = np.exp(zr - m)
    tot = p.sum(axis=1, keepdims=True)
    p = np.divide(p, tot, out=np.zeros_like(p), where=tot > 0)   # all masked: softmax 0
    dz = -p * wsum[rows][:, None]
    where = {int(r): i for i, r in enumerate(rows)}
    for pi in range(pos_row.shape[0]):
        i = where.get(int(pos_row[pi]))
        if i is not None:
            dz[i, pos_tgt[pi]] += dlogp[pi]
    return dz
