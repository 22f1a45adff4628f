"""Reference oracle for the fused loss kernels (fp64, CPU).

TEST INFRASTRUCTURE ONLY: imported by the test suite, ``__graft_entry__``'s
smoke check and bench.py's CPU baseline, never by the product path.

Follows "cross_entropy ve sum_losses — Fused Loss + dLogits"
(https://llm.istanbul/learn/tr/07_loss), sections "Ne Yapar?" (the loss and
gradient formulas with label smoothing alpha and z-loss beta) and "Satır
Satır" (an out-of-range target gives a zero loss and a zero gradient row; the
denominator is floored at 1e-30; sum_losses adds the per-row losses).  Every
step is plain numpy in float64, in the pages' order:

    row_max = max_v l[v]
    denom   = sum_v exp(l[v] - row_max)
    lse     = row_max + log(max(denom, 1e-30))
    p[v]    = exp(l[v] - row_max) / max(denom, 1e-30)
    loss    = lse - (1 - alpha) * l[tgt] - alpha * mean_v l[v] + beta * lse^2
    dl[v]   = ((p[v] - target[v]) + 2 beta lse p[v]) * inv_norm,
              target = (1 - alpha) * one_hot(tgt) + alpha / V

Pinned by tests/test_oracle_loss.py.
"""
from __future__ import annotations

import math

import numpy as np


def cross_entropy(logits, targets, alpha=0.0, beta=0.0, inv_norm=1.0, rows=None):
    """Per-row loss and dLogits of the fused kernel.

    logits: [S, V] float32 (not modified); targets: [S] unsigned integers.
    rows: None (all) or row indices.  Returns (loss [n] float64,
    dlogits [n, V] float64, scale dict) for the selected rows, where the
    scale dict holds the magnitudes the tolerance is relative to: for the
    loss |lse| + (1-alpha)|l[tgt]| + alpha * mean|l| + beta * lse^2, for
    dLogits (p + target + |2 beta lse| p) * |inv_norm|.
    """
    logits = np.asarray(logits)
    S, V = logits.shape
    idx = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    loss = np.zeros(len(idx))
    dl = np.zeros((len(idx), V))
    loss_mag = np.zeros(len(idx))
    dl_mag = np.zeros((len(idx), V))
    for r, s in enumerate(idx):
        tgt = int(targets[s])
        if tgt >= V:
            continue                       # ignored row: loss 0, gradient 0
        l = logits[s].astype(np.float64)
        row_max = l.max()
        e = np.exp(l - row_max)
        denom = max(float(e.sum()), 1e-30)
        lse = row_max + math.log(denom)
        p = e / denom
        mean_l = float(l.sum()) / V
        loss[r] = lse - (1.0 - alpha) * l[tgt] - alpha * mean_l + beta * lse * lse
        loss_mag[r] = abs(lse) + (1.0 - alpha) * abs(l[tgt]) + alpha * float(np.abs(l).mean()) + beta * lse * lse
        target = np.full(V, alpha / V)
        target[tgt] += 1.0 - alpha
        dl[r] = ((p - target) + 2.0 * beta * lse * p) * inv_norm
        dl_mag[r] = (p + target + abs(2.0 * beta * lse) * p) * abs(inv_norm)
    return loss, dl, {"loss": loss_mag, "dlogits": dl_mag}


def sum_losses(losses):
    """The scalar total of the per-row losses (exactly rounded fp64 sum)."""
    return math.fsum(float(x) for x in np.asarray(losses, dtype=np.float64))


# Parity bounds |x - x_ref| <= rel * scale + abs, derived from the fp32
# arithmetic of the kernel: exp and log of arguments up to ~40 in magnitude
# (a few 1e-6 relative), a V-term sum (log2 V roundings), one division.
TOL_LOSS = (1e-5, 1e-6)
TOL_DLOGITS = (1e-5, 1e-9)
