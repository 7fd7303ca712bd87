"""Margin-conditioned inputs: pick the activation draw whose routing is unique.

TEST INFRASTRUCTURE ONLY: part of the plain CPU oracle.

The workloads resample the bf16 activation (next attempt counter of the seeded
generator) until the oracle's top-k logit margin, l_(k) - l_(k+1) on the fp64
logits including any bias, is at least the configured margin; for the LM head
until the top-1 minus top-2 logit gap is.  Under that margin the chosen set
and the argmax are unique, so the GPU must reproduce them exactly.

`draw` is a callable (attempt -> bf16 bits) supplied by the caller; this module
does not import the generator.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64
from .lmhead import lmhead_logits, top2_gap
from .moe import Layer, router_logits, topk_margin


def pick_token(layer: Layer, k: int, margin: float, draw, max_attempts: int = 1000):
    """First attempt whose router margin is >= margin: (x_bits, attempt)."""
    for a in range(max_attempts):
        x = draw(a)
        if topk_margin(router_logits(layer, bf16_to_f64(x)), k) >= margin:
            return x, a
    raise RuntimeError("no draw met the margin")


def pick_hidden(w_q: np.ndarray, w_s: np.ndarray, margin: float, draw, max_attempts: int = 100):
    """One row: first attempt whose top-1/top-2 logit gap is >= margin."""
    X, A = pick_hidden_rows(w_q, w_s, margin, lambda b, a: draw(a), 1, max_attempts)
    return X[0], A[0]


def pick_hidden_rows(w_q: np.ndarray, w_s: np.ndarray, margin: float, draw, B: int, max_attempts: int = 100):
    """B rows, row b drawn as draw(b, attempt) until its gap holds; all
    pending rows are scored together, one pass over the matrix per round."""
    X = [None] * B
    A = [0] * B
    pending = list(range(B))
    for a in range(max_attempts):
        cand = np.stack([draw(b, a) for b in pending])
        gaps = top2_gap(lmhead_logits(w_q, w_s, cand))
        for b, x, g in zip(list(pending), cand, gaps):
            if g >= margin:
                X[b], A[b] = x, a
                pending.remove(b)
        if not pending:
            return np.stack(X), A
    raise RuntimeError("no draw met the gap")
