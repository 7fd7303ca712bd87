"""Plain fp64 oracle of the 4-bit output layer (LM head) with argmax.

TEST INFRASTRUCTURE ONLY: part of the plain CPU oracle.  Nothing in the
product path may import this package.

The pages state that the output layer maps hidden states back to a vocabulary
of about 150,000 tokens, is about an eighth of the per-token work, and is
quantized to 4 bits ("Flint 40B: Best Mid Sized LLM", transcript 03:36-05:39;
mirrorspeed.com page, section "Quantization").  Decoding here is greedy: the
token is the index of the largest logit, the lowest index on ties.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_to_f64, dequant


def lmhead_logits(w_q: np.ndarray, w_s: np.ndarray, x_bits: np.ndarray, rows_per_chunk: int = 8192) -> np.ndarray:
    """z[b, v] = sum_k W[v, k] x[b, k] in fp64 for x of shape [B][d].

    Rows are dequantized a chunk at a time only to bound memory; every logit
    is still one independent dot product."""
    V, half = w_q.shape
    d = 2 * half
    X = bf16_to_f64(np.atleast_2d(x_bits))          # [B][d]
    z = np.empty((X.shape[0], V))
    for v0 in range(0, V, rows_per_chunk):
        W = dequant(w_q[v0:v0 + rows_per_chunk], w_s[v0:v0 + rows_per_chunk], d)
        z[:, v0:v0 + W.shape[0]] = X @ W.T
    return z


def argmax_lowest(z: np.ndarray):
    """(token, max logit) per row: the first index reaching the maximum."""
    z = np.atleast_2d(z)
    tok = np.array([int(np.flatnonzero(row == row.max())[0]) for row in z], dtype=np.int64)
    return tok, z[np.arange(z.shape[0]), tok]


def lmhead_argmax(w_q, w_s, x_bits):
    z = lmhead_logits(w_q, w_s, x_bits)
    tok, zmax = argmax_lowest(z)
    return tok, zmax, z


def top2_gap(z: np.ndarray) -> np.ndarray:
    """Per row: largest minus second-largest logit."""
    s = np.sort(np.atleast_2d(z), axis=1)
    return s[:, -1] - s[:, -2]
