"""Masked scaled dot-product softmax attention in float64.

The pages name attention (Vidu S2 paper read, section 2.2: block-wise causal
attention over reference, condition and history) but print no formula; this is
the textbook definition: O = softmax(Q K^T / sqrt(d) + M) V, softmax over keys,
M = 0 for visible keys and -inf for masked ones.  Also returns the natural-log
sum-exp of every row (LSE), used to check a kernel's normaliser.
"""
from __future__ import annotations

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible=None, row_block: int = 512):
    """q [Nq, d], k [Nk, d], v [Nk, dv] -> (o [Nq, dv], lse [Nq]); all float64.

    `visible` is None (all keys) or a bool array [Nq, Nk].  Queries are taken in
    blocks of `row_block` rows only to bound memory; rows are independent.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, d = q.shape
    o = np.empty((nq, v.shape[1]), dtype=np.float64)
    lse = np.empty(nq, dtype=np.float64)
    scale = 1.0 / np.sqrt(d)
    for r0 in range(0, nq, row_block):
        r1 = min(nq, r0 + row_block)
        s = (q[r0:r1] @ k.T) * scale
        if visible is not None:
            s = np.where(visible[r0:r1], s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        den = e.sum(axis=1, keepdims=True)
        o[r0:r1] = (e @ v) / den
        lse[r0:r1] = (m + np.log(den))[:, 0]
    return o, lse
