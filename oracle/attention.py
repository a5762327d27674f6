"""Attention over a decoded cache (oracle side), for the decode fused into an
attention consumer.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Source: JoLT abstract (arXiv 2607.12550v2), first sentence: the KV cache is
the dominant cost of serving, i.e. of the attention that reads it.  The pages
do not describe the consumer; the reading is plain scaled dot-product
attention of new query vectors over the layer's T cached tokens, grouped as
in GQA (Mistral-7B-v0.3: 4 query heads per KV head; MHA: 1):

    out[hq, s] = softmax_t(q[hq, s] . K[h, t] / sqrt(D)) V[h, t],  h = hq // G,

in fp64 on the decoded K and V (no output rounding: the fused consumer never
stores them).
"""
from __future__ import annotations

import numpy as np


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row-wise softmax; the row maximum is subtracted first (same values,
    no overflow)."""
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def attend(q, K, V, G: int) -> np.ndarray:
    """q [H G, n, D]; K, V [H, T, D]; out [H G, n, D] (fp64)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, n, D = q.shape
    out = np.empty((Hq, n, D))
    for hq in range(Hq):
        h = hq // G
        p = softmax_rows(q[hq] @ K[h].T / np.sqrt(D))        # [n, T]
        out[hq] = p @ V[h]
    return out
