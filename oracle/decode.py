"""fp64 oracle for inference with a key/value cache.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
HIP path.

The model is the one of ``oracle.model`` (architecture list of the release-news
page "Karpathy再放大招…", section 技術細節與問答: multi-query attention, rotary
embeddings, QK norm, logit softcap).  Serving it with a cache of the keys and
values of earlier positions is an evaluation order, not a different function.
By causality the logits at position t depend on tokens 0..t only, so the plain
definition of what prefill and decode must return is the full forward's
softcapped logits row at that position.  The oracle computes exactly that:
``prefix_logits`` runs the forward on the whole prefix, and ``decode_attention``
is the attention of one new position over every cached position (all of them
at or before it, so no mask).
"""
from __future__ import annotations

import numpy as np

from .model import sequence_forward


def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Attention of one query position over n cached positions, one K/V head.

    q: [H, hd] (the new position's query heads, after RoPE and QK norm);
    k, v: [n, hd] (the cached keys and values of positions 0..n-1, the new
    one included).  Returns o [H, hd] with
    o[h] = sum_u softmax_u(q[h] . k[u] * scale) v[u].
    """
    s = (q @ k.T) * scale                      # [H, n]
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    return p @ v


def prefix_logits(cfg, p, ids: np.ndarray) -> np.ndarray:
    """Softcapped logits z' [T, V] at every position of one sequence ids [T]:
    row t is what prefill (t = T-1) or a decode step at position t returns."""
    y = np.zeros_like(ids)
    _, cache = sequence_forward(cfg, p, ids, y, keep_cache=True)
    return cache["zc"]
