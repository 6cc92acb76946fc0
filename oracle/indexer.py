"""Lightning Indexer scores and Top-K selection, as plain definitions.

Test infrastructure only (see package docstring).

Pages: "Deep Dive into Sparse Attention ..." (page 1), section 1: the indexer
scores the relevance of every historical key for each query position and keeps
the Top-K most relevant positions; section 2.1 and "Kimi K3.1 Pro Inference
Acceleration" (page 3), section "Lightning Indexer Three-Stream Coordination":
the three steps are relevance scoring, head-weight weighting and Top-K
selection.  The arithmetic is the task's fixed choice:

    I(t, s) = sum_h w[t, h] * max(0, q[t, h] . k[s]),   0 <= s <= t

with one indexer key per token shared by all H_I heads.  Readings taken:
  * the causal range includes s = t (the query's own key is already cached);
    a decode query of a sequence of length L sits at t = L - 1;
  * -0 and +0 are the same score (I + 0.0 canonicalises);
  * Top-K keeps the K largest scores, ties broken by the lower position; the
    kept positions are reported in ascending order, padded with -1 (scores
    with -inf) when fewer than K positions exist.
"""
from __future__ import annotations

import numpy as np


def indexer_scores(q: np.ndarray, k: np.ndarray, w: np.ndarray, t: int) -> np.ndarray:
    """q [H_I,128] fp64, k [>=t+1,128] fp64, w [H_I] -> I [t+1] fp64."""
    logits = q @ k[:t + 1].T                          # [H_I, t+1]
    I = np.asarray(w, dtype=np.float64) @ np.maximum(logits, 0.0)
    return I + 0.0


def indexer_scores_loops(q, k, w, t) -> np.ndarray:
    """Same definition with explicit Python loops and no BLAS (tiny inputs)."""
    H, D = len(q), len(q[0])
    out = np.zeros(t + 1)
    for s in range(t + 1):
        acc = 0.0
        for h in range(H):
            dot = 0.0
            for i in range(D):
                dot += float(q[h][i]) * float(k[s][i])
            acc += float(w[h]) * (dot if dot > 0.0 else 0.0)
        out[s] = acc + 0.0
    return out


def topk_order(I: np.ndarray) -> np.ndarray:
    """All positions ordered by (score descending, position ascending)."""
    s = np.arange(len(I))
    return np.lexsort((s, -np.asarray(I, dtype=np.float64)))


def topk_select(I: np.ndarray, K: int):
    """-> (idx int32 [K] ascending then -1, score fp64 [K] then -inf)."""
    n = len(I)
    sel = np.sort(topk_order(I)[:min(K, n)])
    idx = np.full(K, -1, dtype=np.int32)
    sc = np.full(K, -np.inf)
    idx[:len(sel)] = sel
    sc[:len(sel)] = np.asarray(I)[sel]
    return idx, sc


def kth_score(I: np.ndarray, K: int) -> float:
    """Score of the K-th selected position (the smallest kept score)."""
    n = len(I)
    return float(np.asarray(I)[topk_order(I)[min(K, n) - 1]])
