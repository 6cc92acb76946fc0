"""Sparse Flash Attention over the selected positions, as a plain definition.

Test infrastructure only (see package docstring).

Pages: "Deep Dive into Sparse Attention ..." (page 1), section 1: SFA runs
attention only on the key-value pairs of the positions the indexer selected,
on top of Multi-Head Latent Attention; "Adapting and Optimizing Kimi K3.1 Pro
..." (page 2), section 2: the attention core reads the cache entries of the
selected indices and gathers them directly.  The arithmetic is the task's
fixed choice: the key of a position is [latent 512 | rope 64] (dequantised
E4M3 latent times its tile scale, bf16 rope), the value is the 512-wide
latent, logits are scaled by 1/sqrt(576), softmax over the selected list, no
further mask.  Readings taken:
  * entries equal to -1 are skipped; duplicate entries count as listed;
  * lse is the natural log of the softmax denominator of the scaled logits
    (max-subtracted form); an empty list gives out = 0 and lse = -inf.
"""
from __future__ import annotations

import math

import numpy as np

D_LATENT = 512
DEFAULT_SCALE = 1.0 / math.sqrt(576.0)


def sparse_attn(q: np.ndarray, latent: np.ndarray, rope: np.ndarray, idx: np.ndarray,
                scale: float = DEFAULT_SCALE):
    """q [H, 576] fp64; latent [n, 512], rope [n, 64] fp64 rows addressed by
    idx (entries < 0 skipped) -> (out [H, 512] fp64, lse [H] fp64)."""
    idx = np.asarray(idx)
    idx = idx[idx >= 0]
    H = q.shape[0]
    if len(idx) == 0:
        return np.zeros((H, D_LATENT)), np.full(H, -np.inf)
    kl = latent[idx]                                   # [m, 512]
    kr = rope[idx]                                     # [m, 64]
    z = scale * (q[:, :D_LATENT] @ kl.T + q[:, D_LATENT:] @ kr.T)   # [H, m]
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    out = (p / l) @ kl
    lse = (m + np.log(l))[:, 0]
    return out, lse


def dense_attn(q: np.ndarray, latent: np.ndarray, rope: np.ndarray, t: int,
               scale: float = DEFAULT_SCALE):
    """Attention over every position 0..t (the L <= K case of SFA)."""
    return sparse_attn(q, latent, rope, np.arange(t + 1), scale)
