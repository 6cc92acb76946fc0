"""End-to-end oracle of one DSA step on synthetic inputs.

Test infrastructure only (see package docstring).

Takes the dictionary of seeded inputs (bf16 bit patterns, fp32 head weights,
sequence lengths, query rows) and produces, per query row, what the hot path
must produce: the indexer scores over 0..t, the Top-K positions and scores,
and the SFA output and log-sum-exp over a given position list.  Everything is
quantised here from the bf16 inputs with this package's own quantisers; the
page layout does not change any value, so this module works on logical token
order (pools.py covers the paged layout on its own).
"""
from __future__ import annotations

from typing import Dict, Iterable

import numpy as np

from . import attention, formats, indexer, quant


class Oracle:
    def __init__(self, inp: Dict[str, np.ndarray]):
        self.inp = inp
        self._kcache: Dict[int, np.ndarray] = {}

    # -- indexer -----------------------------------------------------------
    def q_index(self, r: int) -> np.ndarray:
        codes, e8 = quant.mxfp8_quant(self.inp["q_idx"][r])        # [H_I, 128]
        return quant.mxfp8_dequant(codes, e8)

    def k_index(self, b: int) -> np.ndarray:
        if b not in self._kcache:
            st = int(self.inp["seq_starts"][b])
            L = int(self.inp["seq_lens"][b])
            codes, e8 = quant.mxfp8_quant(self.inp["k_idx"][st:st + L])
            self._kcache[b] = quant.mxfp8_dequant(codes, e8)
        return self._kcache[b]

    def scores(self, r: int) -> np.ndarray:
        b = int(self.inp["row_seq"][r])
        t = int(self.inp["row_pos"][r])
        w = self.inp["w"][r].astype(np.float64)
        return indexer.indexer_scores(self.q_index(r), self.k_index(b), w, t)

    def topk(self, r: int, K: int = None):
        K = int(self.inp["topk"]) if K is None else K
        I = self.scores(r)
        idx, sc = indexer.topk_select(I, K)
        return dict(scores=I, idx=idx, sel_scores=sc, kth=indexer.kth_score(I, K),
                    maxabs=float(np.abs(I).max()))

    def drop_cache(self):
        self._kcache.clear()

    # -- sparse attention ----------------------------------------------------
    def kv_rows(self, b: int, positions: np.ndarray):
        st = int(self.inp["seq_starts"][b])
        rec = quant.kv_quant(self.inp["kv"][st + np.asarray(positions, dtype=np.int64)])
        return quant.kv_dequant(rec)

    def sfa(self, r: int, idx: Iterable[int], scale: float = attention.DEFAULT_SCALE):
        idx = np.asarray(list(idx) if not isinstance(idx, np.ndarray) else idx)
        b = int(self.inp["row_seq"][r])
        valid = idx[idx >= 0]
        uniq, inv = np.unique(valid, return_inverse=True)
        lat, rope = self.kv_rows(b, uniq)
        q = formats.bf16_decode(self.inp["q_sfa"][r])
        return attention.sparse_attn(q, lat, rope, inv, scale)
