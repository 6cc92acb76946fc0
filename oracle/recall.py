"""Synthetic Top-K recall of the MXFP8 Lightning Indexer.

Test infrastructure only (see package docstring).

"Kimi K3.1 Pro Inference Acceleration" (page 3), section "Full MXFP8
Quantization of the Lightning Indexer": quantising the indexer's q and k to
MXFP8 (E4M3, one E8M0 scale per 32 elements) is reported to cost under 0.1%
of accuracy on the page's long-context benchmark.  That benchmark and the
model weights are not available here, so this module measures the quantity
the claim rests on, on the seeded synthetic inputs: how far the Top-K
positions chosen from MXFP8 scores (this package's fp64 indexer on the
dequantised MXFP8 q and k; the HIP path computes the same scores in fp32 on
the scaled fp8 MFMA, within 1e-4 of the row's largest score, and may swap
positions whose scores lie that close to the K-th) agree with the Top-K of the same
indexer evaluated in fp64 on the unquantised bf16 q and k.

Per query row r with history t (n = min(K, t + 1) positions kept):
  recall       |TopK_mx ∩ TopK_ref| / n
  mass recall  sum of I_ref over TopK_mx / sum of I_ref over TopK_ref (how
               much of the reference selection's score the quantised
               selection keeps; 1 when the sets agree).  Read as a fraction
               only where the reference selection's scores are positive: the
               head weights may be negative, and a row whose K-th largest
               score is below zero makes the ratio depend on where zero lies
  score loss   (mean of I_ref over TopK_ref - mean of I_ref over TopK_mx) /
               standard deviation of I_ref over the row's history: the
               average score given up per kept position, in units of the
               row's spread; unchanged by a shift or a positive scale of the
               scores, never negative (TopK_ref has the largest sum), 0 when
               the sets agree
  needles      of the planted needle positions that the reference keeps,
               the fraction the MXFP8 selection keeps too

Run as a module (python -m oracle.recall [config ...]) for the table of the
synthetic workloads.
"""
from __future__ import annotations

import os
import sys
import time
from typing import Dict, Iterable, Optional

import numpy as np

from . import formats, indexer
from .pipeline import Oracle


def reference_scores(inp: Dict[str, np.ndarray], r: int) -> np.ndarray:
    """The indexer on the unquantised bf16 q and k, in fp64 (no MXFP8)."""
    b = int(inp["row_seq"][r])
    t = int(inp["row_pos"][r])
    st = int(inp["seq_starts"][b])
    q = formats.bf16_decode(inp["q_idx"][r])                    # [H_I, 128]
    k = formats.bf16_decode(inp["k_idx"][st:st + t + 1])        # [t+1, 128]
    return indexer.indexer_scores(q, k, inp["w"][r].astype(np.float64), t)


def row_recall(I_mx: np.ndarray, I_ref: np.ndarray, K: int,
               needles: Optional[np.ndarray] = None) -> Dict[str, float]:
    n = min(K, len(I_ref))
    sel_mx = indexer.topk_order(I_mx)[:n]
    sel_ref = indexer.topk_order(I_ref)[:n]
    common = np.intersect1d(sel_mx, sel_ref).size
    out = dict(recall=common / n)
    ref_mass = float(I_ref[sel_ref].sum())
    out["mass_recall"] = float(I_ref[sel_mx].sum()) / ref_mass if ref_mass != 0.0 else 1.0
    sd = float(I_ref.std())
    gap = float(I_ref[sel_ref].sum() - I_ref[sel_mx].sum()) / n
    out["score_loss"] = gap / sd if sd > 0.0 else 0.0
    if needles is not None and len(needles):
        kept_ref = np.intersect1d(needles, sel_ref)
        out["needles_ref"] = int(kept_ref.size)
        out["needle_recall"] = (np.intersect1d(kept_ref, sel_mx).size / kept_ref.size
                                if kept_ref.size else 1.0)
    return out


def study(inp: Dict[str, np.ndarray], rows: Optional[Iterable[int]] = None) -> Dict[str, object]:
    """Per-row recall figures of one input set and their mean / minimum."""
    K = int(inp["topk"])
    o = Oracle(inp)
    rows = list(range(len(inp["row_seq"]))) if rows is None else list(rows)
    per = []
    for r in rows:
        needles = None
        if "needles" in inp:
            b = int(inp["row_seq"][r])
            st = int(inp["seq_starts"][b])
            t = int(inp["row_pos"][r])
            loc = inp["needles"] - st
            needles = loc[(loc >= 0) & (loc <= t)]
        per.append(row_recall(o.scores(r), reference_scores(inp, r), K, needles))
    o.drop_cache()
    summary = dict(rows=len(per),
                   recall_mean=float(np.mean([p["recall"] for p in per])),
                   recall_min=float(np.min([p["recall"] for p in per])),
                   mass_recall_min=float(np.min([p["mass_recall"] for p in per])),
                   score_loss_max=float(np.max([p["score_loss"] for p in per])))
    if per and "needle_recall" in per[0]:
        summary["needles_in_ref_topk"] = int(sum(p["needles_ref"] for p in per))
        summary["needle_recall_min"] = float(np.min([p["needle_recall"] for p in per]))
    summary["per_row"] = per
    return summary


def _rows_for(name: str, R: int):
    if R <= 8:
        return range(R)
    return np.linspace(0, R - 1, 8).astype(int)   # eight rows spread over the config


def main(argv) -> int:
    from sparse_attention_decode_topk_amd import synth    # seeded inputs only
    names = argv or ["decode_8k_needles", "decode_ragged_b32", "decode_128k_b8",
                     "prefill_chunk_8k_of_128k"]
    print(f"{'config':28s} {'rows':>4s} {'recall mean':>11s} {'recall min':>10s} "
          f"{'mass min':>9s} {'loss max':>9s} {'needles':>8s} {'secs':>6s}")
    for name in names:
        cfg = synth.config(name)
        R = len(synth.make(cfg, with_sfa=False, with_index=False)["row_seq"])
        rows = list(_rows_for(name, R))
        t0 = time.perf_counter()
        inp = synth.make(cfg, with_sfa=False, row_subset=rows)
        s = study(inp)
        nd = ("%d/%.3f" % (s["needles_in_ref_topk"], s["needle_recall_min"])
              if "needle_recall_min" in s else "-")
        print(f"{name:28s} {s['rows']:4d} {s['recall_mean']:11.4f} {s['recall_min']:10.4f} "
              f"{s['mass_recall_min']:9.5f} {s['score_loss_max']:9.5f} {nd:>8s} {time.perf_counter() - t0:6.1f}", flush=True)
    return 0


if __name__ == "__main__":
    os.environ.setdefault("OMP_NUM_THREADS", str(len(os.sched_getaffinity(0))))
    sys.exit(main(sys.argv[1:]))
