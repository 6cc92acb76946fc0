"""Parity on further seeds: the shapes of the tiny prefill, decode 8K with
needles and ragged decode workloads drawn from other generator seeds.  The
GPU indexer's selection passes the Top-K rule against the oracle, and SFA
over the GPU's own indices matches the oracle's attention over those same
indices (max abs error <= 1e-3 * max|oracle out|, lse within 1e-3).

In the tiny prefill shape the indexer rule is applied to rows with at least
16 positions: the scaled FP8 MFMA's accumulation error scales with the sum
of |q_i k_i| products, not with the row's largest score, so a row of two or
three positions can sit outside a bar relative to its own max|I| on every
path (such rows are covered by the bit-equality tests between entry
points)."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle.pipeline import Oracle
from sparse_attention_decode_topk_amd import synth
from tests.dsa_state import DeviceState, check_topk_row, say

pytestmark = pytest.mark.gpu

MIN_POSITIONS = 16


@pytest.mark.parametrize("base,seed", [("tiny_prefill", 201), ("tiny_prefill", 202),
                                       ("decode_8k_needles", 203), ("decode_ragged_b32", 204)])
def test_other_seeds_end_to_end(need_gpu, base, seed):
    cfg = dataclasses.replace(synth.CONFIGS[base], index=seed, name=f"{base}_seed{seed}")
    inp = synth.make(cfg)
    st = DeviceState(inp)
    say(f"[seeds] {cfg.name}: R={st.R}")
    idx, sc = st.indexer()
    out, lse = st.sfa(idx)
    torch.cuda.synchronize()
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    o = Oracle(inp)
    pos = inp["row_pos"].astype(np.int64)
    checked = swaps = 0
    for r in range(st.R):
        if pos[r] + 1 >= MIN_POSITIONS:
            swaps += check_topk_row(gi[r], gs[r], o.topk(r), st.topk, int(pos[r]))
            checked += 1
    ref_o, ref_l = zip(*(o.sfa(r, gi[r]) for r in range(st.R)))
    ref_o, ref_l = np.stack(ref_o), np.stack(ref_l)
    err = np.abs(out - ref_o).max()
    bar = 1e-3 * np.abs(ref_o).max()
    say(f"[seeds] {cfg.name}: {checked} rows pass the Top-K rule ({swaps} tolerated swaps); "
        f"SFA max err {err:.3g} vs bar {bar:.3g}")
    assert err <= bar
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(np.abs(lse[fin] - ref_l[fin]) <= 1e-3)
    o.drop_cache()
