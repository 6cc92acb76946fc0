"""Parity over seeded random shapes of the decode path and of prefill
chunks.  Decode: batch, ragged history lengths, indexer and attention head
counts (1 and counts that are not multiples of 16 included), Top-K sizes
and query rows per sequence are drawn per case.  Each case runs the per-row indexer, then the fused decode
entry point (one row per sequence) or the multi-query entry point (several),
both bit-equal to the per-row one, and SFA over the GPU's own indices:
  - a row with no more positions than K must select every position;
  - a longer row of at least 16 positions passes the Top-K rule against the
    oracle; a shorter one is checked for a valid selection (the scaled FP8
    MFMA's accumulation error is bounded by the sum of |q_i k_i|, not by the
    row's largest score, so a bar relative to that score does not hold for
    rows of a handful of positions);
  - SFA within 1e-3 * max|oracle out|, lse within 1e-3."""
import numpy as np
import pytest
import torch

from oracle.pipeline import Oracle
from sparse_attention_decode_topk_amd import ops, synth
from tests.dsa_state import DeviceState, bf16_tensor, check_topk_row, say

pytestmark = pytest.mark.gpu

MIN_POSITIONS = 16
N_CASES = 12


def _case(i):
    rng = np.random.default_rng(500 + i)
    lo = int(rng.integers(4, 2000))
    hi = lo + int(rng.integers(0, 6000))
    return synth.Config(
        300 + i, f"random_{i}", batch=int(rng.integers(1, 7)),
        h_index=int(rng.choice([1, 3, 16, 20, 33, 64])),
        h_attn=int(rng.choice([1, 5, 16, 40, 100, 128])),
        topk=int(rng.choice([1, 17, 64, 300, 1000, 2048])),
        ragged=(lo, hi), q_per_seq=int(rng.choice([1, 1, 2, 4])))


# one head on both sides and histories from 4 tokens, most no longer than K
EXTRA = [synth.Config(320, "one_head", batch=3, h_index=1, h_attn=1, topk=2048, ragged=(4, 3000))]
CASES = [_case(i) for i in range(N_CASES)] + EXTRA


def _check_row(gi, gs, o, r, K, t):
    n = min(K, t + 1)
    if t + 1 <= K:
        assert np.array_equal(gi[:n], np.arange(n)), f"row {r}: every position"
        assert np.all(gi[n:] == -1), f"row {r}: padding"
        return 0
    if t + 1 >= MIN_POSITIONS:
        return check_topk_row(gi, gs, o.topk(r), K, t)
    sel = gi[:n]
    assert np.all(gi[n:] == -1) and np.all(sel >= 0) and np.all(sel <= t), f"row {r}"
    assert np.all(np.diff(sel) > 0), f"row {r}: ascending and unique"
    return 0


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_shape(need_gpu, case):
    cfg = CASES[case]
    inp = synth.make(cfg)
    st = DeviceState(inp)
    K, qps = st.topk, cfg.q_per_seq
    say(f"[random] {cfg.name}: B={cfg.batch} R={st.R} lens={cfg.ragged} H_I={cfg.h_index} "
        f"H={cfg.h_attn} K={K} q_per_seq={qps}")
    a_idx, a_sc = st.indexer()
    if qps == 1:
        new_tok = inp["seq_starts"][inp["row_seq"]].astype(np.int64) + inp["row_pos"].astype(np.int64)
        slots = torch.from_numpy(inp["slot_mapping"][new_tok].astype(np.int64)).cuda()
        kp, kvp = st.k_pool.clone(), st.kv_pool.clone()
        b_idx, b_sc = ops.dsa_decode_indexer_topk(
            bf16_tensor(inp["q_idx"], st.dev), st.w, bf16_tensor(inp["k_idx"][new_tok], st.dev),
            bf16_tensor(inp["kv"][new_tok], st.dev), slots, kp, kvp, st.block_table, st.row_seq,
            st.row_pos, K)
        torch.cuda.synchronize()
        # the new tokens' cache slots already hold their keys and records
        assert torch.equal(kp, st.k_pool) and torch.equal(kvp, st.kv_pool)
    else:
        b_idx, b_sc = ops.dsa_indexer_topk_mq(st.q_fp8, st.q_e8m0, st.w, st.k_pool, st.block_table,
                                              st.row_seq, st.row_pos, qps, K)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)
    out, lse = st.sfa(a_idx)
    torch.cuda.synchronize()
    gi, gs = a_idx.cpu().numpy(), a_sc.cpu().numpy()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    o = Oracle(inp)
    pos = inp["row_pos"].astype(np.int64)
    swaps = sum(_check_row(gi[r], gs[r], o, r, K, int(pos[r])) for r in range(st.R))
    ref_o, ref_l = zip(*(o.sfa(r, gi[r]) for r in range(st.R)))
    ref_o, ref_l = np.stack(ref_o), np.stack(ref_l)
    err = np.abs(out - ref_o).max()
    bar = 1e-3 * np.abs(ref_o).max()
    say(f"[random] {cfg.name}: selection valid on {st.R} rows ({swaps} tolerated swaps); "
        f"SFA max err {err:.3g} vs bar {bar:.3g}")
    assert err <= bar
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(np.abs(lse[fin] - ref_l[fin]) <= 1e-3)
    o.drop_cache()


def _chunk_case(i):
    rng = np.random.default_rng(700 + i)
    L = int(rng.integers(500, 20000))
    count = int(rng.integers(1, 300))
    return synth.Config(
        340 + i, f"random_chunk_{i}", batch=1, ctx=L, rows=(L - count, count),
        h_index=int(rng.choice([1, 5, 16, 40, 64])), h_attn=int(rng.choice([3, 16, 32, 77, 128])),
        topk=(64, 2048, 1, 500, 2048, 300)[i])


CHUNK_CASES = [_chunk_case(i) for i in range(6)]


@pytest.mark.parametrize("case", range(len(CHUNK_CASES)))
def test_random_prefill_chunk(need_gpu, case):
    """The last rows of one sequence as a prefill chunk: the sequence entry
    point bit-equal to the per-row one, the selection rules above on every
    row, and SFA over the GPU's own indices."""
    cfg = CHUNK_CASES[case]
    inp = synth.make(cfg)
    st = DeviceState(inp)
    K = st.topk
    say(f"[random] {cfg.name}: L={cfg.ctx} rows={cfg.rows} H_I={cfg.h_index} H={cfg.h_attn} K={K}")
    a_idx, a_sc = st.indexer()
    b_idx, b_sc = ops.dsa_indexer_topk_seq(st.q_fp8, st.q_e8m0, st.w, st.k_pool,
                                           st.block_table[0].contiguous(), st.row_pos, K)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)
    out, lse = st.sfa(b_idx)
    torch.cuda.synchronize()
    gi, gs = b_idx.cpu().numpy(), b_sc.cpu().numpy()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    o = Oracle(inp)
    pos = inp["row_pos"].astype(np.int64)
    rows = range(st.R) if st.R <= 40 else sorted(set(range(0, st.R, st.R // 20)) | {st.R - 1})
    swaps = sum(_check_row(gi[r], gs[r], o, r, K, int(pos[r])) for r in rows)
    ref_o, ref_l = zip(*(o.sfa(r, gi[r]) for r in rows))
    ref_o, ref_l = np.stack(ref_o), np.stack(ref_l)
    got_o, got_l = out[list(rows)], lse[list(rows)]
    err = np.abs(got_o - ref_o).max()
    bar = 1e-3 * np.abs(ref_o).max()
    say(f"[random] {cfg.name}: {len(rows)} rows checked ({swaps} tolerated swaps); "
        f"SFA max err {err:.3g} vs bar {bar:.3g}")
    assert err <= bar
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(got_l), fin)
    assert np.all(np.abs(got_l[fin] - ref_l[fin]) <= 1e-3)
    o.drop_cache()
