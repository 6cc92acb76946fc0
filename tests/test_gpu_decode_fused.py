"""dsa_decode_indexer_topk (the decode prolog folded into the indexer's
launches) against dsa_decode_prolog followed by dsa_indexer_topk, started
from identical caches whose new-token slots hold stale bytes: the same cache
bytes afterwards and bit-identical indices and scores; plus the Top-K rule
against the oracle on every row."""
import numpy as np
import pytest
import torch

from oracle.pipeline import Oracle
from sparse_attention_decode_topk_amd import ops, synth
from tests.dsa_state import DeviceState, bf16_tensor, check_topk_row, say, stale_caches

pytestmark = pytest.mark.gpu


def _run_both(st, inp, slots_np, K, tag):
    dev = st.dev
    R = st.R
    new_tok = inp["seq_starts"][inp["row_seq"]].astype(np.int64) + inp["row_pos"].astype(np.int64)
    k_new = bf16_tensor(inp["k_idx"][new_tok], dev)
    kv_new = bf16_tensor(inp["kv"][new_tok], dev)
    q_bf = bf16_tensor(inp["q_idx"], dev)
    slots = torch.from_numpy(slots_np).to(dev)
    kpa, kvpa = stale_caches(st, slots_np, 5)
    kpb, kvpb = kpa.clone(), kvpa.clone()
    # A: prolog, then the indexer
    q_fp8, q_e8 = ops.decode_prolog(q_bf, k_new, kv_new, slots, kpa, kvpa)
    a_idx, a_sc = ops.dsa_indexer_topk(q_fp8, q_e8, st.w, kpa, st.block_table, st.row_seq,
                                       st.row_pos, K)
    # B: the fused entry point
    b_idx, b_sc = ops.dsa_decode_indexer_topk(q_bf, st.w, k_new, kv_new, slots, kpb, kvpb,
                                              st.block_table, st.row_seq, st.row_pos, K)
    torch.cuda.synchronize()
    assert torch.equal(kpa, kpb), f"{tag}: K cache bytes differ"
    assert torch.equal(kvpa, kvpb), f"{tag}: KV cache bytes differ"
    assert torch.equal(a_idx, b_idx), f"{tag}: indices differ"
    assert torch.equal(a_sc, b_sc), f"{tag}: scores differ"
    say(f"[fused prolog] {tag}: caches, indices and scores bit-equal on {R} rows")
    return b_idx.cpu().numpy(), b_sc.cpu().numpy()


@pytest.mark.parametrize("cfg", ["decode_8k_needles", "decode_ragged_b32", "decode_128k_b8"])
def test_fused_prolog_matches_prolog_then_indexer(need_gpu, cfg):
    inp = synth.make(cfg)
    st = DeviceState(inp)
    new_tok = inp["seq_starts"][inp["row_seq"]].astype(np.int64) + inp["row_pos"].astype(np.int64)
    slots = inp["slot_mapping"][new_tok].astype(np.int64)
    gi, gs = _run_both(st, inp, slots, st.topk, cfg)
    o = Oracle(inp)
    for r in range(st.R):
        check_topk_row(gi[r], gs[r], o.topk(r), st.topk, int(inp["row_pos"][r]))
    o.drop_cache()


def test_fused_prolog_edge_rows(need_gpu):
    """20 indexer heads (not a multiple of 16), Top-K of 1 and 300, rows
    whose new token sits at offset 0 or 63 of a page, and rows with no new
    token (slot -1 and a slot past the pool)."""
    lens = np.array([65, 128, 1000, 4096, 3333, 64], dtype=np.int32)
    B = len(lens)
    cfg = synth.Config(96, "fused_edge", batch=B, h_index=20, h_attn=16, topk=300,
                       ragged=(int(lens.min()), int(lens.max())))
    rng = np.random.default_rng(19)
    bt, slots_all, starts, npages = synth.page_tables(cfg, lens, rng)
    inp = dict(seq_lens=lens, block_table=bt, slot_mapping=slots_all, seq_starts=starts,
               total_pages=np.int64(npages), topk=np.int32(300),
               row_seq=np.arange(B, dtype=np.int32), row_pos=(lens - 1).astype(np.int32),
               q_idx=synth.f32_to_bf16_bits(rng.standard_normal((B, 20, 128)).astype(np.float32)),
               k_idx=synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 128)).astype(np.float32)),
               w=(rng.standard_normal((B, 20)) / np.sqrt(20)).astype(np.float32),
               q_sfa=synth.f32_to_bf16_bits(rng.standard_normal((B, 16, 576)).astype(np.float32)),
               kv=synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 576)).astype(np.float32)))
    st = DeviceState(inp)
    new_tok = starts.astype(np.int64) + (lens - 1).astype(np.int64)
    slots = slots_all[new_tok].astype(np.int64)
    slots[2] = -1
    slots[4] = npages * 64 + 5
    for K in (300, 1):
        _run_both(st, inp, slots, K, f"edge rows K={K}")


def _subset_matches_batch(st, inp, slots_np, K, nsub, tag):
    """The first nsub rows launched alone (few enough units for the
    work-group scan, four waves on every unit) against the same rows inside
    the whole batch (enough units for the one-wave-per-unit scan): indices
    and scores bit-equal, for dsa_indexer_topk and dsa_decode_indexer_topk."""
    dev = st.dev
    new_tok = inp["seq_starts"][inp["row_seq"]].astype(np.int64) + inp["row_pos"].astype(np.int64)
    k_new = bf16_tensor(inp["k_idx"][new_tok], dev)
    kv_new = bf16_tensor(inp["kv"][new_tok], dev)
    q_bf = bf16_tensor(inp["q_idx"], dev)
    slots = torch.from_numpy(slots_np).to(dev)
    n = nsub
    a_idx, a_sc = ops.dsa_indexer_topk(st.q_fp8, st.q_e8m0, st.w, st.k_pool, st.block_table,
                                       st.row_seq, st.row_pos, K)
    s_idx, s_sc = ops.dsa_indexer_topk(st.q_fp8[:n], st.q_e8m0[:n], st.w[:n], st.k_pool,
                                       st.block_table, st.row_seq[:n], st.row_pos[:n], K)
    kpa, kvpa = st.k_pool.clone(), st.kv_pool.clone()
    b_idx, b_sc = ops.dsa_decode_indexer_topk(q_bf, st.w, k_new, kv_new, slots, kpa, kvpa,
                                              st.block_table, st.row_seq, st.row_pos, K)
    kpb, kvpb = st.k_pool.clone(), st.kv_pool.clone()
    c_idx, c_sc = ops.dsa_decode_indexer_topk(q_bf[:n], st.w[:n], k_new[:n], kv_new[:n], slots[:n],
                                              kpb, kvpb, st.block_table, st.row_seq[:n],
                                              st.row_pos[:n], K)
    torch.cuda.synchronize()
    assert torch.equal(a_idx[:n], s_idx) and torch.equal(a_sc[:n], s_sc), f"{tag}: unfused"
    assert torch.equal(b_idx[:n], c_idx) and torch.equal(b_sc[:n], c_sc), f"{tag}: fused"
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc), f"{tag}: fused vs unfused"
    say(f"[scan forms] {tag}: {n} rows alone equal to the same rows in {st.R}")


def test_wave_scan_matches_workgroup_scan(need_gpu):
    """Ragged decode (64 heads, 32 rows of 4K-64K: 2048 units by the block
    table's width) against its first 4 rows (256 units)."""
    inp = synth.make("decode_ragged_b32")
    st = DeviceState(inp)
    new_tok = inp["seq_starts"] + inp["seq_lens"] - 1
    _subset_matches_batch(st, inp, inp["slot_mapping"][new_tok].astype(np.int64), st.topk, 4,
                          "ragged decode")


def test_wave_scan_edge_rows(need_gpu):
    """160 rows of 20 indexer heads (a partial head tile), lengths 1..4096
    with new tokens at page offsets 0 and 63, rows without a new token (slot
    -1, a slot past the pool) and Top-K of 300 and 1: the batch takes the
    one-wave-per-unit scan (640 units), its first 8 rows the work-group scan."""
    rng = np.random.default_rng(23)
    B = 160
    lens = rng.integers(1, 4097, B).astype(np.int32)
    lens[:6] = [65, 128, 1000, 4096, 3333, 64]
    lens[7] = 1
    cfg = synth.Config(97, "wave_edge", batch=B, h_index=20, h_attn=16, topk=300,
                       ragged=(int(lens.min()), int(lens.max())))
    bt, slots_all, starts, npages = synth.page_tables(cfg, lens, rng)
    assert bt.shape[1] == 64
    inp = dict(seq_lens=lens, block_table=bt, slot_mapping=slots_all, seq_starts=starts,
               total_pages=np.int64(npages), topk=np.int32(300),
               row_seq=np.arange(B, dtype=np.int32), row_pos=(lens - 1).astype(np.int32),
               q_idx=synth.f32_to_bf16_bits(rng.standard_normal((B, 20, 128)).astype(np.float32)),
               k_idx=synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 128)).astype(np.float32)),
               w=(rng.standard_normal((B, 20)) / np.sqrt(20)).astype(np.float32),
               q_sfa=synth.f32_to_bf16_bits(rng.standard_normal((B, 16, 576)).astype(np.float32)),
               kv=synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 576)).astype(np.float32)))
    st = DeviceState(inp)
    new_tok = starts.astype(np.int64) + (lens - 1).astype(np.int64)
    slots = slots_all[new_tok].astype(np.int64)
    slots[2] = -1
    slots[4] = npages * 64 + 5
    slots[100] = -1
    for K in (300, 1):
        _subset_matches_batch(st, inp, slots, K, 8, f"edge rows K={K}")
    # the batch against the oracle on a few rows, the no-new-token ones included
    idx, sc = ops.dsa_decode_indexer_topk(
        bf16_tensor(inp["q_idx"], st.dev), st.w, bf16_tensor(inp["k_idx"][new_tok], st.dev),
        bf16_tensor(inp["kv"][new_tok], st.dev), torch.from_numpy(slots).to(st.dev),
        st.k_pool.clone(), st.kv_pool.clone(), st.block_table, st.row_seq, st.row_pos, 300)
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    o = Oracle(inp)
    for r in (0, 2, 3, 4, 7, 100, B - 1):
        check_topk_row(gi[r], gs[r], o.topk(r), 300, int(lens[r] - 1))



def test_fused_prolog_more_rows_than_one_launch(need_gpu):
    """1100 rows (sequences of 1..300 tokens, 64 indexer heads, Top-K 64)
    take two launches of at most 1024 rows: each launch keeps its quantised
    queries in the workspace region sized for one launch.  The fused entry
    point against the prolog then the indexer."""
    rng = np.random.default_rng(61)
    B, H_I, K = 1100, 64, 64
    lens = rng.integers(1, 301, B).astype(np.int32)
    cfg = synth.Config(99, "fused_many_rows", batch=B, h_index=H_I, h_attn=16, topk=K,
                       ragged=(int(lens.min()), int(lens.max())))
    bt, slots_all, starts, npages = synth.page_tables(cfg, lens, rng)
    inp = dict(seq_lens=lens, block_table=bt, slot_mapping=slots_all, seq_starts=starts,
               total_pages=np.int64(npages), topk=np.int32(K),
               row_seq=np.arange(B, dtype=np.int32), row_pos=(lens - 1).astype(np.int32),
               q_idx=synth.f32_to_bf16_bits(rng.standard_normal((B, H_I, 128)).astype(np.float32)),
               k_idx=synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 128)).astype(np.float32)),
               w=(rng.standard_normal((B, H_I)) / np.sqrt(H_I)).astype(np.float32),
               q_sfa=synth.f32_to_bf16_bits(rng.standard_normal((B, 16, 576)).astype(np.float32)),
               kv=synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 576)).astype(np.float32)))
    st = DeviceState(inp)
    new_tok = starts.astype(np.int64) + (lens - 1).astype(np.int64)
    _run_both(st, inp, slots_all[new_tok].astype(np.int64), K, "1100 rows")
