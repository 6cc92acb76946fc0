"""GPU parity of the fused indexer + Top-K against the oracle.

Scores: within 1e-4 * max|I| of the fp64 oracle.  Selection: the pass rule
of check_topk_row; and, bit-exactly, the kernel's selection equals the exact
Top-K (score desc, position asc) of the kernel's own score rows."""
import functools

import numpy as np
import pytest
import torch

from oracle.pipeline import Oracle
from sparse_attention_decode_topk_amd import ops, synth
from tests.dsa_state import DeviceState, check_topk_row, exact_topk_of, say

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=2)
def state(cfg):
    say(f"[state] building {cfg}")
    return DeviceState(synth.make(cfg, with_sfa=False), with_sfa=False)


def _rows_for(cfg, R):
    if R <= 64:
        return list(range(R))
    rng = np.random.default_rng(1)
    return sorted(set([0, 1, R - 1] + rng.choice(R, 24, replace=False).tolist()))


@pytest.mark.parametrize("cfg", ["tiny_prefill", "decode_8k_needles", "decode_ragged_b32",
                                 "decode_128k_b8"])
def test_indexer_parity(need_gpu, cfg):
    st = state(cfg)
    say(f"[indexer] {cfg} R={st.R} topk={st.topk}")
    idx, sc = st.indexer()
    scores = st.scores()
    torch.cuda.synchronize()
    idx, sc, scores = idx.cpu().numpy(), sc.cpu().numpy(), scores.cpu().numpy()
    o = Oracle(st.inp)
    rows = list(range(st.R)) if cfg == "tiny_prefill" else _rows_for(cfg, st.R)
    swaps = 0
    worst = 0.0   # largest score error as a fraction of max|I|
    for r in rows:
        t = int(st.inp["row_pos"][r])
        ora = o.topk(r)
        # scores of every causal position
        gs = scores[r, :t + 1]
        err = np.abs(gs.astype(np.float64) - ora["scores"])
        worst = max(worst, float(err.max()) / ora["maxabs"] if ora["maxabs"] > 0 else 0.0)
        assert np.all(err <= 1e-4 * ora["maxabs"]), f"row {r} scores"
        assert np.all(np.isneginf(scores[r, t + 1:]))
        swaps += check_topk_row(idx[r], sc[r], ora, st.topk, t)
        # bit-exact: selection == exact Top-K of the kernel's own scores
        assert np.array_equal(idx[r][:min(st.topk, t + 1)], exact_topk_of(scores[r], st.topk)), f"row {r}"
    o.drop_cache()
    say(f"[indexer] {cfg}: {len(rows)} rows ok, {swaps} tolerated swaps, "
        f"max score error {worst:.2e} of max|I| (bar 1e-4)")


def test_indexer_deterministic_and_workspace_reuse(need_gpu):
    st = state("decode_8k_needles")
    ws = ops.indexer_workspace(st.R, st.block_table.shape[1], st.H_I, st.topk)
    a = st.indexer(workspace=ws)
    b = st.indexer(workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    # work counters re-armed for the next call, no page-id error reported
    w = ws.view(torch.int32).cpu().numpy()
    assert w[0] == 0 and w[1] == 0 and (w[2] & 4) == 0


def test_needles_are_selected(need_gpu):
    st = state("decode_8k_needles")
    idx, _ = st.indexer()
    I = st.scores()[0].cpu().numpy()
    sel = set(idx[0].cpu().numpy().tolist())
    nd = st.inp["needles"]
    # every needle whose base score is positive scores x4 and is kept
    kth = np.sort(I[np.isfinite(I)])[::-1][st.topk - 1]
    strong = [n for n in nd if I[n] > kth]
    assert strong and all(n in sel for n in strong)


def test_topk_edge_cases(need_gpu):
    """topk = 1, topk larger than the history, H_I not a multiple of 16,
    and rows with t < 0, on a small ragged batch."""
    say("[indexer] edge cases")
    cfg = synth.Config(90, "edge", batch=3, h_index=20, h_attn=16, topk=1, ragged=(1, 300))
    lens = np.array([1, 300, 129], dtype=np.int32)
    rng = np.random.default_rng(3)
    bt, slots, starts, npages = synth.page_tables(cfg, lens, rng)
    R = 5
    inp = dict(seq_lens=lens, block_table=bt, slot_mapping=slots, seq_starts=starts,
               total_pages=np.int64(npages), topk=np.int32(1),
               row_seq=np.array([0, 1, 1, 2, 1], dtype=np.int32),
               row_pos=np.array([0, 299, 63, 128, 5], dtype=np.int32),
               q_idx=synth.f32_to_bf16_bits(rng.standard_normal((R, 20, 128)).astype(np.float32)),
               k_idx=synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 128)).astype(np.float32)),
               w=(rng.standard_normal((R, 20)) / np.sqrt(20)).astype(np.float32))
    st = DeviceState(inp, with_sfa=False)
    o = Oracle(inp)
    scores = st.scores().cpu().numpy()
    for K in (1, 7, 64, 130, 2048):
        idx, sc = st.indexer(topk=K)
        idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
        for r in range(R):
            t = int(inp["row_pos"][r])
            ora = o.topk(r, K)
            check_topk_row(idx[r], sc[r], ora, K, t)
            assert np.array_equal(idx[r][:min(K, t + 1)], exact_topk_of(scores[r], K))
    # a row with no history: t = -1 -> all -1
    inp2 = dict(inp, row_pos=np.array([-1, 299, 0, 128, 5], dtype=np.int32))
    st2 = DeviceState(inp2, with_sfa=False)
    idx, sc = st2.indexer(topk=16)
    assert np.all(idx[0].cpu().numpy() == -1) and np.all(np.isneginf(sc[0].cpu().numpy()))
    assert idx[2].cpu().numpy()[0] == 0 and np.all(idx[2].cpu().numpy()[1:] == -1)


def test_exact_ties_lower_position_wins(need_gpu):
    """All-zero queries give score 0 everywhere: the K lowest positions win."""
    say("[indexer] exact ties")
    inp = dict(synth.make("decode_8k_needles", with_sfa=False))
    inp["q_idx"] = np.zeros_like(inp["q_idx"])
    st = DeviceState(inp, with_sfa=False)
    idx, sc = st.indexer()
    assert np.array_equal(idx[0].cpu().numpy(), np.arange(st.topk))
    assert np.all(sc[0].cpu().numpy() == 0)


def test_page_permutation_invariance(need_gpu):
    say("[indexer] page permutation")
    inp = synth.make("decode_ragged_b32", with_sfa=False)
    a = DeviceState(inp, with_sfa=False)
    ia, sa = a.indexer()
    ia, sa = ia.cpu().numpy(), sa.cpu().numpy()
    del a
    lens = inp["seq_lens"]
    bt2 = synth.rotate_pages(inp["block_table"], lens, int(inp["total_pages"]), seed=11)
    slots2 = np.concatenate([bt2[b, np.arange(lens[b]) // 64].astype(np.int64) * 64
                             + np.arange(lens[b]) % 64 for b in range(len(lens))])
    b = DeviceState(dict(inp, block_table=bt2, slot_mapping=slots2), with_sfa=False)
    ib, sb = b.indexer()
    assert np.array_equal(ia, ib.cpu().numpy()) and np.array_equal(sa, sb.cpu().numpy())


def test_chunked_prefill_every_64th_row(need_gpu):
    """8192 query rows against a 131072-token cache through the per-row
    entry point; every 64th row (and the last) against the oracle."""
    say("[indexer] chunked prefill 8192 rows")
    inp = synth.make("prefill_chunk_8k_of_128k", with_sfa=False)
    st = DeviceState(inp, with_sfa=False)
    idx, sc = st.indexer()
    torch.cuda.synchronize()
    o = Oracle(inp)
    rows = sorted(set(range(0, 8192, 64)) | {8191})
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    swaps = 0
    for r in rows:
        t = int(inp["row_pos"][r])
        swaps += check_topk_row(idx[r], sc[r], o.topk(r), st.topk, t)
    say(f"[indexer] chunked prefill: {len(rows)} rows ok ({swaps} tolerated swaps)")


def test_block_table_width_not_a_multiple_of_16(need_gpu):
    """Block tables of 129, 135 and 98 pages (the last 16-page unit is 1, 7
    or 2 pages wide): the select's wide layouts read a row's last unit as
    if it were full, and must read nothing past the row's candidate region
    (the last row's region ends the workspace).  Rows: a full-width row, a
    ragged mix, and a launch whose only row is the last of the table."""
    say("[indexer] block-table widths 129, 135, 98")
    rng = np.random.default_rng(17)
    for lens in (np.array([4000, 8256], dtype=np.int32),
                 np.array([8600, 1200, 300, 8640], dtype=np.int32),
                 np.array([6250], dtype=np.int32)):
        B = len(lens)
        cfg = synth.Config(95, "width", batch=B, h_index=64, h_attn=16, topk=2048,
                           ragged=(int(lens.min()), int(lens.max())))
        bt, slots, starts, npages = synth.page_tables(cfg, lens, rng)
        assert bt.shape[1] % 16 != 0
        inp = dict(seq_lens=lens, block_table=bt, slot_mapping=slots, seq_starts=starts,
                   total_pages=np.int64(npages), topk=np.int32(2048),
                   row_seq=np.arange(B, dtype=np.int32), row_pos=(lens - 1).astype(np.int32),
                   q_idx=synth.f32_to_bf16_bits(rng.standard_normal((B, 64, 128)).astype(np.float32)),
                   k_idx=synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 128)).astype(np.float32)),
                   w=(rng.standard_normal((B, 64)) / 8).astype(np.float32))
        st = DeviceState(inp, with_sfa=False)
        o = Oracle(inp)
        scores = st.scores().cpu().numpy()
        for K in (2048, 500):
            ws = ops.indexer_workspace(B, st.block_table.shape[1], st.H_I, K)
            idx, sc = st.indexer(topk=K, workspace=ws)
            idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
            for r in range(B):
                t = int(inp["row_pos"][r])
                check_topk_row(idx[r], sc[r], o.topk(r, K), K, t)
                assert np.array_equal(idx[r][:min(K, t + 1)], exact_topk_of(scores[r], K)), f"row {r} K={K}"
        o.drop_cache()


def test_concentrated_topk_takes_exact_fallback(need_gpu):
    """All head weights positive and the keys of positions 3000..5099 scaled
    by 8: every Top-K position lies in that range, so the unit covering
    3072..4095 holds far more than its quota of the Top-K.  The finisher must
    notice and rescore it; the result still follows the pass rule, the kernel's
    selection equals the exact Top-K of its own scores, and the workspace
    reports that the rescore path ran."""
    say("[indexer] concentrated Top-K (rescore path)")
    inp = dict(synth.make("decode_8k_needles", with_sfa=False))
    inp["w"] = np.abs(inp["w"])
    k = inp["k_idx"].copy()
    k[3000:5100] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(k[3000:5100]) * np.float32(8))
    inp["k_idx"] = k
    st = DeviceState(inp, with_sfa=False)
    ws = ops.indexer_workspace(st.R, st.block_table.shape[1], st.H_I, st.topk)
    idx, sc = st.indexer(workspace=ws)
    scores = st.scores().cpu().numpy()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    flags = int(ws.view(torch.int32)[2].item())
    assert flags & 8, "the rescore path was expected to run"
    o = Oracle(inp)
    ora = o.topk(0)
    t = int(inp["row_pos"][0])
    check_topk_row(idx[0], sc[0], ora, st.topk, t)
    assert np.array_equal(idx[0], exact_topk_of(scores[0], st.topk))
    assert np.sum((idx[0] >= 3000) & (idx[0] < 5100)) > 1900


def _seq_topk(st, q_fp8=None, q_e8m0=None, w=None, row_pos=None, topk=None, workspace=None):
    seqs = np.unique(st.inp["row_seq"])
    assert len(seqs) == 1, "one sequence"
    bt_row = st.block_table[int(seqs[0])].contiguous()
    return ops.dsa_indexer_topk_seq(st.q_fp8 if q_fp8 is None else q_fp8,
                                    st.q_e8m0 if q_e8m0 is None else q_e8m0,
                                    st.w if w is None else w, st.k_pool, bt_row,
                                    st.row_pos if row_pos is None else row_pos,
                                    st.topk if topk is None else topk, workspace=workspace)


@pytest.mark.parametrize("cfg", ["tiny_prefill", "decode_8k_needles", "prefill_chunk_8k_of_128k"])
def test_seq_path_matches_per_row(need_gpu, cfg):
    """The sequence entry point returns the per-row entry point's bits
    (indices and scores) on every row, and passes the oracle rule."""
    st = state(cfg)
    say(f"[indexer seq] {cfg} R={st.R}")
    a_idx, a_sc = st.indexer()
    b_idx, b_sc = _seq_topk(st)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx)
    assert torch.equal(a_sc, b_sc)
    o = Oracle(st.inp)
    rows = list(range(st.R)) if st.R <= 64 else _rows_for(cfg, st.R)
    b_idx, b_sc = b_idx.cpu().numpy(), b_sc.cpu().numpy()
    for r in (rows if st.R <= 64 else rows[:4]):   # bit-equality above covers every row
        check_topk_row(b_idx[r], b_sc[r], o.topk(r), st.topk, int(st.inp["row_pos"][r]))
    o.drop_cache()


def test_seq_path_ragged_rows(need_gpu):
    """Partial last tile, rows with t < 0, rows out of order, short rows and a
    row past the cache: bit-equal to the per-row path."""
    st = state("tiny_prefill")
    say("[indexer seq] ragged rows")
    rng = np.random.default_rng(11)
    R = 37
    pos = rng.integers(-1, 512, size=R).astype(np.int32)
    pos[0], pos[1], pos[2], pos[5] = -1, 511, 0, 2000
    rp = torch.from_numpy(pos).cuda()
    q, qs, w = st.q_fp8[:R].contiguous(), st.q_e8m0[:R].contiguous(), st.w[:R].contiguous()
    rs = torch.zeros(R, dtype=torch.int32, device="cuda")
    for K in (st.topk, 1, 700):
        a_idx, a_sc = ops.dsa_indexer_topk(q, qs, w, st.k_pool, st.block_table, rs, rp, K)
        b_idx, b_sc = _seq_topk(st, q, qs, w, rp, K)
        torch.cuda.synchronize()
        assert torch.equal(a_idx, b_idx), f"K={K}"
        assert torch.equal(a_sc, b_sc), f"K={K}"


def test_seq_path_exact_fallback(need_gpu):
    """The rescoring path of the selection (a unit holding far more than its
    quota) through the sequence entry point: same bits as the per-row path,
    status bit 3 set."""
    say("[indexer seq] concentrated Top-K (rescore path)")
    inp = dict(synth.make("decode_8k_needles", with_sfa=False))
    inp["w"] = np.abs(inp["w"])
    k = inp["k_idx"].copy()
    k[3000:5100] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(k[3000:5100]) * np.float32(8))
    inp["k_idx"] = k
    st = DeviceState(inp, with_sfa=False)
    a_idx, a_sc = st.indexer()
    ws = ops.indexer_seq_workspace(st.R, st.block_table.shape[1], st.H_I, st.topk)
    b_idx, b_sc = _seq_topk(st, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)
    assert (int(ws.view(torch.int32)[2].item()) & 8) != 0


def _mq_topk(st, q_per_seq, topk=None, row_pos=None, workspace=None):
    return ops.dsa_indexer_topk_mq(st.q_fp8, st.q_e8m0, st.w, st.k_pool, st.block_table, st.row_seq,
                                   st.row_pos if row_pos is None else row_pos, q_per_seq,
                                   st.topk if topk is None else topk, workspace=workspace)


def test_multi_query_decode_parity(need_gpu):
    """Multi-query decode at 128K (8 sequences x 4 query tokens): the
    multi-query entry point returns the per-row entry point's bits on every
    row, and sampled rows pass the oracle rule."""
    st = state("decode_mtp4_128k_b8")
    say(f"[indexer mq] decode_mtp4_128k_b8 R={st.R}")
    ws = ops.indexer_workspace(st.R, st.block_table.shape[1], st.H_I, st.topk)
    a_idx, a_sc = st.indexer()
    b_idx, b_sc = _mq_topk(st, 4, workspace=ws)
    c_idx, c_sc = _mq_topk(st, 4, workspace=ws)   # workspace reuse
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)
    assert torch.equal(b_idx, c_idx) and torch.equal(b_sc, c_sc)
    assert int(ws.view(torch.int32)[2].item()) & 4 == 0
    o = Oracle(st.inp)
    b_idx, b_sc = b_idx.cpu().numpy(), b_sc.cpu().numpy()
    for r in (0, 3, 13, 31):
        check_topk_row(b_idx[r], b_sc[r], o.topk(r), st.topk, int(st.inp["row_pos"][r]))
    o.drop_cache()


@pytest.mark.parametrize("q_per_seq,h_index", [(1, 64), (3, 64), (5, 64), (7, 20), (8, 64), (2, 20)])
def test_multi_query_ragged(need_gpu, q_per_seq, h_index):
    """Ragged histories, rows of a group with different limits (short ones,
    t < 0, t beyond the group's longest), several Top-K sizes, a head count
    that is not a multiple of 16: bit-equal to the per-row entry point, and
    the oracle rule on every row."""
    B = 5
    cfg = synth.Config(92, "mq_ragged", batch=B, h_index=h_index, h_attn=16, topk=2048,
                       ragged=(100, 9000), q_per_seq=q_per_seq)
    inp = synth.make(cfg, with_sfa=False)
    rng = np.random.default_rng(q_per_seq)
    pos = inp["row_pos"].copy()
    lens = inp["seq_lens"]
    for r in range(len(pos)):
        b = r // q_per_seq
        pos[r] = rng.integers(-1, int(lens[b]))
    pos[0] = -1
    pos[-1] = int(lens[B - 1]) - 1
    inp["row_pos"] = pos.astype(np.int32)
    st = DeviceState(inp, with_sfa=False)
    say(f"[indexer mq] ragged q_per_seq={q_per_seq} R={st.R}")
    o = Oracle(inp)
    for K in (2048, 1, 300):
        a_idx, a_sc = st.indexer(topk=K)
        b_idx, b_sc = _mq_topk(st, q_per_seq, topk=K)
        torch.cuda.synchronize()
        assert torch.equal(a_idx, b_idx), f"K={K}"
        assert torch.equal(a_sc, b_sc), f"K={K}"
        b_idx, b_sc = b_idx.cpu().numpy(), b_sc.cpu().numpy()
        for r in range(st.R):
            t = int(pos[r])
            if t < 0:
                assert np.all(b_idx[r] == -1)
                continue
            check_topk_row(b_idx[r], b_sc[r], o.topk(r, K), K, t)
    o.drop_cache()


def test_multi_query_mixed_group_flagged(need_gpu):
    """A group whose rows name different sequences sets status bit 4."""
    st = state("decode_ragged_b32")
    say("[indexer mq] mixed group flag")
    ws = ops.indexer_workspace(st.R, st.block_table.shape[1], st.H_I, st.topk)
    _mq_topk(st, 2, workspace=ws)   # rows 2b, 2b+1 belong to different sequences
    torch.cuda.synchronize()
    assert int(ws.view(torch.int32)[2].item()) & 16 != 0


def test_select_layouts(need_gpu):
    """Rows whose units keep many candidates (short histories relative to
    K) take the select's wider register layouts (up to 1024 candidates in
    a unit, two waves per unit): the oracle rule and bit-exact equality with
    the exact Top-K of the kernel's own scores, for several K."""
    say("[indexer] select layouts")
    lens = np.array([2100, 3000, 4100, 5000, 9000, 17000, 26000, 40000, 65600, 70000],
                    dtype=np.int32)
    cfg = synth.Config(93, "layouts", batch=len(lens), h_index=64, h_attn=16, topk=2048,
                       ragged=(int(lens.min()), int(lens.max())))
    rng = np.random.default_rng(5)
    bt, slots, starts, npages = synth.page_tables(cfg, lens, rng)
    R = len(lens)
    inp = dict(seq_lens=lens, block_table=bt, slot_mapping=slots, seq_starts=starts,
               total_pages=np.int64(npages), topk=np.int32(2048),
               row_seq=np.arange(R, dtype=np.int32), row_pos=(lens - 1).astype(np.int32),
               q_idx=synth.f32_to_bf16_bits(rng.standard_normal((R, 64, 128)).astype(np.float32)),
               k_idx=synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 128)).astype(np.float32)),
               w=(rng.standard_normal((R, 64)) / 8).astype(np.float32))
    st = DeviceState(inp, with_sfa=False)
    o = Oracle(inp)
    scores = st.scores().cpu().numpy()
    for K in (2048, 1024, 300):
        ws = ops.indexer_workspace(R, st.block_table.shape[1], st.H_I, K)
        idx, sc = st.indexer(topk=K, workspace=ws)
        idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
        for r in range(R):
            t = int(inp["row_pos"][r])
            check_topk_row(idx[r], sc[r], o.topk(r, K), K, t)
            assert np.array_equal(idx[r][:min(K, t + 1)], exact_topk_of(scores[r], K)), f"row {r} K={K}"
        assert int(ws.view(torch.int32)[2].item()) & 4 == 0
    o.drop_cache()


def test_long_context_rows(need_gpu):
    """Rows past the select's fast layouts (more than 128 units of 1024
    keys): a 1M-token row at the block table's maximum width (16384 pages),
    a 256K row and a 200001-token row.  Against the oracle, and bit-exact
    against the exact Top-K of the kernel's own scores."""
    say("[indexer] long rows: 1048576, 262144, 200001 tokens")
    lens = np.array([1048576, 262144, 200001], dtype=np.int32)
    cfg = synth.Config(94, "long", batch=len(lens), h_index=64, h_attn=16, topk=2048,
                       ragged=(int(lens.min()), int(lens.max())))
    rng = np.random.default_rng(7)
    bt, slots, starts, npages = synth.page_tables(cfg, lens, rng)
    assert bt.shape[1] == 16384
    R = len(lens)
    inp = dict(seq_lens=lens, block_table=bt, slot_mapping=slots, seq_starts=starts,
               total_pages=np.int64(npages), topk=np.int32(2048),
               row_seq=np.arange(R, dtype=np.int32), row_pos=(lens - 1).astype(np.int32),
               q_idx=synth.f32_to_bf16_bits(rng.standard_normal((R, 64, 128)).astype(np.float32)),
               k_idx=synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 128)).astype(np.float32)),
               w=(rng.standard_normal((R, 64)) / 8).astype(np.float32))
    st = DeviceState(inp, with_sfa=False)
    o = Oracle(inp)
    scores = st.scores().cpu().numpy()
    for K in (2048, 300):
        ws = ops.indexer_workspace(R, st.block_table.shape[1], st.H_I, K)
        idx, sc = st.indexer(topk=K, workspace=ws)
        idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
        for r in range(R):
            t = int(inp["row_pos"][r])
            assert np.array_equal(idx[r][:min(K, t + 1)], exact_topk_of(scores[r], K)), f"row {r} K={K}"
            ora = o.topk(r, K)
            gs = scores[r, :t + 1]
            assert np.all(np.abs(gs.astype(np.float64) - ora["scores"]) <= 1e-4 * ora["maxabs"]), f"row {r}"
            check_topk_row(idx[r], sc[r], ora, K, t)
        assert int(ws.view(torch.int32)[2].item()) & 4 == 0
        say(f"[indexer] long rows K={K} ok")
    o.drop_cache()


@pytest.mark.parametrize("q_per_seq", [3, 4])
def test_multi_query_more_rows_than_one_launch(need_gpu, q_per_seq):
    """Several hundred sequences of a few query tokens (histories of 4..300
    tokens, Top-K 64) take two launches of whole sequences of at most 1024
    rows (1023 rows for three tokens per sequence); every launch offsets its
    rows' inputs and outputs: bit-equal to the per-row entry point and the
    oracle rule on rows of both launches."""
    B = 1200 // q_per_seq
    cfg = synth.Config(98, "mq_many", batch=B, h_index=64, h_attn=16, topk=64, ragged=(4, 300),
                       q_per_seq=q_per_seq)
    inp = synth.make(cfg, with_sfa=False)
    st = DeviceState(inp, with_sfa=False)
    say(f"[indexer mq] {st.R} rows, q_per_seq={q_per_seq}")
    a_idx, a_sc = st.indexer()
    b_idx, b_sc = _mq_topk(st, q_per_seq)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)
    o = Oracle(inp)
    gi, gs = b_idx.cpu().numpy(), b_sc.cpu().numpy()
    # rows on both sides of the launch boundary; rows of fewer than 16
    # positions are left to the bit-equality above (their scores' error is
    # bounded by the sum of |q_i k_i|, not by their largest score)
    pos = inp["row_pos"]
    near = [r for r in range(1012, 1036) if pos[r] + 1 >= 16]
    for r in [0, st.R - 1] + near:
        check_topk_row(gi[r], gs[r], o.topk(r), st.topk, int(pos[r]))
