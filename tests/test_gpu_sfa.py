"""GPU parity of Sparse Flash Attention against the oracle.

The position lists come from the oracle (its own Top-K) or are constructed
in the test; both sides read the same quantised cache bytes, each quantising
from the same bf16 inputs.  Bar: max abs error <= 1e-3 * max|oracle out|
over the config's output; lse within 1e-3 absolute (it is a log)."""
import functools

import numpy as np
import pytest
import torch

from oracle.pipeline import Oracle
from sparse_attention_decode_topk_amd import ops, synth
from tests.dsa_state import DeviceState, check_topk_row, say

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def state(cfg):
    say(f"[state] building {cfg}")
    return DeviceState(synth.make(cfg))


def _compare(st, o, idx_np, rows, tag):
    out, lse = st.sfa(torch.from_numpy(idx_np).cuda())
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    ref_o, ref_l = [], []
    for r in rows:
        ro, rl = o.sfa(r, idx_np[r])
        ref_o.append(ro); ref_l.append(rl)
    ref_o = np.stack(ref_o); ref_l = np.stack(ref_l)
    got_o = out[rows]; got_l = lse[rows]
    H = st.inp["q_sfa"].shape[1]
    err = np.abs(got_o - ref_o).max()
    bar = 1e-3 * np.abs(ref_o).max()
    say(f"[sfa] {tag}: max err {err:.3g} vs bar {bar:.3g} (ratio {err / bar:.3f})")
    assert err <= bar
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(got_l), fin)
    assert np.all(np.abs(got_l[fin] - ref_l[fin]) <= 1e-3)
    return out, lse


@pytest.mark.parametrize("cfg", ["tiny_prefill", "decode_8k_needles", "decode_128k_b8"])
def test_sfa_on_oracle_topk(need_gpu, cfg):
    st = state(cfg)
    o = Oracle(st.inp)
    R = st.R
    rows = list(range(R)) if R <= 64 else sorted(set(range(0, R, max(1, R // 48))) | {R - 1})
    idx = np.full((R, st.topk), -1, dtype=np.int32)
    for r in (range(R) if R <= 64 else rows):
        idx[r] = o.topk(r)["idx"]
    o.drop_cache()
    _compare(st, o, idx, rows, cfg)


def test_sfa_all_positions_is_dense(need_gpu):
    """When the history is no longer than K, SFA over every position equals
    dense attention (tiny prefill rows t < 64 select everything)."""
    st = state("tiny_prefill")
    o = Oracle(st.inp)
    R = st.R
    idx = np.full((R, st.topk), -1, dtype=np.int32)
    for r in range(64):
        idx[r, :r + 1] = np.arange(r + 1)[::-1]   # any order
    _compare(st, o, idx, list(range(64)), "dense prefix")


def test_sfa_special_lists(need_gpu):
    """-1 holes, duplicates, a single entry, and an empty row."""
    st = state("tiny_prefill")
    o = Oracle(st.inp)
    R, K = st.R, st.topk
    rng = np.random.default_rng(4)
    idx = np.full((R, K), -1, dtype=np.int32)
    rows = [100, 200, 300, 400, 511]
    idx[100, ::3] = rng.integers(0, 101, size=len(idx[100, ::3]))        # holes + duplicates
    idx[200, 5] = 17                                                       # single entry
    idx[300] = 42                                                          # one position 64 times
    idx[511] = rng.permutation(512)[:K]
    # row 400 stays empty -> out 0, lse -inf
    out, lse = _compare(st, o, idx, rows, "special lists")
    assert np.all(out[400] == 0) and np.all(np.isneginf(lse[400]))


def test_sfa_deterministic(need_gpu):
    st = state("tiny_prefill")
    o = Oracle(st.inp)
    idx = np.stack([o.topk(r)["idx"] for r in range(st.R)])
    t = torch.from_numpy(idx).cuda()
    a = st.sfa(t)
    b = st.sfa(t)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("cfg", ["decode_8k_needles", "decode_ragged_b32", "decode_128k_b8"])
def test_end_to_end_decode(need_gpu, cfg):
    """GPU indexer -> GPU SFA on every row: the selection follows the Top-K
    pass rule, and the attention over the GPU's own indices (which may
    differ from the oracle's by tolerated near-tie swaps) matches the
    oracle's attention over those same indices."""
    st = state(cfg)
    o = Oracle(st.inp)
    idx, sc = st.indexer()
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    swaps = 0
    for r in range(st.R):
        swaps += check_topk_row(gi[r], gs[r], o.topk(r), st.topk, int(st.inp["row_pos"][r]))
    say(f"[e2e] {cfg}: {st.R} rows pass the Top-K rule ({swaps} tolerated swaps)")
    _compare(st, o, gi, list(range(st.R)), f"end to end {cfg}")
    o.drop_cache()


def test_sfa_split_path_with_holes(need_gpu):
    """One row of 128 heads runs as 8 splits of 256 entries combined by the
    second launch.  The list has -1 holes, a run of one duplicated position,
    one split that is entirely empty, and a ragged tail."""
    st = state("decode_8k_needles")
    o = Oracle(st.inp)
    K = st.topk
    idx = o.topk(0)["idx"].copy()
    idx[::5] = -1
    idx[256:512] = -1               # split 1 has no entry at all
    idx[600:650] = idx[701]         # one position listed 50 times
    idx[K - 37:] = -1               # ragged tail of the last split
    out, lse = _compare(st, o, idx[None, :], [0], "split path with holes")
    assert np.all(np.isfinite(out[0]))


def test_sfa_ragged_batch(need_gpu):
    """32 sequences of 4K-64K tokens, 128 heads: two splits per row and the
    combine launch.  Every row's list is 2048 distinct seeded positions of
    its own history (fewer for short rows), with -1 holes."""
    st = state("decode_ragged_b32")
    o = Oracle(st.inp)
    rng = np.random.default_rng(21)
    idx = np.full((st.R, st.topk), -1, dtype=np.int32)
    for r in range(st.R):
        t = int(st.inp["row_pos"][r])
        n = min(st.topk, t + 1)
        idx[r, :n] = rng.choice(t + 1, n, replace=False)
    idx[:, ::9] = -1
    _compare(st, o, idx, list(range(st.R)), "ragged batch")
    o.drop_cache()


def test_sfa_prefill_chunk_every_64th_row(need_gpu):
    """The chunked-prefill shape as bench.py launches it: 8192 query rows of
    128 heads against a 131072-token cache, one split per row (the direct
    output path, 32768 work-groups).  Every 64th row (and the last) carries
    the GPU indexer's own selection, checked against the Top-K rule and then
    through SFA against the oracle's attention over the same indices; the
    rows in between are emptied and must come out as zeros with lse -inf."""
    st = state("prefill_chunk_8k_of_128k")
    o = Oracle(st.inp)
    R = st.R
    rows = sorted(set(range(0, R, 64)) | {R - 1})
    gi, gs = _seq_topk_all(st)
    for r in rows:
        check_topk_row(gi[r], gs[r], o.topk(r), st.topk, int(st.inp["row_pos"][r]))
    say(f"[sfa] prefill chunk: {len(rows)} rows pass the Top-K rule")
    idx = np.full((R, st.topk), -1, dtype=np.int32)
    idx[rows] = gi[rows]
    out, lse = _compare(st, o, idx, rows, f"prefill chunk, {len(rows)} rows")
    empty = [r for r in (2, R // 3, R - 2) if r not in rows]
    assert np.all(out[empty] == 0) and np.all(np.isneginf(lse[empty]))
    o.drop_cache()


@pytest.mark.parametrize("W", [1024, 1100, 2048])
def test_sfa_unsplit_long_lists(need_gpu, W):
    """Lists of at least 1024 entries taken whole by one work-group (8192
    rows of 128 heads: no split; one wave group, two work-groups per CU,
    steps of 32 records).  Index lists of width W with -1 holes, lists of
    95 and 97 entries, a single entry in the last (partial) step, one
    position listed 200 times, and an empty row."""
    st = state("prefill_chunk_8k_of_128k")
    o = Oracle(st.inp)
    R = st.R
    rng = np.random.default_rng(57 + W)
    idx = np.full((R, W), -1, dtype=np.int32)
    t = lambda r: int(st.inp["row_pos"][r])
    idx[0] = rng.choice(t(0) + 1, W, replace=False)
    idx[0, ::5] = -1                                          # holes
    idx[1, :95] = rng.choice(t(1) + 1, 95, replace=False)     # one short of a step boundary
    idx[2, :97] = rng.choice(t(2) + 1, 97, replace=False)     # one past a step boundary
    idx[3, W - 1] = t(3)                                      # last step only
    idx[4] = rng.choice(t(4) + 1, W, replace=False)
    idx[4, 300:500] = idx[4, 77]                              # 200 duplicates
    idx[R - 1] = rng.choice(t(R - 1) + 1, W, replace=False)
    # row 5 stays empty -> out 0, lse -inf
    rows = [0, 1, 2, 3, 4, 5, R - 1]
    out, lse = _compare(st, o, idx, rows, f"unsplit lists of width {W}")
    assert np.all(out[5] == 0) and np.all(np.isneginf(lse[5]))


def test_sfa_unsplit_partial_head_group(need_gpu):
    """24 heads (one head group of 32 with 8 absent heads) over 256 rows of a
    2048-token sequence: one split per row of 1024 entries (the one-group
    form); lists with holes and a ragged last step."""
    cfg = synth.Config(95, "sfa_unsplit_h24", batch=1, h_index=4, h_attn=24, topk=1024, ctx=2048,
                       rows=(1536, 256))
    inp = synth.make(cfg)
    st = DeviceState(inp)
    o = Oracle(inp)
    rng = np.random.default_rng(71)
    R, K = st.R, st.topk
    idx = np.empty((R, K), dtype=np.int32)
    for r in range(R):
        idx[r] = rng.choice(int(inp["row_pos"][r]) + 1, K, replace=False)
    idx[:, ::7] = -1
    idx[R - 1, 1000:] = -1
    rows = [0, 1, 77, 128, 200, R - 1]
    _compare(st, o, idx, rows, "unsplit lists, 24 heads")


def _seq_topk_all(st):
    bt_row = st.block_table[int(st.inp["row_seq"][0])].contiguous()
    idx, sc = ops.dsa_indexer_topk_seq(st.q_fp8, st.q_e8m0, st.w, st.k_pool, bt_row, st.row_pos,
                                       st.topk)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy()


@pytest.mark.parametrize("K", [1, 100, 1000, 2047])
def test_sfa_list_lengths(need_gpu, K):
    """Index lists whose length is not a multiple of the 64-entry step (and
    for 1000 and 2047 not a whole number of splits either)."""
    st = state("decode_8k_needles")
    o = Oracle(st.inp)
    t = int(st.inp["row_pos"][0])
    rng = np.random.default_rng(31 + K)
    idx = rng.choice(t + 1, K, replace=False).astype(np.int32)[None, :]
    _compare(st, o, idx, [0], f"list of {K}")
