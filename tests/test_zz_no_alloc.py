"""The allocation-free indexer entry point (dsa_indexer_topk_noalloc, its
workspace a per-GPU array inside the library) against dsa_indexer_topk with
a caller workspace: bit-identical indices and scores on two calls in a row,
the second with a smaller input (fewer rows, a narrower block table), so the
second call runs on what the first left in the array."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_attention_decode_topk_amd import ops, synth
from tests.dsa_state import DeviceState, say

pytestmark = pytest.mark.gpu


def _noalloc_raw(st, K, rows=None):
    """Calls the C entry point directly through ctypes."""
    q, qs, w = st.q_fp8, st.q_e8m0, st.w
    rs, rp = st.row_seq, st.row_pos
    if rows is not None:
        q, qs, w = q[rows].contiguous(), qs[rows].contiguous(), w[rows].contiguous()
        rs, rp = rs[rows].contiguous(), rp[rows].contiguous()
    R, H = q.shape[0], q.shape[1]
    oi = torch.full((R, K), -7, dtype=torch.int32, device="cuda")
    osc = torch.full((R, K), 7.0, dtype=torch.float32, device="cuda")
    P = ctypes.c_void_p
    st_code = ops.lib().dsa_indexer_topk_noalloc(
        P(q.data_ptr()), P(qs.data_ptr()), P(w.data_ptr()), P(st.k_pool.data_ptr()),
        st.k_pool.shape[0], P(st.block_table.data_ptr()), st.block_table.shape[1],
        P(rs.data_ptr()), P(rp.data_ptr()), R, H, K, P(oi.data_ptr()), P(osc.data_ptr()),
        P(torch.cuda.current_stream().cuda_stream))
    assert st_code == 0, ops.STATUS.get(st_code, st_code)
    return oi, osc, (q, qs, w, rs, rp)


def _with_workspace(st, K, ops_args):
    q, qs, w, rs, rp = ops_args
    return ops.dsa_indexer_topk(q, qs, w, st.k_pool, st.block_table, rs, rp, K)


def test_noalloc_matches_workspace_entry_point(need_gpu):
    # first call: the ragged 32-sequence decode batch (block table of up to
    # 1024 pages); second call: the 8K single-row decode (128 pages) and a
    # subset of the ragged rows, each smaller than the first
    say("[noalloc] ragged decode batch, 32 rows")
    big = DeviceState(synth.make("decode_ragged_b32", with_sfa=False), with_sfa=False)
    K = big.topk
    a_idx, a_sc, args = _noalloc_raw(big, K)
    b_idx, b_sc = _with_workspace(big, K, args)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)
    assert int((a_idx >= 0).sum()) == big.R * K

    say("[noalloc] second call: 5 rows of the same batch, K = 700")
    rows = torch.tensor([3, 9, 17, 22, 30], device="cuda")
    a_idx, a_sc, args = _noalloc_raw(big, 700, rows)
    b_idx, b_sc = _with_workspace(big, 700, args)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)
    del big

    say("[noalloc] third call: decode 8K, one row")
    small = DeviceState(synth.make("decode_8k_needles", with_sfa=False), with_sfa=False)
    a_idx, a_sc, args = _noalloc_raw(small, small.topk)
    b_idx, b_sc = _with_workspace(small, small.topk, args)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)


def test_noalloc_rejects_launches_beyond_its_array(need_gpu):
    """A launch whose workspace would exceed the 64 MiB array returns
    DSA_ERR_WORKSPACE before any device work (8 rows of 16384 pages need
    8 * 16384 * 512 bytes of candidate slots)."""
    assert ops.lib().dsa_indexer_topk_workspace_size(8, 16384, 64, 2048) > (64 << 20)
    t = torch.zeros(16, dtype=torch.uint8, device="cuda")
    P = ctypes.c_void_p
    p = P(t.data_ptr())
    code = ops.lib().dsa_indexer_topk_noalloc(p, p, p, p, 10, p, 16384, p, p, 8, 64, 2048, p, None,
                                              P(torch.cuda.current_stream().cuda_stream))
    assert code == 3


def test_noalloc_more_rows_than_one_launch(need_gpu):
    """1100 rows (histories of 1..300 tokens, Top-K 64) take two launches of
    at most 1024 rows, both on the one array: bit-identical to the entry
    point with a caller workspace."""
    cfg = synth.Config(99, "noalloc_many_rows", batch=1100, h_index=64, h_attn=16, topk=64,
                       ragged=(1, 300))
    st = DeviceState(synth.make(cfg, with_sfa=False), with_sfa=False)
    say(f"[noalloc] {st.R} rows in two launches")
    a_idx, a_sc, args = _noalloc_raw(st, st.topk)
    b_idx, b_sc = _with_workspace(st, st.topk, args)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx) and torch.equal(a_sc, b_sc)
