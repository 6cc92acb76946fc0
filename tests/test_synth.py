"""Host-side checks of the seeded workload generator: shapes, query rows,
page tables and slot mappings of every workload (no method arithmetic)."""
import numpy as np
import pytest

from sparse_attention_decode_topk_amd import synth


@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_rows_and_pages(name):
    cfg = synth.config(name)
    lens = synth.lengths(cfg)
    assert len(lens) == cfg.batch
    if cfg.ragged is None:
        assert np.all(lens == cfg.ctx)
    else:
        assert lens.min() >= cfg.ragged[0] and lens.max() <= cfg.ragged[1]
    row_seq, row_pos = synth.rows_of(cfg, lens)
    assert row_seq.dtype == np.int32 and row_pos.dtype == np.int32
    assert np.all(row_pos < lens[row_seq])
    if cfg.rows == "last":
        q = cfg.q_per_seq
        assert len(row_seq) == cfg.batch * q
        # q consecutive rows per sequence, the sequence's last q positions in order
        assert np.array_equal(row_seq, np.repeat(np.arange(cfg.batch), q))
        assert np.array_equal(row_pos.reshape(cfg.batch, q),
                              lens[:, None] - q + np.arange(q)[None, :])
    bt, slots, starts, total = synth.page_tables(cfg, lens)
    npg = (lens.astype(np.int64) + synth.PAGE - 1) // synth.PAGE
    assert total == int(npg.sum())
    used = np.concatenate([bt[b, :npg[b]] for b in range(cfg.batch)])
    assert np.array_equal(np.sort(used), np.arange(total))          # every page exactly once
    if cfg.identity_pages:
        assert np.array_equal(used, np.arange(total))
    for b in range(cfg.batch):
        s = np.arange(int(lens[b]))
        seg = slots[starts[b]:starts[b] + lens[b]]
        assert np.array_equal(seg, bt[b, s // synth.PAGE].astype(np.int64) * synth.PAGE + s % synth.PAGE)


def test_multi_query_workload_matches_the_decode_batch():
    """The multi-query decode batch has the headline batch's sequences and
    sizes, with four query rows per sequence."""
    a, b = synth.config("decode_128k_b8"), synth.config("decode_mtp4_128k_b8")
    assert (a.batch, a.ctx, a.h_index, a.h_attn, a.topk) == (b.batch, b.ctx, b.h_index, b.h_attn, b.topk)
    assert b.q_per_seq == 4 and a.q_per_seq == 1


def test_draws_are_seeded_and_independent():
    """Same config -> same bits; the streams of a config do not depend on
    which tensors are drawn."""
    x = synth.make("decode_8k_needles", with_sfa=False)
    y = synth.make("decode_8k_needles", with_sfa=True)
    assert np.array_equal(x["q_idx"], y["q_idx"]) and np.array_equal(x["k_idx"], y["k_idx"])
    assert np.array_equal(x["needles"], y["needles"])
    z = synth.make("decode_8k_needles", with_sfa=False)
    assert np.array_equal(x["w"], z["w"])
