"""Pins of the oracle's indexer scores and Top-K selection: explicit-loop
brute force, the single-head special case, the x4 needle invariant, a full
sort, the short-history boundary, exact ties, and page placement."""
import numpy as np
import pytest

from oracle import formats, indexer, pools, quant
from oracle.pipeline import Oracle
from sparse_attention_decode_topk_amd import synth


def _mx(xb):
    c, e = quant.mxfp8_quant(xb)
    return quant.mxfp8_dequant(c, e)


def test_scores_match_explicit_loops():
    rng = np.random.default_rng(0)
    H, L = 4, 40
    q = _mx(synth.f32_to_bf16_bits(rng.standard_normal((H, 128)).astype(np.float32)))
    k = _mx(synth.f32_to_bf16_bits(rng.standard_normal((L, 128)).astype(np.float32)))
    w = rng.standard_normal(H) / 2
    for t in (0, 17, L - 1):
        fast = indexer.indexer_scores(q, k, w, t)
        slow = indexer.indexer_scores_loops(q.tolist(), k.tolist(), w.tolist(), t)
        assert fast.shape == (t + 1,)
        np.testing.assert_allclose(fast, slow, rtol=1e-12, atol=1e-12)


def test_hand_example():
    # two heads, keys along unit directions (all values exact in MXFP8):
    # q0 = e0, q1 = e0 + e1 ; w = [0.5, -1]
    # k0 = 2 e0      -> l = (2, 2)  -> I = 0.5*2 - 1*2 = -1
    # k1 = -e0 + e1  -> l = (-1, 0) -> I = 0
    # k2 = 3 e1      -> l = (0, 3)  -> I = -3
    # k3 = e0        -> l = (1, 1)  -> I = -0.5
    q = np.zeros((2, 128)); q[0, 0] = 1; q[1, 0] = 1; q[1, 1] = 1
    k = np.zeros((4, 128)); k[0, 0] = 2; k[1, 0] = -1; k[1, 1] = 1; k[2, 1] = 3; k[3, 0] = 1
    w = np.array([0.5, -1.0])
    qb = synth.f32_to_bf16_bits(q.astype(np.float32))
    kb = synth.f32_to_bf16_bits(k.astype(np.float32))
    I = indexer.indexer_scores(_mx(qb), _mx(kb), w, 3)
    assert I.tolist() == [-1.0, 0.0, -3.0, -0.5]
    idx, sc = indexer.topk_select(I, 2)
    assert idx.tolist() == [1, 3] and sc.tolist() == [0.0, -0.5]
    idx, sc = indexer.topk_select(I, 6)
    assert idx.tolist() == [0, 1, 2, 3, -1, -1]
    assert sc[4] == -np.inf


def test_single_head_reduces_to_relu_dot():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 128)); k = rng.standard_normal((50, 128))
    I = indexer.indexer_scores(q, k, np.ones(1), 49)
    np.testing.assert_allclose(I, np.maximum(k @ q[0], 0), rtol=1e-13, atol=1e-13)


def test_negative_zero_canonicalised():
    # all logits negative with a negative weight give -0.0 * ... ; score must be +0
    q = np.zeros((1, 128)); q[0, 0] = 1
    k = np.zeros((3, 128)); k[:, 0] = -1
    I = indexer.indexer_scores(q, k, np.array([-1.0]), 2)
    assert np.all(np.signbit(I) == False)  # noqa: E712


def test_needle_x4_is_exact():
    inp = synth.make("decode_8k_needles", with_sfa=False)
    o = Oracle(inp)
    I = o.scores(0)
    # rebuild the same inputs without the x4 and compare at the needles
    base_k = inp["k_idx"].copy()
    nd = inp["needles"]
    base_k[nd] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(base_k[nd]) / np.float32(4))
    o2 = Oracle(dict(inp, k_idx=base_k))
    I2 = o2.scores(0)
    assert np.array_equal(I[nd], 4 * I2[nd])
    mask = np.ones(len(I), bool); mask[nd] = False
    assert np.array_equal(I[mask], I2[mask])
    # quantised bytes identical, scales +2
    c1, e1 = quant.mxfp8_quant(inp["k_idx"][nd]); c2, e2 = quant.mxfp8_quant(base_k[nd])
    assert np.array_equal(c1, c2) and np.array_equal(e1.astype(int), e2.astype(int) + 2)


def _full_sort_topk(I, K):
    order = sorted(range(len(I)), key=lambda s: (-I[s], s))
    return sorted(order[:K])


@pytest.mark.parametrize("seed", range(4))
def test_topk_matches_full_sort_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = 3000
    I = np.round(rng.standard_normal(n) * 3)          # many exact ties
    I[rng.random(n) < 0.3] = 0.0
    I[rng.random(n) < 0.05] = -0.0
    I = I + 0.0
    for K in (1, 64, 700, 2048, 2999, 3000, 5000):
        idx, sc = indexer.topk_select(I, K)
        exp = _full_sort_topk(I.tolist(), K)
        got = idx[idx >= 0].tolist()
        assert got == exp
        assert np.all(idx[len(exp):] == -1)
        assert np.array_equal(sc[:len(exp)], I[exp])


def test_tie_rule_lower_index_wins():
    I = np.array([5.0, 1.0, 3.0, 3.0, 3.0, 0.0, 3.0])
    idx, _ = indexer.topk_select(I, 3)
    assert idx.tolist() == [0, 2, 3]
    assert indexer.kth_score(I, 3) == 3.0


def test_short_history_returns_all_positions():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 128)); k = rng.standard_normal((64, 128))
    for t in (0, 5, 63):
        I = indexer.indexer_scores(q, k, rng.standard_normal(4), t)
        idx, _ = indexer.topk_select(I, 64)
        assert idx[:t + 1].tolist() == list(range(t + 1))
        assert np.all(idx[t + 1:] == -1)


def test_page_placement_does_not_change_scores():
    # same tokens written under two different page permutations and read
    # back through the block table give identical scores
    rng = np.random.default_rng(9)
    cfg = synth.Config(98, "t", batch=2, h_index=4, h_attn=8, topk=32, ragged=(100, 300))
    lens = np.array([300, 190], dtype=np.int32)
    bt, slots, starts, npages = synth.page_tables(cfg, lens, rng)
    bt2 = synth.rotate_pages(bt, lens, npages, seed=5)
    kb = synth.f32_to_bf16_bits(rng.standard_normal((int(lens.sum()), 128)).astype(np.float32))
    codes, e8 = quant.mxfp8_quant(kb)
    slots2 = np.concatenate([bt2[b, np.arange(lens[b]) // 64].astype(np.int64) * 64
                             + np.arange(lens[b]) % 64 for b in range(2)])
    p1 = pools.k_pool_write(codes, e8, slots, npages)
    p2 = pools.k_pool_write(codes, e8, slots2, npages)
    assert not np.array_equal(p1, p2)
    q = rng.standard_normal((4, 128)); w = rng.standard_normal(4)
    for b in range(2):
        c1, x1 = pools.k_pool_read(p1, bt[b], int(lens[b]))
        c2, x2 = pools.k_pool_read(p2, bt2[b], int(lens[b]))
        k1 = quant.mxfp8_dequant(c1, x1); k2 = quant.mxfp8_dequant(c2, x2)
        t = int(lens[b]) - 1
        assert np.array_equal(indexer.indexer_scores(q, k1, w, t),
                              indexer.indexer_scores(q, k2, w, t))


def test_tiny_prefill_has_exact_zero_ties():
    # the tiny prefill workload (H_I = 4, K = 64) has many rows whose K-th
    # score is an exact 0 shared by several positions: the tie rule matters
    inp = synth.make("tiny_prefill", with_sfa=False)
    o = Oracle(inp)
    n_tie_rows = 0
    for r in range(64, 512, 7):
        res = o.topk(r)
        I = res["scores"]
        if res["kth"] == 0.0 and np.sum(I == 0.0) > 1:
            n_tie_rows += 1
            sel = res["idx"]
            zeros_sel = [s for s in sel if s >= 0 and I[s] == 0.0]
            zeros_all = np.flatnonzero(I == 0.0)
            assert zeros_sel == zeros_all[:len(zeros_sel)].tolist()
    assert n_tie_rows > 0
