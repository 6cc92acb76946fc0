"""The synthetic recall study of the MXFP8 indexer (oracle/recall.py).

Pins: on inputs that MXFP8 represents exactly (every value on the E4M3 grid,
every 32-group holding 448 so that its scale is 2^0) the quantised and the
unquantised indexers are the same function, so recall and mass recall are
exactly 1 and the score loss exactly 0 for every row and K; a position list shifted by one, a wrong row
or a dropped head would break that.  On the needle workload the study's
figures are checked against bounds taken from its measured values."""
import numpy as np
import pytest

from oracle import formats, indexer, recall
from sparse_attention_decode_topk_amd import synth


def _e4m3_grid_bf16(rng, shape):
    """bf16 bit patterns of E4M3 values, each 32-group containing +-448."""
    grid = formats.e4m3_decode(np.arange(256, dtype=np.uint8))
    grid = grid[np.isfinite(grid)]
    x = rng.choice(grid, size=shape).astype(np.float32)
    g = x.reshape(-1, 32)
    g[:, 0] = np.where(rng.random(len(g)) < 0.5, 448.0, -448.0)
    return synth.f32_to_bf16_bits(g.reshape(shape))


def _lossless_inputs(seed=5, L=700, H=8, R=5, K=64):
    rng = np.random.default_rng(seed)
    return dict(
        seq_lens=np.array([L], dtype=np.int64), seq_starts=np.array([0], dtype=np.int64),
        row_seq=np.zeros(R, dtype=np.int32),
        row_pos=np.array([0, 10, 63, 64, L - 1], dtype=np.int32)[:R],
        q_idx=_e4m3_grid_bf16(rng, (R, H, 128)), k_idx=_e4m3_grid_bf16(rng, (L, 128)),
        w=(rng.standard_normal((R, H)) / np.sqrt(H)).astype(np.float32),
        topk=np.int32(K))


def test_lossless_inputs_give_identical_scores():
    inp = _lossless_inputs()
    o = recall.Oracle(inp)
    for r in range(len(inp["row_seq"])):
        assert np.array_equal(o.scores(r), recall.reference_scores(inp, r))


@pytest.mark.parametrize("K", [1, 16, 64, 1000])
def test_lossless_recall_is_one(K):
    inp = _lossless_inputs()
    inp["topk"] = np.int32(K)
    s = recall.study(inp)
    assert s["recall_min"] == 1.0 and s["mass_recall_min"] == 1.0
    assert s["score_loss_max"] == 0.0


def test_row_recall_counts_overlap():
    I_ref = np.array([5.0, 4.0, 3.0, 2.0, 1.0])
    I_mx = np.array([5.0, 4.0, 1.0, 2.0, 3.0])     # positions 2 and 4 swap ranks
    r = recall.row_recall(I_mx, I_ref, 3, needles=np.array([0, 2]))
    assert r["recall"] == pytest.approx(2 / 3)
    assert r["mass_recall"] == pytest.approx((5 + 4 + 1) / (5 + 4 + 3))
    assert r["score_loss"] == pytest.approx(((5 + 4 + 3) - (5 + 4 + 1)) / 3 / np.sqrt(2.0))
    assert r["needles_ref"] == 2 and r["needle_recall"] == 0.5
    # K beyond the history keeps everything
    assert recall.row_recall(I_mx, I_ref, 99)["recall"] == 1.0


def test_score_loss_ignores_shift_and_scale():
    rng = np.random.default_rng(3)
    I_ref = rng.standard_normal(500)
    I_mx = I_ref + 0.3 * rng.standard_normal(500)
    a = recall.row_recall(I_mx, I_ref, 40)
    b = recall.row_recall(2.5 * I_mx - 7.0, 2.5 * I_ref - 7.0, 40)
    assert a["score_loss"] > 0.0
    assert b["score_loss"] == pytest.approx(a["score_loss"], rel=1e-12)
    assert b["recall"] == a["recall"]


def test_needle_workload_recall():
    inp = synth.make("decode_8k_needles", with_sfa=False)
    s = recall.study(inp)
    # measured: recall 0.982, mass recall 0.9995, every needle the reference
    # keeps is kept
    assert s["recall_min"] >= 0.97
    assert s["mass_recall_min"] >= 0.999
    assert s["needles_in_ref_topk"] > 0 and s["needle_recall_min"] == 1.0
