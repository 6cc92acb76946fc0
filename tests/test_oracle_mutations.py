"""The pins must catch plausible mistakes in the oracle.

Each case swaps one oracle function for a subtly wrong variant (a dropped
term, a wrong rounding or tie rule, a wrong constant) and checks that at least
one of the pin tests then fails.  Mistakes are planted in the oracle only, on
the CPU."""
import math

import numpy as np
import pytest

import oracle.attention as attention
import oracle.formats as formats
import oracle.indexer as indexer
import oracle.quant as quant

from tests import test_oracle_attention as TA
from tests import test_oracle_formats as TF
from tests import test_oracle_indexer as TI
from tests import test_oracle_pipeline as TP
from oracle.pipeline import Oracle
from tests import test_oracle_quant as TQ


def _encode_ties_away(y):
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, ex = np.frexp(a)
    binade = np.where(a > 0, ex - 1, -6)
    step = np.ldexp(1.0, np.maximum(binade, -6) - 3)
    r = np.minimum(np.floor(a / step + 0.5) * step, 448.0)
    return np.searchsorted(formats.E4M3_POS, r).astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 7)


def _encode_truncate(y):
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, ex = np.frexp(a)
    binade = np.where(a > 0, ex - 1, -6)
    step = np.ldexp(1.0, np.maximum(binade, -6) - 3)
    r = np.minimum(np.floor(a / step) * step, 448.0)
    return np.searchsorted(formats.E4M3_POS, r).astype(np.uint8) | (np.signbit(y).astype(np.uint8) << 7)


def _mx_scale_ocp_floor(amax):
    # floor(log2 amax) - 8: clips elements in (448X, 512X)
    amax = np.asarray(amax, dtype=np.float64)
    safe = np.where(amax > 0, amax, 1.0)
    e = np.floor(np.log2(safe)).astype(np.int64) - 8
    return np.where(amax > 0, np.clip(e, -127, 127), 0)


def _kv_scales_f64(latent_bits):
    x = formats.bf16_decode(latent_bits).reshape(-1, 4, 128)
    amax = np.abs(x).max(axis=2)
    return np.where(amax == 0, 1.0, amax / 448.0).astype(np.float32) * np.float32(1 + 2 ** -20)


def _scores_no_relu(q, k, w, t):
    return np.asarray(w, dtype=np.float64) @ (q @ k[:t + 1].T) + 0.0


def _scores_relu_after_sum(q, k, w, t):
    return np.maximum(np.asarray(w, dtype=np.float64) @ (q @ k[:t + 1].T), 0.0) + 0.0


def _scores_exclusive(q, k, w, t):
    return _orig["indexer_scores"](q, k, w, t - 1) if t > 0 else np.zeros(0)


def _topk_order_high_index(I):
    s = np.arange(len(I))
    return np.lexsort((-s, -np.asarray(I, dtype=np.float64)))


def _sfa_scale_512(q, lat, rope, idx, scale=attention.DEFAULT_SCALE):
    return _orig["sparse_attn"](q, lat, rope, idx, 1 / math.sqrt(512))


def _sfa_no_rope(q, lat, rope, idx, scale=attention.DEFAULT_SCALE):
    return _orig["sparse_attn"](q, lat, np.zeros_like(rope), idx, scale)


def _sfa_dedup(q, lat, rope, idx, scale=attention.DEFAULT_SCALE):
    idx = np.asarray(idx)
    return _orig["sparse_attn"](q, lat, rope, np.unique(idx[idx >= 0]), scale)


def _k_index_no_offset(self, b):
    # the sequence's keys taken from token 0 instead of its own start
    L = int(self.inp["seq_lens"][b])
    codes, e8 = quant.mxfp8_quant(self.inp["k_idx"][:L])
    return quant.mxfp8_dequant(codes, e8)


def _kv_rows_no_offset(self, b, positions):
    rec = quant.kv_quant(self.inp["kv"][np.asarray(positions, dtype=np.int64)])
    return quant.kv_dequant(rec)


_orig = dict(indexer_scores=indexer.indexer_scores, sparse_attn=attention.sparse_attn)

CASES = [
    ("e4m3 ties away from zero", formats, "e4m3_encode", _encode_ties_away,
     [TF.test_e4m3_golden, TF.test_e4m3_encode_matches_exhaustive_search]),
    ("e4m3 truncation", formats, "e4m3_encode", _encode_truncate,
     [TF.test_e4m3_golden, TF.test_e4m3_roundtrip_and_half_ulp]),
    ("MX scale OCP floor rule", quant, "mx_scale_exponent", _mx_scale_ocp_floor,
     [TQ.test_mx_golden_examples, TQ.test_mx_scale_rule_and_error_bound]),
    ("KV scale not the f32 quotient", quant, "kv_tile_scales", _kv_scales_f64,
     [TQ.test_kv_golden_examples, TQ.test_kv_error_bound_and_saturation_free_max]),
    ("indexer without ReLU", indexer, "indexer_scores", _scores_no_relu,
     [TI.test_hand_example, TI.test_scores_match_explicit_loops]),
    ("ReLU after the head sum", indexer, "indexer_scores", _scores_relu_after_sum,
     [TI.test_hand_example, TI.test_scores_match_explicit_loops]),
    ("exclusive causal bound", indexer, "indexer_scores", _scores_exclusive,
     [TI.test_hand_example, TI.test_scores_match_explicit_loops]),
    ("ties to the higher index", indexer, "topk_order", _topk_order_high_index,
     [TI.test_tie_rule_lower_index_wins, TI.test_topk_matches_full_sort_with_ties]),
    ("softmax scale 1/sqrt(512)", attention, "sparse_attn", _sfa_scale_512,
     [TA.test_all_positions_equal_torch_sdpa, TA.test_single_index_returns_latent_row]),
    ("rope dropped from the logits", attention, "sparse_attn", _sfa_no_rope,
     [TA.test_all_positions_equal_torch_sdpa, TA.test_single_index_returns_latent_row]),
    ("duplicates collapsed", attention, "sparse_attn", _sfa_dedup,
     [TA.test_duplicates_count_and_empty_list]),
    ("indexer keys without the sequence offset", Oracle, "k_index", _k_index_no_offset,
     [TP.test_scores_of_every_sequence_through_the_k_pool]),
    ("KV rows without the sequence offset", Oracle, "kv_rows", _kv_rows_no_offset,
     [TP.test_attention_of_every_sequence_through_the_kv_pool]),
]


@pytest.mark.parametrize("name,mod,attr,bad,checks", CASES, ids=[c[0] for c in CASES])
def test_pins_catch_planted_mistake(monkeypatch, name, mod, attr, bad, checks):
    monkeypatch.setattr(mod, attr, bad)
    failed = 0
    for chk in checks:
        args = [0] if "seed" in chk.__code__.co_varnames[:chk.__code__.co_argcount] else []
        try:
            chk(*args)
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, f"no pin caught: {name}"
